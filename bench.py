#!/usr/bin/env python3
"""Throughput of the causal linear-attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One step is one chunked forward of the gated delta rule over the workload
B=4, H=16, T=8192, d_k=d_v=128, bf16 q/k/v, fp32 gates and state, chunk 64
(``la_chunk_fwd``, a single kernel launch).  The decode half of the metric,
one recurrent step of the same rule over B=256 x H=16 heads of fp32 128x128
state (``la_decode_step``), is timed in the same run and reported under
"decode", and the chunked backward pass (``la_chunk_bwd``) of normalized
attention with a per-head decay and of retention at a training shape under
"backward".  Inputs are seeded synthetic data, resident in GPU memory before
timing starts.  Prints ONE JSON line.

Roofline figures use algorithmic counts: bytes the operator must move
(inputs read once, outputs and final state written once) and the matrix
flops of the chunked algorithm, divided by the average kernel duration
measured with HIP events on the launch stream.  The CPU baseline is the
float64 oracle, run on a sample of the same workload's heads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunked fwd tokens/s + TFLOP/s (MFMA %); decode-step state GB/s (HBM %)"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 matrix cores, TFLOP/s
F32_PEAK_TFLOPS = 157.3          # MI355X dense fp32 matrix cores, TFLOP/s

CHUNK_WORKLOAD = "gdr_bf16_b4h16t8192d128"
DECODE_WORKLOAD = "gdr_decode_b256h16d128"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gdr_chunk_b4h16t8192d128_hbm_traffic.txt")
KERNEL_SOURCES = ["la_chunk_gdr.hip", "la_chunk_common.hpp", "la_mfma.hpp", "la_common.hpp"]


def gdr_chunk_flops_per_token_head(d_k: int, d_v: int, C: int) -> float:
    """Matrix flops of the chunked gated delta rule per token and head.

    Per chunk of C tokens: Q K^T and K K^T (2 x 2 C^2 d_k), the triangular
    inverse (~C^3 / 3), Q S0^T and K S0^T (2 x 2 C d_k d_v), T Y and P U
    (2 x 2 C^2 d_v) and the state update (2 C d_k d_v); divided by C.
    """
    per_chunk = 4 * C * C * d_k + C ** 3 / 3 + 4 * C * d_k * d_v + 4 * C * C * d_v + 2 * C * d_k * d_v
    return per_chunk / C


def gdr_chunk_bytes(B, H, T, d_k, d_v, io_bytes=2, with_S0=False):
    """Bytes the forward must move: q, k, v read and out written once (io
    dtype), g and beta read once (fp32), the final state written (fp32)."""
    tok = B * H * T
    b = tok * ((2 * d_k + d_v) * io_bytes + d_v * io_bytes + 8)
    b += B * H * d_v * d_k * 4 * (2 if with_S0 else 1)
    return b


def linear_chunk_flops_per_token_head(d_k, d_v, C, normalized):
    """Matrix flops of chunked (gated) linear attention per token and head:
    phiQ phiK^T and P V over the chunk (2 C (d_k + d_v)), phiQ S0^T and the
    state update (4 d_k d_v), and for the normalized variant the denominator
    (2 d_k + C)."""
    f = 2 * C * (d_k + d_v) + 4 * d_k * d_v
    return f + (2 * d_k + C if normalized else 0)


def linear_chunk_bytes(B, H, T, d_k, d_v, io_bytes, gated, normalized):
    """q, k, v read and out written once; gated: per-channel gates (fp32) read
    once; final state (and normalizer) written once."""
    tok = B * H * T
    b = tok * ((2 * d_k + 2 * d_v) * io_bytes + (d_k * 4 if gated else 0))
    b += B * H * (d_v * d_k + (d_k if normalized else 0)) * 4
    return b


def bwd_bytes(B, H, T, d_k, d_v, io_bytes):
    """Bytes the backward must move: q, k, v and dout read once, dq, dk, dv
    written once (io dtype)."""
    return B * H * T * ((2 * d_k + 2 * d_v) + (2 * d_k + d_v)) * io_bytes


def bwd_flops_per_token_head(d_k, d_v, C):
    """Matrix flops of the chunked backward per token and head: per chunk the
    scores phiQ phiK^T and dO V^T, G phiK, G^T phiQ and A^T dO
    (2 C^2 (3 d_k + 2 d_v)), the state terms of dq, dk, dv and the two state
    increments (5 x 2 C d_k d_v); divided by C."""
    return 2 * C * (3 * d_k + 2 * d_v) + 10 * d_k * d_v


def decode_bytes(B, H, d_k, d_v, io_bytes=2):
    """Bytes of one decode step: the fp32 state read and written once, plus
    q, k, v, out (io dtype) and g, beta (fp32)."""
    per_head = 2 * d_v * d_k * 4 + (2 * d_k + 2 * d_v) * io_bytes + 8
    return B * H * per_head


def source_digest():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_delta_rule_causal_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the chunk kernel from the committed rocprofv3
    counter summary, or None when absent or taken on different sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def to_dev(ht):
    import numpy as np
    import torch
    if ht.dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(ht.data).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(ht.data))
    return t.cuda()


def time_launches(fn, steps, warmup, stream):
    """Run fn warmup + steps times; return (wall seconds of the timed steps,
    mean and per-launch kernel milliseconds from HIP events on `stream`)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall, sum(ms) / len(ms), ms


def cpu_model():
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_peaks(stream, copy_bytes=1 << 30, reps=5):
    """On-box peaks: a hand-written streaming copy of copy_bytes (read once,
    written once; GB/s counts both) and a matrix-core-only bf16 loop
    (libla_probe.so), each timed with HIP events on `stream`."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "gated_delta_rule_causal_amd", "libla_probe.so"))
    lib.la_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.la_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.la_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.la_probe_mfma_flops.restype = ctypes.c_double
    sp = ctypes.c_void_p(stream.cuda_stream)
    src = torch.ones(copy_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def copy():
        assert lib.la_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), copy_bytes, sp) == 0

    _, copy_ms, _ = time_launches(copy, reps, 2, stream)
    assert bool(torch.equal(src[:1024], dst[:1024]))
    del src, dst
    blocks, iters = 256 * 8, 2000
    buf = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")

    def mfma():
        assert lib.la_probe_mfma(ctypes.c_void_p(buf.data_ptr()), blocks, iters, sp) == 0

    _, mfma_ms, _ = time_launches(mfma, reps, 2, stream)
    return {"hbm_copy_gbs": 2 * copy_bytes / (copy_ms * 1e-3) / 1e9, "copy_bytes": copy_bytes,
            "copy_ms": copy_ms,
            "bf16_mfma_tflops": lib.la_probe_mfma_flops(blocks, iters) / (mfma_ms * 1e-3) / 1e12,
            "mfma_ms": mfma_ms}


def cpu_baseline(w, inp, seconds_target=15.0):
    """The float64 oracle on a sample of the workload's heads (full T)."""
    import numpy as np
    import oracle
    import workloads as wl
    nh = w.B * w.H
    n_take = max(1, min(nh, 4 * oracle.num_threads()))

    def sel(name, heads):
        a = inp[name]
        raw = a.data.reshape((nh,) + a.data.shape[2:])[heads]
        return wl.HostTensor(a.dtype, raw).f64()[None]

    heads = np.arange(n_take)
    args = {n: sel(n, heads) for n in ("q", "k", "v", "gate", "beta") if n in inp}
    t0 = time.perf_counter()
    oracle.forward(w.variant, args["q"], args["k"], args["v"], gate=args.get("gate"), beta=args.get("beta"),
                   phi_kind=w.phi_kind)
    dt = time.perf_counter() - t0
    head_tokens_per_s = n_take * w.T / dt
    return {"value": head_tokens_per_s / w.H, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d of %d heads (b*H+h = 0..%d), full T=%d, float64 token recurrence, %.1f s; "
                      "tokens/s counts a token as all H=%d heads" % (n_take, nh, n_take - 1, w.T, dt, w.H)}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=CHUNK_WORKLOAD,
                    help="chunked-forward workload to time (default: the gated delta rule headline)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="also run one probe copy of this many bytes (counter calibration)")
    ap.add_argument("--no-probes", action="store_true", help="skip the on-box peak probes")
    args = ap.parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the operator is measured on one GPU's share; "
              "multi-GPU runs are not supported (got --gpus %d, WORLD_SIZE %d)" % (args.gpus, world),
              file=sys.stderr)
        return 2

    import torch
    import gated_delta_rule_causal_amd as la
    import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    # The decode and backward measurements run first: they bring the GPU's
    # clocks up, so that the headline's warmup steps start from a warm GPU.
    # ---------------- decode step
    wd = wl.WORKLOADS[DECODE_WORKLOAD]
    S = to_dev(wl.decode_state(wd))
    pool = [{k: to_dev(v) for k, v in wl.decode_step_inputs(wd, s).items()} for s in range(8)]
    o = torch.empty((wd.B, wd.H, wd.d_v), dtype=torch.bfloat16, device="cuda")
    it = [0]

    def decode_step():
        x = pool[it[0] % len(pool)]
        it[0] += 1
        la.la_decode_step(x["q"], x["k"], x["v"], S, variant=wd.variant, gate=x["gate"], beta=x["beta"], out=o)

    dwall, dms, _ = time_launches(decode_step, args.decode_steps, 10, stream)
    dbytes = decode_bytes(wd.B, wd.H, wd.d_k, wd.d_v)
    dgbs = dbytes / (dms * 1e-3) / 1e9
    del S, pool

    # control: the same step over B=512 (537 MB of state, twice the 256 MB
    # Infinity Cache), so that the cache cannot hold the state between steps
    Bc = 2 * wd.B
    Sc = to_dev(wl.decode_state(wd, B=Bc))
    poolc = [{k: to_dev(v) for k, v in wl.decode_step_inputs(wd, s, B=Bc).items()} for s in range(4)]
    oc = torch.empty((Bc, wd.H, wd.d_v), dtype=torch.bfloat16, device="cuda")
    itc = [0]

    def decode_step_control():
        x = poolc[itc[0] % len(poolc)]
        itc[0] += 1
        la.la_decode_step(x["q"], x["k"], x["v"], Sc, variant=wd.variant, gate=x["gate"], beta=x["beta"], out=oc)

    _, dmsc, _ = time_launches(decode_step_control, max(20, args.decode_steps // 4), 5, stream)
    dbytesc = decode_bytes(Bc, wd.H, wd.d_k, wd.d_v)
    del Sc, poolc

    # ---------------- backward pass (training)
    backward = []
    for name, wb in wl.BWD_WORKLOADS.items():
        ib = wl.chunk_inputs(wb, head_decay=True)
        cb = wl.backward_cotangents(wb, state=False)
        db = {k: to_dev(v) for k, v in ib.items()}
        dout = to_dev(cb["dout"])
        descb = la.make_desc(wb.variant, la.LA_BF16 if wb.dtype == "bf16" else la.LA_F32, wb.B, wb.H, wb.T, wb.d_k,
                             wb.d_v, 0, wb.phi_kind)
        wsb = torch.empty(la.la_chunk_bwd_workspace(descb), dtype=torch.uint8, device="cuda")
        grads = [torch.empty_like(db["q"]), torch.empty_like(db["k"]), torch.empty_like(db["v"])]

        def bwd_step():
            la.la_chunk_bwd(db["q"], db["k"], db["v"], dout, variant=wb.variant, gate=db.get("gate"),
                            phi=wb.phi_kind, dq=grads[0], dk=grads[1], dv=grads[2], workspace=wsb)

        bwall, bms, _ = time_launches(bwd_step, max(5, args.steps // 2), 3, stream)
        if not all(bool(torch.isfinite(g).all()) for g in grads):
            print("non-finite gradient", file=sys.stderr)
            return 1
        iob = 2 if wb.dtype == "bf16" else 4
        bb = bwd_bytes(wb.B, wb.H, wb.T, wb.d_k, wb.d_v, iob)
        bf = bwd_flops_per_token_head(wb.d_k, wb.d_v, wb.chunk) * wb.B * wb.H * wb.T
        backward.append({"workload": name, "variant": "normalized_linear_attention" if wb.variant == la.LA_NORMALIZED
                         else "retention", "entry": "la_chunk_bwd", "avg_call_ms": bms,
                         "tokens_per_s": wb.B * wb.T / (bms * 1e-3), "workspace_bytes": wsb.numel(),
                         "algorithmic_bytes": bb, "hbm_gbs": bb / (bms * 1e-3) / 1e9,
                         "hbm_frac": bb / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_flops": bf,
                         "tflops": bf / (bms * 1e-3) / 1e12,
                         "mfma_frac": bf / (bms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS})
        del db, dout, wsb, grads

    # ---------------- chunked forward (headline)
    w = wl.WORKLOADS[args.workload] if args.workload in wl.WORKLOADS else wl.EXTRA_WORKLOADS[args.workload]
    assert not w.decode, "--workload names a chunked-forward workload"
    inp = wl.chunk_inputs(w)
    d = {k: to_dev(v) for k, v in inp.items()}
    io_t = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = torch.empty((w.B, w.H, w.T, w.d_v), dtype=io_t, device="cuda")
    S_T = torch.empty((w.B, w.H, w.d_v, w.d_k), dtype=torch.float32, device="cuda")
    z_T = torch.empty((w.B, w.H, w.d_k), dtype=torch.float32, device="cuda") if w.variant == la.LA_NORMALIZED else None
    desc = la.make_desc(w.variant, la.LA_BF16 if w.dtype == "bf16" else la.LA_F32, w.B, w.H, w.T, w.d_k, w.d_v,
                        w.chunk, w.phi_kind)
    ws_bytes = la.la_chunk_fwd_workspace(desc)   # allocated once, outside the timed steps
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda") if ws_bytes else None

    def chunk_step():
        la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=w.variant, gate=d.get("gate"), beta=d.get("beta"),
                        chunk=w.chunk, phi=w.phi_kind, out=out, S_T=S_T, z_T=z_T, workspace=ws)

    wall, ms_avg, _ = time_launches(chunk_step, args.steps, args.warmup, stream)
    if not bool(torch.isfinite(out).all()) or not bool(torch.isfinite(S_T).all()):
        print("non-finite output", file=sys.stderr)
        return 1
    tokens = w.B * w.T
    value = tokens * args.steps / wall
    io_bytes = 2 if w.dtype == "bf16" else 4
    if w.variant == la.LA_GATED_DELTA:
        flops = gdr_chunk_flops_per_token_head(w.d_k, w.d_v, w.chunk) * w.B * w.H * w.T
        nbytes = gdr_chunk_bytes(w.B, w.H, w.T, w.d_k, w.d_v, io_bytes)
        kname, vname = "gdr_chunk_kernel", "gated_delta_rule"
    elif w.variant == la.LA_KDA:
        flops = gdr_chunk_flops_per_token_head(w.d_k, w.d_v, w.chunk) * w.B * w.H * w.T
        # per-channel gates: d_k floats per token instead of one
        nbytes = gdr_chunk_bytes(w.B, w.H, w.T, w.d_k, w.d_v, io_bytes) + w.B * w.H * w.T * (w.d_k - 1) * 4
        kname, vname = "kda_prep_kernel + kda_chain_kernel", "kda"
    else:
        norm = w.variant == la.LA_NORMALIZED
        gated = w.variant == la.LA_GATED
        flops = linear_chunk_flops_per_token_head(w.d_k, w.d_v, w.chunk, norm) * w.B * w.H * w.T
        nbytes = linear_chunk_bytes(w.B, w.H, w.T, w.d_k, w.d_v, io_bytes, gated, norm)
        few_heads = w.B * w.H * (w.d_v // min(w.d_v, 64)) < 256
        if gated:
            kname = "gla_pipelined_kernel"
        elif few_heads and w.d_k in (64, 128) and w.d_v in (64, 128):
            kname = "seg_increment_kernel + seg_attention_kernel"
        else:
            kname = "la_segment_state_kernel + linear_chunk_kernel"
        vname = {la.LA_NORMALIZED: "normalized_linear_attention", la.LA_GATED: "gated_linear_attention",
                 la.LA_RETENTION: "retention"}[w.variant]
    gbs = nbytes / (ms_avg * 1e-3) / 1e9
    tflops = flops / (ms_avg * 1e-3) / 1e12
    traffic = read_traffic() if args.workload == CHUNK_WORKLOAD else None

    peaks = None if args.no_probes else measured_peaks(stream)
    if args.copy_bytes > 0:
        # one probe copy of a known size, for calibrating the traffic counters
        measured_peaks(stream, copy_bytes=args.copy_bytes, reps=1)

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "variant": vname, "B": w.B, "H": w.H, "T": w.T,
                   "d_k": w.d_k, "d_v": w.d_v, "chunk": w.chunk, "global_batch": w.B, "seq_len": w.T,
                   "parallelism": "none (one GPU)"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic},
        "chunk_kernel": {"kernel": kname, "avg_launch_ms": ms_avg, "algorithmic_bytes": nbytes,
                         "algorithmic_flops": flops, "tflops": tflops,
                         "mfma_frac": tflops / (BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS)},
        "decode": {"workload": DECODE_WORKLOAD, "kernel": "decode_kernel", "steps": args.decode_steps,
                   "avg_launch_ms": dms, "tokens_per_s": wd.B * args.decode_steps / dwall,
                   "roofline": {"bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": dgbs / HBM_PEAK_GBS, "algorithmic_bytes": dbytes},
                   "control_b512": {"avg_launch_ms": dmsc, "algorithmic_bytes": dbytesc,
                                    "achieved_gbs": dbytesc / (dmsc * 1e-3) / 1e9,
                                    "frac": dbytesc / (dmsc * 1e-3) / 1e9 / HBM_PEAK_GBS}},
    }
    result["backward"] = backward
    if peaks is not None:
        peaks["chunk_hbm_frac_of_measured"] = gbs / peaks["hbm_copy_gbs"]
        peaks["chunk_mfma_frac_of_measured"] = tflops / peaks["bf16_mfma_tflops"] if w.dtype == "bf16" else None
        peaks["decode_hbm_frac_of_measured"] = dgbs / peaks["hbm_copy_gbs"]
        result["measured_peaks"] = peaks
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
