"""Helpers of the GPU parity tests: host -> device transfer, the parity
metric, and the record of achieved errors."""
import json
import os

import numpy as np
import torch

from workloads import HostTensor

TOL = {"f32": 2e-3, "bf16": 3e-2}   # max relative error (see parity_error)


def dev(ht, device="cuda"):
    """HostTensor (float32 or bfloat16 bit patterns) -> torch tensor on the GPU."""
    if ht is None:
        return None
    if isinstance(ht, HostTensor):
        if ht.dtype == "bf16":
            t = torch.from_numpy(np.ascontiguousarray(ht.data).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(ht.data))
    else:
        t = torch.from_numpy(np.ascontiguousarray(ht))
    return t.to(device)


def host64(t):
    """GPU tensor -> float64 numpy (exact for float32 and bfloat16)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def parity_error(x, ref, lead=2):
    """max over leading slices of max|x - ref| / max|ref|.

    The leading `lead` axes index independent (b, h) slices; the error of a
    slice is its largest absolute deviation divided by its largest absolute
    reference value.
    """
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if x.size == 0:
        return 0.0
    n = int(np.prod(x.shape[:lead]))
    xd = np.abs(x - ref).reshape(n, -1).max(axis=1)
    rm = np.abs(ref).reshape(n, -1).max(axis=1)
    rm = np.where(rm > 0, rm, 1.0)
    return float(np.max(xd / rm))


def record(case, errs, dtype):
    """Append the achieved errors of one parity case (a dict tensor -> error)
    to the JSON-lines file named by LA_PARITY_LOG, when it is set, so that the
    margin to the tolerance is visible and not only pass/fail."""
    path = os.environ.get("LA_PARITY_LOG")
    if not path:
        return
    row = {"case": case, "dtype": dtype, "tol": TOL[dtype]}
    row.update({k: float(v) for k, v in errs.items()})
    with open(path, "a") as f:
        f.write(json.dumps(row) + "\n")
