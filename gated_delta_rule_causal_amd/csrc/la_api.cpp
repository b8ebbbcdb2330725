// la_api.cpp -- the C entry points of include/la.h.
//
// Every argument is checked on the host before any HIP call; a failing check
// returns LA_EINVAL / LA_EUNSUPPORTED, records a message for la_last_error()
// and launches nothing.  Valid calls are forwarded to the kernel launchers
// on the caller's stream without host synchronization or allocation.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "la_internal.hpp"

// Library-held scratch of la_chunk_fwd_noalloc: one array per GPU (each GPU
// holds its own copy at its own address), kept until the process ends.  In
// host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, per device, in scratch_on_current_device().
static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";

la_status fail(la_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

bool supported_head_size(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi); empty when lo == hi
};

Range range(const char *name, const void *p, size_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + bytes : lo};
}

bool overlaps(const Range &a, const Range &b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool misaligned(const void *p, uintptr_t a) { return p && (reinterpret_cast<uintptr_t>(p) % a) != 0; }

// Checks shared by both entry points.  n_tok = tokens per head that the call reads.
la_status check_desc(const la_desc *d, bool chunked) {
    if (!d) return fail(LA_EINVAL, "desc is NULL");
    if (d->variant < LA_NORMALIZED || d->variant > LA_KDA)
        return fail(LA_EINVAL, "variant %d is not a la_variant", d->variant);
    if (d->dtype != LA_F32 && d->dtype != LA_BF16) return fail(LA_EINVAL, "dtype %d is not a la_dtype", d->dtype);
    if (d->phi != LA_PHI_IDENTITY && d->phi != LA_PHI_ELU1) return fail(LA_EINVAL, "phi %d is not a la_phi", d->phi);
    if (d->variant == LA_NORMALIZED && d->phi != LA_PHI_ELU1)
        return fail(LA_EINVAL, "LA_NORMALIZED needs LA_PHI_ELU1 (the normalizer needs positive features)");
    if ((d->variant == LA_GATED_DELTA || d->variant == LA_KDA) && d->phi != LA_PHI_IDENTITY)
        return fail(LA_EINVAL, "the delta rules need LA_PHI_IDENTITY (keys are unit vectors)");
    if (d->B < 0 || d->H < 0) return fail(LA_EINVAL, "B=%d, H=%d must be >= 0", d->B, d->H);
    if (chunked && d->T < 0) return fail(LA_EINVAL, "T=%d must be >= 0", d->T);
    if (d->d_k <= 0 || d->d_v <= 0) return fail(LA_EINVAL, "d_k=%d, d_v=%d must be > 0", d->d_k, d->d_v);
    if (!supported_head_size(d->d_k) || !supported_head_size(d->d_v))
        return fail(LA_EUNSUPPORTED, "head sizes d_k=%d, d_v=%d: supported are 16, 32, 64, 128", d->d_k, d->d_v);
    if (chunked) {
        if (d->chunk < 0) return fail(LA_EINVAL, "chunk=%d must be >= 0", d->chunk);
        if (d->chunk != 0 && d->chunk != 16 && d->chunk != 32 && d->chunk != 64 && d->chunk != 128)
            return fail(LA_EUNSUPPORTED, "chunk=%d: supported are 0 (= 64), 16, 32, 64, 128", d->chunk);
    }
    // element counts must stay far from 64-bit overflow
    const double elems = static_cast<double>(d->B) * d->H * (chunked ? (d->T > 0 ? d->T : 1) : 1) *
                         (d->d_k > d->d_v ? d->d_k : d->d_v);
    if (elems > 4.0e18) return fail(LA_EINVAL, "problem too large");
    return LA_OK;
}

// How a variant's gate is laid out: one decay per head (H,), optional;
// one per token (B,H,T) / (B,H); one per token and key channel.
enum GateKind { GATE_PER_HEAD, GATE_PER_TOKEN, GATE_PER_CHANNEL };
GateKind gate_kind(int variant) {
    if (variant == LA_NORMALIZED || variant == LA_RETENTION) return GATE_PER_HEAD;
    if (variant == LA_GATED_DELTA) return GATE_PER_TOKEN;
    return GATE_PER_CHANNEL;
}
bool has_beta(int variant) { return variant == LA_GATED_DELTA || variant == LA_KDA; }

la_status check_role(const la_desc *d, const float *gate, const float *beta, const float *z_in,
                     const float *z_out, bool need_data) {
    if (d->variant != LA_NORMALIZED && (z_in || z_out))
        return fail(LA_EINVAL, "z must be NULL unless the variant is LA_NORMALIZED");
    if (gate_kind(d->variant) != GATE_PER_HEAD && need_data && !gate)
        return fail(LA_EINVAL, "gate is required for this variant");
    if (!has_beta(d->variant) && beta) return fail(LA_EINVAL, "beta must be NULL for this variant");
    if (has_beta(d->variant) && need_data && !beta) return fail(LA_EINVAL, "beta is required for the delta rules");
    return LA_OK;
}

// Bytes of the gate argument: `per` tokens per head (T, or 1 for decode).
size_t gate_bytes(const la_desc *d, size_t heads, size_t per) {
    switch (gate_kind(d->variant)) {
        case GATE_PER_HEAD: return static_cast<size_t>(d->H) * 4;
        case GATE_PER_TOKEN: return heads * per * 4;
        default: return heads * per * static_cast<size_t>(d->d_k) * 4;
    }
}
// Alignment of the gate argument: scalars per head or token are read one at
// a time, per-channel gates as 16-byte vectors.
uintptr_t gate_align(int variant) { return gate_kind(variant) == GATE_PER_CHANNEL ? 16 : 4; }

// Device address of `scratch` on the current device, resolved once per device
// (with that device current) and kept; nullptr if HIP reports an error.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_on_current_device(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

int la_abi_version(void) { return LA_ABI_VERSION; }

const char *la_status_str(la_status s) {
    switch (s) {
        case LA_OK: return "LA_OK: success";
        case LA_EINVAL: return "LA_EINVAL: invalid argument";
        case LA_EUNSUPPORTED: return "LA_EUNSUPPORTED: no kernel for this configuration";
        case LA_EHIP: return "LA_EHIP: HIP runtime error";
    }
    return "unknown la_status";
}

const char *la_last_error(void) { return g_last_error; }

size_t la_chunk_fwd_workspace(const la_desc *d) {
    if (check_desc(d, true) != LA_OK) return 0;
    la::ChunkArgs a = {};
    a.variant = d->variant; a.dtype = d->dtype; a.phi = d->phi;
    a.B = d->B; a.H = d->H; a.T = d->T; a.d_k = d->d_k; a.d_v = d->d_v;
    a.chunk = d->chunk ? d->chunk : 64;
    return la::chunk_workspace_bytes(a);
}

static la_status chunk_fwd(const la_desc *d, const void *q, const void *k, const void *v, const float *gate,
                           const float *beta, const float *S0, const float *z0, void *out, float *S_T, float *z_T,
                           void *workspace, size_t workspace_bytes, void *stream, bool use_scratch);

la_status la_chunk_fwd(const la_desc *d, const void *q, const void *k, const void *v,
                       const float *gate, const float *beta, const float *S0, const float *z0,
                       void *out, float *S_T, float *z_T, void *workspace, size_t workspace_bytes,
                       void *stream) {
    return chunk_fwd(d, q, k, v, gate, beta, S0, z0, out, S_T, z_T, workspace, workspace_bytes, stream, false);
}

la_status la_chunk_fwd_noalloc(const la_desc *d, const void *q, const void *k, const void *v,
                               const float *gate, const float *beta, const float *S0, const float *z0,
                               void *out, float *S_T, float *z_T, void *stream) {
    return chunk_fwd(d, q, k, v, gate, beta, S0, z0, out, S_T, z_T, nullptr, 0, stream, true);
}

static la_status chunk_fwd(const la_desc *d, const void *q, const void *k, const void *v, const float *gate,
                           const float *beta, const float *S0, const float *z0, void *out, float *S_T, float *z_T,
                           void *workspace, size_t workspace_bytes, void *stream, bool use_scratch) {
    g_last_error[0] = '\0';
    la_status st = check_desc(d, true);
    if (st != LA_OK) return st;
    const size_t heads = static_cast<size_t>(d->B) * d->H;
    const size_t tok = heads * static_cast<size_t>(d->T);
    const bool need_data = tok > 0;
    st = check_role(d, gate, beta, z0, z_T, need_data);
    if (st != LA_OK) return st;
    if (need_data && (!q || !k || !v || !out)) return fail(LA_EINVAL, "q, k, v and out are required when B*H*T > 0");

    const size_t esz = d->dtype == LA_BF16 ? 2 : 4;
    const void *ptrs[] = {q, k, v, gate, beta, S0, z0, out, S_T, z_T, workspace};
    const char *names[] = {"q", "k", "v", "gate", "beta", "S0", "z0", "out", "S_T", "z_T", "workspace"};
    for (int i = 0; i < 11; ++i) {
        // scalar gates (per head or per token) and beta are read with scalar loads
        uintptr_t al = i == 3 ? gate_align(d->variant) : i == 4 ? 4 : 16;
        if (misaligned(ptrs[i], al)) return fail(LA_EINVAL, "%s is not %d-byte aligned", names[i], (int)al);
    }

    la::ChunkArgs a = {};
    a.variant = d->variant; a.dtype = d->dtype; a.phi = d->phi;
    a.B = d->B; a.H = d->H; a.T = d->T; a.d_k = d->d_k; a.d_v = d->d_v;
    a.chunk = d->chunk ? d->chunk : 64;
    const size_t need_ws = la::chunk_workspace_bytes(a);
    if (use_scratch) {
        if (need_ws > LA_NOALLOC_SCRATCH_BYTES)
            return fail(LA_EINVAL, "needs %zu bytes of scratch; la_chunk_fwd_noalloc holds %zu (use la_chunk_fwd)",
                        need_ws, (size_t)LA_NOALLOC_SCRATCH_BYTES);
    } else if (need_ws > 0 && (!workspace || workspace_bytes < need_ws)) {
        return fail(LA_EINVAL, "workspace of %zu bytes required, %zu given", need_ws, workspace ? workspace_bytes : 0);
    }

    const size_t dk = d->d_k, dv = d->d_v;
    const Range r_q = range("q", q, tok * dk * esz), r_k = range("k", k, tok * dk * esz);
    const Range r_v = range("v", v, tok * dv * esz);
    const Range r_g = range("gate", gate, gate_bytes(d, heads, static_cast<size_t>(d->T)));
    const Range r_b = range("beta", beta, tok * 4);
    const Range r_s0 = range("S0", S0, heads * dv * dk * 4), r_z0 = range("z0", z0, heads * dk * 4);
    const Range r_o = range("out", out, tok * dv * esz);
    const Range r_st = range("S_T", S_T, heads * dv * dk * 4), r_zt = range("z_T", z_T, heads * dk * 4);
    const Range r_ws = range("workspace", workspace, need_ws);
    const Range inputs[] = {r_q, r_k, r_v, r_g, r_b, r_s0, r_z0};
    const Range outputs[] = {r_o, r_st, r_zt, r_ws};
    for (const Range &o : outputs) {
        for (const Range &i : inputs) {
            if (!overlaps(o, i)) continue;
            // the final state may replace the initial one exactly (in-place carry)
            if ((o.name == r_st.name && i.name == r_s0.name && o.lo == i.lo) ||
                (o.name == r_zt.name && i.name == r_z0.name && o.lo == i.lo))
                continue;
            return fail(LA_EINVAL, "%s overlaps %s", o.name, i.name);
        }
        for (const Range &o2 : outputs)
            if (&o2 != &o && overlaps(o, o2)) return fail(LA_EINVAL, "%s overlaps %s", o.name, o2.name);
    }
    if (heads == 0) return LA_OK;
    if (use_scratch && need_ws > 0) {
        hipError_t e = scratch_on_current_device(&workspace);
        if (e != hipSuccess) return fail(LA_EHIP, "scratch address: %s", hipGetErrorString(e));
        workspace_bytes = LA_NOALLOC_SCRATCH_BYTES;
    }

    a.q = q; a.k = k; a.v = v; a.gate = gate; a.beta = beta; a.S0 = S0; a.z0 = z0;
    a.out = out; a.S_T = S_T; a.z_T = z_T; a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.stream = static_cast<hipStream_t>(stream);
    hipError_t e = la::launch_chunk(a);
    if (e != hipSuccess) return fail(LA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return LA_OK;
}

static void bwd_args(const la_desc *d, la::BwdArgs &a) {
    a = la::BwdArgs{};
    a.variant = d->variant; a.dtype = d->dtype; a.phi = d->phi;
    a.B = d->B; a.H = d->H; a.T = d->T; a.d_k = d->d_k; a.d_v = d->d_v;
}

size_t la_chunk_bwd_workspace(const la_desc *d) {
    if (check_desc(d, true) != LA_OK) return 0;
    if (d->variant != LA_NORMALIZED && d->variant != LA_RETENTION) return 0;
    la::BwdArgs a;
    bwd_args(d, a);
    return la::bwd_workspace_bytes(a);
}

la_status la_chunk_bwd(const la_desc *d, const void *q, const void *k, const void *v, const float *gate,
                       const float *S0, const float *z0, const void *dout,
                       const float *dS_T, const float *dz_T, void *dq, void *dk, void *dv, float *dgate,
                       float *dS0, float *dz0, void *workspace, size_t workspace_bytes, void *stream) {
    g_last_error[0] = '\0';
    la_status st = check_desc(d, true);
    if (st != LA_OK) return st;
    if (d->variant != LA_NORMALIZED && d->variant != LA_RETENTION)
        return fail(LA_EUNSUPPORTED, "la_chunk_bwd covers LA_NORMALIZED and LA_RETENTION");
    const bool norm = d->variant == LA_NORMALIZED;
    const size_t heads = static_cast<size_t>(d->B) * d->H;
    const size_t tok = heads * static_cast<size_t>(d->T);
    if (!norm && (z0 || dz_T || dz0)) return fail(LA_EINVAL, "z0, dz_T and dz0 must be NULL for LA_RETENTION");
    if (!gate && dgate) return fail(LA_EINVAL, "dgate needs gate (there is no decay to differentiate)");
    if (tok > 0 && (!q || !k || !v || !dout || !dq || !dk || !dv))
        return fail(LA_EINVAL, "q, k, v, dout, dq, dk and dv are required when B*H*T > 0");

    const size_t esz = d->dtype == LA_BF16 ? 2 : 4;
    const void *ptrs[] = {q, k, v, gate, S0, z0, dout, dS_T, dz_T, dq, dk, dv, dgate, dS0, dz0, workspace};
    const char *names[] = {"q", "k", "v", "gate", "S0", "z0", "dout", "dS_T", "dz_T",
                           "dq", "dk", "dv", "dgate", "dS0", "dz0", "workspace"};
    for (int i = 0; i < 16; ++i) {
        // gate and dgate are read or written one float at a time
        const uintptr_t al = (i == 3 || i == 12) ? 4 : 16;
        if (misaligned(ptrs[i], al)) return fail(LA_EINVAL, "%s is not %d-byte aligned", names[i], (int)al);
    }
    la::BwdArgs a;
    bwd_args(d, a);
    const size_t need_ws = la::bwd_workspace_bytes(a);
    if (need_ws > 0 && (!workspace || workspace_bytes < need_ws))
        return fail(LA_EINVAL, "workspace of %zu bytes required, %zu given", need_ws, workspace ? workspace_bytes : 0);

    const size_t dkk = d->d_k, dvv = d->d_v;
    const Range r_q = range("q", q, tok * dkk * esz), r_k = range("k", k, tok * dkk * esz);
    const Range r_v = range("v", v, tok * dvv * esz), r_g = range("gate", gate, static_cast<size_t>(d->H) * 4);
    const Range r_s0 = range("S0", S0, heads * dvv * dkk * 4), r_z0 = range("z0", z0, heads * dkk * 4);
    const Range r_do = range("dout", dout, tok * dvv * esz);
    const Range r_dst = range("dS_T", dS_T, heads * dvv * dkk * 4), r_dzt = range("dz_T", dz_T, heads * dkk * 4);
    const Range r_dq = range("dq", dq, tok * dkk * esz), r_dk = range("dk", dk, tok * dkk * esz);
    const Range r_dv = range("dv", dv, tok * dvv * esz), r_dg = range("dgate", dgate, static_cast<size_t>(d->H) * 4);
    const Range r_ds0 = range("dS0", dS0, heads * dvv * dkk * 4), r_dz0 = range("dz0", dz0, heads * dkk * 4);
    const Range r_ws = range("workspace", workspace, need_ws);
    const Range inputs[] = {r_q, r_k, r_v, r_g, r_s0, r_z0, r_do, r_dst, r_dzt};
    const Range outputs[] = {r_dq, r_dk, r_dv, r_dg, r_ds0, r_dz0, r_ws};
    for (const Range &o : outputs) {
        for (const Range &i : inputs)
            if (overlaps(o, i)) return fail(LA_EINVAL, "%s overlaps %s", o.name, i.name);
        for (const Range &o2 : outputs)
            if (&o2 != &o && overlaps(o, o2)) return fail(LA_EINVAL, "%s overlaps %s", o.name, o2.name);
    }
    if (heads == 0) return LA_OK;

    a.q = q; a.k = k; a.v = v; a.dout = dout;
    a.gate = gate; a.S0 = S0; a.z0 = z0; a.dS_T = dS_T; a.dz_T = dz_T;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dgate = dgate; a.dS0 = dS0; a.dz0 = dz0;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.stream = static_cast<hipStream_t>(stream);
    hipError_t e = la::launch_chunk_bwd(a);
    if (e != hipSuccess) return fail(LA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return LA_OK;
}

la_status la_decode_step(const la_desc *d, const void *q, const void *k, const void *v,
                         const float *gate, const float *beta, float *S, float *z, void *out,
                         void *stream) {
    g_last_error[0] = '\0';
    la_status st = check_desc(d, false);
    if (st != LA_OK) return st;
    const size_t heads = static_cast<size_t>(d->B) * d->H;
    const bool need_data = heads > 0;
    st = check_role(d, gate, beta, z, z, need_data);
    if (st != LA_OK) return st;
    if (need_data && (!q || !k || !v || !out || !S)) return fail(LA_EINVAL, "q, k, v, S and out are required");
    if (need_data && d->variant == LA_NORMALIZED && !z) return fail(LA_EINVAL, "z is required for LA_NORMALIZED");

    const size_t esz = d->dtype == LA_BF16 ? 2 : 4;
    const void *ptrs[] = {q, k, v, gate, beta, S, z, out};
    const char *names[] = {"q", "k", "v", "gate", "beta", "S", "z", "out"};
    for (int i = 0; i < 8; ++i) {
        uintptr_t al = i == 3 ? gate_align(d->variant) : i == 4 ? 4 : 16;
        if (i == 7) al = esz;  // one output element per state row
        if (misaligned(ptrs[i], al)) return fail(LA_EINVAL, "%s is not %d-byte aligned", names[i], (int)al);
    }
    const size_t dk = d->d_k, dv = d->d_v;
    const Range r_q = range("q", q, heads * dk * esz), r_k = range("k", k, heads * dk * esz);
    const Range r_v = range("v", v, heads * dv * esz);
    const Range r_g = range("gate", gate, gate_bytes(d, heads, 1));
    const Range r_b = range("beta", beta, heads * 4);
    const Range r_s = range("S", S, heads * dv * dk * 4), r_z = range("z", z, heads * dk * 4);
    const Range r_o = range("out", out, heads * dv * esz);
    const Range inputs[] = {r_q, r_k, r_v, r_g, r_b};
    const Range outputs[] = {r_s, r_z, r_o};
    for (const Range &o : outputs) {
        for (const Range &i : inputs)
            if (overlaps(o, i)) return fail(LA_EINVAL, "%s overlaps %s", o.name, i.name);
        for (const Range &o2 : outputs)
            if (&o2 != &o && overlaps(o, o2)) return fail(LA_EINVAL, "%s overlaps %s", o.name, o2.name);
    }
    if (heads == 0) return LA_OK;

    la::DecodeArgs a = {};
    a.variant = d->variant; a.dtype = d->dtype; a.phi = d->phi;
    a.B = d->B; a.H = d->H; a.d_k = d->d_k; a.d_v = d->d_v;
    a.q = q; a.k = k; a.v = v; a.gate = gate; a.beta = beta; a.S = S; a.z = z; a.out = out;
    a.stream = static_cast<hipStream_t>(stream);
    hipError_t e = la::launch_decode(a);
    if (e != hipSuccess) return fail(LA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return LA_OK;
}

// Shared checks of la_verify and la_commit: T draft tokens per sequence,
// tensors laid out as the chunked forward's with T tokens; `commit` calls
// take `accepted` and write S (and z) in place, verify calls write `out`.
static la_status multi_token(const la_desc *d, const void *q, const void *k, const void *v, const float *gate,
                             const float *beta, float *S, float *z, void *out, const int32_t *accepted, void *stream,
                             bool commit) {
    g_last_error[0] = '\0';
    la_status st = check_desc(d, false);
    if (st != LA_OK) return st;
    if (d->T < 0) return fail(LA_EINVAL, "T=%d must be >= 0", d->T);
    const size_t heads = static_cast<size_t>(d->B) * d->H;
    const size_t tok = heads * static_cast<size_t>(d->T);
    const bool need_data = tok > 0;
    st = check_role(d, gate, beta, z, z, need_data);
    if (st != LA_OK) return st;
    if (need_data && (!k || !v || !S)) return fail(LA_EINVAL, "k, v and S are required");
    if (need_data && !commit && (!q || !out)) return fail(LA_EINVAL, "q and out are required to verify");
    if (need_data && commit && !accepted) return fail(LA_EINVAL, "accepted is required to commit");
    if (need_data && d->variant == LA_NORMALIZED && !z) return fail(LA_EINVAL, "z is required for LA_NORMALIZED");
    if (commit && out) return fail(LA_EINVAL, "out must be NULL for la_commit");
    if (!commit && accepted) return fail(LA_EINVAL, "accepted must be NULL for la_verify");

    const size_t esz = d->dtype == LA_BF16 ? 2 : 4;
    const void *ptrs[] = {q, k, v, gate, beta, S, z, out, accepted};
    const char *names[] = {"q", "k", "v", "gate", "beta", "S", "z", "out", "accepted"};
    for (int i = 0; i < 9; ++i) {
        uintptr_t al = i == 3 ? gate_align(d->variant) : (i == 4 || i == 8) ? 4 : 16;
        if (i == 7) al = esz;   // one output element per state row
        if (misaligned(ptrs[i], al)) return fail(LA_EINVAL, "%s is not %d-byte aligned", names[i], (int)al);
    }
    const size_t dk = d->d_k, dv = d->d_v;
    const Range r_q = range("q", q, tok * dk * esz), r_k = range("k", k, tok * dk * esz);
    const Range r_v = range("v", v, tok * dv * esz);
    const Range r_g = range("gate", gate, gate_bytes(d, heads, static_cast<size_t>(d->T)));
    const Range r_b = range("beta", beta, tok * 4);
    const Range r_a = range("accepted", accepted, static_cast<size_t>(d->B) * 4);
    const Range r_s = range("S", S, heads * dv * dk * 4), r_z = range("z", z, heads * dk * 4);
    const Range r_o = range("out", out, tok * dv * esz);
    const Range inputs[] = {r_q, r_k, r_v, r_g, r_b, r_a};
    // verify only reads the state; commit writes it; out is written by verify
    const Range written[] = {r_o, commit ? r_s : Range{"S", 0, 0}, commit ? r_z : Range{"z", 0, 0}};
    const Range read_state[] = {r_s, r_z};
    for (const Range &o : written) {
        for (const Range &i : inputs)
            if (overlaps(o, i)) return fail(LA_EINVAL, "%s overlaps %s", o.name, i.name);
        for (const Range &o2 : written)
            if (&o2 != &o && overlaps(o, o2)) return fail(LA_EINVAL, "%s overlaps %s", o.name, o2.name);
        if (!commit)
            for (const Range &s2 : read_state)
                if (overlaps(o, s2)) return fail(LA_EINVAL, "%s overlaps %s", o.name, s2.name);
    }
    if (overlaps(r_s, r_z)) return fail(LA_EINVAL, "S overlaps z");
    if (!need_data) return LA_OK;

    la::DecodeArgs a = {};
    a.variant = d->variant; a.dtype = d->dtype; a.phi = d->phi;
    a.B = d->B; a.H = d->H; a.d_k = d->d_k; a.d_v = d->d_v;
    a.q = q; a.k = k; a.v = v; a.gate = gate; a.beta = beta; a.S = S; a.z = z; a.out = out;
    a.stream = static_cast<hipStream_t>(stream);
    a.mode = commit ? la::DECODE_COMMIT : la::DECODE_VERIFY;
    a.T = d->T;
    a.accepted = accepted;
    hipError_t e = la::launch_decode(a);
    if (e != hipSuccess) return fail(LA_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return LA_OK;
}

la_status la_verify(const la_desc *d, const void *q, const void *k, const void *v, const float *gate,
                    const float *beta, const float *S, const float *z, void *out, void *stream) {
    return multi_token(d, q, k, v, gate, beta, const_cast<float *>(S), const_cast<float *>(z), out, nullptr, stream,
                       false);
}

la_status la_commit(const la_desc *d, const void *k, const void *v, const float *gate, const float *beta,
                    const int32_t *accepted, float *S, float *z, void *stream) {
    return multi_token(d, nullptr, k, v, gate, beta, S, z, nullptr, accepted, stream, true);
}

}  // extern "C"
