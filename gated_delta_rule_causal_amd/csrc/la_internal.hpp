// la_internal.hpp -- argument bundles passed from the validated C entry points
// to the kernel launchers.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "la.h"
#include "la_common.hpp"

namespace la {

enum DecodeMode { DECODE_STEP = 0, DECODE_VERIFY = 1, DECODE_COMMIT = 2 };

struct DecodeArgs {
    int variant, dtype, phi;
    int B, H, d_k, d_v;
    const void *q, *k, *v;
    const float *gate, *beta;
    float *S, *z;
    void *out;
    hipStream_t stream;
    int mode = DECODE_STEP;
    int T = 1;                          // tokens per sequence (verify / commit)
    const int32_t *accepted = nullptr;  // commit: tokens kept per sequence (B,)
};

struct ChunkArgs {
    int variant, dtype, phi;
    int B, H, T, d_k, d_v, chunk;
    const void *q, *k, *v;
    const float *gate, *beta;
    const float *S0, *z0;
    void *out;
    float *S_T, *z_T;
    void *workspace;
    size_t workspace_bytes;
    hipStream_t stream;
};

struct BwdArgs {
    int variant, dtype, phi;
    int B, H, T, d_k, d_v;
    const void *q, *k, *v, *dout;
    const float *gate, *S0, *z0, *dS_T, *dz_T;
    void *dq, *dk, *dv;
    float *dgate, *dS0, *dz0;
    void *workspace;
    size_t workspace_bytes;
    hipStream_t stream;
};

hipError_t launch_decode(const DecodeArgs &a);
hipError_t launch_chunk(const ChunkArgs &a);
hipError_t launch_chunk_kda(const ChunkArgs &a);
size_t chunk_workspace_bytes(const ChunkArgs &a);
size_t kda_workspace_bytes(const ChunkArgs &a);
// normalized / retention over segments held whole in LDS (la_chunk_segment.hip)
bool seg_plan(const ChunkArgs &a, int &seg_len, int &n_seg);
size_t seg_workspace_bytes(const ChunkArgs &a);
hipError_t launch_seg(const ChunkArgs &a);
hipError_t launch_chunk_bwd(const BwdArgs &a);
size_t bwd_workspace_bytes(const BwdArgs &a);
int bwd_chunk_length(const BwdArgs &a);

}  // namespace la
