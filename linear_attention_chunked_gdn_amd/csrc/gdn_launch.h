// Internal interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct PrefillArgs {
    const void *q;          // [T_tot, Hk, 128]
    const void *k;          // [T_tot, Hk, 128]
    const void *v;          // [T_tot, Hv, 128]
    const float *g;         // [T_tot, Hv]
    const float *beta;      // [T_tot, Hv]
    const float *s0;        // [N, Hv, 128, 128] or null
    const int32_t *cu;      // [N+1] or null (single sequence)
    void *o;                // [T_tot, Hv, 128]
    float *sN;              // [N, Hv, 128, 128] or null
    int32_t N, T_tot, Hk, Hv;
    int32_t nslices;        // value-channel slices per (sequence, head)
};

struct DecodeArgs {
    const void *q, *k, *v;  // [B, Hk, 128], [B, Hk, 128], [B, Hv, 128]
    const float *g, *beta;  // [B, Hv]
    float *state;           // [B, Hv, 128, 128]
    void *o;                // [B, Hv, 128]
    int32_t B, Hk, Hv;
};

// Launch the chunked prefill with `grid` workgroups of value-channel width `dvs`.
hipError_t launch_prefill(const PrefillArgs &a, bool bf16, int dvs, int grid, hipStream_t stream);
// LDS bytes of one prefill workgroup, -1 if (bf16, dvs) is not instantiated.
int prefill_lds_bytes(bool bf16, int dvs);
int prefill_threads();
// io: 0 fp32, 1 bf16, 2 fp16 (the gdn_dtype codes)
hipError_t launch_decode(const DecodeArgs &a, int io, hipStream_t stream);
// Software-pipelined bf16 prefill (16 value channels per workgroup).
hipError_t launch_prefill_pipe(const PrefillArgs &a, bool f16, int grid, hipStream_t stream);
int prefill_pipe_lds_bytes();
int prefill_pipe_threads();

}  // namespace gdn
