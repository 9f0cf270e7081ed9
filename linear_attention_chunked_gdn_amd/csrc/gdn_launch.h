// Internal interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

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
    uint32_t prologue;      // GDN_PROLOGUE_* flags (the prologue kernel only)
};

struct DecodeArgs {
    const void *q, *k, *v;  // [B, Hk, 128], [B, Hk, 128], [B, Hv, 128]
    const float *g, *beta;  // [B, Hv]
    float *state;           // [B, Hv, 128, 128]
    void *o;                // [B, Hv, 128]
    int32_t B, Hk, Hv;
    uint32_t prologue;      // GDN_PROLOGUE_* flags
};

// Chunked prefill in two launches (the per-key-channel decay, KDA, with g [T_tot, Hv, 128];
// the scalar gate, with g [T_tot, Hv]).  A map kernel writes one workspace tile per (chunk
// slot, value head); chunk j of sequence n uses slot cu[n] / 64 + n + j, so T_tot / 64 + N
// slots cover every packing of the batch.  The chain kernel reads them.
struct KdaArgs {
    const void *q, *k, *v;  // [T_tot, Hk, 128], [T_tot, Hk, 128], [T_tot, Hv, 128]
    const float *g;         // [T_tot, Hv, 128] (KDA) or [T_tot, Hv] (scalar gate)
    const float *beta;      // [T_tot, Hv]
    const float *s0;        // [N, Hv, 128, 128] or null
    const int32_t *cu;      // [N+1] or null (single sequence)
    void *o;                // [T_tot, Hv, 128]
    float *sN;              // [N, Hv, 128, 128] or null
    char *ws;               // nslots * Hv tiles of Tile<C>::BYTES
    int32_t N, T_tot, Hk, Hv;
    int32_t nslots;         // T_tot / C + N (chunk j of sequence n: slot cu[n] / C + n + j)
    // Segmented chain only (launch_seg_chain, launch_seg_fix): every sequence runs as nseg
    // segments of whole chunks, each from its own start state (see gdn_seg.hip).
    int32_t nseg;
    _Float16 *o0;           // [T_tot, Hv, 128] outputs of segments >= 1 from a zero start
    _Float16 *e;            // [T_tot, Hv, 128] outputs of the identity-state rows
    float *sseg;            // [N, Hv, nseg, 2, 128, 128] segment end states (S and X^T)
    _Float16 *sin16;        // [N, Hv, nseg, 128, 128] start states of segments 1 .. nseg - 1
    uint32_t prologue;      // GDN_PROLOGUE_* flags of the scalar-gate map (0: none)
};
// Workspace tile of one chunk of C tokens and one value head (byte offsets; fp16 except
// gl; row-major), with T = (I + A)^-1 and the decays of the chunk:
//   P   = lower-incl-diagonal(Q K^T (.) decays)      [C tokens][C tokens]
//   W   = T diag(beta) (K (.) exp(Gamma))             [C tokens][128 key channels]
//   Qg  = Q (.) exp(Gamma)                            [C tokens][128 key channels]
//   KlT = (K (.) exp(Gamma_last - Gamma))^T           [128 key channels][C tokens]
//   UT  = (T diag(beta) V)^T                          [128 value channels][C tokens]
//   gl  = exp(Gamma_last)                             [128 key channels] fp32
// Each is laid out so that one chain wave's MFMA fragments are 16-byte row segments.
template <int C> struct Tile {
    static constexpr int P = 0;
    static constexpr int W = C * C * 2;
    static constexpr int QG = W + C * 256;
    static constexpr int KLT = QG + C * 256;
    static constexpr int UT = KLT + C * 256;
    static constexpr int GL = UT + C * 256;
    static constexpr size_t BYTES = (size_t)GL + 512;
};
static_assert(Tile<32>::BYTES % 256 == 0 && Tile<64>::BYTES % 256 == 0 && Tile<128>::BYTES % 256 == 0,
              "tiles keep the workspace's 256-byte alignment");
// The per-key-channel path runs 64-token chunks.
constexpr int WS_OFF_P = Tile<64>::P;
constexpr int WS_OFF_W = Tile<64>::W;
constexpr int WS_OFF_QG = Tile<64>::QG;
constexpr int WS_OFF_KLT = Tile<64>::KLT;
constexpr int WS_OFF_UT = Tile<64>::UT;
constexpr int WS_OFF_GL = Tile<64>::GL;
constexpr size_t WS_TILE_BYTES = Tile<64>::BYTES;
hipError_t launch_kda_map(const KdaArgs &a, bool f16, hipStream_t stream);
// The chain over tiles of `chunk` tokens (32, 64 or 128).
hipError_t launch_kda_chain(const KdaArgs &a, bool f16, int chunk, hipStream_t stream);
int kda_map_lds_bytes();
int kda_chain_lds_bytes();
// The scalar-gate map (KdaArgs::g is [T_tot, Hv]) into the same workspace tiles, read by
// launch_kda_chain.
hipError_t launch_gdn_map(const KdaArgs &a, bool f16, int chunk, hipStream_t stream);
// The segmented chain (the chain kernel in its segment mode), then the two kernels that join
// the segments (gdn_seg.hip): the segments' start states, and the outputs' corrections.
hipError_t launch_seg_chain(const KdaArgs &a, bool f16, int chunk, hipStream_t stream);
hipError_t launch_seg_join(const KdaArgs &a, hipStream_t stream);
hipError_t launch_seg_fix(const KdaArgs &a, bool f16, int chunk, hipStream_t stream);
// one token with a per-key-channel gate: DecodeArgs::g is [B, Hv, 128]
hipError_t launch_kda_decode(const DecodeArgs &a, int io, hipStream_t stream);

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
// The same kernel with the fused input prologue (a.prologue flags).
hipError_t launch_prefill_pipe_prologue(const PrefillArgs &a, bool f16, int grid, hipStream_t stream);
int prefill_pipe_prologue_lds_bytes();

}  // namespace gdn
