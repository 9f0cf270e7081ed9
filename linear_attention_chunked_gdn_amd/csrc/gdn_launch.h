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
    float *sseg;            // [N, Hv, nseg, 2, 128, 128] segment end states: segment 0's S [row][key], later
                            // segments' S from zero and X, both transposed [key][row]
    _Float16 *sin16;        // [N, Hv, nseg, 128, 128] start states of segments 1 .. nseg - 1
    uint32_t prologue;      // GDN_PROLOGUE_* flags of the scalar-gate map (0: none)
};
// Workspace tile of one chunk of C tokens and one value head, with T = (I + A)^-1 and the
// decays of the chunk:
//   WN = -T diag(beta) (K (.) exp(Gamma))            C tokens x 128 key channels
//   QG = Q (.) exp(Gamma)                            C tokens x 128 key channels
//   KL = K (.) exp(Gamma_last - Gamma)               C tokens x 128 key channels
//   P  = lower-incl-diagonal(Q K^T (.) decays)       C tokens x C tokens
//   U  = T diag(beta) V                              C tokens x 128 value channels
//   GL = exp(Gamma_last)                             128 key channels, fp32
// Everything but GL is fp16 and stored as MFMA operand fragments, so that the chain reads
// every operand with one coalesced 16-byte load per lane.  A fragment is 64 lanes x 16
// bytes: lane l = 16 G + m holds, for row m of a 16-row block, the eight entries of a
// 32-wide block kb of the reduction index j = 32 kb + pi(G, e), e = 0..7, with
//   pi(G, e) = 4 G + e (e < 4),   16 + 4 G + (e - 4) (e >= 4),
// the order in which a 16x16 fp32 accumulator pair holds its rows, so that results feed
// the next product without leaving registers.  Fragments:
//   WN, QG: (t, kb), t < C/16 token tiles, kb < 4: row = token 16 t + m, j = key channel
//   KL:     (i, kb), i < 8 key tiles, kb < C/32: row = key channel 16 i + m, j = token
//   P:      (t, kb) for kb <= t/2 only (the rest is zero): row = token 16 t + m, j = token
// and U in the fp32 accumulator order of the value rows: per value slice sl (16 channels)
// and token tile t, lane 16 G + m holds U[16 t + 4 G + r][16 sl + m], r = 0..3 (8 bytes).
template <int C> struct Tile {
    static constexpr int NT = C / 16;
    static constexpr int KB = C / 32;
    static constexpr int FRAG = 1024;
    // P fragments before token tile t: sum over t' < t of (t' / 2 + 1)
    static constexpr int pstart(int t) { return (t / 2) * (t / 2 + 1) + (t % 2) * (t / 2 + 1); }
    static constexpr int NPF = pstart(NT);
    static constexpr int WN = 0;
    static constexpr int QG = WN + NT * 4 * FRAG;
    static constexpr int KL = QG + NT * 4 * FRAG;
    static constexpr int P = KL + 8 * KB * FRAG;
    static constexpr int U = P + NPF * FRAG;
    static constexpr int GL = U + 8 * NT * 512;
    static constexpr size_t BYTES = (size_t)GL + 512;
    static constexpr int wn(int t, int kb) { return WN + (t * 4 + kb) * FRAG; }
    static constexpr int qg(int t, int kb) { return QG + (t * 4 + kb) * FRAG; }
    static constexpr int kl(int i, int kb) { return KL + (i * KB + kb) * FRAG; }
    static constexpr int p(int t, int kb) { return P + (pstart(t) + kb) * FRAG; }
    static constexpr int u(int sl, int t) { return U + (sl * NT + t) * 512; }
};
static_assert(Tile<32>::BYTES % 256 == 0 && Tile<64>::BYTES % 256 == 0 && Tile<128>::BYTES % 256 == 0,
              "tiles keep the workspace's 256-byte alignment");
static_assert(Tile<64>::NPF == 6 && Tile<32>::NPF == 2 && Tile<128>::NPF == 20, "P fragments of the lower triangle");
static_assert(Tile<64>::BYTES == 72192, "the documented tile size at C = 64");
// Byte offset inside a lane's 16-byte fragment piece, and the lane, of reduction index j of
// a 32-wide block (row m): the inverse of pi.
__host__ __device__ constexpr int frag_lane(int j, int m) { return 16 * ((j & 15) >> 2) + m; }
__host__ __device__ constexpr int frag_byte(int j) { return 2 * ((j & 3) + ((j & 16) >> 2)); }
// The per-key-channel path runs 64-token chunks.
constexpr size_t WS_TILE_BYTES = Tile<64>::BYTES;
hipError_t launch_kda_map(const KdaArgs &a, bool f16, hipStream_t stream);
// The chain over tiles of `chunk` tokens (32, 64 or 128); per_channel: GL differs per key
// channel (the KDA map), else one decay per chunk (the scalar-gate map); wide: two 16-value-
// channel slices per workgroup (chunks of up to 64 tokens), else one.
hipError_t launch_kda_chain(const KdaArgs &a, bool f16, int chunk, bool per_channel, bool wide, hipStream_t stream);
int kda_map_lds_bytes();
int kda_chain_lds_bytes();
// The chain kernel's workgroups per (sequence, head): one per 16 value channels, or with
// `wide` (chunks of up to 64 tokens) one per 32, whose two slices share every operand
// fragment (half the workgroups, each about twice as long per chunk).
int chain_workgroups_per_head(int chunk, bool wide);
// The scalar-gate map (KdaArgs::g is [T_tot, Hv]) into the same workspace tiles, read by
// launch_kda_chain.
hipError_t launch_gdn_map(const KdaArgs &a, bool f16, int chunk, hipStream_t stream);
// The segmented chain (the chain kernel in its segment mode), then the two kernels that join
// the segments (gdn_seg.hip): the segments' start states, and the outputs' corrections.
hipError_t launch_seg_chain(const KdaArgs &a, bool f16, int chunk, bool per_channel, bool wide, hipStream_t stream);
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
