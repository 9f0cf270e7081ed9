// Chain half of the two-launch chunked prefill for gfx950 (per-key-channel decay, and the
// scalar gate of gdn_prefill_split), over chunks of C = 32, 64 or 128 tokens.
//
// The map kernels (kda_map.hip, gdn_map.hip) have left, per chunk and value head, the
// products that do not depend on the state: with T = (I + A)^-1,
//   W = T diag(beta) Kg,  U = T diag(beta) V,  P,  Qg,  Kl,  gl = exp(Gamma_last)
// (Kg = K (.) exp(Gamma), Qg = Q (.) exp(Gamma), Kl = K (.) exp(Gamma_last - Gamma)).  What
// remains depends on the state S (Dv x Dk) and runs chunk after chunk, as ops #5-#6 of the
// Map-Reduce-Map pipeline ("Empowering Hybrid Attention Models on NPUs", section 2.1; the
// chunk-first order of section 5):
//
//   v = U - W S^T            (= T diag(beta) (V - Kg S^T), the WY form of the solve)
//   O = Qg S^T + P v,
//   S <- S Diag(gl) + v^T Kl.
//
// With the inverse applied in the map, v is one product with S away from the state, and a
// chunk needs two dependent stages on the chain's critical path instead of three.  The
// chain waves follow gdn_prefill_pipe.hip (the state slice in registers, W S^T and Q S^T
// from a 16-bit copy of it in LDS, the update in place) with every product in fp16.  The
// column-wise split of S is the same: one workgroup per (sequence, value head, 16 value
// channels).
//
// Kl and U come from the map transposed (Kl^T [key][token], U^T [value ch][token]), so
// the update's Kl^T operand and the U term of v are plain row segments in LDS.
//
// Roles: waves 0-3 load the workspace tiles one chunk ahead and commit them to LDS, and
// form the outputs, which nothing downstream in the chunk waits for; waves 4-7 run only
// the recurrence.  Wave W (of either group) owns the 16-token tiles W and W + 4 of the
// chunk (those that exist) for v, Q S^T and O, and key channels [32W, 32W + 32) for the
// update.  A chunk takes two barrier-separated phases:
//   phase 1: chain v(c)        | loaders: commit P, Kl, gl of c; Q S^T(c) from the state copy
//   phase 2: chain S update    | loaders: commit W, Qg, U of c + 1; O(c) = Q S^T + P v
// Each tile is committed after its last reader of the previous chunk and before its
// first reader, so one LDS copy of every tile suffices.  LDS is 74 KB at C = 64 and
// 154 KB at C = 128.
#include "gdn_device.h"
#include "gdn_launch.h"

#include <type_traits>

namespace gdn {
namespace kdachain {

typedef _Float16 hf;

constexpr int DK = 128;
constexpr int DV = 128;
constexpr int DVS = 16;        // value channels per workgroup
constexpr int THREADS = 512;   // 4 loader + 4 chain waves
constexpr int KS = DK + 16;    // fp16 row stride of W, Qg and the state copy (288 B)

template <int C>
struct Cfg {
    static constexpr int NT = C / 16;          // 16-token tiles
    static constexpr int TPW = (NT + 3) / 4;   // tiles per wave (0 for waves 2, 3 at C = 32)
    // (ownership tests are written so that the compiler drops them wherever every wave owns
    // its tiles: a branch around the loaders' loads or stores makes the compiler's count of
    // outstanding vector-memory operations conservative)
    static constexpr int TS = C + 16;          // fp16 row stride of v^T
    static constexpr int TP = C + 8;           // fp16 row stride of P, Kl^T and U^T
    static constexpr int SEGS = C / 8;         // 16-byte segments per C-token row
    static constexpr int KL_N = 128 * SEGS / 256;           // Kl^T segments per loader thread
    static constexpr int P_SEGS = C * SEGS;                 // P segments (128 at C = 32)
    static constexpr int P_N = (P_SEGS + 255) / 256;
    static constexpr int W_N = C * 16 / 256;                // W, Qg segments per loader thread
    static constexpr int U_SEGS = 16 * SEGS;                // the U^T slice's segments
};

template <int C>
struct __align__(16) Smem {
    using F = Cfg<C>;
    hf S[DVS * KS];            // fp16 copy of the state slice [value ch][key ch]
    hf Vh[DVS * F::TS];        // v^T
    hf U[DVS * F::TP];         // U^T slice [value ch][token]
    float gl[DK];              // exp(Gamma_last) per key channel
    hf P[C * F::TP];
    hf W[C * KS];
    hf Qg[C * KS];
    hf Kl[DK * F::TP];         // Kl^T [key ch][token]
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Loader registers: the tiles of one chunk between their load and their commit.
template <int C>
struct StageA {       // P, Kl^T, gl: read in phase 2
    u32x4 p[Cfg<C>::P_N], kl[Cfg<C>::KL_N], gl;
};
template <int C>
struct StageB {       // W, Qg, U^T: read in phase 1
    u32x4 w[Cfg<C>::W_N], qg[Cfg<C>::W_N], u;
};

struct Work {
    const char *ws;       // workspace tile of this (sequence, head) at its first chunk
    size_t slot_stride;   // bytes from one chunk's tile to the next (Hv tiles)
    int bos, eos, nchunks, h, dv0;
};

__device__ __forceinline__ int chunk_clamp(const Work &wk, int c) { return min(c, wk.nchunks - 1); }

// Loader thread ld (0..255).  Where a tile has fewer segments than threads, the rest read
// its last segment again and do not commit.
template <int C>
__device__ __forceinline__ void load_a(StageA<C> &st, const Work &wk, int c, int ld) {
    using F = Cfg<C>;
    const char *tile = wk.ws + (size_t)chunk_clamp(wk, c) * wk.slot_stride;
#pragma unroll
    for (int p = 0; p < F::P_N; ++p)
        st.p[p] = *reinterpret_cast<const u32x4 *>(
            tile + Tile<C>::P + (F::P_SEGS % 256 != 0 ? min(ld + 256 * p, F::P_SEGS - 1) : ld + 256 * p) * 16);
#pragma unroll
    for (int p = 0; p < F::KL_N; ++p)
        st.kl[p] = *reinterpret_cast<const u32x4 *>(tile + Tile<C>::KLT + (ld + 256 * p) * 16);
    st.gl = *reinterpret_cast<const u32x4 *>(tile + Tile<C>::GL + (ld & 31) * 16);
}

template <int C>
__device__ __forceinline__ void commit_a(const StageA<C> &st, Smem<C> &s, int ld) {
    using F = Cfg<C>;
#pragma unroll
    for (int p = 0; p < F::P_N; ++p) {
        const int idx = ld + 256 * p, row = idx / F::SEGS, seg = idx % F::SEGS;
        // a guard only where P has fewer segments than threads (C = 32): a branch here
        // would make the compiler's count of outstanding loads conservative
        if constexpr (F::P_SEGS % 256 != 0) {
            if (idx < F::P_SEGS) *reinterpret_cast<u32x4 *>(&s.P[row * F::TP + seg * 8]) = st.p[p];
        } else {
            *reinterpret_cast<u32x4 *>(&s.P[row * F::TP + seg * 8]) = st.p[p];
        }
    }
#pragma unroll
    for (int p = 0; p < F::KL_N; ++p) {
        const int idx = ld + 256 * p, row = idx / F::SEGS, seg = idx % F::SEGS;
        *reinterpret_cast<u32x4 *>(&s.Kl[row * F::TP + seg * 8]) = st.kl[p];
    }
    if (ld < 32) *reinterpret_cast<u32x4 *>(&s.gl[ld * 4]) = st.gl;
}

template <int C>
__device__ __forceinline__ void load_b(StageB<C> &st, const Work &wk, int c, int ld) {
    using F = Cfg<C>;
    const char *tile = wk.ws + (size_t)chunk_clamp(wk, c) * wk.slot_stride;
#pragma unroll
    for (int p = 0; p < F::W_N; ++p) {
        st.w[p] = *reinterpret_cast<const u32x4 *>(tile + Tile<C>::W + (ld + 256 * p) * 16);
        st.qg[p] = *reinterpret_cast<const u32x4 *>(tile + Tile<C>::QG + (ld + 256 * p) * 16);
    }
    // U^T slice: 16 rows (value channels dv0 ..) x C / 8 segments
    const int ui = F::U_SEGS >= 256 ? ld : (ld & (F::U_SEGS - 1)), ur = ui / F::SEGS, us = ui % F::SEGS;
    st.u = *reinterpret_cast<const u32x4 *>(tile + Tile<C>::UT + ((wk.dv0 + ur) * C + 8 * us) * 2);
}

template <int C>
__device__ __forceinline__ void commit_b(const StageB<C> &st, Smem<C> &s, int ld) {
    using F = Cfg<C>;
#pragma unroll
    for (int p = 0; p < F::W_N; ++p) {
        const int idx = ld + 256 * p, row = idx >> 4, seg = idx & 15;
        *reinterpret_cast<u32x4 *>(&s.W[row * KS + seg * 8]) = st.w[p];
        *reinterpret_cast<u32x4 *>(&s.Qg[row * KS + seg * 8]) = st.qg[p];
    }
    if (ld < F::U_SEGS) *reinterpret_cast<u32x4 *>(&s.U[(ld / F::SEGS) * F::TP + 8 * (ld % F::SEGS)]) = st.u;
}

// Phase 1, chain wave W: v = ukeep U - W S^T for its token tiles (lane = value channel, rows
// = tokens), stored transposed.  ukeep is 1, or 0 for the identity rows of a segment.
template <int C>
__device__ __forceinline__ void chain_v(Smem<C> &s, int W, int l16, int g4, float ukeep) {
    using F = Cfg<C>;
    const hf *srow = s.S + l16 * KS + 8 * g4;
    Frag<hf> fs[4];
#pragma unroll
    for (int k = 0; k < F::TPW; ++k) {
        const int t = W + 4 * k;
        if (F::NT >= 4 * (k + 1) || t < F::NT) {   // compile-time true unless C = 32
            const hf *wrow = s.W + (16 * t + l16) * KS + 8 * g4;
            f32x4 ws = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                if (k == 0) fs[kb].load8(srow + 32 * kb);   // interleaved with the first tile's
                Frag<hf> fw;
                fw.load8(wrow + 32 * kb);
                mma(ws, fw, fs[kb]);
            }
            const int t0 = 16 * t + 4 * g4;
            const f16x4 u = *reinterpret_cast<const f16x4 *>(&s.U[l16 * F::TP + t0]);
            f16x4 x;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (hf)(ukeep * (float)u[i] - ws[i]);
            *reinterpret_cast<f16x4 *>(&s.Vh[l16 * F::TS + t0]) = x;
        }
    }
}

// Phase 1, loader wave W (off the chain's critical path): (Q S^T)^T = S Qg^T for its
// token tiles (lane = token, rows = value channels 4G..4G+3), from the state copy, which
// holds the chunk's starting state until phase 2.
template <int C>
__device__ __forceinline__ void loader_QS(const Smem<C> &s, int W, int l16, int g4, f32x4 (&qs)[Cfg<C>::TPW]) {
    using F = Cfg<C>;
    const hf *srow = s.S + l16 * KS + 8 * g4;
    Frag<hf> fs[4];
#pragma unroll
    for (int k = 0; k < F::TPW; ++k) {
        const int t = W + 4 * k;
        qs[k] = zero4();
        if (F::NT >= 4 * (k + 1) || t < F::NT) {   // compile-time true unless C = 32
            const hf *qrow = s.Qg + (16 * t + l16) * KS + 8 * g4;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                if (k == 0) fs[kb].load8(srow + 32 * kb);
                Frag<hf> fq;
                fq.load8(qrow + 32 * kb);
                mma(qs[k], fs[kb], fq);
            }
        }
    }
}

// Phase 2, loader wave W: O^T = S Qg^T + v^T P^T for its token tiles, stored as IO to o.
// In the segment mode `kind` picks the destination, all [token][head][channel]: 0 IO to o
// (segment 0), 1 fp16 to a.o0 (value rows of later segments), 2 fp16 to a.e (identity
// rows); one 8-byte store for each, with no branch between them (a branch around stores
// here would make the compiler's count of outstanding vector-memory operations
// conservative).
template <typename IO, int C, bool SEG>
__device__ __forceinline__ void loader_O(const Smem<C> &s, const KdaArgs &a, int W, int l16, int g4,
                                         const f32x4 (&qs)[Cfg<C>::TPW], int h, int dv0, int tok0, int nval,
                                         int kind) {
    using F = Cfg<C>;
#pragma unroll
    for (int k = 0; k < F::TPW; ++k) {
        const int t = W + 4 * k;
        if (F::NT >= 4 * (k + 1) || t < F::NT) {   // compile-time true unless C = 32
            f32x4 acc = qs[k];
            const hf *ph = s.P + (16 * t + l16) * F::TP + 8 * g4;
#pragma unroll
            for (int kb = 0; kb < (C >= 64 ? 2 : 1) + 2 * k; ++kb) {
                // tokens 32kb ..: past the diagonal P is zero (tiles W < 2 at C = 64 take
                // the zero block rather than a branch)
                Frag<hf> fp, fv;
                fp.load8(ph + 32 * kb);
                fv.load8(s.Vh + l16 * F::TS + 32 * kb + 8 * g4);
                mma(acc, fv, fp);
            }
            const int tok = 16 * t + l16;
            const size_t at = ((size_t)(tok0 + tok) * a.Hv + h) * DV + dv0 + 4 * g4;
            if constexpr (SEG) {
                typename Vec4<IO>::type yio;
                f16x4 yh;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    yio[i] = Cvt<IO>::from_f32(acc[i]);
                    yh[i] = (hf)acc[i];
                }
                typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
                const u32x2 bits = kind == 0 ? __builtin_bit_cast(u32x2, yio) : __builtin_bit_cast(u32x2, yh);
                char *base = kind == 0 ? (char *)a.o : kind == 1 ? (char *)a.o0 : (char *)a.e;
                if (tok < nval) *reinterpret_cast<u32x2 *>(base + at * 2) = bits;
            } else if (tok < nval) {
                typename Vec4<IO>::type y;
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = Cvt<IO>::from_f32(acc[i]);
                *reinterpret_cast<typename Vec4<IO>::type *>(reinterpret_cast<IO *>(a.o) + at) = y;
            }
        }
    }
}

// Phase 2, chain wave W: the update of key channels [32W, 32W + 32) of the state slice:
// S^T rows (key channels) 32W + 16mt + 4G + r, column = value channel.
template <int C>
__device__ __forceinline__ void chain_update(Smem<C> &s, int W, int l16, int g4, f32x4 (&st)[2]) {
    using F = Cfg<C>;
    Frag<hf> fv[C / 32];   // v^T rows (value channel l16), tokens 32kb + 8g4 .. + 7
#pragma unroll
    for (int kb = 0; kb < C / 32; ++kb) fv[kb].load8(s.Vh + l16 * F::TS + 32 * kb + 8 * g4);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        // Kl^T rows 32W + 16mt + l16 (key channels), tokens 32kb + 8g4 .. + 7
        const hf *kr = s.Kl + (32 * W + 16 * mt + l16) * F::TP + 8 * g4;
        const int kc = 32 * W + 16 * mt + 4 * g4;
        const f32x4 gl = *reinterpret_cast<const f32x4 *>(&s.gl[kc]);
        f32x4 acc = st[mt] * gl;
#pragma unroll
        for (int kb = 0; kb < C / 32; ++kb) {
            Frag<hf> fk;
            fk.load8(kr + 32 * kb);
            mma(acc, fk, fv[kb]);
        }
        st[mt] = acc;
        f16x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (hf)acc[i];
        *reinterpret_cast<f16x4 *>(&s.S[l16 * KS + kc]) = x;
    }
}

// The sequence of rank r when the N <= 64 sequences of cu are ordered by decreasing length
// (ties by index), by one wave: lane i counts the sequences ahead of sequence i.
__device__ __forceinline__ int longest_first(const int32_t *cu, int N, int r, int lane) {
    const int len = lane < N ? cu[lane + 1] - cu[lane] : -1;
    int rank = 0;
    for (int j = 0; j < N; ++j) {
        const int lj = __shfl(len, j, 64);
        rank += (lj > len || (lj == len && j < lane)) ? 1 : 0;
    }
    const unsigned long long hit = __ballot(lane < N && rank == r);
    return hit ? __builtin_ctzll(hit) : r;
}

// SEG: the segment mode of the Chunk-Seg-Seg mapping ("Empowering Hybrid Attention Models on
// NPUs", section 4, Figure 7): each sequence's chunks split into a.nseg runs.  Per
// (sequence, head), segment 0 has the 8 value slices, from the initial state; every later
// segment has 8 value slices from a zero state and 8 slices of identity rows (state X = I
// and no U term), whose outputs E and end state X carry the segment's dependence on its
// real start state.  Segment 0 stores its outputs to o; later segments store theirs as
// fp16 to a.o0 (value rows) or a.e (identity rows); end states go to a.sseg (X
// transposed).  gdn_seg.hip joins them.
template <typename IO, int C, bool SEG>
__global__ __launch_bounds__(THREADS) void kda_chain_kernel(const KdaArgs a) {
    using F = Cfg<C>;
    __shared__ Smem<C> s;
    const int tid = threadIdx.x;
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_loader = wave < 4;
    const int W = wave & 3;

    constexpr int NSL = DV / DVS;
    // XCD-aware mapping.  Workgroups are dispatched to the 8 XCDs in turn (blockIdx % 8).
    // The GS workgroups that read the same tiles (a head's 8 slices; in the segment mode a
    // segment's value and identity slices) form a group, and group g runs on XCD g % 8, so
    // its tiles are fetched into one L2.  The grid is padded to whole rounds of 8 groups;
    // the padding workgroups leave at once.
    constexpr int GS = SEG ? 2 * NSL : NSL;
    const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
    const int item = GS * (xcd + 8 * (kx / GS)) + kx % GS;
    if (item >= a.N * a.Hv * (SEG ? GS * a.nseg : NSL)) return;
    int slice, h, n, seg = 0;
    bool ident = false;
    if constexpr (SEG) {
        const int per = GS * a.nseg;   // item slots per (sequence, head)
        const int i = item % per;
        h = (item / per) % a.Hv;
        n = item / (per * a.Hv);
        seg = i / GS;
        ident = i % GS >= NSL;
        slice = i % NSL;
        if (seg == 0 && ident) return;   // segment 0 runs from the real state: no identity rows
    } else {
        slice = item % NSL;
        h = (item / NSL) % a.Hv;
        n = item / (NSL * a.Hv);
        // A packed batch of up to 64 sequences runs longest first, so that the longest
        // chains start in the first round of workgroups: item rank n takes the sequence
        // with the n-th most tokens (ties by index).
        if (a.cu && a.N > 1 && a.N <= 64) n = longest_first(a.cu, a.N, n, lane);
    }
    Work wk;
    wk.h = h;
    wk.dv0 = slice * DVS;
    const int bos = a.cu ? a.cu[n] : 0, eos = a.cu ? a.cu[n + 1] : a.T_tot;
    const int len = eos > bos ? eos - bos : 0;
    const int nc = (len + C - 1) / C;
    // segment `seg`: chunks [seg nc / nseg, (seg + 1) nc / nseg) of the sequence
    const int c0 = SEG ? (int)((long long)seg * nc / a.nseg) : 0;
    const int c1 = SEG ? (int)((long long)(seg + 1) * nc / a.nseg) : nc;
    wk.bos = bos + c0 * C;
    wk.eos = SEG ? min(eos, bos + c1 * C) : eos;
    wk.nchunks = c1 - c0;
    wk.slot_stride = (size_t)a.Hv * Tile<C>::BYTES;
    wk.ws = a.ws + ((size_t)(bos / C + n + c0) * a.Hv + h) * Tile<C>::BYTES;
    const int kind = seg == 0 ? 0 : ident ? 2 : 1;
    const float ukeep = ident ? 0.f : 1.f;

    f32x4 st[2];
    const size_t sbase = ((size_t)n * a.Hv + h) * (size_t)DV * DK;
    if (!is_loader) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int dk = 32 * W + 16 * mt + 4 * g4;
            f32x4 x = zero4();
            if (seg == 0 && a.s0) x = *reinterpret_cast<const f32x4 *>(a.s0 + sbase + (size_t)(wk.dv0 + l16) * DK + dk);
            if (ident) {
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = dk + i == wk.dv0 + l16 ? 1.f : 0.f;
            }
            st[mt] = x;
            f16x4 y;
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = (hf)x[i];
            *reinterpret_cast<f16x4 *>(&s.S[l16 * KS + dk]) = y;
        }
    }

    if (wk.nchunks > 0) {
        StageA<C> sa;
        StageB<C> sb;
        if (is_loader) {
            load_b(sb, wk, 0, tid);
            commit_b(sb, s, tid);
            load_a(sa, wk, 0, tid);
            load_b(sb, wk, 1, tid);
        }
        __syncthreads();
        if (is_loader) {
            for (int c = 0; c < wk.nchunks; ++c) {
                const int tok0 = wk.bos + c * C;
                const int nval = min(C, wk.eos - tok0);
                commit_a(sa, s, tid);
                load_a(sa, wk, c + 1, tid);
                f32x4 qs[F::TPW];
                loader_QS(s, W, l16, g4, qs);
                __syncthreads();
                commit_b(sb, s, tid);
                load_b(sb, wk, c + 2, tid);
                loader_O<IO, C, SEG>(s, a, W, l16, g4, qs, h, wk.dv0, tok0, nval, kind);
                __syncthreads();
            }
        } else {
            for (int c = 0; c < wk.nchunks; ++c) {
                chain_v(s, W, l16, g4, SEG ? ukeep : 1.f);
                __syncthreads();
                chain_update(s, W, l16, g4, st);
                __syncthreads();
            }
        }
    }

    if constexpr (SEG) {
        if (!is_loader) {
            float *sb = a.sseg + ((((size_t)n * a.Hv + h) * a.nseg + seg) * 2 + (ident ? 1 : 0)) * DV * DK;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int dk = 32 * W + 16 * mt + 4 * g4, r = wk.dv0 + l16;
                if (ident) {   // X^T [key][row]
#pragma unroll
                    for (int i = 0; i < 4; ++i) sb[(size_t)(dk + i) * DV + r] = st[mt][i];
                } else {
                    *reinterpret_cast<f32x4 *>(sb + (size_t)r * DK + dk) = st[mt];
                }
            }
        }
    } else if (a.sN && !is_loader) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int dk = 32 * W + 16 * mt + 4 * g4;
            *reinterpret_cast<f32x4 *>(a.sN + sbase + (size_t)(wk.dv0 + l16) * DK + dk) = st[mt];
        }
    }
}

}  // namespace kdachain

namespace {

template <bool SEG>
hipError_t chain_launch(const KdaArgs &a, bool f16, int chunk, hipStream_t stream) {
    // groups of GS workgroups (see the kernel), padded to whole rounds of 8 groups
    constexpr unsigned long long GS = (kdachain::DV / kdachain::DVS) * (SEG ? 2 : 1);
    const unsigned long long groups = (unsigned long long)a.N * a.Hv * (SEG ? (unsigned long long)a.nseg : 1ull);
    const unsigned long long wgs = 8 * GS * ((groups + 7) / 8);
    if (wgs > 0x7fffffffULL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs), block(kdachain::THREADS);
#define KDA_CHAIN_LAUNCH(C)                                                                                   \
    do {                                                                                                      \
        if (f16) hipLaunchKernelGGL((kdachain::kda_chain_kernel<_Float16, C, SEG>), grid, block, 0, stream, a); \
        else hipLaunchKernelGGL((kdachain::kda_chain_kernel<__bf16, C, SEG>), grid, block, 0, stream, a);      \
    } while (0)
    switch (chunk) {
        case 32: KDA_CHAIN_LAUNCH(32); break;
        case 64: KDA_CHAIN_LAUNCH(64); break;
        case 128: KDA_CHAIN_LAUNCH(128); break;
        default: return hipErrorInvalidValue;
    }
#undef KDA_CHAIN_LAUNCH
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kda_chain(const KdaArgs &a, bool f16, int chunk, hipStream_t stream) {
    return chain_launch<false>(a, f16, chunk, stream);
}

hipError_t launch_seg_chain(const KdaArgs &a, bool f16, int chunk, hipStream_t stream) {
    if (a.nseg < 1) return hipErrorInvalidValue;
    return chain_launch<true>(a, f16, chunk, stream);
}

int kda_chain_lds_bytes() { return (int)sizeof(kdachain::Smem<64>); }

}  // namespace gdn
