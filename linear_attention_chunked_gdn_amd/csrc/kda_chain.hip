// Chain half of the two-launch chunked prefill for gfx950 (per-key-channel decay, and the
// scalar gate of gdn_prefill_split), over chunks of C = 32, 64 or 128 tokens.
//
// The map kernels (kda_map.hip, gdn_map.hip) have left, per chunk and value head, the
// products that do not depend on the state: with T = (I + A)^-1,
//   WN = -T diag(beta) Kg,  U = T diag(beta) V,  P,  Qg,  Kl,  gl = exp(Gamma_last)
// (Kg = K (.) exp(Gamma), Qg = Q (.) exp(Gamma), Kl = K (.) exp(Gamma_last - Gamma)), as
// MFMA operand fragments (gdn_launch.h, Tile).  What remains depends on the state S
// (Dv x Dk) and runs chunk after chunk, as ops #5-#6 of the Map-Reduce-Map pipeline
// ("Empowering Hybrid Attention Models on NPUs", section 2.1; the chunk-first order of
// section 5):
//
//   v = U + WN S^T           (= T diag(beta) (V - Kg S^T), the WY form of the solve)
//   O = Qg S^T + P v,
//   S <- S Diag(gl) + v^T Kl.
//
// Value channels are independent in all three (S's rows never mix), so one workgroup
// owns 16 of them for one (sequence, value head) and needs nothing from the others.
//
// The recurrence runs on ONE wave and never leaves its registers.  It holds S^T (128 key
// x 16 value channels) as eight fp32 16x16 accumulators; read in pairs, an accumulator's
// rows are the eight reduction slots of an MFMA operand (the slot order pi of the tile
// layout), so fp16 copies of S^T are the B operands of v = U + WN S^T as they stand, and
// v's token tiles are likewise the B operands of the update S^T <- gl S^T + Kl^T v.  A
// chunk is 4 x C/16 + 8 x C/32 MFMAs (32 at C = 64) on one SIMD with no barrier between
// them.  Their A operands (WN, Kl, U, gl: 34.5 KB at C = 64) come from LDS: a wave64
// 16-byte global load holds the issuing wave ~16 cycles in the address unit, so the
// recurrence issues none.  Two loader waves (operand halves A: WN, U, gl and B: Kl)
// stream each chunk's tiles from L2 into a two-buffer LDS ring, issued two chunks ahead
// into a second register set.  (Each of a head's 8 workgroups reads the same tiles; a
// head's workgroups share one XCD and so one L2.)
//
// Two output waves form O^T = S Qg^T + v^T P^T, half of the token tiles each, from the
// fp16 state and v fragments the recurrence wave leaves in one of two LDS exchange slots
// per chunk, their Qg and P fragments loaded a chunk ahead from L2.  O^T puts four
// consecutive value channels of one token in a lane: one 8-byte store.
//
// One barrier per chunk orders the roles.  Between barriers c - 1 and c (barrier -1 ends
// the loaders' prologue, which puts chunk 0 in the ring): the recurrence wave reads ring
// buffer c % 2 and fills exchange slot c % 2; the loaders put chunk c + 1 into buffer
// (c + 1) % 2, which the recurrence wave last read before barrier c - 1; the output waves
// read exchange slot (c - 1) % 2, filled before barrier c - 1 and refilled after barrier c.
//
// Measured and not kept (H16 T4096): three ring buffers with the next chunk's operands
// read in the shadow of the update products; progress counters in LDS instead of
// barriers; loaders and output waves split by chunk parity; the recurrence split over
// two waves by key halves with a partial-v exchange.  Each was slower: the operand
// stream, not the recurrence's issue, sets the chunk period (the tiles come from the
// Infinity Cache or HBM, whose round trip the two-chunk prefetch barely covers).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace kdachain {

typedef _Float16 hf;
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int DK = 128;
constexpr int DV = 128;
constexpr int DVS = 16;         // value channels per workgroup
constexpr int NSL = DV / DVS;   // workgroups per (sequence, head)
// wave 0: the recurrence; 1, 2: the outputs; 3, 4: the loaders (operand halves A, B)
constexpr int THREADS = 320;

template <int C>
struct Cfg {
    static constexpr int NT = C / 16;             // 16-token tiles
    static constexpr int KB = C / 32;             // 32-token reduction blocks
    static constexpr int OT = NT / 2;             // token tiles per output wave
    // loaders and output waves keep a second register set (loads issued two chunks
    // ahead) up to C = 64; at C = 128 one chunk's operands are already 128 registers
    static constexpr bool DB = C <= 64;
    // output wave o's k-th tile (the two waves take tiles 0, 3, 4, 7 and 1, 2, 5, 6, which
    // gives both the same number of P fragments) and its P fragment count
    __device__ static constexpr int tile(int k, int o) { return 4 * (k >> 1) + ((k & 1) ? 3 - o : o); }
    static constexpr int npf(int k) { return 2 * (k >> 1) + (k & 1) + 1; }
    static constexpr int NPO = OT == 1 ? 1 : OT == 2 ? 3 : 10;   // P fragments per output wave
};
static_assert(Cfg<64>::npf(0) + Cfg<64>::npf(1) == Cfg<64>::NPO, "");
static_assert(Cfg<128>::npf(0) + Cfg<128>::npf(1) + Cfg<128>::npf(2) + Cfg<128>::npf(3) == Cfg<128>::NPO, "");

__device__ __forceinline__ f32x4 mfma(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// LDS: the exchange slots and the operand ring (81 KB at C = 64, 153 KB at C = 128).
template <int C>
struct __align__(16) Smem {
    using F = Cfg<C>;
    f16x8 xs[2][(4 + F::KB) * 64];   // S^T (4) and v (KB) fragments, lane-major
    struct Ops {
        f16x8 w[F::NT * 4 * 64];  // WN fragments (t, kb), lane-major
        f16x8 kl[8 * F::KB * 64]; // Kl fragments (i, kb)
        u32x2 u[F::NT * 64];      // the workgroup's U slice, per token tile
        f32x4 gl[32];             // exp(Gamma_last) per key channel
    } ob[2];
};
static_assert(sizeof(Smem<128>) <= 160 * 1024 && sizeof(Smem<64>) <= 160 * 1024, "the LDS holds the ring");

struct Work {
    const char *ws;       // workspace tile of this (sequence, head) at its first chunk
    size_t slot_stride;   // bytes from one chunk's tile to the next (Hv tiles)
    int bos, eos, nchunks, h, dv0, slice;
};

// The workspace tile of chunk c as a buffer (clamped to the last chunk: prefetches past the
// end read it again).  Operands are read with buffer loads: a lane's byte offset is one
// VGPR for every load, the tile and the fragment offsets are scalars, so no load needs a
// 64-bit address computed in vector registers, and every access is bounded by the tile.
template <int C>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const Work &wk, int c) {
    const char *tile = wk.ws + (size_t)min(c, wk.nchunks - 1) * wk.slot_stride;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(tile), 0, (int)Tile<C>::BYTES, 0x00020000);
}

__device__ __forceinline__ f16x8 ld_frag(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// ---- loaders ------------------------------------------------------------------------

// The loaders' registers for one chunk: A takes gl, U and WN, B takes Kl.
template <int C, bool A>
struct LoadRegs;
template <int C>
struct LoadRegs<C, true> {
    f16x8 w[Cfg<C>::NT * 4];
    u32x2 u[Cfg<C>::NT];
    f32x4 gl;                 // lanes 0..31: 4 key channels each
};
template <int C>
struct LoadRegs<C, false> {
    f16x8 kl[8 * Cfg<C>::KB];
};

template <int C, bool A>
__device__ __forceinline__ void load_ops(LoadRegs<C, A> &rg, const Work &wk, int c, int lane) {
    using F = Cfg<C>;
    using TL = Tile<C>;
    const __amdgpu_buffer_rsrc_t r = tile_rsrc<C>(wk, c);
    if constexpr (A) {
        rg.gl = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (lane & 31), TL::GL, 0));
#pragma unroll
        for (int t = 0; t < F::NT; ++t)
            rg.u[t] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, 8 * lane, TL::u(wk.slice, t), 0));
#pragma unroll
        for (int t = 0; t < F::NT; ++t)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) rg.w[t * 4 + kb] = ld_frag(r, 16 * lane, TL::wn(t, kb));
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int kb = 0; kb < F::KB; ++kb) rg.kl[i * F::KB + kb] = ld_frag(r, 16 * lane, TL::kl(i, kb));
    }
}

template <int C, bool A>
__device__ __forceinline__ void store_ops(const LoadRegs<C, A> &rg, typename Smem<C>::Ops &ob, int lane) {
    using F = Cfg<C>;
    if constexpr (A) {
        if (lane < 32) ob.gl[lane] = rg.gl;
#pragma unroll
        for (int t = 0; t < F::NT; ++t) ob.u[t * 64 + lane] = rg.u[t];
#pragma unroll
        for (int j = 0; j < F::NT * 4; ++j) ob.w[j * 64 + lane] = rg.w[j];
    } else {
#pragma unroll
        for (int j = 0; j < 8 * F::KB; ++j) ob.kl[j * 64 + lane] = rg.kl[j];
    }
}

// A loader wave's run: before barrier c it puts chunk c + 1 into buffer (c + 1) % 2 from
// registers loaded two chunks earlier, and issues the loads of chunk c + 3 into them (one
// register set at C = 128: chunk c + 2, loaded right after).
template <int C, bool A>
__device__ __forceinline__ void loader_run(Smem<C> &sm, const Work &wk, int lane) {
    const int n = wk.nchunks;
    if constexpr (Cfg<C>::DB) {
        LoadRegs<C, A> r0, r1;
        load_ops(r0, wk, 0, lane);
        load_ops(r1, wk, 1, lane);
        store_ops(r0, sm.ob[0], lane);
        load_ops(r0, wk, 2, lane);
        __syncthreads();
        for (int c = 0; c < n; c += 2) {
            store_ops(r1, sm.ob[1], lane);
            load_ops(r1, wk, c + 3, lane);
            __syncthreads();
            if (c + 1 >= n) break;
            store_ops(r0, sm.ob[0], lane);
            load_ops(r0, wk, c + 4, lane);
            __syncthreads();
        }
    } else {
        LoadRegs<C, A> r0;
        load_ops(r0, wk, 0, lane);
        store_ops(r0, sm.ob[0], lane);
        load_ops(r0, wk, 1, lane);
        __syncthreads();
        for (int c = 0; c < n; ++c) {
            store_ops(r0, sm.ob[(c + 1) & 1], lane);
            load_ops(r0, wk, c + 2, lane);
            __syncthreads();
        }
    }
}

// ---- the recurrence -------------------------------------------------------------------

// One chunk c of the recurrence: v = ukeep U + WN S^T, then S^T <- gl S^T + Kl^T v, with
// the operands from ring buffer c % 2.  The fp16 S^T and v fragments go to exchange slot
// c % 2.  ukeep is 1, or 0 for the identity rows of a segment (no U term).
template <int C, bool PERCH>
__device__ __forceinline__ void chain_step(f32x4 (&st)[8], Smem<C> &sm, int c, int lane, bool ukeep) {
    using F = Cfg<C>;
    const typename Smem<C>::Ops &ob = sm.ob[c & 1];
    const int g4 = lane >> 4;
    // the v phase's operands first, then the update's (LDS returns them in order)
    f16x8 w[F::NT][4];
    u32x2 u[F::NT];
#pragma unroll
    for (int t = 0; t < F::NT; ++t) u[t] = ob.u[t * 64 + lane];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int t = 0; t < F::NT; ++t) w[t][kb] = ob.w[(t * 4 + kb) * 64 + lane];
    f32x4 gl[PERCH ? 8 : 1];
    if constexpr (PERCH) {
#pragma unroll
        for (int i = 0; i < 8; ++i) gl[i] = ob.gl[4 * i + g4];
    } else {
        gl[0] = ob.gl[0];
    }
    f16x8 kl[8][F::KB];
#pragma unroll
    for (int kb = 0; kb < F::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) kl[i][kb] = ob.kl[(i * F::KB + kb) * 64 + lane];

    f16x8 *xs = sm.xs[c & 1];
    f16x8 sb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sb[kb][e] = (hf)st[2 * kb][e];
            sb[kb][4 + e] = (hf)st[2 * kb + 1][e];
        }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) xs[kb * 64 + lane] = sb[kb];
    f32x4 v[F::NT];
#pragma unroll
    for (int t = 0; t < F::NT; ++t) {
        const f16x4 uu = __builtin_bit_cast(f16x4, u[t]);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[t][q] = ukeep ? (float)uu[q] : 0.f;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int t = 0; t < F::NT; ++t) v[t] = mfma(w[t][kb], sb[kb], v[t]);
    // the decay of the state (off the v products' path)
    if constexpr (PERCH) {
#pragma unroll
        for (int i = 0; i < 8; ++i) st[i] *= gl[i];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) st[i] *= gl[0][0];
    }
    f16x8 vb[F::KB];
#pragma unroll
    for (int kb = 0; kb < F::KB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vb[kb][e] = (hf)v[2 * kb][e];
            vb[kb][4 + e] = (hf)v[2 * kb + 1][e];
        }
#pragma unroll
    for (int kb = 0; kb < F::KB; ++kb) xs[(4 + kb) * 64 + lane] = vb[kb];
#pragma unroll
    for (int kb = 0; kb < F::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 8; ++i) st[i] = mfma(kl[i][kb], vb[kb], st[i]);
}

// ---- the outputs ----------------------------------------------------------------------

template <int C>
struct OutOps {
    using F = Cfg<C>;
    f16x8 qg[F::OT][4];
    f16x8 p[F::NPO];
};

template <int C>
__device__ __forceinline__ void load_out(OutOps<C> &op, const Work &wk, int c, int o, int lane) {
    using F = Cfg<C>;
    using TL = Tile<C>;
    const __amdgpu_buffer_rsrc_t r = tile_rsrc<C>(wk, c);
    int pi = 0;
#pragma unroll
    for (int k = 0; k < F::OT; ++k) {
        const int t = F::tile(k, o);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) op.qg[k][kb] = ld_frag(r, 16 * lane, TL::qg(t, kb));
#pragma unroll
        for (int j = 0; j < F::npf(k); ++j) op.p[pi++] = ld_frag(r, 16 * lane, TL::p(t, j));
    }
}

// Chunk c's outputs on output wave o: O^T = S Qg^T + v^T P^T for its token tiles, from the
// exchange slot.  In the segment mode `kind` picks the destination, all
// [token][head][channel]: 0 IO to o (segment 0), 1 fp16 to a.o0 (value rows of later
// segments), 2 fp16 to a.e (identity rows); one 8-byte store for each, with no branch
// between them.
template <typename IO, int C, bool SEG>
__device__ __forceinline__ void out_step(const OutOps<C> &op, const Smem<C> &sm, int c, const KdaArgs &a, int o,
                                         int lane, int h, int dv0, int tok0, int nval, int kind) {
    using F = Cfg<C>;
    const int l16 = lane & 15, g4 = lane >> 4;
    const f16x8 *xs = sm.xs[c & 1];
    f16x8 sb[4], vb[F::KB];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) sb[kb] = xs[kb * 64 + lane];
#pragma unroll
    for (int kb = 0; kb < F::KB; ++kb) vb[kb] = xs[(4 + kb) * 64 + lane];
    int pi = 0;
#pragma unroll
    for (int k = 0; k < F::OT; ++k) {
        const int t = F::tile(k, o);
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc = mfma(sb[kb], op.qg[k][kb], acc);
#pragma unroll
        for (int j = 0; j < F::npf(k); ++j) acc = mfma(vb[j], op.p[pi++], acc);
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

// Output wave o's run: after barrier c it forms chunk c's outputs; before barrier c it
// issues the loads of chunk c + 1 into its other register set (one set at C = 128).
template <typename IO, int C, bool SEG>
__device__ __forceinline__ void output_run(const Smem<C> &sm, const KdaArgs &a, const Work &wk, int o, int lane,
                                           int kind) {
    using F = Cfg<C>;
    const int n = wk.nchunks;
    auto step = [&](const OutOps<C> &op, int c) {
        const int tok0 = wk.bos + c * C;
        out_step<IO, C, SEG>(op, sm, c, a, o, lane, wk.h, wk.dv0, tok0, min(C, wk.eos - tok0), kind);
    };
    if constexpr (F::DB) {
        OutOps<C> op0, op1;
        load_out(op0, wk, 0, o, lane);
        __syncthreads();
        for (int c = 0; c < n; c += 2) {
            load_out(op1, wk, c + 1, o, lane);
            __syncthreads();
            step(op0, c);
            if (c + 1 >= n) break;
            load_out(op0, wk, c + 2, o, lane);
            __syncthreads();
            step(op1, c + 1);
        }
    } else {
        OutOps<C> op0;
        __syncthreads();
        for (int c = 0; c < n; ++c) {
            load_out(op0, wk, c, o, lane);
            __syncthreads();
            step(op0, c);
        }
    }
}

// ---- the kernel ------------------------------------------------------------------------

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
template <typename IO, int C, bool SEG, bool PERCH>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void kda_chain_kernel(const KdaArgs a) {
    __shared__ Smem<C> sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

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
    wk.slice = slice;
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
    const size_t sbase = ((size_t)n * a.Hv + h) * (size_t)DV * DK;
    const int l16 = lane & 15, g4 = lane >> 4;

    if (wave == 0) {
        // S^T rows (key channels) 16 i + 4 G + q, column = value channel dv0 + m
        f32x4 st[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int dk = 16 * i + 4 * g4;
            f32x4 x = zero4();
            if (seg == 0 && a.s0) x = *reinterpret_cast<const f32x4 *>(a.s0 + sbase + (size_t)(wk.dv0 + l16) * DK + dk);
            if (ident) {
#pragma unroll
                for (int q = 0; q < 4; ++q) x[q] = dk + q == wk.dv0 + l16 ? 1.f : 0.f;
            }
            st[i] = x;
        }
        if (wk.nchunks > 0) {
            __syncthreads();   // the loaders' prologue: chunk 0 is in the ring
            for (int c = 0; c < wk.nchunks; ++c) {
                chain_step<C, PERCH>(st, sm, c, lane, !ident);
                __syncthreads();
            }
        }
        if constexpr (SEG) {
            float *sb = a.sseg + ((((size_t)n * a.Hv + h) * a.nseg + seg) * 2 + (ident ? 1 : 0)) * DV * DK;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int dk = 16 * i + 4 * g4, r = wk.dv0 + l16;
                if (ident) {   // X^T [key][row]
#pragma unroll
                    for (int q = 0; q < 4; ++q) sb[(size_t)(dk + q) * DV + r] = st[i][q];
                } else {
                    *reinterpret_cast<f32x4 *>(sb + (size_t)r * DK + dk) = st[i];
                }
            }
        } else if (a.sN) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<f32x4 *>(a.sN + sbase + (size_t)(wk.dv0 + l16) * DK + 16 * i + 4 * g4) = st[i];
        }
    } else if (wk.nchunks > 0 && wave < 3) {
        output_run<IO, C, SEG>(sm, a, wk, wave - 1, lane, kind);
    } else if (wk.nchunks > 0) {
        if (wave == 3) loader_run<C, true>(sm, wk, lane);
        else loader_run<C, false>(sm, wk, lane);
    }
}

}  // namespace kdachain

namespace {

template <bool SEG, bool PERCH>
hipError_t chain_launch(const KdaArgs &a, bool f16, int chunk, hipStream_t stream) {
    // groups of GS workgroups (see the kernel), padded to whole rounds of 8 groups
    constexpr unsigned long long GS = kdachain::NSL * (SEG ? 2 : 1);
    const unsigned long long groups = (unsigned long long)a.N * a.Hv * (SEG ? (unsigned long long)a.nseg : 1ull);
    const unsigned long long wgs = 8 * GS * ((groups + 7) / 8);
    if (wgs > 0x7fffffffULL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs), block(kdachain::THREADS);
#define KDA_CHAIN_LAUNCH(C)                                                                                           \
    do {                                                                                                              \
        if (f16) hipLaunchKernelGGL((kdachain::kda_chain_kernel<_Float16, C, SEG, PERCH>), grid, block, 0, stream, a); \
        else hipLaunchKernelGGL((kdachain::kda_chain_kernel<__bf16, C, SEG, PERCH>), grid, block, 0, stream, a);      \
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

hipError_t launch_kda_chain(const KdaArgs &a, bool f16, int chunk, bool per_channel, hipStream_t stream) {
    return per_channel ? chain_launch<false, true>(a, f16, chunk, stream) : chain_launch<false, false>(a, f16, chunk, stream);
}

hipError_t launch_seg_chain(const KdaArgs &a, bool f16, int chunk, bool per_channel, hipStream_t stream) {
    if (a.nseg < 1) return hipErrorInvalidValue;
    return per_channel ? chain_launch<true, true>(a, f16, chunk, stream) : chain_launch<true, false>(a, f16, chunk, stream);
}

int kda_chain_lds_bytes() { return (int)sizeof(kdachain::Smem<64>); }

}  // namespace gdn
