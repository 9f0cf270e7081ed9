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
// owns 16 of them (or 32, as two slices) for one (sequence, value head) and needs nothing
// from the others.
//
// Eight waves share a workgroup (ten with two slices), one barrier per chunk:
//
// * Waves 0 .. 2 SPW - 1, the recurrence, two per slice of 16 value channels, one per half
//   of the key channels.  The wave of slice s and key half h holds rows 64 h .. 64 h + 63
//   of that slice's S^T as four fp32 16x16 accumulators that never leave its registers;
//   read in pairs, an accumulator's rows are the eight reduction slots of an MFMA operand
//   (the slot order pi of the tile layout), so fp16 copies of S^T are B operands as they
//   stand.  Per chunk, the wave reads its key half of WN and Kl from the LDS ring, forms
//   the partial p_h = WN[:, half h] S^T[half h], plus U on its half of the token tiles,
//   and writes it and its fp16 copy of S^T into exchange slot c % 2; after the barrier it
//   reads the other key half's partial, forms v = p_0 + p_1 in fp16 (addition commutes
//   exactly, so every wave that forms v gets the same values) and updates its half,
//   S^T[half h] <- gl S^T[half h] + Kl[half h]^T v, with v's token tiles as B operands.
//   U and gl come with WN and Kl through the ring (at C = 128 from L2 into registers, a
//   chunk ahead).
// * The next four waves, the outputs, one 16-token tile each (two at C = 128).  After
//   barrier c a wave reads slot c % 2 (S^T and both partials) and forms
//   O^T = S Qg^T + v^T P^T, its Qg and P fragments loaded from L2 into registers a chunk
//   ahead.  O^T puts four
//   consecutive value channels of one token in a lane; the tiles go out through LDS as
//   16-byte stores (a vector-memory instruction costs the CU's address and data path
//   about the same whatever its width): with two slices a wave's own tile (32 channels
//   per token), with one slice at C = 64 two waves' tiles after the next barrier.
// * The last two waves, the loaders, stream WN (with U) and Kl (with gl) into an NB-buffer
//   LDS ring with direct global-to-LDS loads, chunk c + NB into buffer c % NB after barrier c.
//
// Each of a head's workgroups reads the same tiles; they run on one XCD and so share one
// L2, from which a workgroup moves about 56 KB per chunk at C = 64.  With two slices per
// workgroup every WN, Kl, Qg and P fragment serves both: about the same bytes per chunk
// for twice the value channels, twice the output work, and two more recurrence waves.
//
// Measured and not kept (chain kernel at H16 T4096, against 44 us): one recurrence wave
// fed from the ring (47 us: its LDS reads of 34.5 KB per chunk set the period); the two
// recurrence waves loading their own WN and Kl from L2 (47.8 us); two barriers per chunk
// (65 us); Qg and P through a second LDS ring filled by two more loader waves (48-54 us);
// Qg replaced by the raw q rows, the decay applied by the output waves (62.8 us: a load
// instruction then touches 16 rows).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace kdachain {

typedef _Float16 hf;
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int DK = 128;
constexpr int DV = 128;

template <int C, int SPW_ = 1>
struct Cfg {
    static constexpr int NT = C / 16;             // 16-token tiles
    static constexpr int KB = C / 32;             // 32-token reduction blocks
    // 16-value-channel slices per workgroup: one, or two (their WN, Kl, Qg and P operands
    // shared in the same registers; up to C = 64, two would not fit the LDS at 128)
    static constexpr int SPW = SPW_;
    static_assert(SPW == 1 || (SPW == 2 && C <= 64), "two slices up to C = 64");
    static constexpr int DVS = 16 * SPW;          // value channels per workgroup
    // waves 0 .. NRW - 1: the recurrence (slice s = w / 2, key half w % 2); then four output
    // waves (token tiles t = 4 k + o) and two loaders (WN, Kl)
    static constexpr int NRW = 2 * SPW;
    static constexpr int THREADS = 64 * (NRW + 6);
    static constexpr int WPE = (NRW + 6 + 3) / 4;   // waves per SIMD
    static constexpr int NSL = DV / DVS;          // workgroups per (sequence, head)
    static constexpr int NW = NT * 4;             // WN fragments per chunk
    static constexpr int NK = 8 * KB;             // Kl fragments per chunk
    // U (the workgroup's slices) and gl travel with WN and Kl through the ring where the
    // LDS holds them (C <= 64): NU 1 KB pieces of U and one of gl per chunk.  At C = 128
    // the recurrence waves load them from L2 into registers.
    static constexpr bool URING = C <= 64;
    static constexpr int NU = URING ? SPW * NT / 2 : 0;
    static constexpr int NG = URING ? 1 : 0;
    // 1 KB direct-to-LDS loads per chunk of the WN loader (with U) and the Kl loader (with gl)
    static constexpr int nload(bool kl) { return kl ? NK + NG : NW + NU; }
    // operand ring depth: chunk c + NB - 1 is loaded while chunk c runs
    static constexpr int NB = C == 32 ? 4 : C == 64 ? 3 : 2;
    static constexpr int OT = NT >= 4 ? NT / 4 : 1;   // token tiles per output wave
    // P fragments of token tile t (its 32-token blocks up to its own), and of output wave o
    static constexpr int npf(int t) { return t / 2 + 1; }
    static constexpr int npo(int o) {
        int n = 0;
        for (int k = 0; k < OT; ++k)
            if (4 * k + o < NT) n += npf(4 * k + o);
        return n;
    }
};

__device__ __forceinline__ f32x4 mfma(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// LDS: the operand ring, two exchange slots and the output staging (125 KB at C = 64 with
// one slice, 147 KB with two, 152 KB at C = 128).
template <int C, int SPW>
struct __align__(16) Smem {
    using F = Cfg<C, SPW>;
    struct Ops {
        f16x8 w[F::NW * 64];   // WN fragments (t, kb), lane-major, as in the tile
        f16x8 kl[F::NK * 64];  // Kl fragments (i, kb)
        // the workgroup's U fragments (slice, token tile) as in the tile, then gl's 512
        // bytes (in a 1 KB piece)
        f16x8 ug[F::URING ? (F::NU + F::NG) * 64 : 1];
    } ob[F::NB];
    f16x8 xs[2][F::SPW * 4 * 64];             // S^T fragments (slice, key block)
    u32x2 pv[2][2][F::SPW][F::NT * 64];       // the recurrence waves' partials, fp16 (wave, slice, token tile)
    // output tiles on their way to 16-byte stores: with two slices each output wave's tile
    // (16 tokens x 32 channels, 1 KB); with one slice at C = 64 every wave's tile (16 x 16,
    // 512 B) of chunk c in half c % 2, stored with its neighbour's after the next barrier
    f16x8 ot[F::SPW == 2 || C == 64 ? 256 : 1];
};
static_assert(sizeof(Smem<32, 2>) <= 160 * 1024 && sizeof(Smem<64, 2>) <= 160 * 1024 && sizeof(Smem<128, 1>) <= 160 * 1024,
              "the LDS holds the ring");

struct Work {
    const char *ws;       // workspace tile of this (sequence, head) at its first chunk
    size_t slot_stride;   // bytes from one chunk's tile to the next (Hv tiles)
    int bos, eos, nchunks, h, dv0, slice;
};

// The workspace tile of chunk c as a buffer (clamped to the last chunk: prefetches past the
// end read it again).  Operands are read with buffer loads: a lane's byte offset is one
// VGPR for every load, the tile and the fragment offsets are scalars, so no load needs a
// 64-bit address computed in vector registers, and every access is bounded by the tile.
template <int C, int SPW>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const Work &wk, int c) {
    const char *tile = wk.ws + (size_t)min(c, wk.nchunks - 1) * wk.slot_stride;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(tile), 0, (int)Tile<C>::BYTES, 0x00020000);
}

__device__ __forceinline__ f16x8 ld_frag(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// ---- the loaders ---------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void;

// vmcnt(N) alone (gfx9 encoding: expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Chunk c's WN (KL false) or Kl fragments into ring buffer c % NB, one 1 KB fragment per
// instruction, global to LDS directly (lane l's 16 bytes land at 16 l: the fragment
// layout of the tile is kept).  The workgroups reading one tile start at different
// fragments (slice s at fragment 2 s), so that they do not all ask the L2 for the same
// lines at once.
template <int C, int SPW, bool KL>
__device__ __forceinline__ void dma_chunk(Smem<C, SPW> &sm, const Work &wk, int c, int lane) {
    using F = Cfg<C, SPW>;
    using TL = Tile<C>;
    const __amdgpu_buffer_rsrc_t r = tile_rsrc<C, SPW>(wk, c);
    typename Smem<C, SPW>::Ops &ob = sm.ob[c % F::NB];
    f16x8 *dst = KL ? ob.kl : ob.w;
    constexpr int NF = KL ? F::NK : F::NW;
    constexpr int SRC = KL ? TL::KL : TL::WN;
    static_assert((NF & (NF - 1)) == 0, "fragment counts are powers of two");
    const int rot = __builtin_amdgcn_readfirstlane(2 * wk.slice);
#pragma unroll
    for (int f0 = 0; f0 < NF; ++f0) {
        const int f = (f0 + rot) & (NF - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + 64 * f), 16, 16 * lane, SRC + 1024 * f, 0, 0);
    }
    if constexpr (F::URING) {
        if constexpr (KL) {   // gl's 512 bytes, the tile's last: lanes 0 .. 31
            if (lane < 32)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(ob.ug + 64 * F::NU), 16, TL::GL + 16 * lane, 0, 0, 0);
        } else {              // U of the workgroup's slices, contiguous in the tile
            const int u0 = __builtin_amdgcn_readfirstlane(TL::u(wk.slice * F::SPW, 0));
#pragma unroll
            for (int j = 0; j < F::NU; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(ob.ug + 64 * j), 16, 16 * lane, u0 + 1024 * j, 0, 0);
        }
    }
}

// A loader wave's run.  Chunk c's operands are read by the recurrence waves between
// barriers c - 1 and c, so chunk c + NB goes into buffer c % NB after barrier c, and
// chunk c + 1 must have landed before barrier c: the loads have NB - 1 chunks to land.
// Plain s_barrier: the waits on this wave's own loads are explicit (vmcnt counts them in
// issue order); it writes LDS only through the loads.
template <int C, int SPW, bool KL>
__device__ __forceinline__ void loader_run(Smem<C, SPW> &sm, const Work &wk, int lane) {
    using F = Cfg<C, SPW>;
    constexpr int NF = F::nload(KL);
#pragma unroll
    for (int j = 0; j < F::NB; ++j) dma_chunk<C, SPW, KL>(sm, wk, j, lane);
    wait_vmcnt<(F::NB - 1) * NF>();   // chunk 0
    __builtin_amdgcn_s_barrier();
    for (int c = 0; c < wk.nchunks; ++c) {
        wait_vmcnt<(F::NB - 2) * NF>();   // chunk c + 1
        __builtin_amdgcn_s_barrier();
        dma_chunk<C, SPW, KL>(sm, wk, c + F::NB, lane);
    }
    wait_vmcnt<0>();   // nothing in flight into the LDS when the workgroup ends
}

// ---- the recurrence -------------------------------------------------------------------

// The per-chunk operands besides WN and Kl of the recurrence wave of slice s and key half
// h: half of the token tiles of U's slice s (tiles h NT / 2 .. (h + 1) NT / 2 - 1, which
// its partials add) and its keys' decays gl (one value for the scalar gate).  From the ring where it carries
// them (ring_rec); at C = 128 from L2 a chunk ahead (load_rec: the same loads on both
// waves, so that the compiler's load counts are exact).  A vector-memory instruction
// costs the CU's address and data path about as much whatever its width, and these small
// loads on the recurrence waves took ~7 % of the chain's time at C = 64.
template <int C, int SPW, bool PERCH>
struct RecRegs {
    u32x2 u[Cfg<C, SPW>::NT / 2];
    f32x4 gl[PERCH ? 4 : 1];
};

template <int C, int SPW, bool PERCH>
__device__ __forceinline__ void load_rec(RecRegs<C, SPW, PERCH> &rg, const Work &wk, int c, int s, int h, int lane) {
    using F = Cfg<C, SPW>;
    using TL = Tile<C>;
    const __amdgpu_buffer_rsrc_t r = tile_rsrc<C, SPW>(wk, c);
#pragma unroll
    for (int t = 0; t < F::NT / 2; ++t)
        rg.u[t] = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, 8 * lane, TL::u(wk.slice * F::SPW + s, h * F::NT / 2 + t), 0));
    if constexpr (PERCH) {
        // keys 64 h + 16 i + 4 G + q: 16 bytes at GL + 4 (16 (4 h + i) + 4 G)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            rg.gl[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (lane >> 4),
                                                                                       TL::GL + 64 * (4 * h + i), 0));
    } else {
        rg.gl[0][0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 0, TL::GL, 0));
    }
}

template <int C, int SPW, bool PERCH>
__device__ __forceinline__ void ring_rec(RecRegs<C, SPW, PERCH> &rg, const Smem<C, SPW> &sm, int c, int s, int h,
                                         int lane) {
    using F = Cfg<C, SPW>;
    const typename Smem<C, SPW>::Ops &ob = sm.ob[c % F::NB];
    const u32x2 *u = reinterpret_cast<const u32x2 *>(ob.ug);
#pragma unroll
    for (int t = 0; t < F::NT / 2; ++t) rg.u[t] = u[(s * F::NT + h * F::NT / 2 + t) * 64 + lane];
    if constexpr (PERCH) {
        const f32x4 *g = reinterpret_cast<const f32x4 *>(ob.ug + 64 * F::NU);
#pragma unroll
        for (int i = 0; i < 4; ++i) rg.gl[i] = g[4 * (4 * h + i) + (lane >> 4)];
    } else {
        rg.gl[0][0] = reinterpret_cast<const float *>(ob.ug + 64 * F::NU)[0];
    }
}

// Key half h of WN and Kl for one chunk, from its ring buffer.
template <int C, int SPW>
struct RingRegs {
    f16x8 w[Cfg<C, SPW>::NT][2];
    f16x8 kl[4][Cfg<C, SPW>::KB];
};

template <int C, int SPW>
__device__ __forceinline__ void read_ring_w(RingRegs<C, SPW> &rr, const Smem<C, SPW> &sm, int c, int h, int lane) {
    using F = Cfg<C, SPW>;
    const typename Smem<C, SPW>::Ops &ob = sm.ob[c % F::NB];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int t = 0; t < F::NT; ++t) rr.w[t][j] = ob.w[(4 * t + 2 * h + j) * 64 + lane];
}

template <int C, int SPW>
__device__ __forceinline__ void read_ring_kl(RingRegs<C, SPW> &rr, const Smem<C, SPW> &sm, int c, int h, int lane) {
    using F = Cfg<C, SPW>;
    const typename Smem<C, SPW>::Ops &ob = sm.ob[c % F::NB];
#pragma unroll
    for (int kb = 0; kb < F::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) rr.kl[i][kb] = ob.kl[((4 * h + i) * F::KB + kb) * 64 + lane];
}

// Chunk c on the recurrence wave of slice s and key half h, around barrier c: its halves
// of WN and Kl from ring buffer c % NB, then the partial, the exchange with the other key
// half's wave, the update.  with_u is 0 for the identity rows of a segment (no U term).
template <int C, int SPW, bool PERCH>
__device__ __forceinline__ void rec_step(f32x4 (&st)[4], const RecRegs<C, SPW, PERCH> &rg, Smem<C, SPW> &sm, int c,
                                         int s, int h, int lane, bool with_u) {
    using F = Cfg<C, SPW>;
    RingRegs<C, SPW> cur;
    read_ring_w(cur, sm, c, h, lane);
    read_ring_kl(cur, sm, c, h, lane);
    f16x8 sb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sb[j][e] = (hf)st[2 * j][e];
            sb[j][4 + e] = (hf)st[2 * j + 1][e];
        }
    // U on this wave's half of the token tiles
    f32x4 p[F::NT];
#pragma unroll
    for (int t = 0; t < F::NT; ++t) {
        const f16x4 uu = __builtin_bit_cast(f16x4, rg.u[t % (F::NT / 2)]);
        const bool add = with_u && t / (F::NT / 2) == h;
#pragma unroll
        for (int q = 0; q < 4; ++q) p[t][q] = add ? (float)uu[q] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int t = 0; t < F::NT; ++t) p[t] = mfma(cur.w[t][j], sb[j], p[t]);
    f16x8 *xs = sm.xs[c & 1];
#pragma unroll
    for (int j = 0; j < 2; ++j) xs[(4 * s + 2 * h + j) * 64 + lane] = sb[j];
    // the decay of the state (off the partial's path)
    if constexpr (PERCH) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st[i] *= rg.gl[i];
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) st[i] *= rg.gl[0][0];
    }
    f16x4 ph[F::NT];
#pragma unroll
    for (int t = 0; t < F::NT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) ph[t][q] = (hf)p[t][q];
#pragma unroll
    for (int t = 0; t < F::NT; ++t) sm.pv[c & 1][h][s][t * 64 + lane] = __builtin_bit_cast(u32x2, ph[t]);
    __syncthreads();
    // v = p_0 + p_1 from the fp16 partials (addition commutes exactly: every wave that
    // forms v gets the same values), then the update
    f16x4 po[F::NT];
#pragma unroll
    for (int t = 0; t < F::NT; ++t) po[t] = __builtin_bit_cast(f16x4, sm.pv[c & 1][h ^ 1][s][t * 64 + lane]);
    f16x8 vb[F::KB];
#pragma unroll
    for (int kb = 0; kb < F::KB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vb[kb][e] = (hf)((float)ph[2 * kb][e] + (float)po[2 * kb][e]);
            vb[kb][4 + e] = (hf)((float)ph[2 * kb + 1][e] + (float)po[2 * kb + 1][e]);
        }
#pragma unroll
    for (int kb = 0; kb < F::KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[i] = mfma(cur.kl[i][kb], vb[kb], st[i]);
}

// The run of the recurrence wave of slice s and key half h: barrier -1 (chunk 0 in the
// ring), then a barrier per chunk; U and gl of chunk c come with its ring buffer, or
// (C = 128) those of chunk c + 1 are loaded while chunk c runs.
template <int C, int SPW, bool PERCH>
__device__ __forceinline__ void rec_run(f32x4 (&st)[4], Smem<C, SPW> &sm, const Work &wk, int s, int h, int lane,
                                        bool with_u) {
    const int n = wk.nchunks;
    if constexpr (Cfg<C, SPW>::URING) {
        __syncthreads();
        for (int c = 0; c < n; c += 2) {   // two chunks per trip, as below
            RecRegs<C, SPW, PERCH> r0, r1;
            ring_rec(r0, sm, c, s, h, lane);
            rec_step(st, r0, sm, c, s, h, lane, with_u);
            if (c + 1 >= n) break;
            ring_rec(r1, sm, c + 1, s, h, lane);
            rec_step(st, r1, sm, c + 1, s, h, lane, with_u);
        }
        return;
    }
    RecRegs<C, SPW, PERCH> r0, r1;
    load_rec(r0, wk, 0, s, h, lane);
    __syncthreads();
    for (int c = 0; c < n; c += 2) {
        load_rec(r1, wk, c + 1, s, h, lane);
        rec_step(st, r0, sm, c, s, h, lane, with_u);
        if (c + 1 >= n) break;
        load_rec(r0, wk, c + 2, s, h, lane);
        rec_step(st, r1, sm, c + 1, s, h, lane, with_u);
    }
}

// ---- the outputs ----------------------------------------------------------------------

// Output wave O's operands for one chunk: Qg and P fragments of its token tiles 4 k + O.
template <int C, int SPW, int O>
struct OutOps {
    using F = Cfg<C, SPW>;
    f16x8 qg[F::OT][4];
    f16x8 p[F::npo(O) > 0 ? F::npo(O) : 1];
};

template <int C, int SPW, int O>
__device__ __forceinline__ void load_out(OutOps<C, SPW, O> &op, const Work &wk, int c, int lane) {
    using F = Cfg<C, SPW>;
    using TL = Tile<C>;
    const __amdgpu_buffer_rsrc_t r = tile_rsrc<C, SPW>(wk, c);
    int pi = 0;
#pragma unroll
    for (int k = 0; k < F::OT; ++k) {
        const int t = 4 * k + O;
        if (t >= F::NT) continue;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) op.qg[k][kb] = ld_frag(r, 16 * lane, TL::qg(t, kb));
#pragma unroll
        for (int j = 0; j < F::npf(t); ++j) op.p[pi++] = ld_frag(r, 16 * lane, TL::p(t, j));
    }
}

// Chunk c's outputs on output wave O: O^T = S Qg^T + v^T P^T for its token tiles, from the
// exchange slot (S^T and the two partials of v).  In the segment mode `kind` picks the
// destination, all [token][head][channel]: 0 IO to o (segment 0), 1 fp16 to a.o0 (value
// rows of later segments), 2 fp16 to a.e (identity rows), with the same stores for each
// (bits and base pointer selected, no branch between them).
template <typename IO, int C, int SPW, bool SEG, int O>
__device__ __forceinline__ void out_step(const OutOps<C, SPW, O> &op, Smem<C, SPW> &sm, int c, const KdaArgs &a,
                                         int lane, int h, int dv0, int tok0, int nval, int kind, char *obase, bool last) {
    using F = Cfg<C, SPW>;
    // one slice at C = 64: the even output waves store chunk c - 1's tiles O and O + 1 (a
    // chunk before the last is whole), 16 bytes per lane: token 16 O + lane / 2, channels
    // dv0 + 8 (lane % 2) ..
    constexpr bool PAIR = SPW == 1 && C == 64;
    char *const stg = reinterpret_cast<char *>(sm.ot);
    if constexpr (PAIR) {
        if (O % 2 == 0 && c > 0) {
            const f16x8 row = *reinterpret_cast<const f16x8 *>(stg + ((c - 1) & 1) * 2048 + O * 512 + 16 * lane);
            const int tk = 16 * O + (lane >> 1);
            *reinterpret_cast<f16x8 *>(obase + (((size_t)(tok0 - C + tk) * a.Hv + h) * DV + dv0 + 8 * (lane & 1)) * 2) = row;
        }
    }
    const int l16 = lane & 15, g4 = lane >> 4;
    constexpr int TMAX = 4 * (F::OT - 1) + O;                   // its last token tile
    constexpr int VB = (TMAX < F::NT ? TMAX : F::NT - 1) / 2 + 1;  // v blocks it needs
    const f16x8 *xs = sm.xs[c & 1];
    f16x8 sb[SPW][4], vb[SPW][VB];
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sb[s][kb] = xs[(4 * s + kb) * 64 + lane];
    // v = p_0 + p_1, as the recurrence waves form it
#pragma unroll
    for (int s = 0; s < SPW; ++s)
#pragma unroll
        for (int kb = 0; kb < VB; ++kb)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const f16x4 a0 = __builtin_bit_cast(f16x4, sm.pv[c & 1][0][s][(2 * kb + j) * 64 + lane]);
                const f16x4 a1 = __builtin_bit_cast(f16x4, sm.pv[c & 1][1][s][(2 * kb + j) * 64 + lane]);
#pragma unroll
                for (int e = 0; e < 4; ++e) vb[s][kb][4 * j + e] = (hf)((float)a0[e] + (float)a1[e]);
            }
    int pi = 0;
#pragma unroll
    for (int k = 0; k < F::OT; ++k) {
        const int t = 4 * k + O;
        if (t >= F::NT) continue;
        f32x4 accs[SPW];
#pragma unroll
        for (int s = 0; s < SPW; ++s) accs[s] = zero4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int s = 0; s < SPW; ++s) accs[s] = mfma(sb[s][kb], op.qg[k][kb], accs[s]);
#pragma unroll
        for (int j = 0; j < F::npf(t); ++j) {
#pragma unroll
            for (int s = 0; s < SPW; ++s) accs[s] = mfma(vb[s][j], op.p[pi], accs[s]);
            ++pi;
        }
        const int tok = 16 * t + l16;
        if constexpr (SPW == 2) {
            // the tile's 32 channels per token through the wave's staging rows (64 bytes per
            // token): one 16-byte store per lane (token 16 t + lane / 4, channels
            // dv0 + 8 (lane % 4) ..) instead of two 8-byte ones
#pragma unroll
            for (int s = 0; s < SPW; ++s) {
                typename Vec4<IO>::type yio;
                f16x4 yh;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    yio[i] = Cvt<IO>::from_f32(accs[s][i]);
                    yh[i] = (hf)accs[s][i];
                }
                const u32x2 bits = !SEG || kind == 0 ? __builtin_bit_cast(u32x2, yio) : __builtin_bit_cast(u32x2, yh);
                *reinterpret_cast<u32x2 *>(stg + 1024 * O + 64 * l16 + 32 * s + 8 * g4) = bits;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const f16x8 row = *reinterpret_cast<const f16x8 *>(stg + 1024 * O + 16 * lane);
            const int tk = 16 * t + (lane >> 2);
            if (tk < nval) *reinterpret_cast<f16x8 *>(obase + (((size_t)(tok0 + tk) * a.Hv + h) * DV + dv0 + 8 * (lane & 3)) * 2) = row;
            continue;
        }
#pragma unroll
        for (int s = 0; s < SPW; ++s) {
        const f32x4 &acc = accs[s];
        const size_t at = ((size_t)(tok0 + tok) * a.Hv + h) * DV + dv0 + 16 * s + 4 * g4;
        if constexpr (SEG) {
            typename Vec4<IO>::type yio;
            f16x4 yh;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                yio[i] = Cvt<IO>::from_f32(acc[i]);
                yh[i] = (hf)acc[i];
            }
            const u32x2 bits = kind == 0 ? __builtin_bit_cast(u32x2, yio) : __builtin_bit_cast(u32x2, yh);
            if (tok < nval) *reinterpret_cast<u32x2 *>(obase + at * 2) = bits;
        } else {
            typename Vec4<IO>::type y;
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = Cvt<IO>::from_f32(acc[i]);
            if (PAIR && !last)
                *reinterpret_cast<typename Vec4<IO>::type *>(stg + (c & 1) * 2048 + O * 512 + 32 * l16 + 8 * g4) = y;
            else if (tok < nval)
                *reinterpret_cast<typename Vec4<IO>::type *>(reinterpret_cast<IO *>(a.o) + at) = y;
        }
        }
    }
}

// Output wave O's run: barrier -1, then after barrier c it forms chunk c's outputs; the
// loads of chunk c + 1 are issued before barrier c.  A wave with no token tile (O >= NT,
// at C = 32) takes part in the barriers only.
template <typename IO, int C, int SPW, bool SEG, int O>
__device__ __forceinline__ void output_run(Smem<C, SPW> &sm, const KdaArgs &a, const Work &wk, int lane, int kind) {
    using F = Cfg<C, SPW>;
    const int n = wk.nchunks;
    if constexpr (O >= F::NT) {
        for (int c = 0; c <= n; ++c) __syncthreads();
        return;
    }
    // the destination (segment mode: o, a.o0 or a.e by the workgroup's kind), picked once
    char *obase = (char *)a.o;
    if constexpr (SEG) obase = kind == 1 ? (char *)a.o0 : kind == 2 ? (char *)a.e : obase;
    auto step = [&](const OutOps<C, SPW, O> &op, int c) {
        const int tok0 = wk.bos + c * C;
        out_step<IO, C, SPW, SEG, O>(op, sm, c, a, lane, wk.h, wk.dv0, tok0, min(C, wk.eos - tok0), kind, obase,
                                     c + 1 >= n);
    };
    OutOps<C, SPW, O> op0, op1;
    load_out(op0, wk, 0, lane);
    __syncthreads();
    for (int c = 0; c < n; c += 2) {
        load_out(op1, wk, c + 1, lane);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        step(op0, c);
        if (c + 1 >= n) break;
        load_out(op0, wk, c + 2, lane);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        step(op1, c + 1);
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
template <typename IO, int C, int SPW, bool SEG, bool PERCH>
__global__ __launch_bounds__((Cfg<C, SPW>::THREADS))
__attribute__((amdgpu_waves_per_eu(Cfg<C, SPW>::WPE, Cfg<C, SPW>::WPE))) void kda_chain_kernel(const KdaArgs a) {
    __shared__ Smem<C, SPW> sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // XCD-aware mapping.  Workgroups are dispatched to the 8 XCDs in turn (blockIdx % 8).
    // The GS workgroups that read the same tiles (a head's 8 slices; in the segment mode a
    // segment's value and identity slices) form a group, and group g runs on XCD g % 8, so
    // its tiles are fetched into one L2.  The grid is padded to whole rounds of 8 groups;
    // the padding workgroups leave at once.
    using F = Cfg<C, SPW>;
    constexpr int NSL = F::NSL, DVS = F::DVS;
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

    if (wave < F::NRW) {
        const int kh = wave & 1, sl = wave >> 1;   // key half, slice
        // S^T rows (key channels) 64 kh + 16 i + 4 G + q, column = value channel r
        const int r = wk.dv0 + 16 * sl + l16;
        f32x4 st[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int dk = 64 * kh + 16 * i + 4 * g4;
            f32x4 x = zero4();
            if (seg == 0 && a.s0) x = *reinterpret_cast<const f32x4 *>(a.s0 + sbase + (size_t)r * DK + dk);
            if (ident) {
#pragma unroll
                for (int q = 0; q < 4; ++q) x[q] = dk + q == r ? 1.f : 0.f;
            }
            st[i] = x;
        }
        if (wk.nchunks > 0) rec_run<C, SPW, PERCH>(st, sm, wk, sl, kh, lane, !ident);
        if constexpr (SEG) {
            // segment 0's end state [row][key]; later segments' end states from zero and
            // from the identity (X) transposed, [key][row], as the join reads them
            float *sb = a.sseg + ((((size_t)n * a.Hv + h) * a.nseg + seg) * 2 + (ident ? 1 : 0)) * DV * DK;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int dk = 64 * kh + 16 * i + 4 * g4;
                if (seg > 0) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) sb[(size_t)(dk + q) * DV + r] = st[i][q];
                } else {
                    *reinterpret_cast<f32x4 *>(sb + (size_t)r * DK + dk) = st[i];
                }
            }
        } else if (a.sN) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<f32x4 *>(a.sN + sbase + (size_t)r * DK + 64 * kh + 16 * i + 4 * g4) = st[i];
        }
    } else if (wk.nchunks > 0 && wave < F::NRW + 4) {
        switch (wave - F::NRW) {
            case 0: output_run<IO, C, SPW, SEG, 0>(sm, a, wk, lane, kind); break;
            case 1: output_run<IO, C, SPW, SEG, 1>(sm, a, wk, lane, kind); break;
            case 2: output_run<IO, C, SPW, SEG, 2>(sm, a, wk, lane, kind); break;
            default: output_run<IO, C, SPW, SEG, 3>(sm, a, wk, lane, kind); break;
        }
    } else if (wk.nchunks > 0) {
        if (wave == F::NRW + 4) loader_run<C, SPW, false>(sm, wk, lane);
        else loader_run<C, SPW, true>(sm, wk, lane);
    }
}

}  // namespace kdachain

namespace {

template <int C, int SPW, bool SEG, bool PERCH>
hipError_t chain_launch_c(const KdaArgs &a, bool f16, hipStream_t stream) {
    // groups of GS workgroups (see the kernel), padded to whole rounds of 8 groups
    constexpr unsigned long long GS = kdachain::Cfg<C, SPW>::NSL * (SEG ? 2 : 1);
    const unsigned long long groups = (unsigned long long)a.N * a.Hv * (SEG ? (unsigned long long)a.nseg : 1ull);
    const unsigned long long wgs = 8 * GS * ((groups + 7) / 8);
    if (wgs > 0x7fffffffULL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)wgs), block(kdachain::Cfg<C, SPW>::THREADS);
    if (f16) hipLaunchKernelGGL((kdachain::kda_chain_kernel<_Float16, C, SPW, SEG, PERCH>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((kdachain::kda_chain_kernel<__bf16, C, SPW, SEG, PERCH>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <bool SEG, bool PERCH>
hipError_t chain_launch(const KdaArgs &a, bool f16, int chunk, bool wide, hipStream_t stream) {
    switch (chunk) {
        case 32: return wide ? chain_launch_c<32, 2, SEG, PERCH>(a, f16, stream) : chain_launch_c<32, 1, SEG, PERCH>(a, f16, stream);
        case 64: return wide ? chain_launch_c<64, 2, SEG, PERCH>(a, f16, stream) : chain_launch_c<64, 1, SEG, PERCH>(a, f16, stream);
        case 128: return wide ? hipErrorInvalidValue : chain_launch_c<128, 1, SEG, PERCH>(a, f16, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_kda_chain(const KdaArgs &a, bool f16, int chunk, bool per_channel, bool wide, hipStream_t stream) {
    return per_channel ? chain_launch<false, true>(a, f16, chunk, wide, stream)
                       : chain_launch<false, false>(a, f16, chunk, wide, stream);
}

hipError_t launch_seg_chain(const KdaArgs &a, bool f16, int chunk, bool per_channel, bool wide, hipStream_t stream) {
    if (a.nseg < 1) return hipErrorInvalidValue;
    return per_channel ? chain_launch<true, true>(a, f16, chunk, wide, stream)
                       : chain_launch<true, false>(a, f16, chunk, wide, stream);
}

int kda_chain_lds_bytes() { return (int)sizeof(kdachain::Smem<64, 1>); }

int chain_workgroups_per_head(int chunk, bool wide) { return wide && chunk <= 64 ? 4 : 8; }

}  // namespace gdn
