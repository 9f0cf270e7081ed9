// Map half of the chunked prefill with a per-key-channel decay (KDA) for gfx950.
//
// KDA is the delta rule of gdn_prefill.hip with the head's scalar decay replaced by one
// decay per key channel ("Empowering Hybrid Attention Models on NPUs", section 2.1 and
// the peak-memory discussion of section 7.5: the cumulative gate is 128x the GDN one):
//
//   S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t.
//
// Per chunk of n_c <= 64 tokens with Gamma = cumsum(log a) (a [n_c, 128] matrix now),
//   A[r, s] = beta_r sum_j k_rj k_sj exp(Gamma_rj - Gamma_sj)   (r > s),
//   P[r, s] = sum_j q_rj k_sj exp(Gamma_rj - Gamma_sj)          (r >= s),
//   T = (I + A)^-1,
// and the S-dependent half (kda_chain.hip) needs W = T diag(beta) (K (.) exp(Gamma)),
// U = T diag(beta) V, Q (.) exp(Gamma), K (.) exp(Gamma_last - Gamma) and
// exp(Gamma_last), stored as its MFMA operand fragments (gdn_launch.h, Tile).  None of this depends on the state, so every chunk of every head is
// one independent workgroup here (the Map phases #1-#4 of the page's Map-Reduce-Map
// pipeline), and the results go to a workspace tile the chain kernel reads: with a
// per-channel gate this map is several times the chain's work, and doing it once per
// chunk instead of once per value-channel slice of the chain is what makes the split pay.
//
// Decays without overflow.  exp(Gamma_rj - Gamma_sj) is rank one per channel,
// f_rj * f'_sj, for any reference point between s and r: with f_rj = prod of a over
// (ref, r] and f'_sj = prod of a over (s, ref], both factors are <= 1 whenever a <= 1,
// so the MFMA operands k (.) f stay in [-1, 1] in fp16 and underflow only where the
// decay really is negligible.  Each pair (r > s) of the chunk is assigned to the level
// at which r and s fall in different halves of an aligned segment -- 32, 16, 8, 4, 2
// or 1 tokens -- and the reference is the last token of the first half.  Levels 32 and
// 16 cover the six 16x16 tiles below the diagonal whole; levels 8..1 split the four
// diagonal tiles, each computed in full per level and masked to its own pairs.  Every
// factor is a product of per-token decays a = exp(g), computed once.
//
// One workgroup = 4 wave64s; wave b owns token block b (16 tokens) while the factors
// are formed, each lane two key channels.  LDS stays under half a CU's (two factor tiles
// per round, A and T overlaid on them once the grams are done), so two workgroups
// share a CU and hide each other's load and barrier latency.
#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_wy.h"

#include <type_traits>

namespace gdn {
namespace kdamap {

typedef _Float16 hf;
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int CH = 64;
constexpr int DK = 128;
constexpr int THREADS = 256;
constexpr int XS = DK + 16;   // 16-bit row stride of k, q and the factor tiles (288 B)
constexpr int AS = CH + 8;    // fp32 row stride of A and T (288 B)
constexpr float LOG2E = 1.4426950408889634f;

template <typename IO>
struct __align__(16) Smem {
    union {
        struct {
            hf K[CH * XS];    // k rows of the chunk in fp16 (rows past its end repeat the last)
            hf Q[CH * XS];
        } kq;
        struct {              // once the grams are done: diag(beta) Kg, diag(beta) V
            hf Kb[CH * WY_S];
            hf Vb[CH * WY_S];
        } wy;
    };
    union {
        hf F[2][CH * XS];     // decay factors of two reference levels (grams)
        struct {
            float A[CH * AS];     // beta-scaled, strictly lower (solve)
            float T[CH * AS];     // (I + A)^-1
            float Y[3][16 * 16];  // partial products of the block solve
        } sv;
    };
    float blk[4][DK];         // per 16-token block: product of a over the block
    float beta[CH];           // 0 past the chunk's end
};

// Factors inside a 16-token block for half-segment length L (8, 4, 2, 1): tokens in the
// first half of each aligned 2L segment get the product of a over (i, first-half end],
// tokens in the second half the product over [second-half start, i].
template <int L>
__device__ __forceinline__ void level_factors(const float (&a)[16], float (&f)[16]) {
#pragma unroll
    for (int s0 = 0; s0 < 16; s0 += 2 * L) {
        float c = 1.f;
#pragma unroll
        for (int i = s0 + L - 1; i >= s0; --i) {
            f[i] = c;
            c *= a[i];
        }
        float r = 1.f;
#pragma unroll
        for (int i = s0 + L; i < s0 + 2 * L; ++i) {
            r *= a[i];
            f[i] = r;
        }
    }
}

__device__ __forceinline__ void put_pair(hf *tile, int t, int ch, float x0, float x1) {
    f16x2 v;
    v[0] = (hf)x0;
    v[1] = (hf)x1;
    *reinterpret_cast<f16x2 *>(&tile[t * XS + ch]) = v;
}

// MFMA operand: 16 tokens (rows 16X + l16) x 32 key channels (32kb + 8g4 + e) of x, times
// the factor tile f: one fp16 multiply per element (packed two to an instruction).  x and
// f are fp16, so their exact product fits fp32 and the fp16 multiply rounds it once, as
// forming it in fp32 and converting would; k and q go to fp16 as they are staged, which is
// exact for bf16 values within fp16's normal range.
__device__ __forceinline__ Frag<hf> frag_scaled(const hf *x, const hf *f, int X, int kb, int l16, int g4) {
    const int off = (16 * X + l16) * XS + 32 * kb + 8 * g4;
    Frag<hf> r;
    r.v = *reinterpret_cast<const f16x8 *>(x + off) * *reinterpret_cast<const f16x8 *>(f + off);
    return r;
}

__device__ __forceinline__ Frag<hf> frag_raw(const hf *x, int X, int kb, int l16, int g4) {
    Frag<hf> r;
    r.v = *reinterpret_cast<const f16x8 *>(x + (16 * X + l16) * XS + 32 * kb + 8 * g4);
    return r;
}

// P tile (I, J), J <= I, as the lane holds it (row 16I + l16, columns 16J + 4g4 + i)
__device__ __forceinline__ void store_p(char *tile, int I, int J, int l16, int g4, const f32x4 &x) {
    f16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (hf)x[i];
    store_p_frag<CH>(tile, I, J, l16, g4, v);
}

// Tile (I, J), I > J, of A and P at one reference level, whole.  The product is taken
// transposed (K_J X_I^T), so the lane holds row r = 16I + l16 and columns
// 16J + 4g4 .. 16J + 4g4 + 3.  P goes to the workspace; A (beta-scaled) is returned and
// written to LDS once the factor tiles it would overlay are no longer read.
template <typename IO>
__device__ __forceinline__ f32x4 offdiag_tile(const Smem<IO> &s, char *tile, int I, int J, const hf *f, int l16,
                                              int g4) {
    f32x4 accA = zero4(), accP = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const Frag<hf> kj = frag_scaled(s.kq.K, f, J, kb, l16, g4);
        const Frag<hf> ki = frag_scaled(s.kq.K, f, I, kb, l16, g4);
        const Frag<hf> qi = frag_scaled(s.kq.Q, f, I, kb, l16, g4);
        mma(accA, kj, ki);
        mma(accP, kj, qi);
    }
    store_p(tile, I, J, l16, g4, accP);
    return accA * s.beta[16 * I + l16];
}

// Diagonal tile X at level 2^LB: the full 16x16 products, of which this level keeps the
// pairs (r, s) whose local indices first differ in bit LB (r's bit set).
template <int LB, typename IO>
__device__ __forceinline__ void diag_level(const Smem<IO> &s, int X, const hf *f, int l16, int g4,
                                           f32x4 &selA, f32x4 &selP) {
    f32x4 accA = zero4(), accP = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const Frag<hf> kx = frag_scaled(s.kq.K, f, X, kb, l16, g4);
        const Frag<hf> qx = frag_scaled(s.kq.Q, f, X, kb, l16, g4);
        mma(accA, kx, kx);
        mma(accP, kx, qx);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int sl = 4 * g4 + i, d = l16 ^ sl;
        if (l16 > sl && (31 - __builtin_clz(d)) == LB) {
            selA[i] = accA[i];
            selP[i] = accP[i];
        }
    }
}

template <typename IO>
__global__ __launch_bounds__(THREADS, 2) void kda_map_kernel(const KdaArgs a) {
    __shared__ Smem<IO> s;
    const int tid = threadIdx.x;
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slot = blockIdx.x / a.Hv, h = blockIdx.x % a.Hv, hk = h % a.Hk;

    // the sequence of this slot: the last n with cu[n] / 64 + n <= slot
    int n = 0;
    if (a.cu) {
        int lo = 0, hi = a.N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.cu[mid] / CH + mid <= slot) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
    }
    const int bos = a.cu ? a.cu[n] : 0, eos = a.cu ? a.cu[n + 1] : a.T_tot;
    const int tok0 = bos + CH * (slot - (bos / CH + n));
    if (tok0 >= eos) return;   // a slot no chunk uses (the whole workgroup leaves)
    const int nval = min(CH, eos - tok0);
    char *tile = a.ws + ((size_t)slot * a.Hv + h) * WS_TILE_BYTES;

    // beta for wave 0 (lane = token, clamped into the chunk) before the gate's loads, to
    // LDS after them: its round trip overlaps theirs
    static_assert(CH == 64, "one wave holds the chunk's beta");
    float braw = 0.f;
    if (wave == 0) braw = a.beta[(size_t)(tok0 + min(lane, nval - 1)) * a.Hv + h];

    // k and q rows of this wave's 16-token block straight to LDS in fp16, four rows per load
    // (lane: row 4 p + lane / 16 of the block, channels 8 (lane % 16) .. + 7)
    const int b = wave, ch = 2 * lane;
    {
        typedef IO v8 __attribute__((ext_vector_type(8)));
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int t = 16 * b + 4 * p + (lane >> 4), c8 = 8 * (lane & 15);
            const size_t kq = ((size_t)(tok0 + min(t, nval - 1)) * a.Hk + hk) * DK + c8;
            const v8 kk = *reinterpret_cast<const v8 *>(reinterpret_cast<const IO *>(a.k) + kq);
            const v8 qq = *reinterpret_cast<const v8 *>(reinterpret_cast<const IO *>(a.q) + kq);
            f16x8 kh, qh;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                kh[e] = (hf)Cvt<IO>::to_f32(kk[e]);
                qh[e] = (hf)Cvt<IO>::to_f32(qq[e]);
            }
            *reinterpret_cast<f16x8 *>(&s.kq.K[t * XS + c8]) = kh;
            *reinterpret_cast<f16x8 *>(&s.kq.Q[t * XS + c8]) = qh;
        }
    }
    // #1 Gate, per channel: a = exp(g) for this lane's two channels and 16 tokens
    float a0[16], a1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = 16 * b + i;
        const size_t tok = (size_t)(tok0 + min(t, nval - 1));
        const f32x2 gg = *reinterpret_cast<const f32x2 *>(a.g + (tok * a.Hv + h) * DK + ch);
        const bool ok = t < nval;
        a0[i] = ok ? exp2f(gg[0] * LOG2E) : 1.f;
        a1[i] = ok ? exp2f(gg[1] * LOG2E) : 1.f;
    }
    if (wave == 0) s.beta[lane] = lane < nval ? braw : 0.f;
    // products inside the block: F inclusive from the block start, B exclusive to its end
    float F0[16], F1[16], B0[16], B1[16];
    F0[0] = a0[0];
    F1[0] = a1[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) {
        F0[i] = F0[i - 1] * a0[i];
        F1[i] = F1[i - 1] * a1[i];
    }
    B0[15] = B1[15] = 1.f;
#pragma unroll
    for (int i = 14; i >= 0; --i) {
        B0[i] = B0[i + 1] * a0[i + 1];
        B1[i] = B1[i + 1] * a1[i + 1];
    }
    s.blk[b][ch] = F0[15];
    s.blk[b][ch + 1] = F1[15];
    __syncthreads();
    float pre0 = 1.f, pre1 = 1.f, post0 = 1.f, post1 = 1.f;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
        const float x0 = s.blk[bb][ch], x1 = s.blk[bb][ch + 1];
        if (bb < b) { pre0 *= x0; pre1 *= x1; }
        if (bb > b) { post0 *= x0; post1 *= x1; }
    }
    // operands of the chain: Q (.) exp(Gamma), K (.) exp(Gamma_last - Gamma); and
    // diag(beta) (K (.) exp(Gamma)) kept for the WY products
    f16x2 kgb[16];
    {
        f16x4 kl[2][4];   // Kl of channels ch, ch + 1 over this block's 16 tokens, 4 at a time
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 16 * b + i;
            const f16x2 kv = *reinterpret_cast<const f16x2 *>(&s.kq.K[t * XS + ch]);
            const f16x2 qv = *reinterpret_cast<const f16x2 *>(&s.kq.Q[t * XS + ch]);
            const float k0 = (float)kv[0], k1 = (float)kv[1];
            const float e0 = pre0 * F0[i], e1 = pre1 * F1[i];
            const float l0 = B0[i] * post0, l1 = B1[i] * post1;
            const float bt = s.beta[t];
            kgb[i][0] = (hf)(k0 * e0 * bt);
            kgb[i][1] = (hf)(k1 * e1 * bt);
            f16x2 x;
            x[0] = (hf)((float)qv[0] * e0); x[1] = (hf)((float)qv[1] * e1);
            // Qg's rows of this wave, staged in F[0] (unused until the gram factors)
            *reinterpret_cast<f16x2 *>(&s.F[0][t * XS + ch]) = x;
            kl[0][i >> 2][i & 3] = (hf)(k0 * l0);
            kl[1][i >> 2][i & 3] = (hf)(k1 * l1);
        }
        // Kl(key tile c / 16, token block b / 2): lane (G, c % 16), half b % 2
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int c = ch + j;
#pragma unroll
            for (int G = 0; G < 4; ++G)
                *reinterpret_cast<f16x4 *>(tile + Tile<CH>::kl(c >> 4, b >> 1) + 16 * (16 * G + (c & 15)) + 8 * (b & 1)) =
                    kl[j][G];
        }
        // Qg(b, kb) from the staged rows, one 16-byte store per fragment: lane (G, m) takes
        // token 16 b + m, channels 32 kb + 4 G .. + 3 and 32 kb + 16 + 4 G .. + 3.  The rows
        // are this wave's own, and only its own gram factors overwrite them after.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        {
            const hf *row = &s.F[0][(16 * b + l16) * XS];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const f16x4 lo = *reinterpret_cast<const f16x4 *>(row + 32 * kb + 4 * g4);
                const f16x4 hi = *reinterpret_cast<const f16x4 *>(row + 32 * kb + 16 + 4 * g4);
                *reinterpret_cast<f16x8 *>(tile + Tile<CH>::qg(b, kb) + 16 * lane) =
                    f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (b == 0) {
            f32x2 gl;
            gl[0] = F0[15] * post0;
            gl[1] = F1[15] * post1;
            *reinterpret_cast<f32x2 *>(tile + Tile<CH>::GL + ch * 4) = gl;
        }
    }

    // #2 grams in three rounds of two reference levels each.  Round 1: levels 32 and 16,
    // the six tiles below the diagonal (blocks 0, 1 hold columns at level 32, with
    // products to token 31; blocks 2, 3 rows, from token 32; at level 16 even blocks
    // hold columns and odd blocks rows).
    {
        const float m0 = b == 0 ? s.blk[1][ch] : (b == 3 ? s.blk[2][ch] : 1.f);
        const float m1 = b == 0 ? s.blk[1][ch + 1] : (b == 3 ? s.blk[2][ch + 1] : 1.f);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 16 * b + i;
            put_pair(s.F[0], t, ch, (b < 2 ? B0[i] : F0[i]) * m0, (b < 2 ? B1[i] : F1[i]) * m1);
            put_pair(s.F[1], t, ch, (b & 1) ? F0[i] : B0[i], (b & 1) ? F1[i] : B1[i]);
        }
    }
    __syncthreads();
    f32x4 offA0 = zero4(), offA1 = zero4();   // this wave's tiles below the diagonal
    switch (wave) {
        case 0: offA0 = offdiag_tile(s, tile, 1, 0, s.F[1], l16, g4); break;
        case 1:
            offA0 = offdiag_tile(s, tile, 2, 0, s.F[0], l16, g4);
            offA1 = offdiag_tile(s, tile, 2, 1, s.F[0], l16, g4);
            break;
        case 2:
            offA0 = offdiag_tile(s, tile, 3, 0, s.F[0], l16, g4);
            offA1 = offdiag_tile(s, tile, 3, 1, s.F[0], l16, g4);
            break;
        default: offA0 = offdiag_tile(s, tile, 3, 2, s.F[1], l16, g4); break;
    }
    __syncthreads();
    // round 2: levels 8 and 4 inside the diagonal tiles
    f32x4 selA = zero4(), selP = zero4();
    {
        float f0[16], f1[16], h0[16], h1[16];
        level_factors<8>(a0, f0);
        level_factors<8>(a1, f1);
        level_factors<4>(a0, h0);
        level_factors<4>(a1, h1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 16 * b + i;
            put_pair(s.F[0], t, ch, f0[i], f1[i]);
            put_pair(s.F[1], t, ch, h0[i], h1[i]);
        }
    }
    __syncthreads();
    diag_level<3>(s, wave, s.F[0], l16, g4, selA, selP);
    diag_level<2>(s, wave, s.F[1], l16, g4, selA, selP);
    __syncthreads();
    // round 3: levels 2 and 1, and the diagonal of P itself; v of this thread's tokens and
    // channels is fetched here for the WY products
    // (four rows per load: lane = row 4 p + lane / 16 of the block, channels 8 (lane % 16) ..)
    typedef IO v8 __attribute__((ext_vector_type(8)));
    v8 vp[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const size_t tok = (size_t)(tok0 + min(16 * b + 4 * p + (lane >> 4), nval - 1));
        vp[p] = *reinterpret_cast<const v8 *>(reinterpret_cast<const IO *>(a.v) + (tok * a.Hv + h) * DK + 8 * (lane & 15));
    }
    {
        float f0[16], f1[16], h0[16], h1[16];
        level_factors<2>(a0, f0);
        level_factors<2>(a1, f1);
        level_factors<1>(a0, h0);
        level_factors<1>(a1, h1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 16 * b + i;
            put_pair(s.F[0], t, ch, f0[i], f1[i]);
            put_pair(s.F[1], t, ch, h0[i], h1[i]);
        }
    }
    __syncthreads();
    diag_level<1>(s, wave, s.F[0], l16, g4, selA, selP);
    diag_level<0>(s, wave, s.F[1], l16, g4, selA, selP);
    {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mma(acc, frag_raw(s.kq.K, wave, kb, l16, g4), frag_raw(s.kq.Q, wave, kb, l16, g4));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (l16 == 4 * g4 + i) selP[i] = acc[i];
    }
    __syncthreads();   // the factor tiles and k, q are dead; A and T overlay the former,
                       // the WY right-hand sides the latter
#pragma unroll
    for (int i = 0; i < 16; ++i) *reinterpret_cast<f16x2 *>(&s.wy.Kb[(16 * b + i) * WY_S + ch]) = kgb[i];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int t = 16 * b + 4 * p + (lane >> 4);
        const float bt = s.beta[t];
        f16x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (hf)(Cvt<IO>::to_f32(vp[p][e]) * bt);
        *reinterpret_cast<f16x8 *>(&s.wy.Vb[t * WY_S + 8 * (lane & 15)]) = x;
    }
    {
        // A: this wave's diagonal tile, its tiles below the diagonal, zeros right of the
        // diagonal; P: the diagonal tile and the zeros (the tiles below went out above)
        float *A = s.sv.A;
        const int r = 16 * wave + l16;
        *reinterpret_cast<f32x4 *>(&A[r * AS + 16 * wave + 4 * g4]) = selA * s.beta[r];
        store_p(tile, wave, wave, l16, g4, selP);   // (and the zero half of an even diagonal's fragment)
        for (int J = wave + 1; J < 4; ++J) *reinterpret_cast<f32x4 *>(&A[r * AS + 16 * J + 4 * g4]) = zero4();
        switch (wave) {
            case 0: *reinterpret_cast<f32x4 *>(&A[(16 + l16) * AS + 4 * g4]) = offA0; break;
            case 1:
                *reinterpret_cast<f32x4 *>(&A[(32 + l16) * AS + 4 * g4]) = offA0;
                *reinterpret_cast<f32x4 *>(&A[(32 + l16) * AS + 16 + 4 * g4]) = offA1;
                break;
            case 2:
                *reinterpret_cast<f32x4 *>(&A[(48 + l16) * AS + 4 * g4]) = offA0;
                *reinterpret_cast<f32x4 *>(&A[(48 + l16) * AS + 16 + 4 * g4]) = offA1;
                break;
            default: *reinterpret_cast<f32x4 *>(&A[(48 + l16) * AS + 32 + 4 * g4]) = offA0; break;
        }
        for (int i = tid; i < CH * AS; i += THREADS) s.sv.T[i] = 0.f;
    }
    __syncthreads();

    // #3 Solve, T = (I + A)^-1: the diagonal 16x16 blocks by substitution (all four on wave
    // 0: lane group g4 solves block g4, lane l16 one column), then the blocks below them by
    // distance from the diagonal, T_IJ = -T_II (sum_{J <= m < I} A_Im T_mJ), one block per
    // wave on fp32 MFMAs (16x16x4: lane l supplies row / column l % 16 at k = l / 16).
    const float *A = s.sv.A;
    float *T = s.sv.T;
    if (wave == 0) {
        const int X = g4, c = l16;
        const float *arow = &A[16 * X * AS + 16 * X];
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = r == c ? 1.f : 0.f;
#pragma unroll
            for (int q = 0; q < r; ++q) acc -= arow[r * AS + q] * x[q];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) T[(16 * X + r) * AS + 16 * X + c] = x[r];
    }
    __syncthreads();
    for (int d = 1; d < 4; ++d) {
        const int J = wave, I = J + d;
        if (I < 4) {
            f32x4 y = zero4();
            for (int kk = 16 * J; kk < 16 * I; kk += 4)
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(A[(16 * I + l16) * AS + kk + g4],
                                                         T[(kk + g4) * AS + 16 * J + l16], y, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) s.sv.Y[J][(4 * g4 + i) * 16 + l16] = y[i];
        }
        __syncthreads();
        if (I < 4) {
            f32x4 t = zero4();
#pragma unroll
            for (int v = 0; v < 16; v += 4)
                t = __builtin_amdgcn_mfma_f32_16x16x4f32(T[(16 * I + l16) * AS + 16 * I + v + g4],
                                                         s.sv.Y[J][(v + g4) * 16 + l16], t, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) T[(16 * I + 4 * g4 + i) * AS + 16 * J + l16] = -t[i];
        }
        __syncthreads();
    }
    // #4 W = T diag(beta) Kg and U = T diag(beta) V to the workspace
    wy_products<CH>(s.sv.T, AS, s.wy.Kb, s.wy.Vb, tile, wave, l16, g4);
}

}  // namespace kdamap

hipError_t launch_kda_map(const KdaArgs &a, bool f16, hipStream_t stream) {
    const dim3 grid((unsigned)a.nslots * (unsigned)a.Hv), block(kdamap::THREADS);
    if (f16)
        hipLaunchKernelGGL(kdamap::kda_map_kernel<_Float16>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(kdamap::kda_map_kernel<__bf16>, grid, block, 0, stream, a);
    return hipGetLastError();
}

int kda_map_lds_bytes() { return (int)sizeof(kdamap::Smem<__bf16>); }

}  // namespace gdn
