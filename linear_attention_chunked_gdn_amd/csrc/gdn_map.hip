// Chunk-parallel map of the scalar-gate prefill for gfx950: the Map phases #1-#4 of the
// Map-Reduce-Map pipeline ("Empowering Hybrid Attention Models on NPUs", section 2.1,
// Figure 1(b)) for every chunk of every value head at once, into the workspace tiles that
// kda_chain.hip's state recurrence reads.  Chunks of C = 32, 64 or 128 tokens.
//
// Per chunk of n_c <= C tokens, with Gamma = cumsum(g), gamma = exp(Gamma),
// lambda_r = exp(Gamma_last - Gamma_r) and D[r][s] = exp(Gamma_r - Gamma_s) for r >= s:
//
//   A = strictly-lower(diag(beta) K K^T .* D),   T = (I + A)^-1,
//   P = lower-incl-diagonal(Q K^T .* D),
//   W = T diag(beta gamma) K (stored negated),  U = T diag(beta) V,
//   Qg = diag(gamma) Q,  Kl = diag(lambda) K,  gl = gamma_last,
//
// all as the chain's MFMA operand fragments (gdn_launch.h, Tile), so that the chain's
// v = U - W S^T (= T diag(beta) (V - diag(gamma) K S^T)),
// O = Qg S^T + P v and S <- gl S + v^T Kl are the scalar-gate chunk formulas with the
// decays and the inverse already in the operands (the per-key-channel gate of
// kda_map.hip with every channel's decay equal).
// None of this depends on the state.  The in-kernel map of gdn_prefill_pipe.hip repeats
// it for each of a head's eight value-channel slices on the chain's critical path; done
// here once per (chunk, head) over the whole chip, it leaves the chain kernel only the
// S-dependent products, which is the shorter per-chunk period when the (sequence, head,
// slice) chains alone cannot fill the compute units.
//
// The grams take the stored q, k exactly (bf16 or fp16 MFMAs, fp32 accumulation) and the
// decays as fp32 scalars on the accumulators; D is formed only for r >= s, never as
// exp(Gamma_r) * exp(-Gamma_s).  gamma and lambda are <= 1 for g <= 0, so the decayed
// fp16 operands underflow only where the decay really is negligible.
//
// Fused input prologue (PRO, with the GDN_PROLOGUE_* flags of the call): q and k arrive
// unnormalised and beta, g as logits.  The 16 lanes holding a q or k row reduce its L2
// norm in fp32 from the registers it was loaded into; 1 / ||row|| is kept per token and
// folded into the per-row factors applied anyway (the grams' decays, gamma on Qg and in
// W's right-hand side, lambda on Kl), so q and k stay exact 16-bit MFMA operands.  The
// gate scan applies beta = sigmoid(x) and g = -softplus(x).
//
// One workgroup = 4 wave64s per (chunk slot, value head).  One LDS region is reused
// three times: the k and q tiles (grams); then M, T in its lower triangle and A^T in its
// strict upper one (A is held in registers until every wave is done with k and q); then
// T in fp16 and the right-hand sides diag(beta gamma) K and diag(beta) V of the W/U
// products, from the k and v rows each thread keeps in registers since its first load.
// The map moves 122 KB per item and waits mostly on memory, so the item count per CU
// decides its time: at C = 64 (37.9 KB, the right-hand sides one after the other, at
// most 128 VGPRs) four workgroups fit on a CU, one round for 1,024 items on 256 CUs.
// C = 32 takes 19 KB, C = 128 105 KB.
#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_wy.h"

namespace gdn {
namespace gdnmap {

typedef _Float16 hf;
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int DK = 128;
constexpr int THREADS = 256;
constexpr int XS = DK + 8;   // 16-bit row stride of the k and q tiles (272 B)

template <typename IO, int C>
struct Cfg {
    static constexpr int NT = C / 16;            // 16-token tiles
    static constexpr int AS = C + 8;             // fp32 row stride of M (T and A^T)
    static constexpr int TS = C + 8;             // fp16 row stride of T for the W/U products
    static constexpr int KQ_BYTES = 2 * C * XS * (int)sizeof(IO);
    static constexpr int M_BYTES = C * AS * 4;
    static constexpr int Y_OFF = M_BYTES;                 // after M
    static constexpr int RHS_BYTES = C * WY_S * 2;
    // At C = 64 the right-hand sides take turns in one buffer, which keeps the workgroup
    // under a quarter of the CU's LDS (four per CU); elsewhere that gains no workgroup
    // and both are staged at once.
    static constexpr bool TWO_PASS = C == 64;
    static constexpr int RHS_ALL = TWO_PASS ? RHS_BYTES : 2 * RHS_BYTES;
    static constexpr int T16_OFF = RHS_ALL > M_BYTES ? RHS_ALL : M_BYTES;   // past M and the RHS
    static constexpr int T16_BYTES = C * TS * 2;
    static constexpr int R0 = KQ_BYTES > Y_OFF + 4096 ? (KQ_BYTES > T16_OFF + T16_BYTES ? KQ_BYTES : T16_OFF + T16_BYTES)
                                                      : (Y_OFF + 4096 > T16_OFF + T16_BYTES ? Y_OFF + 4096 : T16_OFF + T16_BYTES);
};

// One LDS region, overlaid in turn by
//   the k and q tiles (grams);
//   M, fp32: T = (I + A)^-1 in its lower triangle (diagonal included) and the beta-scaled
//     A transposed in its strict upper triangle (A is strictly lower, so the two never
//     meet), then the solve's per-wave partial products Y;
//   T in fp16, placed past M so that it is written while M is read, and the right-hand
//     sides of the W/U products, diag(beta gamma) K and diag(beta) V (at C = 64 one at a
//     time).
template <typename IO, int C, bool PRO>
struct __align__(16) Smem {
    using F = Cfg<IO, C>;
    __align__(16) char r0[F::R0];
    float gcum[C];            // Gamma (flat past the chunk's end)
    float gam[C];             // exp(Gamma)
    float lam[C];             // exp(Gamma_last - Gamma)
    float beta[C];            // 0 past the chunk's end
    float rn[PRO ? 2 : 1][PRO ? C : 1];   // prologue: 1 / ||k_t||, 1 / ||q_t|| (1 without the norm)
    __device__ IO *K() { return reinterpret_cast<IO *>(r0); }
    __device__ IO *Q() { return reinterpret_cast<IO *>(r0) + C * XS; }
    __device__ const IO *K() const { return reinterpret_cast<const IO *>(r0); }
    __device__ const IO *Q() const { return reinterpret_cast<const IO *>(r0) + C * XS; }
    __device__ float *M() { return reinterpret_cast<float *>(r0); }
    __device__ float *Y(int w) { return reinterpret_cast<float *>(r0 + F::Y_OFF) + 256 * w; }
    __device__ hf *T16() { return reinterpret_cast<hf *>(r0 + F::T16_OFF); }
    __device__ hf *RHS() { return reinterpret_cast<hf *>(r0); }
};

static_assert(Cfg<__bf16, 64>::T16_OFF >= Cfg<__bf16, 64>::M_BYTES &&
                  Cfg<__bf16, 128>::T16_OFF >= Cfg<__bf16, 128>::M_BYTES &&
                  Cfg<__bf16, 32>::T16_OFF >= Cfg<__bf16, 32>::M_BYTES,
              "T's fp16 copy is written while M is read");
static_assert(sizeof(Smem<__bf16, 64, true>) <= 160 * 1024 / 4 && sizeof(Smem<_Float16, 64, true>) <= 160 * 1024 / 4,
              "four chunk-64 workgroups share a CU's LDS");

// Tiles (I, 2 kb) and (I, 2 kb + 1) of A and P, the second only where it is on or below
// the diagonal (2 kb + 1 <= I).  The products are taken transposed (K_J X_I^T), so the
// lane holds row r = 16I + l16 and columns 16J + 4g4 .. 16J + 4g4 + 3 of each; both P
// tiles go to the workspace as fp16 in one 16-byte piece of fragment P(I, kb) (zeros for
// a missing second tile), the beta-scaled A tiles are returned (they go to LDS once every
// wave is done reading the k and q tiles they would overlay).
template <typename IO, int C, bool PRO>
__device__ __forceinline__ void gram_pair(const Smem<IO, C, PRO> &s, char *tile, int I, int kb, int l16, int g4,
                                          f32x4 (&va)[2]) {
    const bool two = 2 * kb + 1 <= I;
    f32x4 accA[2] = {zero4(), zero4()}, accP[2] = {zero4(), zero4()};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        Frag<IO> ki, qi, kj;
        ki.load8(s.K() + (16 * I + l16) * XS + 32 * k + 8 * g4);
        qi.load8(s.Q() + (16 * I + l16) * XS + 32 * k + 8 * g4);
        kj.load8(s.K() + (32 * kb + l16) * XS + 32 * k + 8 * g4);
        mma(accA[0], kj, ki);
        mma(accP[0], kj, qi);
        if (two) {
            kj.load8(s.K() + (32 * kb + 16 + l16) * XS + 32 * k + 8 * g4);
            mma(accA[1], kj, ki);
            mma(accP[1], kj, qi);
        }
    }
    const int r = 16 * I + l16;
    const float gr = s.gcum[r], br = s.beta[r];
    f16x8 hp = {};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c0 = 32 * kb + 16 * h + 4 * g4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = c0 + i;
            const float d = c <= r ? __expf(gr - s.gcum[c]) : 0.f;
            float da = d, dp = d;
            if constexpr (PRO) {   // the rows' and columns' reciprocal norms
                da *= s.rn[0][r] * s.rn[0][c];
                dp *= s.rn[1][r] * s.rn[0][c];
            }
            va[h][i] = c < r ? br * accA[h][i] * da : 0.f;
            hp[4 * h + i] = (hf)(accP[h][i] * dp);
        }
    }
    // a missing second tile lies above the diagonal: d = 0 there, so its half is zeros
    *reinterpret_cast<f16x8 *>(tile + Tile<C>::p(I, kb) + 16 * (16 * g4 + l16)) = hp;
}

// The pairs (I, kb) of P fragments, numbered for the waves: first those with two tiles
// (2 kb + 1 <= I, row by row), then the diagonal fragments of even I with one; job j <->
// (I, kb).  Row I has (I + 1) / 2 pairs of the first kind.
template <int NT>
__device__ __forceinline__ void pair_of_job(int j, int &I, int &kb) {
    constexpr int N2 = (NT / 2) * (NT / 2);   // sum over I < NT of (I + 1) / 2
    if (j >= N2) {
        I = 2 * (j - N2);
        kb = j - N2;
        return;
    }
    I = 1;
    while (j >= (I + 1) / 2) {
        j -= (I + 1) / 2;
        ++I;
    }
    kb = j;
}

template <typename IO, int C, bool PRO>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(C <= 64 ? 4 : 1))) void gdn_map_kernel(const KdaArgs a) {
    using F = Cfg<IO, C>;
    constexpr int NT = F::NT, AS = F::AS;
    constexpr int NJOBS = Tile<C>::NPF;       // P fragments: pairs of gram tiles
    constexpr int JPW = (NJOBS + 3) / 4;   // gram jobs per wave
    __shared__ Smem<IO, C, PRO> s;
    const int tid = threadIdx.x;
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slot = blockIdx.x / a.Hv, h = blockIdx.x % a.Hv, hk = h % a.Hk;

    // the sequence of this slot: the last n with cu[n] / C + n <= slot
    int n = 0;
    if (a.cu) {
        int lo = 0, hi = a.N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.cu[mid] / C + mid <= slot) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
    }
    const int bos = a.cu ? a.cu[n] : 0, eos = a.cu ? a.cu[n + 1] : a.T_tot;
    const int tok0 = bos + C * (slot - (bos / C + n));
    if (tok0 >= eos) return;   // a slot no chunk uses (the whole workgroup leaves)
    const int nval = min(C, eos - tok0);
    char *tile = a.ws + ((size_t)slot * a.Hv + h) * Tile<C>::BYTES;

    // wave 0's gate operands first (lane = token, clamped into the chunk), so that their
    // round trip overlaps the k, q, v loads instead of following them
    constexpr int GB = C > 64 ? C / 64 : 1;
    float graw[GB], braw[GB];
    if (wave == 0) {
#pragma unroll
        for (int b = 0; b < GB; ++b) {
            const size_t gi = (size_t)(tok0 + min(64 * b + lane, nval - 1)) * a.Hv + h;
            graw[b] = a.g[gi];
            braw[b] = a.beta[gi];
        }
    }

    // k, q rows to LDS, and kept in registers with the v rows: C rows x 16 segments of 8
    typedef IO v8 __attribute__((ext_vector_type(8)));
    v8 kv[C / 16], qv[C / 16], vv[C / 16];
#pragma unroll
    for (int p = 0; p < C / 16; ++p) {
        const int idx = tid + THREADS * p, row = idx >> 4, seg = idx & 15;
        const size_t tr = (size_t)(tok0 + min(row, nval - 1));
        const size_t off = (tr * a.Hk + hk) * DK + 8 * seg;
        kv[p] = *reinterpret_cast<const v8 *>(reinterpret_cast<const IO *>(a.k) + off);
        qv[p] = *reinterpret_cast<const v8 *>(reinterpret_cast<const IO *>(a.q) + off);
        vv[p] = *reinterpret_cast<const v8 *>(reinterpret_cast<const IO *>(a.v) + (tr * a.Hv + h) * DK + 8 * seg);
        *reinterpret_cast<v8 *>(&s.K()[row * XS + 8 * seg]) = kv[p];
        *reinterpret_cast<v8 *>(&s.Q()[row * XS + 8 * seg]) = qv[p];
    }
    if constexpr (PRO) {   // the 16 lanes of a DPP row hold one token's k (q) row
        const bool norm = a.prologue & GDN_PROLOGUE_QK_L2NORM;
#pragma unroll
        for (int p = 0; p < C / 16; ++p) {
            const int idx = tid + THREADS * p, row = idx >> 4;
            const float rk = norm ? row_rnorm<IO>(kv[p]) : 1.f, rq = norm ? row_rnorm<IO>(qv[p]) : 1.f;
            if ((idx & 15) == 0) {
                s.rn[0][row] = rk;
                s.rn[1][row] = rq;
            }
        }
    }
    // #1 Gate on wave 0, lane = token (64 at a time): inclusive prefix sum, flat past the
    // chunk's end
    if (wave == 0) {
        float carry = 0.f;
#pragma unroll
        for (int base = 0; base < C; base += 64) {
            const int t = base + lane;
            const bool ok = t < nval;
            float x = ok ? graw[base / 64] : 0.f;
            float b = ok ? braw[base / 64] : 0.f;
            if constexpr (PRO) {
                if (ok && (a.prologue & GDN_PROLOGUE_BETA_SIGMOID)) b = prologue_sigmoid(b);
                if (ok && (a.prologue & GDN_PROLOGUE_G_SOFTPLUS)) x = prologue_neg_softplus(x);
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            x += carry;
            carry = __shfl(x, 63, 64);
            if (t < C) {
                s.gcum[t] = x;
                s.beta[t] = b;
                if constexpr (C <= 64) {   // one pass: carry is already Gamma_last
                    s.gam[t] = __expf(x);
                    s.lam[t] = __expf(carry - x);
                }
            }
        }
        // carry is now Gamma_last (C = 32: lanes 32..63 added zeros)
        if constexpr (C > 64) {
#pragma unroll
            for (int base = 0; base < C; base += 64) {
                const int t = base + lane;
                const float x = s.gcum[t];
                s.gam[t] = __expf(x);
                s.lam[t] = __expf(carry - x);
            }
        }
        const float gl = __expf(carry);
        *reinterpret_cast<float2 *>(tile + Tile<C>::GL + 8 * lane) = make_float2(gl, gl);
    }
    __syncthreads();

    // the decayed operands of the chain, fp16, from the rows in registers and LDS, as operand
    // fragments (gdn_launch.h, Tile), each as 16-byte pieces (one fragment lane's eight
    // entries).  Qg by the threads that loaded the row: the piece of lane (G, row) holds
    // channels 32 kb + 4 G .. + 3 and 32 kb + 16 + 4 G .. + 3, which row segments seg and
    // seg ^ 2 (lanes l and l ^ 2) hold, so the two swap one half and each stores one piece.
    // Kl by key channel (lane: channel 64 x + lane) and pair of token tiles kb: the piece of
    // lane (G, channel) holds tokens 32 kb + 4 G .. + 3 and 32 kb + 16 + 4 G .. + 3.
    {
#pragma unroll
        for (int p = 0; p < C / 16; ++p) {
            const int idx = tid + THREADS * p, row = idx >> 4, seg = idx & 15;
            const float gm = PRO ? s.gam[row] * s.rn[1][row] : s.gam[row];
            f16x4 xq[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int e = 0; e < 4; ++e) xq[h2][e] = (hf)(Cvt<IO>::to_f32(qv[p][4 * h2 + e]) * gm);
            // channel j = 8 seg + 4 h2: G = 2 (seg & 1) + h2, upper half of the piece iff
            // seg & 2, block kb = seg / 4
            const int up = (seg >> 1) & 1;
            const u32x2 send = __builtin_bit_cast(u32x2, up ? xq[0] : xq[1]);
            u32x2 recv;
            recv[0] = from_lane_xor2(send[0]);
            recv[1] = from_lane_xor2(send[1]);
            const f16x4 other = __builtin_bit_cast(f16x4, recv);
            const f16x4 lo = up ? other : xq[0], hi = up ? xq[1] : other;
            const f16x8 piece = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const int G = 2 * (seg & 1) + up;
            *reinterpret_cast<f16x8 *>(tile + Tile<C>::qg(row >> 4, seg >> 2) + 16 * (16 * G + (row & 15))) = piece;
        }
        for (int it = wave; it < 2 * (C / 32); it += 4) {
            const int kb = it >> 1, ch = 64 * (it & 1) + lane;
            f16x8 kl[4];
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const int t = 32 * kb + i;
                const float lm = PRO ? s.lam[t] * s.rn[0][t] : s.lam[t];
                kl[(i & 15) >> 2][4 * (i >> 4) + (i & 3)] = (hf)(Cvt<IO>::to_f32(s.K()[t * XS + ch]) * lm);
            }
#pragma unroll
            for (int G = 0; G < 4; ++G)
                *reinterpret_cast<f16x8 *>(tile + Tile<C>::kl(ch >> 4, kb) + 16 * (16 * G + (ch & 15))) = kl[G];
        }
    }

    // #2 the lower 16x16 tiles of A and P, in pairs per P fragment (pair_of_job's order),
    // round-robin over the waves; zeros for P's tiles above the diagonal.  A stays in
    // registers until every wave is done with k and q.
    f32x4 av[JPW][2];
#pragma unroll
    for (int k = 0; k < JPW; ++k) {
        const int j = wave + 4 * k;
        if (j < NJOBS) {
            int I, kb;
            pair_of_job<NT>(j, I, kb);
            gram_pair(s, tile, I, kb, l16, g4, av[k]);
        }
    }
    __syncthreads();   // k and q are dead: A and T go over them
    // A^T into M's upper triangle: the lane's A[r][c0 + i] to M[c0 + i][r] (a diagonal
    // tile's zeros land on the lower half, which the solve then fills)
    float *const M = s.M();
#pragma unroll
    for (int k = 0; k < JPW; ++k) {
        const int j = wave + 4 * k;
        if (j < NJOBS) {
            int I, kb;
            pair_of_job<NT>(j, I, kb);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int J = 2 * kb + h;
                if (J > I) break;
#pragma unroll
                for (int i = 0; i < 4; ++i) M[(16 * J + 4 * g4 + i) * AS + 16 * I + l16] = av[k][h][i];
            }
        }
    }
    __syncthreads();

    // #3 Solve, T = (I + A)^-1: the diagonal 16x16 blocks by substitution, four at once on
    // one wave (lane group g4 of wave w takes block 4 w + g4, lane l16 one column; the
    // other waves wait at the barrier, leaving their SIMDs to the CU's other workgroups),
    // then the blocks below them by distance d from the diagonal,
    // T_IJ = -T_II (sum_{J <= m < I} A_Im T_mJ), on fp32 MFMAs (16x16x4: lane l supplies
    // row / column l % 16 at k = l / 16).  One barrier per distance: the sums read only
    // blocks of smaller distance; each wave keeps its partial product in its own Y.
    if (wave < (NT + 3) / 4 && 4 * wave + g4 < NT) {
        const int X = 4 * wave + g4, c = l16;
        const float *blk = &M[16 * X * AS + 16 * X];   // A[16X + r][16X + q] = blk[q AS + r]
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = r == c ? 1.f : 0.f;
#pragma unroll
            for (int q = 0; q < r; ++q) acc -= blk[q * AS + r] * x[q];
            x[r] = acc;
        }
        // the lower half with the diagonal; rows above it (x[r] = 0, over A^T) go to a
        // slot of Y, unused until the levels below
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float *dst = r >= c ? &M[(16 * X + r) * AS + 16 * X + c] : s.Y(g4) + 16 * wave + c;
            *dst = x[r];
        }
    }
    __syncthreads();
    for (int d = 1; d < NT; ++d) {
        for (int J = wave; J + d < NT; J += 4) {
            const int I = J + d;
            f32x4 y = zero4();
            for (int kk = 16 * J; kk < 16 * I; kk += 4)
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(M[(kk + g4) * AS + 16 * I + l16],
                                                         kk + g4 >= 16 * J + l16 ? M[(kk + g4) * AS + 16 * J + l16] : 0.f,
                                                         y, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) s.Y(wave)[(4 * g4 + i) * 16 + l16] = y[i];
            f32x4 t = zero4();
#pragma unroll
            for (int v = 0; v < 16; v += 4)
                t = __builtin_amdgcn_mfma_f32_16x16x4f32(v + g4 <= l16 ? M[(16 * I + l16) * AS + 16 * I + v + g4] : 0.f,
                                                         s.Y(wave)[(v + g4) * 16 + l16], t, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) M[(16 * I + 4 * g4 + i) * AS + 16 * J + l16] = -t[i];
        }
        __syncthreads();
    }

    // T to fp16 for the products (the MFMA operand type), zeros above the diagonal
    constexpr int TS = F::TS;
    for (int i = tid; i < C * C / 8; i += THREADS) {
        const int r = i / (C / 8), c = 8 * (i % (C / 8));
        const f32x4 t0 = *reinterpret_cast<const f32x4 *>(&M[r * AS + c]);
        const f32x4 t1 = *reinterpret_cast<const f32x4 *>(&M[r * AS + c + 4]);
        f16x8 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            y[e] = (hf)(c + e <= r ? t0[e] : 0.f);
            y[4 + e] = (hf)(c + 4 + e <= r ? t1[e] : 0.f);
        }
        *reinterpret_cast<f16x8 *>(&s.T16()[r * TS + c]) = y;
    }
    __syncthreads();   // M is dead: the right-hand sides go over it, one at a time

    // #4 W = T diag(beta gamma) K and U = T diag(beta) V to the workspace
    hf *const rhs = s.RHS();
#pragma unroll
    for (int p = 0; p < C / 16; ++p) {
        const int idx = tid + THREADS * p, row = idx >> 4, seg = idx & 15;
        const float bk = s.beta[row] * s.gam[row] * (PRO ? s.rn[0][row] : 1.f);
        f16x8 xk;
#pragma unroll
        for (int e = 0; e < 8; ++e) xk[e] = (hf)(Cvt<IO>::to_f32(kv[p][e]) * bk);
        *reinterpret_cast<f16x8 *>(&rhs[row * WY_S + 8 * seg]) = xk;
    }
    hf *const vb = F::TWO_PASS ? rhs : rhs + C * WY_S;
    if constexpr (F::TWO_PASS) {
        __syncthreads();
        wy_products<C, hf, true, false>(s.T16(), TS, rhs, nullptr, tile, wave, l16, g4);
        __syncthreads();
    }
#pragma unroll
    for (int p = 0; p < C / 16; ++p) {
        const int idx = tid + THREADS * p, row = idx >> 4, seg = idx & 15;
        const float bv = s.beta[row];
        f16x8 xv;
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] = (hf)(Cvt<IO>::to_f32(vv[p][e]) * bv);
        *reinterpret_cast<f16x8 *>(&vb[row * WY_S + 8 * seg]) = xv;
    }
    __syncthreads();
    if constexpr (F::TWO_PASS)
        wy_products<C, hf, false, true>(s.T16(), TS, nullptr, vb, tile, wave, l16, g4);
    else
        wy_products<C, hf, true, true>(s.T16(), TS, rhs, vb, tile, wave, l16, g4);
}

}  // namespace gdnmap

hipError_t launch_gdn_map(const KdaArgs &a, bool f16, int chunk, hipStream_t stream) {
    const dim3 grid((unsigned)a.nslots * (unsigned)a.Hv), block(gdnmap::THREADS);
#define GDN_MAP_LAUNCH(C)                                                                                    \
    do {                                                                                                     \
        if (a.prologue) {                                                                                    \
            if (f16) hipLaunchKernelGGL((gdnmap::gdn_map_kernel<_Float16, C, true>), grid, block, 0, stream, a); \
            else hipLaunchKernelGGL((gdnmap::gdn_map_kernel<__bf16, C, true>), grid, block, 0, stream, a);      \
        } else {                                                                                             \
            if (f16) hipLaunchKernelGGL((gdnmap::gdn_map_kernel<_Float16, C, false>), grid, block, 0, stream, a); \
            else hipLaunchKernelGGL((gdnmap::gdn_map_kernel<__bf16, C, false>), grid, block, 0, stream, a);      \
        }                                                                                                    \
    } while (0)
    switch (chunk) {
        case 32: GDN_MAP_LAUNCH(32); break;
        case 64: GDN_MAP_LAUNCH(64); break;
        case 128: GDN_MAP_LAUNCH(128); break;
        default: return hipErrorInvalidValue;
    }
#undef GDN_MAP_LAUNCH
    return hipGetLastError();
}

}  // namespace gdn
