// Chunked gated delta-rule prefill for gfx950 (MI355X).
//
// Method ("Empowering Hybrid Attention Models on NPUs", section 2.1, Figure 1(b)):
// the sequence is cut into chunks of 64 tokens; per chunk a Map phase builds
// chunk-local quantities (#1 Gate, #2 KKT, #3 Solve, #4 W/U), a Reduce phase
// carries the state across chunks (#5 H) and a second Map phase forms the outputs
// (#6 O).  With, inside one chunk of n_c tokens and state S (Dv x Dk):
//
//   Gamma = cumsum(g), gamma = exp(Gamma), lambda_r = exp(Gamma_last - Gamma_r)
//   D[r][s] = exp(Gamma_r - Gamma_s) for r >= s (masked before the exponential)
//   A = strictly-lower(diag(beta) K K^T .* D)           (#2)
//   T = (I + A)^-1                                       (#3, the UT transform)
//   R = diag(beta) V - diag(beta .* gamma) K S^T         (#4 with the inverse factored
//   v = T R                                               out, section 5, Figure 11)
//   O = diag(gamma) Q S^T + (lower-incl-diagonal(Q K^T) .* D) v      (#6)
//   S <- gamma_last S + v^T diag(lambda) K                (#5-update)
//
// O is formed before S is overwritten (chunk-first order 5-read -> 6 -> 5-update,
// section 5, Figure 10), so the state is updated in place and never has two copies.
//
// Mapping onto the chip.  One workgroup (4 wave64s) owns one (sequence, value
// head, slice of DVS value channels) and walks that sequence's chunks in order,
// keeping its DVS x 128 fp32 state slice in MFMA accumulator registers for the
// whole sequence.  Different value channels of S never interact, so slicing S by
// value channel needs no cross-workgroup reduction ("Empowering Hybrid Attention
// Models on NPUs", section 4, column-wise partitioning, Figure 8(b)).  On MI355X
// that split is the primary source of parallelism (256 CUs against 16-64 heads),
// not only a fix for tail heads; each slice recomputes the chunk's gate, grams and
// inverse, which do not depend on S.
//
// Per chunk, inside the workgroup (wave w, lane l, lane group G = l / 16):
//   grams   : the 10 lower 16x16 tiles of K K^T and of Q K^T, 5 tiles per wave
//   R, QS^T : wave w owns tokens [16w, 16w+16)
//   solve   : wave w inverts diagonal 16x16 block w by substitution (one column per
//             lane), then forms the blocks below it, T_iw = -T_ii sum_j A_ij T_jw,
//             with MFMAs whose B operands never leave registers
//   v = T R, O : wave w owns tokens [16w, 16w+16)
//   update  : wave w owns key channels [32w, 32w+32) of its state slice
// q/k/v/g/beta of chunk c+1 are fetched into registers while chunk c computes.
//
// Precision (bf16 I/O).  q, k, v enter the MFMAs exactly (they are bf16 already) and
// every product accumulates in fp32; the state is fp32 in registers.  Operands the
// kernel computes are rounded to bf16 to enter an MFMA: the state copy used by
// K S^T and Q S^T, and T, are single bf16; R, v, lambda*v and P are split into two
// bf16 halves (x = hi + lo) and their products take two or three MFMAs, since a
// single rounding of those dominated the output error.  The fp32 I/O path uses fp32
// MFMAs throughout.
#include "gdn_device.h"
#include "gdn_launch.h"

#include <type_traits>

namespace gdn {

constexpr int CH = 64;       // chunk length
constexpr int DK = 128;      // key head dimension
constexpr int DV = 128;      // value head dimension
constexpr int THREADS = 256; // 4 wave64s

template <bool BF16, int DVS>
struct Cfg {
    using CT = typename std::conditional<BF16, __bf16, float>::type;   // MFMA operand type
    using IO = typename std::conditional<BF16, uint16_t, float>::type; // storage of q/k/v/o
    static constexpr int PAD = 16 / (int)sizeof(CT);
    static constexpr int KS = DK + PAD;  // row stride: K, Q tiles and the state snapshot
    static constexpr int TS = CH + PAD;  // row stride: T, P, R^T, v^T, (lambda v)^T
    static constexpr int AS = CH + 4;    // row stride: A (fp32)
    static constexpr int NT = DVS / 16;  // 16-wide value-channel tiles per slice
    // global -> register staging of one chunk
    static constexpr int KQ_SPR = DK * (int)sizeof(IO) / 16;            // 16B segments per row
    static constexpr int KQ_VEC = CH * KQ_SPR / THREADS;                // per thread per tile
    static constexpr int V_SPR = DVS * (int)sizeof(IO) / 16;
    static constexpr int V_VEC = (CH * V_SPR + THREADS - 1) / THREADS;
    static constexpr int IO_PER_SEG = 16 / (int)sizeof(IO);
    // bf16 path: computed MFMA operands (R, v, lambda*v, P) are carried as a pair
    // hi + lo of bf16 values, hi = bf16(x), lo = bf16(x - hi), so that products with
    // them keep about 16 significant bits instead of 8.
    static constexpr bool SPLIT = BF16;
    static constexpr int LO = SPLIT ? 1 : 0;
};

template <bool BF16, int DVS>
struct __align__(16) Smem {
    using C = Cfg<BF16, DVS>;
    using CT = typename C::CT;
    CT K[CH * C::KS];      // keys of the chunk      [token][key channel]
    CT Q[CH * C::KS];      // queries of the chunk   [token][key channel]
    CT S[DVS * C::KS];     // operand copy of the state slice [value ch][key ch]
    CT Tm[CH * C::TS];     // T = (I + A)^-1         [token][token]
    CT Pm[CH * C::TS];     // (Q K^T) .* D, lower    [token][token]
    CT Rt[DVS * C::TS];    // R^T                    [value ch][token]
    CT Vt[DVS * C::TS];    // v^T                    [value ch][token]
    CT Vlt[DVS * C::TS];   // (diag(lambda) v)^T     [value ch][token]
    // low halves of the split operands (bf16 path only)
    CT Pm_lo[C::LO ? CH * C::TS : 8];
    CT Rt_lo[C::LO ? DVS * C::TS : 8];
    CT Vt_lo[C::LO ? DVS * C::TS : 8];
    CT Vlt_lo[C::LO ? DVS * C::TS : 8];
    float A[CH * C::AS];   // A, strictly lower, fp32
    float V[CH * DVS];     // value slice, fp32      [token][value ch]
    float graw[CH], gcum[CH], gam[CH], lam[CH], beta[CH];
};

template <bool BF16, int DVS>
struct Stage {
    using C = Cfg<BF16, DVS>;
    uint4 k[C::KQ_VEC];
    uint4 q[C::KQ_VEC];
    uint4 v[C::V_VEC];
    float g, b;
};

// Fetch chunk [tok0, tok0 + nval) of one (sequence, head, slice) into registers.
// Rows at and beyond nval are zero (g = beta = 0 too), which makes a short last
// chunk behave exactly like a full one whose extra tokens have no effect.
template <bool BF16, int DVS>
__device__ __forceinline__ void stage_load(Stage<BF16, DVS> &st, const PrefillArgs &a,
                                           int tok0, int nval, int h, int hk, int dv0, int tid) {
    using C = Cfg<BF16, DVS>;
    using IO = typename C::IO;
    const size_t kq_row = (size_t)a.Hk * DK * sizeof(IO);
    const char *kb = reinterpret_cast<const char *>(a.k) + (size_t)hk * DK * sizeof(IO);
    const char *qb = reinterpret_cast<const char *>(a.q) + (size_t)hk * DK * sizeof(IO);
#pragma unroll
    for (int i = 0; i < C::KQ_VEC; ++i) {
        const int f = tid + THREADS * i;
        const int row = f / C::KQ_SPR, seg = f % C::KQ_SPR;
        const size_t off = (size_t)(tok0 + row) * kq_row + (size_t)seg * 16;
        uint4 zk = make_uint4(0, 0, 0, 0), zq = zk;
        if (row < nval) {
            zk = *reinterpret_cast<const uint4 *>(kb + off);
            zq = *reinterpret_cast<const uint4 *>(qb + off);
        }
        st.k[i] = zk;
        st.q[i] = zq;
    }
    const size_t v_row = (size_t)a.Hv * DV * sizeof(IO);
    const char *vb = reinterpret_cast<const char *>(a.v) + ((size_t)h * DV + dv0) * sizeof(IO);
#pragma unroll
    for (int i = 0; i < C::V_VEC; ++i) {
        const int f = tid + THREADS * i;
        const int row = f / C::V_SPR, seg = f % C::V_SPR;
        uint4 z = make_uint4(0, 0, 0, 0);
        if (row < CH && row < nval)
            z = *reinterpret_cast<const uint4 *>(vb + (size_t)(tok0 + row) * v_row + (size_t)seg * 16);
        st.v[i] = z;
    }
    st.g = 0.f;
    st.b = 0.f;
    if (tid < CH && tid < nval) {
        st.g = a.g[(size_t)(tok0 + tid) * a.Hv + h];
        st.b = a.beta[(size_t)(tok0 + tid) * a.Hv + h];
    }
}

template <bool BF16, int DVS>
__device__ __forceinline__ void stage_commit(const Stage<BF16, DVS> &st, Smem<BF16, DVS> &s, int tid) {
    using C = Cfg<BF16, DVS>;
    using CT = typename C::CT;
    using IO = typename C::IO;
    constexpr int CT_PER_SEG = 16 / (int)sizeof(CT);
#pragma unroll
    for (int i = 0; i < C::KQ_VEC; ++i) {
        const int f = tid + THREADS * i;
        const int row = f / C::KQ_SPR, seg = f % C::KQ_SPR;
        *reinterpret_cast<uint4 *>(&s.K[row * C::KS + seg * CT_PER_SEG]) = st.k[i];
        *reinterpret_cast<uint4 *>(&s.Q[row * C::KS + seg * CT_PER_SEG]) = st.q[i];
    }
#pragma unroll
    for (int i = 0; i < C::V_VEC; ++i) {
        const int f = tid + THREADS * i;
        const int row = f / C::V_SPR, seg = f % C::V_SPR;
        if (row < CH) {
            const IO *e = reinterpret_cast<const IO *>(&st.v[i]);
#pragma unroll
            for (int j = 0; j < C::IO_PER_SEG; ++j) {
                float x;
                if constexpr (BF16) x = bf16_bits_to_f32(e[j]);
                else x = e[j];
                s.V[row * DVS + seg * C::IO_PER_SEG + j] = x;
            }
        }
    }
    if (tid < CH) {
        s.graw[tid] = st.g;
        s.beta[tid] = st.b;
    }
}

// Four consecutive CT values from fp32, written as one vector store.
template <typename CT>
__device__ __forceinline__ void store4(CT *p, float a0, float a1, float a2, float a3) {
    if constexpr (std::is_same<CT, float>::value) {
        *reinterpret_cast<f32x4 *>(p) = f32x4{a0, a1, a2, a3};
    } else {
        bf16x4 t;
        t[0] = f32_to_bf16(a0); t[1] = f32_to_bf16(a1);
        t[2] = f32_to_bf16(a2); t[3] = f32_to_bf16(a3);
        *reinterpret_cast<bf16x4 *>(p) = t;
    }
}

// Four consecutive values stored as the split pair (hi, lo) on the bf16 path, or
// plainly on the fp32 path.
template <bool SPLIT, typename CT>
__device__ __forceinline__ void store4s(CT *hi, CT *lo, float a0, float a1, float a2, float a3) {
    if constexpr (SPLIT) {
        const CT h0 = Cvt<CT>::from_f32(a0), h1 = Cvt<CT>::from_f32(a1);
        const CT h2 = Cvt<CT>::from_f32(a2), h3 = Cvt<CT>::from_f32(a3);
        store4<CT>(hi, Cvt<CT>::to_f32(h0), Cvt<CT>::to_f32(h1), Cvt<CT>::to_f32(h2), Cvt<CT>::to_f32(h3));
        store4<CT>(lo, a0 - Cvt<CT>::to_f32(h0), a1 - Cvt<CT>::to_f32(h1), a2 - Cvt<CT>::to_f32(h2),
                   a3 - Cvt<CT>::to_f32(h3));
    } else {
        (void)lo;
        store4<CT>(hi, a0, a1, a2, a3);
    }
}

// Blocks T_iw (i > W) of column block W of T = (I + A)^-1:
//   T_iw = -T_ii * sum_{j=W}^{i-1} A_ij T_jw .
// tcol[j] holds T_jw in accumulator layout, which is also the B-operand layout, so
// the partial results stay in registers; only T_ii and A_ij are read from LDS.
template <bool BF16, int DVS, int W>
__device__ __forceinline__ void solve_column_block(Smem<BF16, DVS> &s, const f32x4 &tdiag,
                                                   int l16, int g4) {
    using C = Cfg<BF16, DVS>;
    using CT = typename C::CT;
    f32x4 tcol[4];
    tcol[W] = tdiag;
#pragma unroll
    for (int i = W + 1; i < 4; ++i) {
        f32x4 X = zero4();
#pragma unroll
        for (int j = W; j < i; j += 2) {
            Frag<CT> fa, fb;
            const float *ar = &s.A[(16 * i + l16) * C::AS + 16 * j + 4 * g4];
            const f32x4 a0 = *reinterpret_cast<const f32x4 *>(ar);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                fa.set(e, a0[e]);
                fb.set(e, tcol[j][e]);
            }
            if (j + 1 < i) {
                const f32x4 a1 = *reinterpret_cast<const f32x4 *>(ar + 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    fa.set(4 + e, a1[e]);
                    fb.set(4 + e, tcol[j + 1][e]);
                }
            } else {
#pragma unroll
                for (int e = 4; e < 8; ++e) {
                    fa.set(e, 0.f);
                    fb.set(e, 0.f);
                }
            }
            mma(X, fa, fb);
        }
        Frag<CT> fa, fb;
        fa.zero();
        fb.zero();
        fa.load4(0, &s.Tm[(16 * i + l16) * C::TS + 16 * i + 4 * g4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) fb.set(e, -X[e]);
        f32x4 Y = zero4();
        mma(Y, fa, fb);
        tcol[i] = Y;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            s.Tm[(16 * i + 4 * g4 + r) * C::TS + 16 * W + l16] = Cvt<CT>::from_f32(Y[r]);
    }
}

template <bool BF16, int DVS>
__global__ __launch_bounds__(THREADS) void gdn_prefill_kernel(const PrefillArgs a) {
    using C = Cfg<BF16, DVS>;
    using CT = typename C::CT;
    using IO = typename C::IO;
    constexpr int NT = C::NT;
    __shared__ Smem<BF16, DVS> s;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, l16 = lane & 15, g4 = lane >> 4;

    // Work item.  Consecutive items are the slices of one head; when the grid is a
    // multiple of 8 they are numbered so that a head's slices share an XCD (whose
    // L2 then serves that head's q/k tiles to all of them).
    const int G = gridDim.x;
    int item = blockIdx.x;
    if ((G & 7) == 0) item = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const int slice = item % a.nslices;
    const int h = (item / a.nslices) % a.Hv;
    const int n = item / (a.nslices * a.Hv);
    const int hk = h % a.Hk;
    const int dv0 = slice * DVS;
    int bos = 0, eos = a.T_tot;
    if (a.cu) {
        bos = a.cu[n];
        eos = a.cu[n + 1];
    }
    const int len = eos > bos ? eos - bos : 0;
    const int nchunks = (len + CH - 1) / CH;

    // State slice: st[mt][nt] holds S^T rows (key channels) 32w + 16mt + 4G + r,
    // column (value channel) dv0 + 16nt + l16.
    f32x4 st[2][NT];
    const size_t sbase = ((size_t)n * a.Hv + h) * (size_t)DV * DK;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int dv = dv0 + 16 * nt + l16, dk = 32 * w + 16 * mt + 4 * g4;
            f32x4 x = zero4();
            if (a.s0) x = *reinterpret_cast<const f32x4 *>(a.s0 + sbase + (size_t)dv * DK + dk);
            st[mt][nt] = x;
            store4<CT>(&s.S[(16 * nt + l16) * C::KS + dk], x[0], x[1], x[2], x[3]);
        }
    for (int i = tid; i < CH * C::TS; i += THREADS) {
        s.Tm[i] = Cvt<CT>::from_f32(0.f);
        s.Pm[i] = Cvt<CT>::from_f32(0.f);
        if constexpr (C::SPLIT) s.Pm_lo[i] = Cvt<CT>::from_f32(0.f);
    }

    Stage<BF16, DVS> stg;
    if (nchunks > 0) stage_load<BF16, DVS>(stg, a, bos, min(CH, len), h, hk, dv0, tid);

    for (int c = 0; c < nchunks; ++c) {
        const int tok0 = bos + c * CH;
        const int nval = min(CH, eos - tok0);
        stage_commit<BF16, DVS>(stg, s, tid);
        if (c + 1 < nchunks)
            stage_load<BF16, DVS>(stg, a, tok0 + CH, min(CH, eos - tok0 - CH), h, hk, dv0, tid);
        __syncthreads();

        // #1 Gate: inclusive prefix sum of g over the chunk, lane = token.
        if (w == 0) {
            float x = s.graw[lane];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            const float last = __shfl(x, 63, 64);
            s.gcum[lane] = x;
            s.gam[lane] = __expf(x);
            s.lam[lane] = __expf(last - x);
        }
        __syncthreads();

        // #2 KKT and the Q K^T gram: 10 lower tiles each, 5 tile jobs per wave.
        for (int job = w; job < 20; job += 4) {
            const bool isq = job >= 10;
            const int tt = isq ? job - 10 : job;
            const int bi = (int)((0x3333222110ull >> (4 * tt)) & 0xF);
            const int bj = (int)((0x3210210100ull >> (4 * tt)) & 0xF);
            const CT *arow = (isq ? s.Q : s.K) + (16 * bi + l16) * C::KS + 8 * g4;
            const CT *brow = s.K + (16 * bj + l16) * C::KS + 8 * g4;
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                Frag<CT> fa, fb;
                fa.load8(arow + 32 * kb);
                fb.load8(brow + 32 * kb);
                mma(acc, fa, fb);
            }
            const int sc = 16 * bj + l16;
            const float gs = s.gcum[sc];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rr = 16 * bi + 4 * g4 + r;
                const float gr = s.gcum[rr];
                if (!isq) {
                    const float d = (sc < rr) ? __expf(gr - gs) : 0.f;
                    s.A[rr * C::AS + sc] = (sc < rr) ? s.beta[rr] * acc[r] * d : 0.f;
                } else {
                    const float d = (sc <= rr) ? __expf(gr - gs) : 0.f;
                    const float p = (sc <= rr) ? acc[r] * d : 0.f;
                    const CT ph = Cvt<CT>::from_f32(p);
                    s.Pm[rr * C::TS + sc] = ph;
                    if constexpr (C::SPLIT) s.Pm_lo[rr * C::TS + sc] = Cvt<CT>::from_f32(p - Cvt<CT>::to_f32(ph));
                }
            }
        }

        // R = beta V - beta gamma (K S^T) and Q S^T for tokens [16w, 16w + 16).
        f32x4 qs[NT];
        {
            const CT *krow = s.K + (16 * w + l16) * C::KS + 8 * g4;
            const CT *qrow = s.Q + (16 * w + l16) * C::KS + 8 * g4;
            f32x4 ks[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                ks[nt] = zero4();
                qs[nt] = zero4();
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                Frag<CT> fk, fq;
                fk.load8(krow + 32 * kb);
                fq.load8(qrow + 32 * kb);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    Frag<CT> fs;
                    fs.load8(s.S + (16 * nt + l16) * C::KS + 32 * kb + 8 * g4);
                    mma(ks[nt], fk, fs);
                    mma(qs[nt], fq, fs);
                }
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int nn = 16 * nt + l16;
                float rv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * w + 4 * g4 + r;
                    rv[r] = s.beta[t] * (s.V[t * DVS + nn] - s.gam[t] * ks[nt][r]);
                }
                store4s<C::SPLIT, CT>(&s.Rt[nn * C::TS + 16 * w + 4 * g4],
                                      &s.Rt_lo[C::LO * (nn * C::TS + 16 * w + 4 * g4)],
                                      rv[0], rv[1], rv[2], rv[3]);
            }
        }
        __syncthreads();

        // #3 Solve, part 1: wave w inverts the unit lower-triangular diagonal block
        // I + A_ww by substitution; lane l16 computes column l16 of the inverse.
        f32x4 tdiag;
        {
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = (i == l16) ? 1.f : 0.f;
                const float *ar = &s.A[(16 * w + i) * C::AS + 16 * w];
#pragma unroll
                for (int j = 0; j < i; ++j) acc -= ar[j] * x[j];
                x[i] = acc;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = g4 == 0 ? x[r] : g4 == 1 ? x[4 + r] : g4 == 2 ? x[8 + r] : x[12 + r];
                tdiag[r] = v;
                s.Tm[(16 * w + 4 * g4 + r) * C::TS + 16 * w + l16] = Cvt<CT>::from_f32(v);
            }
        }
        __syncthreads();

        // #3 Solve, part 2: blocks below the diagonal, wave w fills column block w.
        switch (w) {
            case 0: solve_column_block<BF16, DVS, 0>(s, tdiag, l16, g4); break;
            case 1: solve_column_block<BF16, DVS, 1>(s, tdiag, l16, g4); break;
            case 2: solve_column_block<BF16, DVS, 2>(s, tdiag, l16, g4); break;
            default: break;
        }
        __syncthreads();

        // #5-read: v = T R for tokens [16w, 16w + 16).  T is lower triangular, so
        // only the first w/2 + 1 blocks of 32 columns contribute.
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 acc = zero4();
            const CT *trow = s.Tm + (16 * w + l16) * C::TS + 8 * g4;
            const CT *rrow = s.Rt + (16 * nt + l16) * C::TS + 8 * g4;
            for (int kb = 0; kb <= (w >> 1); ++kb) {
                Frag<CT> fa, fb;
                fa.load8(trow + 32 * kb);
                fb.load8(rrow + 32 * kb);
                mma(acc, fa, fb);
                if constexpr (C::SPLIT) {
                    fb.load8(s.Rt_lo + (16 * nt + l16) * C::TS + 8 * g4 + 32 * kb);
                    mma(acc, fa, fb);
                }
            }
            const int nn = 16 * nt + l16;
            const int t0 = 16 * w + 4 * g4;
            const int lo_off = C::LO * (nn * C::TS + t0);
            store4s<C::SPLIT, CT>(&s.Vt[nn * C::TS + t0], &s.Vt_lo[lo_off], acc[0], acc[1], acc[2], acc[3]);
            store4s<C::SPLIT, CT>(&s.Vlt[nn * C::TS + t0], &s.Vlt_lo[lo_off], s.lam[t0] * acc[0],
                                  s.lam[t0 + 1] * acc[1], s.lam[t0 + 2] * acc[2], s.lam[t0 + 3] * acc[3]);
        }
        __syncthreads();

        // #6 O = diag(gamma) Q S^T + P v for tokens [16w, 16w + 16), stored.
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 acc = zero4();
            const CT *prow = s.Pm + (16 * w + l16) * C::TS + 8 * g4;
            const CT *vrow = s.Vt + (16 * nt + l16) * C::TS + 8 * g4;
            for (int kb = 0; kb <= (w >> 1); ++kb) {
                Frag<CT> fa, fb;
                fa.load8(prow + 32 * kb);
                fb.load8(vrow + 32 * kb);
                mma(acc, fa, fb);
                if constexpr (C::SPLIT) {
                    Frag<CT> fal, fbl;
                    fal.load8(s.Pm_lo + (16 * w + l16) * C::TS + 8 * g4 + 32 * kb);
                    fbl.load8(s.Vt_lo + (16 * nt + l16) * C::TS + 8 * g4 + 32 * kb);
                    mma(acc, fa, fbl);
                    mma(acc, fal, fb);
                }
            }
            IO *ob = reinterpret_cast<IO *>(a.o) + (size_t)h * DV + dv0 + 16 * nt + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * w + 4 * g4 + r;
                if (t < nval) {
                    const float y = s.gam[t] * qs[nt][r] + acc[r];
                    IO out;
                    if constexpr (BF16) out = __builtin_bit_cast(uint16_t, f32_to_bf16(y));
                    else out = y;
                    ob[(size_t)(tok0 + t) * a.Hv * DV] = out;
                }
            }
        }

        // #5-update: S^T[key ch][value ch] = gamma_last S^T + K^T (lambda v), wave w
        // updating key channels [32w, 32w + 32).  The K^T operand is gathered from
        // the token-major K tile (slot e of group G <-> token 32kb + 8G + e).
        {
            const float glast = s.gam[CH - 1];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                Frag<CT> ka[2];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        ka[kb].set_raw(e, s.K[(32 * kb + 8 * g4 + e) * C::KS + 32 * w + 16 * mt + l16]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    f32x4 acc = st[mt][nt] * glast;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        Frag<CT> fb;
                        fb.load8(s.Vlt + (16 * nt + l16) * C::TS + 32 * kb + 8 * g4);
                        mma(acc, ka[kb], fb);
                        if constexpr (C::SPLIT) {
                            fb.load8(s.Vlt_lo + (16 * nt + l16) * C::TS + 32 * kb + 8 * g4);
                            mma(acc, ka[kb], fb);
                        }
                    }
                    st[mt][nt] = acc;
                    store4<CT>(&s.S[(16 * nt + l16) * C::KS + 32 * w + 16 * mt + 4 * g4],
                               acc[0], acc[1], acc[2], acc[3]);
                }
            }
        }
        __syncthreads();
    }

    if (a.sN) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int dv = dv0 + 16 * nt + l16, dk = 32 * w + 16 * mt + 4 * g4;
                *reinterpret_cast<f32x4 *>(a.sN + sbase + (size_t)dv * DK + dk) = st[mt][nt];
            }
    }
}

template <bool BF16, int DVS>
static hipError_t launch_t(const PrefillArgs &a, int grid, hipStream_t stream) {
    hipLaunchKernelGGL((gdn_prefill_kernel<BF16, DVS>), dim3(grid), dim3(THREADS), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &a, bool bf16, int dvs, int grid, hipStream_t stream) {
    if (bf16) {
        switch (dvs) {
            case 16: return launch_t<true, 16>(a, grid, stream);
            case 32: return launch_t<true, 32>(a, grid, stream);
        }
    } else {
        switch (dvs) {
            case 16: return launch_t<false, 16>(a, grid, stream);
        }
    }
    return hipErrorInvalidValue;
}

int prefill_threads() { return THREADS; }

int prefill_lds_bytes(bool bf16, int dvs) {
    if (bf16) {
        switch (dvs) {
            case 16: return (int)sizeof(Smem<true, 16>);
            case 32: return (int)sizeof(Smem<true, 32>);
        }
    } else {
        switch (dvs) {
            case 16: return (int)sizeof(Smem<false, 16>);
        }
    }
    return -1;
}

}  // namespace gdn
