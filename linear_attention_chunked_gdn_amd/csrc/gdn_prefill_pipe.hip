// Wave-specialised, software-pipelined chunked gated delta-rule prefill for gfx950,
// bf16 or fp16 I/O (the kernel is a template on the 16-bit I/O type IO).
//
// The chunkwise formulas and the column-wise split of the state are those of
// gdn_prefill.hip (see there), scheduled so the two halves of the Map-Reduce-Map
// pipeline ("Empowering Hybrid Attention Models on NPUs", section 2.1, Figure 1(b))
// run side by side.  Operand precision of the products (fp32 accumulation always):
//   * q, k, v and the state copy used by K S^T and Q S^T: the I/O type (q, k, v
//     exactly);
//   * T, R, v and P, which the kernel computes: fp16 (11-bit significand), one MFMA
//     per product; a single bf16 rounding of R, v or P would cost 1.4-3.6 % of the
//     output RMS, fp16 costs a quarter of that.  They stay far inside fp16's range
//     for L2-normalised q and k (|P| <= 1) and values of ordinary size;
//   * lambda v, multiplied with K^T in the update: bf16 hi + lo for bf16 I/O, one fp16
//     operand for fp16 I/O.
//
// Roles:
//
//   * four "map" waves do the S-independent work of chunk c+1 -- the gate scan (#1),
//     the K K^T and Q K^T grams (#2) and the (I + A)^-1 solve (#3);
//   * four "chain" waves hold the fp32 state slice in registers and do the
//     S-dependent work of chunk c -- R = beta V - beta gamma K S^T, v = T R
//     (#4/#5-read), the output (#6) and the in-place update (#5-update).
//
// Waves i and i+4 share SIMD i, so each SIMD interleaves one map and one chain
// wave and the latency of one hides behind the other.  A chunk costs three
// workgroup barriers:
//
//   phase 1:  chain R(c), Q S^T(c)       | map: T(c) blocks below the diagonal (waves
//                                        |      0-2), diagonal tiles of A(c+1) (2, 3)
//             all waves: k, v of chunk c+2 into LDS (gate scan: wave 1); fetch c+3
//   phase 2:  chain v(c) = T(c) R(c)     | map: A(c+1) below the diagonal (waves 0-2),
//                                        |      first half of the diagonal solve (3)
//             all waves: q of chunk c+1 into LDS (q of c is dead); fetch q of c+2
//   phase 3:  chain O(c), S update       | map: Q K^T(c+1) -> P(c+1) (waves 0-2), rest
//                                        |      of the diagonal blocks of T(c+1) (3)
//
// LDS holds three buffers (chunk mod 3) of the k and v tiles, the gates and P, so k of
// chunk c+1 is in place when phase 1 starts; q, T and A are single-buffered because
// their lifetimes do not overlap across the phases (the diagonal tiles of A(c+1) and
// the blocks of A(c) below it, read in the same phase, are disjoint).
// One workgroup = 8 wave64s = one (sequence, value head, 16 value channels).
//
// Fused input prologue (the kernel's PRO template parameter; each setting is a kernel of
// its own, with its own registers and LDS layout): q and k arrive unnormalised and
// beta, g as their logits.  The gate scan applies beta = sigmoid(x) and g = -softplus(x).
// The L2 norms of the q and k rows are reduced in fp32 while the rows are staged (the
// 16 lanes that commit a row), and 1 / ||row|| is kept per token; q and k stay exact
// 16-bit MFMA operands and the reciprocal norms are folded into the per-row factors the
// kernel applies anyway: the grams' decay factors (r_row * r_col), beta gamma in R,
// lambda in the update and gamma on Q S^T.
#include "gdn_device.h"
#include "gdn_launch.h"

#include <type_traits>

namespace gdn {
namespace pipe {

constexpr int CH = 64;        // chunk length
constexpr int DK = 128;
constexpr int DV = 128;
constexpr int DVS = 16;       // value channels per workgroup
constexpr int THREADS = 512;   // 4 map + 4 chain waves
// LDS row strides, chosen by measurement on gfx950: 16-lane groups reading 16 B
// from 16 consecutive rows are conflict-free when the row stride in bytes is 32
// modulo 64 (288 B, 160 B); 8-byte writes across rows prefer an odd multiple of 8 B
// (P, written in 8-byte pieces and read less often, uses 144 B).
constexpr int KS = DK + 16;   // bf16 row stride of K and the state copy (288 B)
constexpr int TS = CH + 16;   // bf16 row stride of T, R^T, v^T, (lambda v)^T (160 B)
constexpr int TP = CH + 8;    // bf16 row stride of P (144 B)
constexpr int VS = DVS;       // bf16 row stride of the value tile (32 B)
constexpr int NBUF = 3;       // buffers of the per-chunk tiles (k, v, gates, P)
constexpr int AS = CH + 8;    // fp32 row stride of A (288 B)
constexpr float LOG2E = 1.4426950408889634f;

typedef __bf16 bf;
typedef _Float16 hf;

// Per-chunk gate quantities, computed once by one map wave from the staged g.
// Decays inside a chunk are exp(Gamma_r - Gamma_s), r >= s.  For r and s in different
// 16-token blocks (r in block i > block of s) they are formed as u_r * w[i-1]_s with
// u_r = exp(Gamma_r - Gamma_16i') (i' the block of r) and w[i-1]_s = exp(Gamma_16i -
// Gamma_s): both exponents are <= 0 when g <= 0, so neither factor can overflow.
template <bool PRO>
struct Gate {
    float beta[CH];   // beta (0 past the chunk's end)
    float gam[CH];    // gamma_t = exp(Gamma_t)
    float lam[CH];    // lambda_t = exp(Gamma_last - Gamma_t)
    float g2[CH];     // Gamma_t * log2(e)
    float u[CH];      // exp(Gamma_t - Gamma at the first token of t's 16-token block)
    float w[3][CH];   // w[i-1][s] = exp(Gamma_16i - Gamma_s) for s < 16i, else 0
    float rn[PRO ? 2 : 0][CH];  // 1 / ||k_t|| and 1 / ||q_t|| (input prologue only)
};

template <typename IO, bool PRO>
struct __align__(16) Smem {
    // The small tiles come first: a DS instruction's immediate offset reaches 64 KiB,
    // so these are addressed from one base register plus constants.
    float A[CH * AS];              // A of the chunk being mapped, strictly lower
    hf T[CH * TS];                 // T = (I + A)^-1
    IO S[DVS * KS];                // copy of the state slice [value ch][key ch] in IO's type
    hf Rh[DVS * TS];               // R^T
    hf Vh[DVS * TS];               // v^T
    IO Wh[DVS * TS], Wl[DVS * TS];  // (diag(lambda) v)^T (hi + lo for bf16 I/O)
    Gate<PRO> gate[NBUF];
    IO V[NBUF][CH * VS];
    IO K[NBUF][CH * KS];
    IO Q[CH * KS];
    hf Ph[NBUF][CH * TP];          // P
};

__device__ __forceinline__ float to_f(bf x) { return bf16_to_f32(x); }

template <typename IO> constexpr bool IS_F16 = std::is_same<IO, hf>::value;

// Four values rounded to IO and written with one 8-byte store.
template <typename IO>
__device__ __forceinline__ void store4_io(IO *p, const f32x4 &x) {
    typename Vec4<IO>::type t;
#pragma unroll
    for (int r = 0; r < 4; ++r) t[r] = Cvt<IO>::from_f32(x[r]);
    *reinterpret_cast<typename Vec4<IO>::type *>(p) = t;
}

// ds_read_b64_tr_b16 for either 16-bit element type.
__device__ __forceinline__ bf16x4 ds_read_tr4(const bf *p) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
}
__device__ __forceinline__ f16x4 ds_read_tr4(const hf *p) {
    typedef __fp16 fp16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)p));
}

// Four consecutive values as split bf16 pairs (hi, lo).
__device__ __forceinline__ void store4_split(bf *hi, bf *lo, float a0, float a1, float a2, float a3) {
    bf16x4 h, l;
    h[0] = f32_to_bf16(a0); h[1] = f32_to_bf16(a1); h[2] = f32_to_bf16(a2); h[3] = f32_to_bf16(a3);
    l[0] = f32_to_bf16(a0 - to_f(h[0])); l[1] = f32_to_bf16(a1 - to_f(h[1]));
    l[2] = f32_to_bf16(a2 - to_f(h[2])); l[3] = f32_to_bf16(a3 - to_f(h[3]));
    *reinterpret_cast<bf16x4 *>(hi) = h;
    *reinterpret_cast<bf16x4 *>(lo) = l;
}

// Four consecutive values as fp16.
__device__ __forceinline__ void store4_h(hf *p, float a0, float a1, float a2, float a3) {
    *reinterpret_cast<f16x4 *>(p) = f16x4{(hf)a0, (hf)a1, (hf)a2, (hf)a3};
}

// Column-per-lane results into a row-major fp16 tile with 4-byte writes.  Lane pairs
// (2k, 2k+1) hold columns 2k and 2k+1 of the same rows; for each pair of rows the pair
// swaps one value (DPP quad_perm [1,0,3,2]) so the even lane writes row r and the odd
// lane row r+1, each as two adjacent bf16.  Two lanes writing the halves of one LDS
// dword with 2-byte stores is several times slower.  `col0` points at (row 0, the
// lane's column); rows are `stride` elements apart; NR is even.
template <int NR>
__device__ __forceinline__ void store_cols_paired(hf *col0, int stride, const float (&x)[NR], int l16) {
    const bool odd = l16 & 1;
    hf *p = col0 + (odd ? stride - 1 : 0);
#pragma unroll
    for (int r = 0; r < NR; r += 2) {
        const float send = odd ? x[r] : x[r + 1];
        const float recv = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, true));
        f16x2 w;
        w[0] = (hf)(odd ? recv : x[r]);
        w[1] = (hf)(odd ? x[r + 1] : recv);
        *reinterpret_cast<f16x2 *>(p + r * stride) = w;
    }
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP shifts inside each row of 16
// lanes, then the totals of the earlier rows are added.
__device__ __forceinline__ float wave_inclusive_scan(float x, int lane) {
    // row_shr:n (dpp_ctrl 0x110 + n); lanes with no source in their row read 0
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
    const int row = lane >> 4;
    x += (row >= 1 ? r0 : 0.f) + (row >= 2 ? r1 : 0.f) + (row >= 3 ? r2 : 0.f);
    return x;
}

struct Work {
    size_t kq_base;         // byte offset of this key head in q and k
    size_t kq_row;          // bytes between tokens in q/k
    size_t v_row;           // bytes between tokens in v
    size_t v_off;           // byte offset of (head, slice) in v
    unsigned kq_row32, v_row32;   // the same strides as 32-bit values (row offsets < 2^32)
    int h, bos, eos;
};

// Staged copy of one chunk's k, v, g and beta, fetched a chunk ahead.  Loads are
// unconditional: rows past the chunk's end read the last valid token instead (finite
// values), because a load under a branch would make the compiler wait for it at the
// branch join.  Those rows need no zeros: their g and beta are set to 0 when the gate
// is computed, so their rows of A, R and v vanish, and their k and v then contribute
// nothing; their q only reaches outputs that are not stored.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct Stage {
    u32x4 k0, k1;   // native vectors so the stage always lives in registers
    unsigned v;
    float g, b;
    int nval;
};
struct StageQ {
    u32x4 q0, q1;
};

// Rows of the staged tiles a thread loads: k and q rows tid/16 and tid/16 + 32 (16-byte
// segment tid%16); v row tid/8 (4-byte piece tid%8); g, beta row tid%64.  Every thread
// loads and commits the same amount, with no branch around a load or an LDS write,
// so the compiler's wait for a staged value covers exactly that value and not the
// younger prefetches.  The chunk's base address is wave-uniform (scalar registers)
// and each lane adds a 32-bit offset; rows are clamped only in a sequence's short
// last chunk.
__device__ __forceinline__ void stage_load(Stage &st, const PrefillArgs &a, const Work &wk, int tok0,
                                           int nval, int tid) {
    const char *kb = reinterpret_cast<const char *>(a.k) + wk.kq_base + (size_t)tok0 * wk.kq_row;
    const char *vb = reinterpret_cast<const char *>(a.v) + wk.v_off + (size_t)tok0 * wk.v_row;
    const float *gb = a.g + (size_t)tok0 * a.Hv + wk.h;
    const float *bb = a.beta + (size_t)tok0 * a.Hv + wk.h;
    int r0 = tid >> 4, r1 = (tid + THREADS) >> 4, rv = tid >> 3, rg = tid & (CH - 1);
    if (nval < CH) {
        r0 = min(r0, nval - 1);
        r1 = min(r1, nval - 1);
        rv = min(rv, nval - 1);
        rg = min(rg, nval - 1);
    }
    const unsigned seg = (tid & 15) * 16;
    st.k0 = *reinterpret_cast<const u32x4 *>(kb + ((unsigned)r0 * wk.kq_row32 + seg));
    st.k1 = *reinterpret_cast<const u32x4 *>(kb + ((unsigned)r1 * wk.kq_row32 + seg));
    st.v = *reinterpret_cast<const unsigned *>(vb + ((unsigned)rv * wk.v_row32 + (tid & 7) * 4));
    st.g = gb[(unsigned)rg * (unsigned)a.Hv];
    st.b = bb[(unsigned)rg * (unsigned)a.Hv];
    st.nval = nval;
}

__device__ __forceinline__ void stage_load_q(StageQ &st, const PrefillArgs &a, const Work &wk, int tok0,
                                             int nval, int tid) {
    const char *qb = reinterpret_cast<const char *>(a.q) + wk.kq_base + (size_t)tok0 * wk.kq_row;
    int r0 = tid >> 4, r1 = (tid + THREADS) >> 4;
    if (nval < CH) {
        r0 = min(r0, nval - 1);
        r1 = min(r1, nval - 1);
    }
    const unsigned seg = (tid & 15) * 16;
    st.q0 = *reinterpret_cast<const u32x4 *>(qb + ((unsigned)r0 * wk.kq_row32 + seg));
    st.q1 = *reinterpret_cast<const u32x4 *>(qb + ((unsigned)r1 * wk.kq_row32 + seg));
}

// First token of the chunk to prefetch.  Past the sequence's last chunk the last chunk
// is fetched again (in bounds, never used), so every loop trip issues the same loads
// and commits; the commits then land in the LDS buffer or q tile that no wave reads
// any more.
__device__ __forceinline__ int prefetch_tok(const Work &wk, int c, int nchunks) {
    return wk.bos + min(c, nchunks - 1) * CH;
}

template <typename IO, bool PRO>
__device__ __forceinline__ void stage_commit(const Stage &st, Smem<IO, PRO> &s, int buf, int tid, unsigned pro) {
    const int seg = tid & 15;
    *reinterpret_cast<u32x4 *>(&s.K[buf][(tid >> 4) * KS + seg * 8]) = st.k0;
    *reinterpret_cast<u32x4 *>(&s.K[buf][((tid + THREADS) >> 4) * KS + seg * 8]) = st.k1;
    *reinterpret_cast<unsigned *>(&s.V[buf][(tid >> 3) * VS + (tid & 7) * 2]) = st.v;
    if constexpr (PRO) {
        const bool norm = pro & GDN_PROLOGUE_QK_L2NORM;
        const float r0 = norm ? row_rnorm<IO>(st.k0) : 1.f, r1 = norm ? row_rnorm<IO>(st.k1) : 1.f;
        if (seg == 0) {
            s.gate[buf].rn[0][tid >> 4] = r0;
            s.gate[buf].rn[0][(tid + THREADS) >> 4] = r1;
        }
    } else {
        (void)pro;
    }
}

template <typename IO, bool PRO>
__device__ __forceinline__ void stage_commit_q(const StageQ &st, Smem<IO, PRO> &s, int buf, int tid, unsigned pro) {
    const int seg = tid & 15;
    *reinterpret_cast<u32x4 *>(&s.Q[(tid >> 4) * KS + seg * 8]) = st.q0;
    *reinterpret_cast<u32x4 *>(&s.Q[((tid + THREADS) >> 4) * KS + seg * 8]) = st.q1;
    if constexpr (PRO) {
        const bool norm = pro & GDN_PROLOGUE_QK_L2NORM;
        const float r0 = norm ? row_rnorm<IO>(st.q0) : 1.f, r1 = norm ? row_rnorm<IO>(st.q1) : 1.f;
        if (seg == 0) {
            s.gate[buf].rn[1][tid >> 4] = r0;
            s.gate[buf].rn[1][(tid + THREADS) >> 4] = r1;
        }
    } else {
        (void)buf;
        (void)pro;
    }
}

// #1 Gate for the chunk staged in buffer buf, by map wave 3 (lane = token): the
// inclusive scan of g and every decay factor the grams and the chain need.
template <typename IO, bool PRO>
__device__ __forceinline__ void gate_scan(const Stage &st, Smem<IO, PRO> &s, int buf, int lane, unsigned pro) {
    const bool valid = lane < st.nval;
    float g = st.g, beta = st.b;
    if constexpr (PRO) {
        // beta = sigmoid(x); g = -softplus(x) = -(max(x, 0) + log(1 + e^-|x|))
        if (pro & GDN_PROLOGUE_BETA_SIGMOID) beta = prologue_sigmoid(beta);
        if (pro & GDN_PROLOGUE_G_SOFTPLUS) g = prologue_neg_softplus(g);
    } else {
        (void)pro;
    }
    const float x2 = wave_inclusive_scan(valid ? g : 0.f, lane) * LOG2E;
    const float last2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x2), 63));
    const float b16 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x2), 16));
    const float b32 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x2), 32));
    const float b48 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x2), 48));
    const float b0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x2), 0));
    const int blk = lane >> 4;
    const float start = blk == 0 ? b0 : blk == 1 ? b16 : blk == 2 ? b32 : b48;
    Gate<PRO> &gt = s.gate[buf];
    gt.beta[lane] = valid ? beta : 0.f;
    gt.g2[lane] = x2;
    gt.gam[lane] = __builtin_amdgcn_exp2f(x2);
    gt.lam[lane] = __builtin_amdgcn_exp2f(last2 - x2);
    // u and w share one reference per 16-token block, the inclusive Gamma at the
    // block's first token, so u_r * w_s = exp(Gamma_r - Gamma_s) exactly.
    gt.u[lane] = __builtin_amdgcn_exp2f(x2 - start);
    gt.w[0][lane] = lane < 16 ? __builtin_amdgcn_exp2f(b16 - x2) : 0.f;
    gt.w[1][lane] = lane < 32 ? __builtin_amdgcn_exp2f(b32 - x2) : 0.f;
    gt.w[2][lane] = lane < 48 ? __builtin_amdgcn_exp2f(b48 - x2) : 0.f;
}

// ---------------------------------------------------------------------------------
// Map: grams of the chunk in buffer nb.  The ten lower 16x16 tiles of K K^T (phase 2)
// are spread over the four map waves, those of Q K^T (phase 3) over waves 1-3.  Tiles
// are computed transposed (K_j X_i^T with X = K or Q), so each lane ends with one row
// and four consecutive columns and writes them with one vector store.
// ---------------------------------------------------------------------------------
// Per-element factor of tile (bi, bj) for this lane's row and four columns: the decay,
// times beta of the row for K K^T.  Computed before the tile's products so the gate
// reads overlap the MFMAs.
template <bool ISQ, typename IO, bool PRO>
__device__ __forceinline__ f32x4 gram_scale(const Smem<IO, PRO> &s, int nb, int bi, int bj, int l16, int g4) {
    const Gate<PRO> &gt = s.gate[nb];
    const int rr = 16 * bi + l16;          // row of this lane
    const int c0 = 16 * bj + 4 * g4;       // first of its four columns
    f32x4 d;
    if (bi == bj) {
        // same 16-token block: direct exponent differences, masked before use
        const float gr = gt.g2[rr];
        const f32x4 gc = *reinterpret_cast<const f32x4 *>(&gt.g2[c0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool keep = ISQ ? (c0 + r <= rr) : (c0 + r < rr);
            d[r] = keep ? __builtin_amdgcn_exp2f(gr - gc[r]) : 0.f;
        }
    } else {
        const float ur = gt.u[rr];
        const f32x4 wc = *reinterpret_cast<const f32x4 *>(&gt.w[bi - 1][c0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) d[r] = ur * wc[r];
    }
    if constexpr (!ISQ) {
        const float br = gt.beta[rr];
#pragma unroll
        for (int r = 0; r < 4; ++r) d[r] *= br;
    }
    if constexpr (PRO) {
        const float rrow = s.gate[nb].rn[ISQ ? 1 : 0][rr];
        const f32x4 rcol = *reinterpret_cast<const f32x4 *>(&s.gate[nb].rn[0][c0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) d[r] *= rrow * rcol[r];
    }
    return d;
}

// A goes to s.A (fp32), P to s.Ph[nb] (fp16).
template <bool ISQ, typename IO, bool PRO>
__device__ __forceinline__ void gram_store(Smem<IO, PRO> &s, int nb, int bi, int bj, const f32x4 &acc, const f32x4 &d,
                                          int l16, int g4) {
    const int rr = 16 * bi + l16;
    const int c0 = 16 * bj + 4 * g4;
    if constexpr (!ISQ) {
        *reinterpret_cast<f32x4 *>(&s.A[rr * AS + c0]) =
            f32x4{acc[0] * d[0], acc[1] * d[1], acc[2] * d[2], acc[3] * d[3]};
    } else {
        store4_h(&s.Ph[nb][rr * TP + c0], acc[0] * d[0], acc[1] * d[1], acc[2] * d[2], acc[3] * d[3]);
    }
}

// Up to four tiles of one gram, each given as 4 * (row block) + (column block), -1 for
// none.  Operand fragments shared by several tiles are read once per step.
template <bool ISQ, int T0, int T1, int T2, int T3, typename IO, bool PRO>
__device__ __forceinline__ void gram_tiles(Smem<IO, PRO> &s, int nb, int l16, int g4) {
    constexpr int tl[4] = {T0, T1, T2, T3};
    constexpr int NT = (T0 >= 0) + (T1 >= 0) + (T2 >= 0) + (T3 >= 0);
    f32x4 c[NT], d[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        c[t] = zero4();
        d[t] = gram_scale<ISQ>(s, nb, tl[t] >> 2, tl[t] & 3, l16, g4);
    }
    const IO *xs = ISQ ? s.Q : s.K[nb];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            // tile (bi, bj) is computed transposed, K_bj X_bi^T
            Frag<IO> kj, x;
            kj.load8(s.K[nb] + (16 * (tl[t] & 3) + l16) * KS + 32 * kb + 8 * g4);
            x.load8(xs + (16 * (tl[t] >> 2) + l16) * KS + 32 * kb + 8 * g4);
            mma(c[t], kj, x);
        }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) gram_store<ISQ>(s, nb, tl[t] >> 2, tl[t] & 3, c[t], d[t], l16, g4);
}

// K K^T of the chunk in buffer nb, all ten tiles over the four map waves (first chunk).
template <typename IO, bool PRO>
__device__ __forceinline__ void map_gram_kk(Smem<IO, PRO> &s, int nb, int m, int l16, int g4) {
    switch (m) {
        case 0: gram_tiles<false, 12, 13, -1, -1>(s, nb, l16, g4); break;   // (3,0) (3,1)
        case 1: gram_tiles<false, 14, 15, 0, -1>(s, nb, l16, g4); break;    // (3,2) (3,3) (0,0)
        case 2: gram_tiles<false, 8, 9, 10, -1>(s, nb, l16, g4); break;     // (2,0) (2,1) (2,2)
        default: gram_tiles<false, 4, 5, -1, -1>(s, nb, l16, g4); break;    // (1,0) (1,1)
    }
}

// K K^T tiles below the diagonal, over map waves 0-2 (the diagonal tiles are computed
// one phase earlier by wave 3, which then solves the diagonal blocks of T from them).
template <typename IO, bool PRO>
__device__ __forceinline__ void map_gram_kk_below(Smem<IO, PRO> &s, int nb, int m, int l16, int g4) {
    switch (m) {
        case 0: gram_tiles<false, 12, 13, -1, -1>(s, nb, l16, g4); break;   // (3,0) (3,1)
        case 1: gram_tiles<false, 14, 8, -1, -1>(s, nb, l16, g4); break;    // (3,2) (2,0)
        default: gram_tiles<false, 9, 4, -1, -1>(s, nb, l16, g4); break;    // (2,1) (1,0)
    }
}

// Q K^T of the chunk in buffer nb (q in the single q buffer), ten tiles over three map
// waves: m = 1..3 for the first chunk, m = 0..2 in the loop.
template <typename IO, bool PRO>
__device__ __forceinline__ void map_gram_qk(Smem<IO, PRO> &s, int nb, int m, int l16, int g4) {
    switch (m) {
        case 0: gram_tiles<true, 12, 13, 14, 15>(s, nb, l16, g4); break;    // row block 3
        case 1: gram_tiles<true, 8, 9, 10, -1>(s, nb, l16, g4); break;      // row block 2
        default: gram_tiles<true, 0, 4, 5, -1>(s, nb, l16, g4); break;      // row blocks 0, 1
    }
}

// ---------------------------------------------------------------------------------
// Map: the four diagonal 16x16 blocks of T = (I + A)^-1 by substitution, all in one
// wave: lane group G solves block G, lane l16 computing column l16 of its inverse.
// Each block is solved as two 8-row halves (rows 0-7, then rows 8-15 after the
// independent update by the lower-left 8x8 block), each half read into registers
// first and solved right-looking, so the updates of one step are independent.  The
// first half runs in one phase, the update, the second half and the stores in the
// next; x carries the columns across the barrier.
// ---------------------------------------------------------------------------------
// Rows 8+R0 .. 8+R1-1 of a diagonal block minus the lower-left 8x8 block times rows
// 0-7 (the update between the two halves of the substitution).
template <int R0, int R1, typename IO, bool PRO>
__device__ __forceinline__ void diag_update_rows(const Smem<IO, PRO> &s, int g4, float (&x)[16]) {
    const float *bblk = &s.A[(16 * g4 + 8) * AS + 16 * g4];
    float b[8][8];
#pragma unroll
    for (int r = R0; r < R1; ++r)
#pragma unroll
        for (int q = 0; q < 8; q += 4) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(bblk + r * AS + q);
#pragma unroll
            for (int e = 0; e < 4; ++e) b[r][q + e] = t[e];
        }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = R0; r < R1; ++r) x[8 + r] -= b[r][j] * x[j];
}

// rows of the update done in the first phase of the solve, the rest in the second
constexpr int DIAG_SPLIT = 0;

template <typename IO, bool PRO>
__device__ __forceinline__ void diag_solve_first(const Smem<IO, PRO> &s, int l16, int g4, float (&x)[16]) {
    const float *ablk = &s.A[(16 * g4) * AS + 16 * g4];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == l16) ? 1.f : 0.f;
    float a[8][8];
#pragma unroll
    for (int r = 1; r < 8; ++r)
#pragma unroll
        for (int q = 0; q < r; q += 4) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(ablk + r * AS + q);
#pragma unroll
            for (int e = 0; e < 4; ++e) a[r][q + e] = t[e];
        }
#pragma unroll
    for (int j = 0; j < 7; ++j)
#pragma unroll
        for (int r = j + 1; r < 8; ++r) x[r] -= a[r][j] * x[j];
    diag_update_rows<0, DIAG_SPLIT>(s, g4, x);
}

template <typename IO, bool PRO>
__device__ __forceinline__ void diag_solve_second(Smem<IO, PRO> &s, int l16, int g4, float (&x)[16]) {
    diag_update_rows<DIAG_SPLIT, 8>(s, g4, x);
    const float *ablk = &s.A[(16 * g4 + 8) * AS + 16 * g4 + 8];
    float a[8][8];
#pragma unroll
    for (int r = 1; r < 8; ++r)
#pragma unroll
        for (int q = 0; q < r; q += 4) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(ablk + r * AS + q);
#pragma unroll
            for (int e = 0; e < 4; ++e) a[r][q + e] = t[e];
        }
#pragma unroll
    for (int j = 0; j < 7; ++j)
#pragma unroll
        for (int r = j + 1; r < 8; ++r) x[8 + r] -= a[r][j] * x[8 + j];
    store_cols_paired<16>(&s.T[(16 * g4) * TS + 16 * g4 + l16], TS, x, l16);
}

// ---------------------------------------------------------------------------------
// Map: blocks of column block CB below the diagonal, T_i,CB = -T_ii sum_j A_ij T_j,CB.
// Results stay in registers (accumulator layout == B-operand layout) between steps.
// ---------------------------------------------------------------------------------
template <int CB, typename IO, bool PRO>
__device__ __forceinline__ void map_merges(Smem<IO, PRO> &s, int l16, int g4) {
    // every operand read from LDS up front, so the three dependent levels wait on one
    // round of loads instead of one per level
    f32x4 a[4][4];       // a[i][j]: A_ij, row 16i + l16, columns 16j + 4G..+3
    f16x4 tii[4];        // row 16i + l16 of T_ii, columns 16i + 4G..+3
    f32x4 tcol[4];
#pragma unroll
    for (int i = CB + 1; i < 4; ++i) {
#pragma unroll
        for (int j = CB; j < i; ++j)
            a[i][j] = *reinterpret_cast<const f32x4 *>(&s.A[(16 * i + l16) * AS + 16 * j + 4 * g4]);
        tii[i] = *reinterpret_cast<const f16x4 *>(&s.T[(16 * i + l16) * TS + 16 * i + 4 * g4]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) tcol[CB][r] = (float)s.T[(16 * CB + 4 * g4 + r) * TS + 16 * CB + l16];
#pragma unroll
    for (int i = CB + 1; i < 4; ++i) {
        f32x4 X = zero4();
#pragma unroll
        for (int j = CB; j < i; j += 2) {
            Frag<hf> fa, fb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                fa.set(e, a[i][j][e]);
                fb.set(e, tcol[j][e]);
                fa.set(4 + e, j + 1 < i ? a[i][j + 1][e] : 0.f);
                fb.set(4 + e, j + 1 < i ? tcol[j + 1][e] : 0.f);
            }
            mma(X, fa, fb);
        }
        Frag<hf> fa, fb;
        fa.zero();
        fb.zero();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            fa.set_raw(e, tii[i][e]);
            fb.set(e, -X[e]);
        }
        f32x4 Y = zero4();
        mma(Y, fa, fb);
        tcol[i] = Y;
        const float y[4] = {Y[0], Y[1], Y[2], Y[3]};
        store_cols_paired<4>(&s.T[(16 * i + 4 * g4) * TS + 16 * CB + l16], TS, y, l16);
    }
}

// ---------------------------------------------------------------------------------
// Chain, phase 1: R = beta V - beta gamma (K S^T) for tokens [16W, 16W+16).  The S
// fragments are returned for Q S^T.
// ---------------------------------------------------------------------------------
template <typename IO, bool PRO>
__device__ __forceinline__ void chain_R(Smem<IO, PRO> &s, int buf, int W, int l16, int g4, Frag<IO> (&fs)[4]) {
    const IO *krow = s.K[buf] + (16 * W + l16) * KS + 8 * g4;
    const IO *srow = s.S + l16 * KS + 8 * g4;
    // R = beta V - (beta gamma) (K S^T): the gate and V terms are read before the products
    const int t0 = 16 * W + 4 * g4;
    const f32x4 b = *reinterpret_cast<const f32x4 *>(&s.gate[buf].beta[t0]);
    const f32x4 gm = *reinterpret_cast<const f32x4 *>(&s.gate[buf].gam[t0]);
    f32x4 bv, bg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bv[i] = b[i] * Cvt<IO>::to_f32(s.V[buf][(t0 + i) * VS + l16]);
        bg[i] = b[i] * gm[i];
    }
    if constexpr (PRO) bg *= *reinterpret_cast<const f32x4 *>(&s.gate[buf].rn[0][t0]);
    f32x4 ks = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        Frag<IO> fk;
        fs[kb].load8(srow + 32 * kb);
        fk.load8(krow + 32 * kb);
        mma(ks, fk, fs[kb]);      // (K S^T): lane = value channel, rows = tokens
    }
    float r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = bv[i] - bg[i] * ks[i];
    store4_h(&s.Rh[l16 * TS + t0], r[0], r[1], r[2], r[3]);
}

// Chain, phase 1: (Q S^T)^T = S Q^T for tokens [16W, 16W+16) (lane = token, rows =
// value channels), from the S fragments loaded by chain_R.
template <typename IO, bool PRO>
__device__ __forceinline__ f32x4 chain_QS(const Smem<IO, PRO> &s, int W, int l16, int g4, const Frag<IO> (&fs)[4]) {
    const IO *qrow = s.Q + (16 * W + l16) * KS + 8 * g4;
    f32x4 qs = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        Frag<IO> fq;
        fq.load8(qrow + 32 * kb);
        mma(qs, fs[kb], fq);
    }
    return qs;
}

// Chain, phase 2: v = T R for tokens [16W, 16W+16); T is lower triangular, so only
// the first W/2 + 1 blocks of 32 columns contribute.
template <typename IO, bool PRO>
__device__ __forceinline__ void chain_v(Smem<IO, PRO> &s, int buf, int W, int l16, int g4) {
    const int t0 = 16 * W + 4 * g4;
    f32x4 lm = *reinterpret_cast<const f32x4 *>(&s.gate[buf].lam[t0]);
    if constexpr (PRO) lm *= *reinterpret_cast<const f32x4 *>(&s.gate[buf].rn[0][t0]);
    f32x4 acc = zero4();
    const hf *trow = s.T + (16 * W + l16) * TS + 8 * g4;
    for (int kb = 0; kb <= (W >> 1); ++kb) {
        Frag<hf> fa, fr;
        fa.load8(trow + 32 * kb);
        fr.load8(s.Rh + l16 * TS + 32 * kb + 8 * g4);
        mma(acc, fa, fr);
    }
    store4_h(&s.Vh[l16 * TS + t0], acc[0], acc[1], acc[2], acc[3]);
    // lambda v multiplies K^T in IO's type: one fp16 operand for fp16 I/O, bf16 hi + lo
    // for bf16 I/O
    if constexpr (IS_F16<IO>)
        store4_io(&s.Wh[l16 * TS + t0], lm * acc);
    else
        store4_split(&s.Wh[l16 * TS + t0], &s.Wl[l16 * TS + t0], lm[0] * acc[0], lm[1] * acc[1],
                     lm[2] * acc[2], lm[3] * acc[3]);
}

// Chain, phase 3: output rows of wave W, then the update of key channels
// [32W, 32W+32) of the state slice.
template <typename IO, bool PRO>
__device__ __forceinline__ void chain_out_update(Smem<IO, PRO> &s, const PrefillArgs &a, int buf, int W, int l16,
                                                 int g4, const f32x4 &qs, f32x4 (&st)[2], int h,
                                                 int dv0, int tok0, int nval) {
    const int t = 16 * W + l16;
    float gm = s.gate[buf].gam[t];
    if constexpr (PRO) gm *= s.gate[buf].rn[1][t];
    const float glast = s.gate[buf].gam[CH - 1];
    {
        // O^T = S Q^T diag(gamma) + v^T P^T: lane = token 16W + l16, rows = value
        // channels 4G..4G+3, so each lane stores four consecutive outputs at once
        f32x4 acc = qs * gm;
        const hf *ph = s.Ph[buf] + (16 * W + l16) * TP + 8 * g4;
        for (int kb = 0; kb <= (W >> 1); ++kb) {
            Frag<hf> fp, fv;
            fp.load8(ph + 32 * kb);
            fv.load8(s.Vh + l16 * TS + 32 * kb + 8 * g4);
            mma(acc, fv, fp);
        }
        if (t < nval)
            store4_io(reinterpret_cast<IO *>(a.o) + ((size_t)(tok0 + t) * a.Hv + h) * DV + dv0 + 4 * g4, acc);
    }
    {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            // K^T fragments (slot e of group G = token 32kb + 8G + e, row = key channel
            // 32W + 16mt + l16) with ds_read_b64_tr_b16: in each 16-lane group, source
            // lane a points at 4 key channels of token t0 + a/4, and result lane m then
            // holds key channel m of tokens t0..t0+3.
            Frag<IO> ka[2];
            const int a_tok = l16 >> 2, a_ch = 32 * W + 16 * mt + 4 * (l16 & 3);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int t0 = 32 * kb + 8 * g4 + 4 * hh;
                    const auto v = ds_read_tr4(&s.K[buf][(t0 + a_tok) * KS + a_ch]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) ka[kb].set_raw(4 * hh + e, v[e]);
                }
            f32x4 acc = st[mt] * glast;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                Frag<IO> fh;
                fh.load8(s.Wh + l16 * TS + 32 * kb + 8 * g4);
                mma(acc, ka[kb], fh);
                if constexpr (!IS_F16<IO>) {
                    Frag<IO> fl;
                    fl.load8(s.Wl + l16 * TS + 32 * kb + 8 * g4);
                    mma(acc, ka[kb], fl);
                }
            }
            st[mt] = acc;
            store4_io(&s.S[l16 * KS + 32 * W + 16 * mt + 4 * g4], acc);
        }
    }
}

template <typename IO, bool PRO>
__global__ __launch_bounds__(THREADS) void gdn_prefill_pipe_kernel(const PrefillArgs a) {
    __shared__ Smem<IO, PRO> s;
    const int tid = threadIdx.x;
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_map = wave < 4;
    const int W = wave & 3;   // map: block / gram job index; chain: token tile and key block

    const int G = gridDim.x;
    int item = blockIdx.x;
    if ((G & 7) == 0) item = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    const int slice = item % a.nslices;
    const int h = (item / a.nslices) % a.Hv;
    const int n = item / (a.nslices * a.Hv);
    const int hk = h % a.Hk;
    const int dv0 = slice * DVS;
    Work wk;
    wk.kq_base = (size_t)hk * DK * 2;
    wk.kq_row = (size_t)a.Hk * DK * 2;
    wk.v_row = (size_t)a.Hv * DV * 2;
    wk.v_off = ((size_t)h * DV + dv0) * 2;
    wk.kq_row32 = (unsigned)wk.kq_row;
    wk.v_row32 = (unsigned)wk.v_row;
    wk.h = h;
    wk.bos = 0;
    wk.eos = a.T_tot;
    if (a.cu) {
        wk.bos = a.cu[n];
        wk.eos = a.cu[n + 1];
    }
    const int len = wk.eos > wk.bos ? wk.eos - wk.bos : 0;
    const int nchunks = (len + CH - 1) / CH;

    // State slice, held by the chain waves: S^T rows (key channels) 32W + 16mt + 4G + r,
    // column (value channel) dv0 + l16.
    f32x4 st[2];
    const size_t sbase = ((size_t)n * a.Hv + h) * (size_t)DV * DK;
    if (!is_map) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int dk = 32 * W + 16 * mt + 4 * g4;
            f32x4 x = zero4();
            if (a.s0) x = *reinterpret_cast<const f32x4 *>(a.s0 + sbase + (size_t)(dv0 + l16) * DK + dk);
            st[mt] = x;
            store4_io(&s.S[l16 * KS + dk], x);
        }
    }

    if (nchunks > 0) {
        for (int i = tid; i < CH * TS; i += THREADS) s.T[i] = (hf)0.f;
        for (int i = tid; i < CH * TP; i += THREADS) s.Ph[0][i] = s.Ph[1][i] = s.Ph[2][i] = (hf)0.f;
        Stage stg;
        StageQ stq;
        stage_load(stg, a, wk, wk.bos, min(CH, len), tid);
        stage_load_q(stq, a, wk, wk.bos, min(CH, len), tid);
        stage_commit(stg, s, 0, tid, a.prologue);
        stage_commit_q(stq, s, 0, tid, a.prologue);
        if (wave == 2) gate_scan(stg, s, 0, lane, a.prologue);
        {
            const int t1 = prefetch_tok(wk, 1, nchunks), n1 = min(CH, wk.eos - t1);
            stage_load(stg, a, wk, t1, n1, tid);
            stage_load_q(stq, a, wk, t1, n1, tid);
            stage_commit(stg, s, 1, tid, a.prologue);
            if (wave == 2) gate_scan(stg, s, 1, lane, a.prologue);
            const int t2 = prefetch_tok(wk, 2, nchunks), n2 = min(CH, wk.eos - t2);
            stage_load(stg, a, wk, t2, n2, tid);
        }
        __syncthreads();

        // The two roles run separate loops with the same barrier sequence (three per
        // chunk), so values one role keeps across a barrier do not occupy registers in
        // the other role's code.  All 512 threads stage the tiles of later chunks: k, v,
        // g, beta two chunks ahead (committed in phase 1), q one chunk ahead (phase 2).
        // Each loop trip runs three chunks, so the LDS buffer (chunk mod 3) of every
        // access is a compile-time constant.
        using B0 = std::integral_constant<int, 0>;
        using B1 = std::integral_constant<int, 1>;
        using B2 = std::integral_constant<int, 2>;
        if (is_map) {
            // first chunk: K K^T, then Q K^T and the diagonal blocks of T
            float xd[16];   // wave 3: columns of the diagonal blocks of T, across a barrier
            map_gram_kk(s, 0, W, l16, g4);
            __syncthreads();
            if (W != 0) {
                map_gram_qk(s, 0, W - 1, l16, g4);
            } else {
                diag_solve_first(s, l16, g4, xd);
                diag_solve_second(s, l16, g4, xd);
            }
            __syncthreads();
            auto step = [&](auto bufc, int c) {
                constexpr int b0 = decltype(bufc)::value, b1 = (b0 + 1) % NBUF, b2 = (b0 + 2) % NBUF;
                const bool has_next = c + 1 < nchunks;
                const int tq = prefetch_tok(wk, c + 2, nchunks), nq = min(CH, wk.eos - tq);
                const int t3 = prefetch_tok(wk, c + 3, nchunks), n3 = min(CH, wk.eos - t3);
                // phase 1: T(c) below the diagonal; diagonal tiles of A(c+1); k, v and
                // gates of chunk c+2 (their buffers held chunk c-1, finished last step)
                switch (W) {
                    case 0: map_merges<0>(s, l16, g4); break;
                    case 1: map_merges<1>(s, l16, g4); break;
                    case 2:
                        map_merges<2>(s, l16, g4);
                        if (has_next) gram_tiles<false, 15, -1, -1, -1>(s, b1, l16, g4);
                        break;
                    default:
                        if (has_next) gram_tiles<false, 0, 5, 10, -1>(s, b1, l16, g4);
                        break;
                }
                stage_commit(stg, s, b2, tid, a.prologue);
                if (wave == 1) gate_scan(stg, s, b2, lane, a.prologue);
                stage_load(stg, a, wk, t3, n3, tid);
                __syncthreads();
                // phase 2: A(c+1) below the diagonal; first half of its diagonal solve
                if (has_next) {
                    if (W == 3) diag_solve_first(s, l16, g4, xd);
                    else map_gram_kk_below(s, b1, W, l16, g4);
                }
                stage_commit_q(stq, s, b1, tid, a.prologue);
                stage_load_q(stq, a, wk, tq, nq, tid);
                __syncthreads();
                // phase 3: P(c+1); second half of the diagonal solve of T(c+1)
                if (has_next) {
                    if (W == 3) diag_solve_second(s, l16, g4, xd);
                    else map_gram_qk(s, b1, W, l16, g4);
                }
                __syncthreads();
            };
            for (int c = 0; c < nchunks; c += 3) {
                step(B0{}, c);
                if (c + 1 < nchunks) step(B1{}, c + 1);
                if (c + 2 < nchunks) step(B2{}, c + 2);
            }
        } else {
            __syncthreads();
            __syncthreads();
            auto step = [&](auto bufc, int c) {
                constexpr int b0 = decltype(bufc)::value, b1 = (b0 + 1) % NBUF, b2 = (b0 + 2) % NBUF;
                const int tok0 = wk.bos + c * CH;
                const int nval = min(CH, wk.eos - tok0);
                const int tq = prefetch_tok(wk, c + 2, nchunks), nq = min(CH, wk.eos - tq);
                const int t3 = prefetch_tok(wk, c + 3, nchunks), n3 = min(CH, wk.eos - t3);
                // phase 1
                Frag<IO> fs[4];
                chain_R(s, b0, W, l16, g4, fs);
                const f32x4 qs = chain_QS(s, W, l16, g4, fs);
                stage_commit(stg, s, b2, tid, a.prologue);
                stage_load(stg, a, wk, t3, n3, tid);
                __syncthreads();
                // phase 2
                chain_v(s, b0, W, l16, g4);
                stage_commit_q(stq, s, b1, tid, a.prologue);
                stage_load_q(stq, a, wk, tq, nq, tid);
                __syncthreads();
                // phase 3
                chain_out_update(s, a, b0, W, l16, g4, qs, st, h, dv0, tok0, nval);
                __syncthreads();
            };
            for (int c = 0; c < nchunks; c += 3) {
                step(B0{}, c);
                if (c + 1 < nchunks) step(B1{}, c + 1);
                if (c + 2 < nchunks) step(B2{}, c + 2);
            }
        }
    }

    if (a.sN && !is_map) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int dk = 32 * W + 16 * mt + 4 * g4;
            *reinterpret_cast<f32x4 *>(a.sN + sbase + (size_t)(dv0 + l16) * DK + dk) = st[mt];
        }
    }
}

}  // namespace pipe

hipError_t launch_prefill_pipe(const PrefillArgs &a, bool f16, int grid, hipStream_t stream) {
    if (f16)
        hipLaunchKernelGGL((pipe::gdn_prefill_pipe_kernel<pipe::hf, false>), dim3(grid), dim3(pipe::THREADS), 0, stream, a);
    else
        hipLaunchKernelGGL((pipe::gdn_prefill_pipe_kernel<pipe::bf, false>), dim3(grid), dim3(pipe::THREADS), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_prefill_pipe_prologue(const PrefillArgs &a, bool f16, int grid, hipStream_t stream) {
    if (f16)
        hipLaunchKernelGGL((pipe::gdn_prefill_pipe_kernel<pipe::hf, true>), dim3(grid), dim3(pipe::THREADS), 0, stream, a);
    else
        hipLaunchKernelGGL((pipe::gdn_prefill_pipe_kernel<pipe::bf, true>), dim3(grid), dim3(pipe::THREADS), 0, stream, a);
    return hipGetLastError();
}

int prefill_pipe_lds_bytes() { return (int)sizeof(pipe::Smem<pipe::bf, false>); }

int prefill_pipe_prologue_lds_bytes() { return (int)sizeof(pipe::Smem<pipe::bf, true>); }

int prefill_pipe_threads() { return pipe::THREADS; }

}  // namespace gdn
