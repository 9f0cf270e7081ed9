// The WY products of the two-launch prefill's map kernels (gdn_map.hip, kda_map.hip):
// with T = (I + A)^-1 of one chunk of C tokens,
//
//   W = T diag(beta) Kg   (C tokens x 128 key channels),
//   U = T diag(beta) V    (C tokens x 128 value channels),
//
// so that the chain only forms v = U - W S^T.  This is the solve applied to the two
// right-hand sides that do not depend on the state (the W/U form of op #4, "Empowering
// Hybrid Attention Models on NPUs", section 2.1).
#pragma once

#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

// fp16 row stride of the right-hand sides [token][channel] (288 B)
constexpr int WY_S = 128 + 16;

// Operand^T as an MFMA A operand from a token-major fp16 tile x (row stride WY_S): row =
// channel c0 + l16, slots 4hh..4hh+3 of group G = tokens 32kb + 8G + 4hh .. +3, by
// ds_read_b64_tr_b16 (source lane a of a 16-lane group addresses 4 channels of token
// t + a / 4; result lane m then holds channel c0 + m of tokens t .. t + 3).
__device__ __forceinline__ Frag<_Float16> wy_frag_t(const _Float16 *x, int c0, int kb, int l16, int g4) {
    typedef __fp16 fp16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;
    Frag<_Float16> f;
    const int a_tok = l16 >> 2, a_ch = c0 + 4 * (l16 & 3);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int t = 32 * kb + 8 * g4 + 4 * hh;
        const f16x4 v = __builtin_bit_cast(
            f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)&x[(t + a_tok) * WY_S + a_ch]));
#pragma unroll
        for (int e = 0; e < 4; ++e) f.v[4 * hh + e] = v[e];
    }
    return f;
}

// T: fp32 or fp16 (TT), row stride `as`, lower triangular (zeros above the diagonal),
// rounded to fp16 as an MFMA operand.  kg, vb: diag(beta) Kg and diag(beta) V, fp16
// [token][channel] with row stride WY_S, in LDS.  Wave `wave` (0..3) forms channel tiles
// 2 wave and 2 wave + 1 of both products and writes them to the workspace tile in the
// chain's operand layout (gdn_launch.h, Tile): W is taken transposed (Kg^T T^T), so a
// lane holds token 16 I + l16 and four consecutive key channels of each of the two
// channel tiles, which together are its 16-byte piece of fragment WN(I, wave) (stored
// negated); U is taken as it stands (T (diag(beta) V)), so a lane holds four consecutive
// tokens of one value channel, its 8-byte piece of U(slice, I) for each of the wave's two
// slices: lanes l and l ^ 1 swap one of them, so that the even lane stores both lanes'
// pieces of the first slice and the odd lane both of the second, 16 bytes each.  DW / DU
// select the products formed (kg or vb may be null for the other).
template <int C, typename TT = float, bool DW = true, bool DU = true>
__device__ __forceinline__ void wy_products(const TT *T, int as, const _Float16 *kg, const _Float16 *vb,
                                            char *tile, int wave, int l16, int g4) {
    typedef _Float16 hf;
    const int lane = 16 * g4 + l16;
#pragma unroll
    for (int I = 0; I < C / 16; ++I) {
        f32x4 acc[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[j][0] = acc[j][1] = zero4();
#pragma unroll
        for (int kb = 0; kb <= (I >> 1); ++kb) {
            // T's row 16I + l16 as an A operand, or T^T's column as a B operand: slots =
            // tokens 32kb + 8G + e
            const TT *tr = T + (16 * I + l16) * as + 32 * kb + 8 * g4;
            Frag<hf> ft;
            if constexpr (sizeof(TT) == 2) {
                ft.load8(reinterpret_cast<const hf *>(tr));
            } else {
                const f32x4 t0 = *reinterpret_cast<const f32x4 *>(tr);
                const f32x4 t1 = *reinterpret_cast<const f32x4 *>(tr + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ft.v[e] = (hf)t0[e];
                    ft.v[4 + e] = (hf)t1[e];
                }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int c0 = 16 * (2 * wave + j);
                if constexpr (DW) mma(acc[j][0], wy_frag_t(kg, c0, kb, l16, g4), ft);
                if constexpr (DU) mma(acc[j][1], ft, wy_frag_t(vb, c0, kb, l16, g4));
            }
        }
        if constexpr (DW) {   // -W[16I + l16][32 wave + 4 g4 + e] (e < 4), [32 wave + 16 + 4 g4 + e - 4]
            f16x8 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[i] = (hf)(-acc[0][0][i]);
                w[4 + i] = (hf)(-acc[1][0][i]);
            }
            *reinterpret_cast<f16x8 *>(tile + Tile<C>::wn(I, wave) + 16 * lane) = w;
        }
        if constexpr (DU) {   // U[16I + 4 g4 + i][16 (2 wave + j) + l16]
            typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
            f16x4 u[2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) u[j][i] = (hf)acc[j][1][i];
            const int odd = lane & 1;
            const u32x2 send = __builtin_bit_cast(u32x2, odd ? u[0] : u[1]);
            u32x2 recv;
            recv[0] = from_lane_xor1(send[0]);
            recv[1] = from_lane_xor1(send[1]);
            const f16x4 other = __builtin_bit_cast(f16x4, recv);
            const f16x4 lo = odd ? other : u[0], hi = odd ? u[1] : other;
            const f16x8 piece = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            *reinterpret_cast<f16x8 *>(tile + Tile<C>::u(2 * wave + odd, I) + 8 * (lane & ~1)) = piece;
        }
    }
}

// P[16I + l16][16J + 4 g4 + i], i = 0..3 (a 16x16 gram tile taken transposed) into the
// lane's half of fragment P(I, J / 2).  J <= I; for even I the diagonal tile's fragment
// also covers tile (I, I + 1), above the diagonal, whose half is zeroed with it.
template <int C>
__device__ __forceinline__ void store_p_frag(char *tile, int I, int J, int l16, int g4, const f16x4 &x) {
    char *pf = tile + Tile<C>::p(I, J >> 1) + 16 * (16 * g4 + l16) + 8 * (J & 1);
    if (J == I && (I & 1) == 0)
        *reinterpret_cast<f16x8 *>(pf) = f16x8{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
    else
        *reinterpret_cast<f16x4 *>(pf) = x;
}

}  // namespace gdn
