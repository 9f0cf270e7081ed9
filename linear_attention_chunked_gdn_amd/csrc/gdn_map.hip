// Chunk-parallel map of the scalar-gate prefill for gfx950: the Map phases #1-#4 of the
// Map-Reduce-Map pipeline ("Empowering Hybrid Attention Models on NPUs", section 2.1,
// Figure 1(b)) for every chunk of every value head at once, into the workspace tiles that
// kda_chain.hip's state recurrence reads.
//
// Per chunk of n_c <= 64 tokens, with Gamma = cumsum(g), gamma = exp(Gamma),
// lambda_r = exp(Gamma_last - Gamma_r) and D[r][s] = exp(Gamma_r - Gamma_s) for r >= s:
//
//   A = strictly-lower(diag(beta) K K^T .* D),   T = (I + A)^-1,
//   P = lower-incl-diagonal(Q K^T .* D),
//   W = T diag(beta gamma) K,  U = T diag(beta) V (stored transposed),
//   Qg = diag(gamma) Q,  Kl = diag(lambda) K (stored transposed),  gl = gamma_last,
//
// so that the chain's v = U - W S^T (= T diag(beta) (V - diag(gamma) K S^T)),
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
// One workgroup = 4 wave64s per (chunk slot, value head); 76 KiB of LDS, two per CU.
#include "gdn_device.h"
#include "gdn_launch.h"
#include "gdn_wy.h"

namespace gdn {
namespace gdnmap {

typedef _Float16 hf;

constexpr int CH = 64;
constexpr int DK = 128;
constexpr int THREADS = 256;
constexpr int XS = DK + 16;   // 16-bit row stride of the k and q tiles (288 B)
constexpr int AS = CH + 8;    // fp32 row stride of A and T (288 B)

template <typename IO>
struct __align__(16) Smem {
    union {
        struct {
            IO K[CH * XS];    // k rows of the chunk (rows past its end repeat the last)
            IO Q[CH * XS];
        } kq;
        struct {              // once the grams are done: diag(beta gamma) K, diag(beta) V
            hf Kb[CH * WY_S];
            hf Vb[CH * WY_S];
        } wy;
    };
    float A[CH * AS];         // beta-scaled, strictly lower
    float T[CH * AS];         // (I + A)^-1
    float Y[3][16 * 16];      // partial products of the block solve
    float gcum[CH];           // Gamma (flat past the chunk's end)
    float gam[CH];            // exp(Gamma)
    float lam[CH];            // exp(Gamma_last - Gamma)
    float beta[CH];           // 0 past the chunk's end
};

// Tile (I, J), I >= J, of A and P.  The product is taken transposed (K_J X_I^T), so the
// lane holds row r = 16I + l16 and columns 16J + 4g4 .. 16J + 4g4 + 3; P goes to the
// workspace as fp16, A (fp32) to LDS.
template <typename IO>
__device__ __forceinline__ void gram_tile(Smem<IO> &s, char *tile, int I, int J, int l16, int g4) {
    f32x4 accA = zero4(), accP = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        Frag<IO> kj, ki, qi;
        kj.load8(s.kq.K + (16 * J + l16) * XS + 32 * kb + 8 * g4);
        ki.load8(s.kq.K + (16 * I + l16) * XS + 32 * kb + 8 * g4);
        qi.load8(s.kq.Q + (16 * I + l16) * XS + 32 * kb + 8 * g4);
        mma(accA, kj, ki);
        mma(accP, kj, qi);
    }
    const int r = 16 * I + l16, c0 = 16 * J + 4 * g4;
    const float gr = s.gcum[r], br = s.beta[r];
    f32x4 va, vp;
    f16x4 hp;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = c0 + i;
        const float d = c <= r ? __expf(gr - s.gcum[c]) : 0.f;
        va[i] = c < r ? br * accA[i] * d : 0.f;
        vp[i] = accP[i] * d;
        hp[i] = (hf)vp[i];
    }
    *reinterpret_cast<f32x4 *>(&s.A[r * AS + c0]) = va;
    *reinterpret_cast<f16x4 *>(tile + WS_OFF_P + (r * CH + c0) * 2) = hp;
}

template <typename IO>
__global__ __launch_bounds__(THREADS, 2) void gdn_map_kernel(const KdaArgs a) {
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

    // k, q (and v) rows to LDS and registers: 64 rows x 16 segments of 8 values, 4 per thread
    typedef IO v8 __attribute__((ext_vector_type(8)));
    v8 kv[4], qv[4], vv[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int idx = tid + THREADS * p, row = idx >> 4, seg = idx & 15;
        const size_t trow = (size_t)(tok0 + min(row, nval - 1));
        const size_t off = (trow * a.Hk + hk) * DK + 8 * seg;
        kv[p] = *reinterpret_cast<const v8 *>(reinterpret_cast<const IO *>(a.k) + off);
        qv[p] = *reinterpret_cast<const v8 *>(reinterpret_cast<const IO *>(a.q) + off);
        vv[p] = *reinterpret_cast<const v8 *>(reinterpret_cast<const IO *>(a.v) + (trow * a.Hv + h) * DK + 8 * seg);
        *reinterpret_cast<v8 *>(&s.kq.K[row * XS + 8 * seg]) = kv[p];
        *reinterpret_cast<v8 *>(&s.kq.Q[row * XS + 8 * seg]) = qv[p];
    }
    // #1 Gate on wave 0, lane = token: inclusive prefix sum, flat past the chunk's end
    if (wave == 0) {
        const bool ok = lane < nval;
        const size_t gi = (size_t)(tok0 + min(lane, nval - 1)) * a.Hv + h;
        float x = ok ? a.g[gi] : 0.f;
        const float b = ok ? a.beta[gi] : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        const float last = __shfl(x, 63, 64);
        s.gcum[lane] = x;
        s.gam[lane] = __expf(x);
        s.lam[lane] = __expf(last - x);
        s.beta[lane] = b;
        const float gl = __expf(last);
        *reinterpret_cast<float2 *>(tile + WS_OFF_GL + 8 * lane) = make_float2(gl, gl);
    }
    for (int i = tid; i < CH * AS; i += THREADS) s.T[i] = 0.f;
    __syncthreads();

    // the decayed operands of the chain, fp16: Qg token-major from the registers; Kl
    // transposed from the k tile in LDS (wave b: tokens 16b .. 16b + 15, lane: channels
    // 2 lane and 2 lane + 1, two 16-byte row segments of Kl^T per channel)
    {
        hf *qg = reinterpret_cast<hf *>(tile + WS_OFF_QG);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int idx = tid + THREADS * p, row = idx >> 4;
            const float gm = s.gam[row];
            f16x8 xq;
#pragma unroll
            for (int e = 0; e < 8; ++e) xq[e] = (hf)(Cvt<IO>::to_f32(qv[p][e]) * gm);
            *reinterpret_cast<f16x8 *>(qg + 8 * idx) = xq;
        }
        typedef IO v2 __attribute__((ext_vector_type(2)));
        const int ch = 2 * lane;
        f16x8 kl[2][2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 16 * wave + i;
            const v2 kk = *reinterpret_cast<const v2 *>(&s.kq.K[t * XS + ch]);
            const float lm = s.lam[t];
            kl[0][i >> 3][i & 7] = (hf)(Cvt<IO>::to_f32(kk[0]) * lm);
            kl[1][i >> 3][i & 7] = (hf)(Cvt<IO>::to_f32(kk[1]) * lm);
        }
        hf *klt = reinterpret_cast<hf *>(tile + WS_OFF_KLT);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            *reinterpret_cast<f16x8 *>(klt + (ch + j) * CH + 16 * wave) = kl[j][0];
            *reinterpret_cast<f16x8 *>(klt + (ch + j) * CH + 16 * wave + 8) = kl[j][1];
        }
    }

    // #2 the ten lower 16x16 tiles of A and P (waves 0, 1: three tiles; 2, 3: two), and
    // zeros for P's six tiles above the diagonal
    switch (wave) {
        case 0: gram_tile(s, tile, 0, 0, l16, g4); gram_tile(s, tile, 1, 0, l16, g4); gram_tile(s, tile, 3, 3, l16, g4); break;
        case 1: gram_tile(s, tile, 1, 1, l16, g4); gram_tile(s, tile, 2, 0, l16, g4); gram_tile(s, tile, 3, 0, l16, g4); break;
        case 2: gram_tile(s, tile, 2, 1, l16, g4); gram_tile(s, tile, 2, 2, l16, g4); break;
        default: gram_tile(s, tile, 3, 1, l16, g4); gram_tile(s, tile, 3, 2, l16, g4); break;
    }
    if (tid < 192) {
        // upper tiles (I, J) = (0,1) (0,2) (0,3) (1,2) (1,3) (2,3): 16 rows x 2 segments each
        const int b = tid >> 5, row = (tid >> 1) & 15, half = tid & 1;
        const int I = b < 3 ? 0 : (b < 5 ? 1 : 2);
        const int J = b < 3 ? b + 1 : (b < 5 ? b - 1 : 3);
        f16x8 z;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (hf)0.f;
        *reinterpret_cast<f16x8 *>(tile + WS_OFF_P + ((16 * I + row) * CH + 16 * J + 8 * half) * 2) = z;
    }
    __syncthreads();
    // k and q are dead: diag(beta gamma) K and diag(beta) V go over them (read by the WY
    // products once the solve is done, after its barriers)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int idx = tid + THREADS * p, row = idx >> 4, seg = idx & 15;
        const float bk = s.beta[row] * s.gam[row], bv = s.beta[row];
        f16x8 xk, xv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            xk[e] = (hf)(Cvt<IO>::to_f32(kv[p][e]) * bk);
            xv[e] = (hf)(Cvt<IO>::to_f32(vv[p][e]) * bv);
        }
        *reinterpret_cast<f16x8 *>(&s.wy.Kb[row * WY_S + 8 * seg]) = xk;
        *reinterpret_cast<f16x8 *>(&s.wy.Vb[row * WY_S + 8 * seg]) = xv;
    }

    // #3 Solve, T = (I + A)^-1: the diagonal 16x16 blocks by substitution (wave X solves
    // block X, lane l16 one column), then the blocks below them by distance from the
    // diagonal, T_IJ = -T_II (sum_{J <= m < I} A_Im T_mJ), one block per wave on fp32
    // MFMAs (16x16x4: lane l supplies row / column l % 16 at k = l / 16).
    {
        const int X = wave, c = l16;
        const float *arow = &s.A[16 * X * AS + 16 * X];
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = r == c ? 1.f : 0.f;
#pragma unroll
            for (int q = 0; q < r; ++q) acc -= arow[r * AS + q] * x[q];
            x[r] = acc;
        }
        if (g4 == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s.T[(16 * X + r) * AS + 16 * X + c] = x[r];
        }
    }
    __syncthreads();
    for (int d = 1; d < 4; ++d) {
        const int J = wave, I = J + d;
        if (I < 4) {
            f32x4 y = zero4();
            for (int kk = 16 * J; kk < 16 * I; kk += 4)
                y = __builtin_amdgcn_mfma_f32_16x16x4f32(s.A[(16 * I + l16) * AS + kk + g4],
                                                         s.T[(kk + g4) * AS + 16 * J + l16], y, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) s.Y[J][(4 * g4 + i) * 16 + l16] = y[i];
        }
        __syncthreads();
        if (I < 4) {
            f32x4 t = zero4();
#pragma unroll
            for (int v = 0; v < 16; v += 4)
                t = __builtin_amdgcn_mfma_f32_16x16x4f32(s.T[(16 * I + l16) * AS + 16 * I + v + g4],
                                                         s.Y[J][(v + g4) * 16 + l16], t, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) s.T[(16 * I + 4 * g4 + i) * AS + 16 * J + l16] = -t[i];
        }
        __syncthreads();
    }
    // #4 W = T diag(beta gamma) K and U = T diag(beta) V to the workspace
    wy_products(s.T, AS, s.wy.Kb, s.wy.Vb, tile + WS_OFF_W, tile + WS_OFF_UT, wave, l16, g4);
}

}  // namespace gdnmap

hipError_t launch_gdn_map(const KdaArgs &a, bool f16, hipStream_t stream) {
    const dim3 grid((unsigned)a.nslots * (unsigned)a.Hv), block(gdnmap::THREADS);
    if (f16)
        hipLaunchKernelGGL(gdnmap::gdn_map_kernel<_Float16>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(gdnmap::gdn_map_kernel<__bf16>, grid, block, 0, stream, a);
    return hipGetLastError();
}

int gdn_map_lds_bytes() { return (int)sizeof(gdnmap::Smem<__bf16>); }

}  // namespace gdn
