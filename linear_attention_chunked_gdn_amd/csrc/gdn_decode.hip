// Single-token gated delta-rule step (decoding) for gfx950.
//
// For each (sequence b, value head h) with key head h % Hk, one token updates the
// fp32 state in place and reads the output from the updated state ("Empowering
// Hybrid Attention Models on NPUs", section 2.1: token-by-token recurrence serves
// decoding; the state is updated with k_t, v_t, then read with q_t):
//
//   S <- alpha S (I - beta k k^T) + beta v k^T = alpha S - alpha beta (S k) k^T + beta v k^T
//   o  = S q
//
// Every value-channel row of S evolves independently given k, q and its own v
// entry, so the kernel is row-parallel: 16 lanes own one row (8 key channels each,
// two 16-byte loads), the two dot products are reduced across those 16 lanes, and
// a 256-thread workgroup covers 16 rows.  The step is bound by the state's read and
// write (128 KiB per head).
//
// With a per-key-channel gate (KDA: g is [B, Hv, 128]) the scalar alpha becomes
// Diag(a), a_j = exp(g_j), on the key index, applied before the erase:
//   S <- S Diag(a) (I - beta k k^T) + beta v k^T:  D = S Diag(a), S = D - beta (D k) k^T + beta v k^T.
//
// DecodeArgs::prologue (GDN_PROLOGUE_* flags) applies the input prologue first: q and k
// divided by max(||x||_2, 1e-12) (the norms reduced over the row's 16 lanes), beta =
// sigmoid(beta), g = -softplus(g) (per channel for the per-channel gate).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

constexpr int DEC_D = 128;
constexpr int DEC_ROWS = 16;   // rows per workgroup

template <typename IO>
__device__ __forceinline__ void load8_io(const void *base, size_t off, float *x) {
    if constexpr (sizeof(IO) == 2) {
        typedef IO v8 __attribute__((ext_vector_type(8)));
        const v8 u = *reinterpret_cast<const v8 *>(reinterpret_cast<const IO *>(base) + off);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = Cvt<IO>::to_f32(u[i]);
    } else {
        const float *p = reinterpret_cast<const float *>(base) + off;
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
    }
}

__device__ __forceinline__ float sum16(float x) {
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m, 16);
    return x;
}

// softplus(x) = max(x, 0) + log(1 + e^-|x|), which cannot overflow
__device__ __forceinline__ float softplus_f(float x) { return fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x))); }

template <typename IO, bool PER_CHANNEL>
__global__ __launch_bounds__(256) void gdn_decode_kernel(const DecodeArgs a) {
    constexpr int RB = DEC_D / DEC_ROWS;
    const int rb = blockIdx.x % RB;
    const int bh = blockIdx.x / RB;
    const int h = bh % a.Hv, b = bh / a.Hv, hk = h % a.Hk;
    const int row = rb * DEC_ROWS + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;

    float *srow = a.state + (((size_t)b * a.Hv + h) * DEC_D + row) * DEC_D + 8 * l;
    float S[8], kk[8], qq[8];
    {
        const f32x4 s0 = *reinterpret_cast<const f32x4 *>(srow);
        const f32x4 s1 = *reinterpret_cast<const f32x4 *>(srow + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { S[i] = s0[i]; S[4 + i] = s1[i]; }
    }
    const size_t koff = ((size_t)b * a.Hk + hk) * DEC_D + 8 * l;
    load8_io<IO>(a.k, koff, kk);
    load8_io<IO>(a.q, koff, qq);
    const size_t voff = ((size_t)b * a.Hv + h) * DEC_D + row;
    const float vi = Cvt<IO>::to_f32(reinterpret_cast<const IO *>(a.v)[voff]);
    if (a.prologue & GDN_PROLOGUE_QK_L2NORM) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sk += kk[i] * kk[i];
            sq += qq[i] * qq[i];
        }
        const float rk = 1.f / fmaxf(sqrtf(sum16(sk)), 1e-12f);
        const float rq = 1.f / fmaxf(sqrtf(sum16(sq)), 1e-12f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kk[i] *= rk;
            qq[i] *= rq;
        }
    }
    float beta = a.beta[(size_t)b * a.Hv + h];
    if (a.prologue & GDN_PROLOGUE_BETA_SIGMOID) beta = 1.f / (1.f + __expf(-beta));
    const bool do_softplus = a.prologue & GDN_PROLOGUE_G_SOFTPLUS;
    float o = 0.f;
    if constexpr (PER_CHANNEL) {
        float gg[8];
        load8_io<float>(a.g, ((size_t)b * a.Hv + h) * DEC_D + 8 * l, gg);
        float u = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (do_softplus) gg[i] = -softplus_f(gg[i]);
            S[i] *= __expf(gg[i]);                // S Diag(a)
            u += S[i] * kk[i];
        }
        u = sum16(u);                               // (S Diag(a) k)_row
        const float erase = beta * u;
        const float write = beta * vi;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            S[i] = S[i] - erase * kk[i] + write * kk[i];
            o += S[i] * qq[i];
        }
    } else {
        float gs = a.g[(size_t)b * a.Hv + h];
        if (do_softplus) gs = -softplus_f(gs);
        const float alpha = __expf(gs);
        float u = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) u += S[i] * kk[i];
        u = sum16(u);                               // (S k)_row, state before the token
        const float erase = alpha * beta * u;
        const float write = beta * vi;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            S[i] = alpha * S[i] - erase * kk[i] + write * kk[i];
            o += S[i] * qq[i];
        }
    }
    o = sum16(o);                               // (S q)_row, updated state
    *reinterpret_cast<f32x4 *>(srow) = f32x4{S[0], S[1], S[2], S[3]};
    *reinterpret_cast<f32x4 *>(srow + 4) = f32x4{S[4], S[5], S[6], S[7]};
    if (l == 0) reinterpret_cast<IO *>(a.o)[voff] = Cvt<IO>::from_f32(o);
}

template <bool PER_CHANNEL>
hipError_t launch_decode_kind(const DecodeArgs &a, int io, hipStream_t stream) {
    const int grid = a.B * a.Hv * (DEC_D / DEC_ROWS);
    if (io == 1)
        hipLaunchKernelGGL((gdn_decode_kernel<__bf16, PER_CHANNEL>), dim3(grid), dim3(256), 0, stream, a);
    else if (io == 2)
        hipLaunchKernelGGL((gdn_decode_kernel<_Float16, PER_CHANNEL>), dim3(grid), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((gdn_decode_kernel<float, PER_CHANNEL>), dim3(grid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, int io, hipStream_t stream) {
    return launch_decode_kind<false>(a, io, stream);
}

hipError_t launch_kda_decode(const DecodeArgs &a, int io, hipStream_t stream) {
    return launch_decode_kind<true>(a, io, stream);
}

}  // namespace gdn
