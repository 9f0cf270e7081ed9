// Fix-up of the segmented chain (the Chunk-Seg-Seg mapping of "Empowering Hybrid Attention
// Models on NPUs", section 4, Figure 7): the state recurrence of one sequence split into
// segments that run at the same time, each from its own start state, then joined here.
//
// Per chunk the state map is affine, S -> S M + B (M = Diag(gl) - W^T Kl, B = U^T Kl), so a
// segment run from a zero state and from the identity (in place of S, with no B term)
// gives everything needed to restart it from any state S_in:
//   X          product of the segment's M (the identity rows' end state),
//   S0_end     its end state from zero,
//   O0, E      outputs of the value rows from zero, and of the identity rows, per token,
// and then, exactly up to rounding,
//   S_end = S_in X + S0_end,      O = O0 + E S_in^T.
// The chain kernel's segment mode writes O0, E, S0_end and X^T; this kernel composes the
// start state of every segment (S_in of segment 0 is the initial state, so its end state
// is the first S_in) and writes o and the final state.
//
// One 256-thread workgroup per (chunk slot, value head, 16 value channels) corrects that
// chunk's outputs; N * Hv * 8 more compose the final state.  Each composes the 16 rows of
// S_in it needs in LDS, one fp32 MFMA product per earlier segment.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace gdnseg {

constexpr int D = 128;
constexpr int ROWS = 16;        // value channels per workgroup
constexpr int RS = D + 4;       // fp32 row stride of the S_in rows in LDS
constexpr int THREADS = 256;

template <typename IO, int C>
__global__ __launch_bounds__(THREADS) void gdn_seg_fix_kernel(const KdaArgs a) {
    __shared__ __align__(16) float R[ROWS * RS];
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int NSL = D / ROWS;
    const long long nout = (long long)a.nslots * a.Hv * NSL;
    const bool final_item = (long long)blockIdx.x >= nout;

    int n, h, slice, upto, tok0 = 0, eos = 0;
    if (!final_item) {
        const int slot = blockIdx.x / (a.Hv * NSL), rem = blockIdx.x % (a.Hv * NSL);
        h = rem / NSL;
        slice = rem % NSL;
        // the sequence of this slot: the last n with cu[n] / C + n <= slot
        n = 0;
        if (a.cu) {
            int lo = 0, hi = a.N - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (a.cu[mid] / C + mid <= slot) lo = mid;
                else hi = mid - 1;
            }
            n = lo;
        }
        const int bos = a.cu ? a.cu[n] : 0;
        eos = a.cu ? a.cu[n + 1] : a.T_tot;
        const int j = slot - (bos / C + n);
        tok0 = bos + C * j;
        if (tok0 >= eos) return;   // a slot no chunk uses
        const int nc = (eos - bos + C - 1) / C;
        // the segment holding chunk j: the largest s with s nc / nseg <= j
        upto = (int)(((long long)(j + 1) * a.nseg + nc - 1) / nc) - 1;
    } else {
        const int b = (int)((long long)blockIdx.x - nout);
        slice = b % NSL;
        h = (b / NSL) % a.Hv;
        n = b / (NSL * a.Hv);
        upto = a.nseg;   // through every segment
    }
    const int dv0 = slice * ROWS;
    const float *sb = a.sseg + ((size_t)n * a.Hv + h) * a.nseg * 2 * D * D;

    // S_in of segment 1 = the end state of segment 0, rows dv0 .. dv0 + 15
    for (int i = tid; i < ROWS * D / 4; i += THREADS) {
        const int r = i / (D / 4), c = 4 * (i % (D / 4));
        *reinterpret_cast<f32x4 *>(&R[r * RS + c]) =
            *reinterpret_cast<const f32x4 *>(sb + (size_t)(dv0 + r) * D + c);
    }
    __syncthreads();
    // S_in of segment s + 1 = S_in(s) X_s + S0_end(s); wave w forms key columns [32w, 32w + 32)
    for (int s = 1; s < upto; ++s) {
        const float *s0e = sb + (size_t)s * 2 * D * D, *xt = s0e + D * D;
        f32x4 acc[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int col = 32 * wave + 16 * ct + l16;
            // lane: rows dv0 + 4 g4 + i, key column col
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[ct][i] = s0e[(size_t)(dv0 + 4 * g4 + i) * D + col];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                // slot (g4, e) = row r = 32 kb + 8 g4 + e of X: R[.][r] and X^T[col][r]
                Frag<float> fa, fb;
                fa.load8(&R[l16 * RS + 32 * kb + 8 * g4]);
                fb.load8(xt + (size_t)col * D + 32 * kb + 8 * g4);
                mma(acc[ct], fa, fb);
            }
        }
        __syncthreads();
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) R[(4 * g4 + i) * RS + 32 * wave + 16 * ct + l16] = acc[ct][i];
        __syncthreads();
    }

    if (final_item) {
        if (a.sN) {
            float *dst = a.sN + ((size_t)n * a.Hv + h) * D * D;
            for (int i = tid; i < ROWS * D / 4; i += THREADS) {
                const int r = i / (D / 4), c = 4 * (i % (D / 4));
                *reinterpret_cast<f32x4 *>(dst + (size_t)(dv0 + r) * D + c) =
                    *reinterpret_cast<const f32x4 *>(&R[r * RS + c]);
            }
        }
        return;
    }

    // O^T (value channels x tokens) = O0^T + S_in E^T for the chunk's 16-token tiles
    for (int t = wave; t < C / 16; t += 4) {
        const int tok = tok0 + 16 * t + l16;
        const int tc = min(tok, eos - 1);   // rows past the sequence are read in bounds, not stored
        const size_t row = ((size_t)tc * a.Hv + h) * D;
        f32x4 acc = *reinterpret_cast<const f32x4 *>(a.o0 + row + dv0 + 4 * g4);
        if (upto > 0) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                Frag<float> fa, fb;
                fa.load8(&R[l16 * RS + 32 * kb + 8 * g4]);
                fb.load8(a.e + row + 32 * kb + 8 * g4);
                mma(acc, fa, fb);
            }
        }
        if (tok < eos) {
            typename Vec4<IO>::type y;
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = Cvt<IO>::from_f32(acc[i]);
            *reinterpret_cast<typename Vec4<IO>::type *>(reinterpret_cast<IO *>(a.o) + ((size_t)tok * a.Hv + h) * D +
                                                         dv0 + 4 * g4) = y;
        }
    }
}

}  // namespace gdnseg

hipError_t launch_seg_fix(const KdaArgs &a, bool f16, int chunk, hipStream_t stream) {
    constexpr unsigned NSL = gdnseg::D / gdnseg::ROWS;
    const unsigned long long items = ((unsigned long long)a.nslots + (unsigned long long)a.N) * a.Hv * NSL;
    if (a.nseg < 1 || items > 0x7fffffffULL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)items), block(gdnseg::THREADS);
#define SEG_FIX_LAUNCH(C)                                                                                \
    do {                                                                                                 \
        if (f16) hipLaunchKernelGGL((gdnseg::gdn_seg_fix_kernel<_Float16, C>), grid, block, 0, stream, a); \
        else hipLaunchKernelGGL((gdnseg::gdn_seg_fix_kernel<__bf16, C>), grid, block, 0, stream, a);      \
    } while (0)
    switch (chunk) {
        case 32: SEG_FIX_LAUNCH(32); break;
        case 64: SEG_FIX_LAUNCH(64); break;
        case 128: SEG_FIX_LAUNCH(128); break;
        default: return hipErrorInvalidValue;
    }
#undef SEG_FIX_LAUNCH
    return hipGetLastError();
}

}  // namespace gdn
