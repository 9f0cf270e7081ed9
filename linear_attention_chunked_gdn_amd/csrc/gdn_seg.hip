// Joining the segments of the segmented chain (the Chunk-Seg-Seg mapping of "Empowering
// Hybrid Attention Models on NPUs", section 4, Figure 7): the state recurrence of one
// sequence split into segments that run at the same time, each from its own start state.
//
// Per chunk the state map is affine, S -> S M + B (M = Diag(gl) - W^T Kl, B = U^T Kl), so a
// segment run from a zero state and from the identity (in place of S, with no B term)
// gives everything needed to restart it from any state S_in:
//   X          product of the segment's M (the identity rows' end state),
//   S0_end     its end state from zero,
//   O0, E      outputs of the value rows from zero, and of the identity rows, per token,
// and then, exactly up to rounding,
//   S_end = S_in X + S0_end,      O = O0 + E S_in^T.
// The chain kernel's segment mode writes O0 and E (fp16), S0_end and X^T; segment 0
// starts from the real initial state and writes its outputs directly.
//
// gdn_seg_join_kernel: one 512-thread workgroup per (sequence, value head, 16 value
// channels) walks the segments in order, S_in(s + 1) = S_in(s) X_s + S0_end(s) with one
// fp32 MFMA product each (X_{s+1} and S0_end(s + 1) loaded while segment s is joined),
// stores every S_in as fp16 (a.sin16) and the last one as the final state.
// gdn_seg_fix_kernel: one 512-thread workgroup per (chunk slot, value head) of segments
// >= 1 issues all its loads at once (E and O0 rows, 16 bytes per lane, and S_in
// fragments), stages the chunk's E and O0 rows in LDS; wave w forms O = O0 + E S_in^T for
// value channels [16w, 16w + 16) (fp16 MFMA, fp32 accumulation) into the O0 rows' place,
// and the workgroup stores the o rows 16 bytes per lane.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {
namespace gdnseg {

constexpr int D = 128;
constexpr int ROWS = 16;        // value channels per workgroup
constexpr int RS = D + 4;       // fp32 row stride of the S_in rows in LDS
constexpr int JOIN_THREADS = 512;   // 8 waves: one per 16 key columns

// S_in(s + 1) = S_in(s) X_s + S0_end(s) for the workgroup's 16 rows, held in LDS; wave w
// forms key columns [16 w, 16 w + 16).
__global__ __launch_bounds__(JOIN_THREADS) void gdn_seg_join_kernel(const KdaArgs a) {
    __shared__ __align__(16) float R[ROWS * RS];
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int NSL = D / ROWS;
    const int slice = blockIdx.x % NSL, h = (blockIdx.x / NSL) % a.Hv, n = blockIdx.x / (NSL * a.Hv);
    const int dv0 = slice * ROWS;
    float *sb = a.sseg + ((size_t)n * a.Hv + h) * a.nseg * 2 * D * D;

    // fp16 copies of S_in(1) .. S_in(nseg - 1), [nseg][128][128] per (sequence, head)
    _Float16 *s16 = a.sin16 + ((size_t)n * a.Hv + h) * a.nseg * D * D;
    {   // S_in(1): segment 0's end state (thread t: row t / 32, keys 4 (t % 32) .. + 3)
        const int r = tid >> 5, c = 4 * (tid & 31);
        const f32x4 x = *reinterpret_cast<const f32x4 *>(sb + (size_t)(dv0 + r) * D + c);
        *reinterpret_cast<f32x4 *>(&R[r * RS + c]) = x;
        f16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (_Float16)x[e];
        *reinterpret_cast<f16x4 *>(s16 + (size_t)(dv0 + r) * D + c) = y;
    }
    __syncthreads();
    // Segment s's operands, loaded one segment ahead: the wave's 16 key columns of X_s^T (B
    // fragments; slot (g4, e) = row r = 32 kb + 8 g4 + e of X) and of S0_end(s)^T (rows
    // dv0 + 4 g4 .. + 3 of a column: 16 bytes).
    const int col = 16 * wave + l16;
    struct StepOps {
        Frag<float> fb[4];
        f32x4 s0;
    };
    auto load_step = [&](StepOps &op, int s) {
        const float *s0e = sb + (size_t)s * 2 * D * D;
        const float *xt = s0e + D * D;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) op.fb[kb].load8(xt + (size_t)col * D + 32 * kb + 8 * g4);
        op.s0 = *reinterpret_cast<const f32x4 *>(s0e + (size_t)col * D + dv0 + 4 * g4);
    };
    auto step = [&](const StepOps &op, int s) {
        // lane: rows dv0 + 4 g4 + i, key column col; the sum over a row of X in two halves
        // (two accumulators) for a shorter dependent chain
        f32x4 acc[2];
        acc[0] = op.s0;
        acc[1] = zero4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            Frag<float> fa;
            fa.load8(&R[l16 * RS + 32 * kb + 8 * g4]);
            mma(acc[kb & 1], fa, op.fb[kb]);
        }
        __syncthreads();   // every wave has read R
#pragma unroll
        for (int i = 0; i < 4; ++i) R[(4 * g4 + i) * RS + col] = acc[0][i] + acc[1][i];
        __syncthreads();
        // S_in(s + 1) from R, row-major (thread t: row t / 32, keys 4 (t % 32) .. + 3): as
        // fp16 for the fix-up, or in fp32 as the final state after the last segment.  (The
        // next step only reads R before its first barrier, as these reads do.)
        const int r = tid >> 5, c = 4 * (tid & 31);
        const f32x4 y = *reinterpret_cast<const f32x4 *>(&R[r * RS + c]);
        const size_t at = (size_t)(dv0 + r) * D + c;
        if (s + 1 < a.nseg) {
            f16x4 yh;
#pragma unroll
            for (int e = 0; e < 4; ++e) yh[e] = (_Float16)y[e];
            *reinterpret_cast<f16x4 *>(s16 + (size_t)s * D * D + at) = yh;
        } else if (a.sN) {
            *reinterpret_cast<f32x4 *>(a.sN + ((size_t)n * a.Hv + h) * D * D + at) = y;
        }
    };
    StepOps op0, op1;
    if (a.nseg > 1) load_step(op0, 1);
    for (int s = 1; s < a.nseg; s += 2) {
        if (s + 1 < a.nseg) load_step(op1, s + 1);
        step(op0, s);
        if (s + 1 >= a.nseg) break;
        if (s + 2 < a.nseg) load_step(op0, s + 2);
        step(op1, s + 1);
    }
    if (a.nseg == 1 && a.sN) {   // one segment: its end state is the final state
        const int r = tid >> 5, c = 4 * (tid & 31);
        *reinterpret_cast<f32x4 *>(a.sN + ((size_t)n * a.Hv + h) * D * D + (size_t)(dv0 + r) * D + c) =
            *reinterpret_cast<const f32x4 *>(&R[r * RS + c]);
    }
}

constexpr int FIX_THREADS = 512;   // 8 waves: one per 16 value channels

template <typename IO, int C>
__global__ __launch_bounds__(FIX_THREADS) void gdn_seg_fix_kernel(const KdaArgs a) {
    constexpr int ES = D + 8;   // 16-bit row stride of the staged E, O0 and o rows
    __shared__ __align__(16) _Float16 Es[C * ES];
    __shared__ __align__(16) _Float16 Os[C * ES];   // O0 rows, then o's (IO) in place
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slot = blockIdx.x / a.Hv, h = blockIdx.x % a.Hv;
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
    const int j = slot - (bos / C + n);
    const int tok0 = bos + C * j;
    if (tok0 >= eos) return;   // a slot no chunk uses
    const int nc = (eos - bos + C - 1) / C;
    // the segment holding chunk j: the largest s with s nc / nseg <= j
    const int seg = (int)(((long long)(j + 1) * a.nseg + nc - 1) / nc) - 1;
    if (seg == 0) return;      // segment 0 stored its outputs itself
    const int dv0 = ROWS * wave;
    const int nval = min(C, eos - tok0);

    // E and O0 rows of the chunk, 16 bytes per lane (rows clamped into the sequence: E's
    // past it become zero in LDS, O0's are not stored), and S_in, all issued before any
    // is waited for
    constexpr int EPT = C * D / 8 / FIX_THREADS;   // 16-byte row segments per thread
    static_assert(EPT * FIX_THREADS * 8 == C * D, "row segments split evenly over the threads");
    f16x8 ev[EPT], ov[EPT];
#pragma unroll
    for (int p = 0; p < EPT; ++p) {
        const int i = tid + FIX_THREADS * p, t = i / (D / 8), c = 8 * (i % (D / 8));
        const size_t at = ((size_t)(tok0 + min(t, nval - 1)) * a.Hv + h) * D + c;
        ev[p] = *reinterpret_cast<const f16x8 *>(a.e + at);
        ov[p] = *reinterpret_cast<const f16x8 *>(a.o0 + at);
    }
    // S_in(seg) rows dv0 + l16 as A operands (slots = identity rows 32 kb + 8 g4 + e)
    const _Float16 *sin = a.sin16 + (((size_t)n * a.Hv + h) * a.nseg + (seg - 1)) * D * D;
    Frag<_Float16> fs[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) fs[kb].load8(sin + (size_t)(dv0 + l16) * D + 32 * kb + 8 * g4);
#pragma unroll
    for (int p = 0; p < EPT; ++p) {
        const int i = tid + FIX_THREADS * p, t = i / (D / 8), c = 8 * (i % (D / 8));
        const f16x8 zero = {};
        *reinterpret_cast<f16x8 *>(&Es[t * ES + c]) = t < nval ? ev[p] : zero;
        *reinterpret_cast<f16x8 *>(&Os[t * ES + c]) = ov[p];
    }
    __syncthreads();

    // O^T (value channels x tokens) = O0^T + S_in E^T, one 16-token tile at a time; o back
    // into the wave's own columns of Os
#pragma unroll
    for (int t = 0; t < C / 16; ++t) {
        _Float16 *orow = &Os[(16 * t + l16) * ES + dv0 + 4 * g4];
        const f16x4 o0 = *reinterpret_cast<const f16x4 *>(orow);
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = (float)o0[i];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            Frag<_Float16> fe;
            fe.load8(&Es[(16 * t + l16) * ES + 32 * kb + 8 * g4]);
            mma(acc, fs[kb], fe);
        }
        typename Vec4<IO>::type y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = Cvt<IO>::from_f32(acc[i]);
        *reinterpret_cast<typename Vec4<IO>::type *>(orow) = y;
    }
    __syncthreads();
    // o rows of the chunk's tokens, 16 bytes per lane
#pragma unroll
    for (int p = 0; p < EPT; ++p) {
        const int i = tid + FIX_THREADS * p, t = i / (D / 8), c = 8 * (i % (D / 8));
        if (t < nval)
            *reinterpret_cast<f16x8 *>(reinterpret_cast<IO *>(a.o) + ((size_t)(tok0 + t) * a.Hv + h) * D + c) =
                *reinterpret_cast<const f16x8 *>(&Os[t * ES + c]);
    }
}

}  // namespace gdnseg

hipError_t launch_seg_join(const KdaArgs &a, hipStream_t stream) {
    constexpr unsigned NSL = gdnseg::D / gdnseg::ROWS;
    const unsigned long long items = (unsigned long long)a.N * a.Hv * NSL;
    if (a.nseg < 1 || items > 0x7fffffffULL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gdnseg::gdn_seg_join_kernel, dim3((unsigned)items), dim3(gdnseg::JOIN_THREADS), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_seg_fix(const KdaArgs &a, bool f16, int chunk, hipStream_t stream) {
    const unsigned long long items = (unsigned long long)a.nslots * a.Hv;
    if (a.nseg < 1 || items > 0x7fffffffULL) return hipErrorInvalidValue;
    if (items == 0) return hipSuccess;
    const dim3 grid((unsigned)items), block(gdnseg::FIX_THREADS);
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
