// Device-side helpers for the gfx950 gated delta-rule kernels: element types,
// conversions and the 16x16 MFMA tile abstraction.
//
// MFMA operand convention used throughout.  A 16x16 output tile is computed by
// steps that each contract 32 values of the reduction index k.  In one step, lane
// l supplies for its row m = l % 16 (A operand) or column n = l % 16 (B operand)
// eight "slots" e = 0..7 of lane group G = l / 16.  Slot (G, e) stands for one k
// index; which k it stands for is chosen by the caller, and the A and B operands of
// a step must use the same choice.  The product is the same for every choice
// because the MFMA pairs A slot (G, e) with B slot (G, e) and sums over all 32.
//
//   bf16 path: one v_mfma_f32_16x16x32_bf16 per step (8 bf16 slots per lane).
//   fp16 path: one v_mfma_f32_16x16x32_f16 per step (8 fp16 slots per lane).
//   fp32 path: eight v_mfma_f32_16x16x4_f32 per step, MFMA e taking slot e.
//
// The accumulator layout is the common 16x16 one: lane l holds rows 4*(l/16)+r,
// r = 0..3, of column l % 16.  Read as a B operand, the four rows a lane holds in
// each of two stacked tiles are exactly eight slots of one column, which lets a
// result feed the next product without leaving registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// A lane's value from lane l ^ 2 and from lane l ^ 1 of its group of four, by DPP quad
// permutations (2, 3, 0, 1) and (1, 0, 3, 2): a VALU move, no LDS round trip.
__device__ __forceinline__ unsigned from_lane_xor2(unsigned x) {
    return (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ unsigned from_lane_xor1(unsigned x) {
    return (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
}

__device__ __forceinline__ float bf16_to_f32(__bf16 x) {
    return __uint_as_float(static_cast<uint32_t>(__builtin_bit_cast(uint16_t, x)) << 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
// round-to-nearest-even (hardware conversion on gfx950)
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return static_cast<__bf16>(x); }

template <typename CT> struct Cvt;
template <> struct Cvt<__bf16> {
    __device__ static __forceinline__ float to_f32(__bf16 x) { return bf16_to_f32(x); }
    __device__ static __forceinline__ __bf16 from_f32(float x) { return f32_to_bf16(x); }
};
template <> struct Cvt<_Float16> {
    __device__ static __forceinline__ float to_f32(_Float16 x) { return (float)x; }
    __device__ static __forceinline__ _Float16 from_f32(float x) { return (_Float16)x; }
};
template <> struct Cvt<float> {
    __device__ static __forceinline__ float to_f32(float x) { return x; }
    __device__ static __forceinline__ float from_f32(float x) { return x; }
};

// Four-element vectors of a 16-bit element type (one 8-byte access).
template <typename CT> struct Vec4;
template <> struct Vec4<__bf16> { typedef bf16x4 type; };
template <> struct Vec4<_Float16> { typedef f16x4 type; };

// Eight slots of one MFMA step operand.
template <typename CT> struct Frag;

template <> struct Frag<__bf16> {
    bf16x8 v;
    __device__ __forceinline__ void zero() {
        for (int e = 0; e < 8; ++e) v[e] = f32_to_bf16(0.f);
    }
    __device__ __forceinline__ void set(int e, float x) { v[e] = f32_to_bf16(x); }
    __device__ __forceinline__ void set_raw(int e, __bf16 x) { v[e] = x; }
    // eight consecutive elements, 16-byte aligned
    __device__ __forceinline__ void load8(const __bf16 *p) {
        v = *reinterpret_cast<const bf16x8 *>(p);
    }
    // four consecutive elements into slots [4h, 4h+4), 8-byte aligned
    __device__ __forceinline__ void load4(int h, const __bf16 *p) {
        bf16x4 t = *reinterpret_cast<const bf16x4 *>(p);
        for (int e = 0; e < 4; ++e) v[4 * h + e] = t[e];
    }
};

template <> struct Frag<_Float16> {
    f16x8 v;
    __device__ __forceinline__ void zero() {
        for (int e = 0; e < 8; ++e) v[e] = (_Float16)0.f;
    }
    __device__ __forceinline__ void set(int e, float x) { v[e] = (_Float16)x; }
    __device__ __forceinline__ void set_raw(int e, _Float16 x) { v[e] = x; }
    __device__ __forceinline__ void load8(const _Float16 *p) {
        v = *reinterpret_cast<const f16x8 *>(p);
    }
    __device__ __forceinline__ void load4(int h, const _Float16 *p) {
        f16x4 t = *reinterpret_cast<const f16x4 *>(p);
        for (int e = 0; e < 4; ++e) v[4 * h + e] = t[e];
    }
};

template <> struct Frag<float> {
    float v[8];
    __device__ __forceinline__ void zero() {
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    __device__ __forceinline__ void set(int e, float x) { v[e] = x; }
    __device__ __forceinline__ void set_raw(int e, float x) { v[e] = x; }
    __device__ __forceinline__ void load8(const float *p) {
        f32x4 a = *reinterpret_cast<const f32x4 *>(p);
        f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
        for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
    }
    __device__ __forceinline__ void load4(int h, const float *p) {
        f32x4 a = *reinterpret_cast<const f32x4 *>(p);
        for (int e = 0; e < 4; ++e) v[4 * h + e] = a[e];
    }
};

__device__ __forceinline__ void mma(f32x4 &acc, const Frag<__bf16> &a, const Frag<__bf16> &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4 &acc, const Frag<_Float16> &a, const Frag<_Float16> &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4 &acc, const Frag<float> &a, const Frag<float> &b) {
    for (int e = 0; e < 8; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Steps of the fused input prologue (GDN_PROLOGUE_* flags).
constexpr float kLog2e = 1.4426950408889634f;
// beta = sigmoid(x)
__device__ __forceinline__ float prologue_sigmoid(float x) { return 1.f / (1.f + __builtin_amdgcn_exp2f(-x * kLog2e)); }
// g = -softplus(x) = -(max(x, 0) + log(1 + e^-|x|))
__device__ __forceinline__ float prologue_neg_softplus(float x) {
    return -(fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e)) / kLog2e);
}
// 1 / max(||x||_2, 1e-12) for the row whose 16-byte pieces (8 values each) the 16 lanes
// of this lane's DPP row hold; every lane of the row gets the result (row rotations).
// (`piece`: any 16-byte vector holding 8 values of type IO)
template <typename IO, typename V>
__device__ __forceinline__ float row_rnorm(const V &piece) {
    typedef IO v8 __attribute__((ext_vector_type(8)));
    static_assert(sizeof(V) == sizeof(v8), "a row piece is 8 values");
    const v8 x = __builtin_bit_cast(v8, piece);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float f = Cvt<IO>::to_f32(x[e]);
        ss += f * f;
    }
    // row_ror:8, 4, 2, 1 (dpp_ctrl 0x120 + n)
    ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x128, 0xF, 0xF, false));
    ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x124, 0xF, 0xF, false));
    ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x122, 0xF, 0xF, false));
    ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x121, 0xF, 0xF, false));
    return __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));   // 1 / max(||x||, 1e-12)
}

}  // namespace gdn
