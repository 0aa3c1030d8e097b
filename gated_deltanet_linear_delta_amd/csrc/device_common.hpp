// Device-side helpers shared by the gfx950 kernels of libgdn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;

// Element access for the two input dtypes.  bf16 -> f32 is exact; f32 -> bf16 rounds to nearest
// even (clang's __bf16 conversion, a v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 16-byte global load/store through a 4-float vector.
__device__ __forceinline__ floatx4 ld4(const float* p) { return *reinterpret_cast<const floatx4*>(p); }
__device__ __forceinline__ void st4(float* p, floatx4 v) { *reinterpret_cast<floatx4*>(p) = v; }

// Four consecutive elements of an input tensor as floats (8-byte load for bf16, 16 for f32).
__device__ __forceinline__ floatx4 load4f(const float* p) { return ld4(p); }
__device__ __forceinline__ floatx4 load4f(const bf16* p) {
    bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ void store4f(float* p, floatx4 v) { st4(p, v); }
__device__ __forceinline__ void store4f(bf16* p, floatx4 v) {
    bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    *reinterpret_cast<bf16x4*>(p) = o;
}

// A log decay g = log alpha as the chunk kernels use it: raised to at least -100.  The chunk
// algebra exponentiates differences of in-chunk cumulative sums of g, so g = -inf (alpha = 0,
// which clears the state: "Gated Attention Architectures", section 3) would give -inf - -inf =
// NaN.  exp(-100) is below every float32 normal (the smallest is about exp(-87.3)), so the floor
// changes no product by more than float32's own rounding.  A floored token moves the cumsum by
// about -100, where float32's spacing is 8e-6, so later differences keep that accuracy; a chunk
// of 64 floored tokens sums to -6400, far from float32's range limits.
__device__ __forceinline__ float log_decay(float g) { return fmaxf(g, -100.f); }

// Butterfly sum over lanes whose ids differ only in bits [lo_mask .. 32]: used to reduce the
// row-partials of one column group held by several lanes of a wave.
__device__ __forceinline__ float xor_sum(float x, int stride_lo) {
    for (int s = stride_lo; s < 64; s <<= 1) x += __shfl_xor(x, s, 64);
    return x;
}

}  // namespace gdn
