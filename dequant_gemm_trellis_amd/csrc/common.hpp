// Device-side building blocks shared by the trellis kernels (gfx950).
//
// Pages cited: diff views of "@mlx-bun/inference" 0.0.0-stage -> 1.0.0,
// page 60 (tiled-prefill.ts weight-tile decode, vector-expand.ts) and
// page 59 (scatter.ts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace trellis {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 256;           // weights per block
constexpr int kL = 12;            // window bits
constexpr int kLutEntries = 4096; // 2^L codebook entries
constexpr int kWave = 64;

// Words per 256-weight block.
template <int K> struct Bits {
    static constexpr int wpb = kT * K / 32;   // 16 / 24 / 32
};

// Copy the 16 KB float32 codebook into LDS with 16-byte loads
// (page 59 scatter.ts stages the LUT into threadgroup memory once per group).
template <int NTHREADS>
__device__ __forceinline__ void stage_lut(float* __restrict__ lut_s, const float* __restrict__ lut) {
    const float4* src = reinterpret_cast<const float4*>(lut);
    float4* dst = reinterpret_cast<float4*>(lut_s);
#pragma unroll
    for (int i = threadIdx.x; i < kLutEntries / 4; i += NTHREADS) dst[i] = src[i];
}

// Compile-time loop: f(std::integral_constant<int, I>{}) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Byte offset into the LDS codebook of the window that starts at bit O of a
// little-endian word array: ((bits >> O) & 0xFFF) * 4, formed as
// (bits >> (O - 2)) & 0x3FFC so the x4 costs nothing. O is a template
// constant, so every word index is known at compile time and the array stays
// in registers; the words read are w[(O-2)/32] and, if the window crosses a
// word boundary, the next one.
template <int O, int N>
__device__ __forceinline__ uint32_t lut_byte_offset(const uint32_t (&w)[N]) {
    if constexpr (O < 2) {
        return (w[0] << (2 - O)) & 0x3FFCu;
    } else {
        constexpr int s = O - 2, wi = s >> 5, sh = s & 31;
        if constexpr (sh + 14 <= 32) {
            return (w[wi] >> sh) & 0x3FFCu;
        } else {
            static_assert(wi + 1 < N, "window runs past the loaded words");
            return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & 0x3FFCu;
        }
    }
}

__device__ __forceinline__ float lds_lut(const float* lut_s, uint32_t byte_off) {
    return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lut_s) + byte_off);
}

// Two decoded weights packed as bf16x2 (low half = first): each is the float32
// product value*scale rounded to bf16, nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_weights(float v0, float v1, float scale) {
    floatx2 p = {v0 * scale, v1 * scale};
    bf16x2 h = __builtin_convertvector(p, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint16_t round_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ floatx4 mfma16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace trellis
