// Device-side helpers shared by the MoE kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 255;   // groups = experts + shared expert fit one 256-thread scan
constexpr int kMaxTopk = 8;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float -> bfloat16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) { return f2bf(lo) | (f2bf(hi) << 16); }

__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float sigmoidf_(float a) { return 1.0f / (1.0f + __expf(-a)); }

// Per-expert matrix addressing: single grouped tensor or a device pointer table.
struct MatRef {
  const uint8_t* base;     // bytes
  const uint8_t* const* table;
  int64_t estride_bytes;
  int64_t ld_bytes;
  int64_t row_offset;      // rows
  __device__ __forceinline__ const uint8_t* row(int e, int64_t r) const {
    const uint8_t* b = table ? table[e] : base + (int64_t)e * estride_bytes;
    return b + (row_offset + r) * ld_bytes;
  }
};

struct GradRef {
  float* base;
  float* const* table;
  int64_t estride;         // elements
  int64_t ld;              // elements
  int64_t row_offset;
  __device__ __forceinline__ float* row(int e, int64_t r) const {
    float* b = table ? table[e] : base + (int64_t)e * estride;
    return b + (row_offset + r) * ld;
  }
};

}  // namespace moe
