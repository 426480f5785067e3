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

// Two floats -> packed bfloat16 bits (lo in bits 0-15), round to nearest even, NaN stays
// NaN: one v_cvt_pk_bf16_f32.  Over every float bit pattern (FP32 denormals preserved,
// the compiler's default) it gives the same bits as rounding the float's bits by hand
// (add 0x7fff plus the kept LSB, keep the top half), and a NaN for every NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f2bf(float f) { return pack_bf2(f, 0.0f) & 0xffffu; }

__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// logistic function with the hardware reciprocal (1 ulp) instead of an IEEE division
__device__ __forceinline__ float sigmoidf_(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

// ----------------------------------------------------------------------------- MXFP8
// Block exponent of a 32-element MX block: the smallest e in [-127, 127] with
// amax * 2^-e <= 448 (E4M3's largest finite magnitude), taken from the float's bits:
// amax = (1 + m / 2^23) 2^(b - 127) gives e = b - 135, plus one when the significand
// exceeds 1.75 (= 448 / 2^8).  amax == 0 (or subnormal) -> -127.
__device__ __forceinline__ int mx_block_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int b = (int)((u >> 23) & 0xffu);
  if (b == 0) return -127;
  const int e = b - 135 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Four floats (already scaled into [-448, 448]) -> four E4M3 codes (round to nearest even).
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Max over the 4 lanes 4q .. 4q + 3 (one 32-element MX block held as 4 pieces of 8).
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 1));
  return fmaxf(v, __shfl_xor(v, 2));
}

// 8 floats of a 32-element block whose |max| is amax -> 8 E4M3 codes; returns the E8M0 byte.
__device__ __forceinline__ uint32_t mx_quantize8(const float (&v)[8], float amax, uint2& q) {
  const int e = mx_block_exp(amax);
  const float inv = ldexpf(1.0f, -e);
  q.x = pack_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  q.y = pack_e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  return (uint32_t)(e + 127);
}

__device__ __forceinline__ float absmax8(const float (&v)[8]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  return m;
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& v, float* f) {
  f[0] = lo_bf(v.x); f[1] = hi_bf(v.x); f[2] = lo_bf(v.y); f[3] = hi_bf(v.y);
  f[4] = lo_bf(v.z); f[5] = hi_bf(v.z); f[6] = lo_bf(v.w); f[7] = hi_bf(v.w);
}

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

// MXFP8 operand of a routed weight: payload rows and their E8M0 scale rows.
struct MxRef {
  MatRef data;    // E4M3 payload (bytes)
  MatRef scale;   // E8M0 bytes; for a columnwise copy its rows are blocks of 32 weight rows
};

// main_grad of one weight: FP32 or BF16 elements (ES = 4 or 2 bytes).
struct GradRef {
  uint8_t* base;
  uint8_t* const* table;
  int64_t estride;         // elements
  int64_t ld;              // elements
  int64_t row_offset;
  template <int ES>
  __device__ __forceinline__ uint8_t* row(int e, int64_t r) const {
    uint8_t* b = table ? table[e] : base + (int64_t)e * estride * ES;
    return b + (row_offset + r) * ld * ES;
  }
};

}  // namespace moe
