// Per-token row kernels: dispatch gather, probability-weighted combine, the
// backward's weighted gather of dy fused with the router-probability gradient,
// and the data-gradient combine.  All are HBM-bound row copies/reductions with
// 16-byte accesses; every sum runs in a fixed order (no float atomics).
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kRowThreads = 256;

__device__ __forceinline__ void load_slots(const int32_t* __restrict__ slot_of, int t, int K,
                                           int (&s)[kMaxTopk]) {
#pragma unroll
  for (int k = 0; k < kMaxTopk; ++k) s[k] = (k < K) ? slot_of[(int64_t)t * K + k] : -1;
}

// xp[slot_of[t,k]] = x[t] for every valid route (dispatch into expert-contiguous rows).
// With Q, the row is also quantised to MXFP8 along H (one E8M0 scale per 32 elements)
// into xq / xs, the A operand of the scaled-FP8 FC1.  One thread per 32-element block.
template <bool Q>
__global__ __launch_bounds__(kRowThreads) void k_gather_rows(
    const uint16_t* __restrict__ x, int H, int K, const int32_t* __restrict__ slot_of,
    uint16_t* __restrict__ xp, uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
  const int t = blockIdx.x;
  int s[kMaxTopk];
  load_slots(slot_of, t, K, s);
  const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * H);
  for (int c = threadIdx.x; c < H / 32; c += kRowThreads) {
    uint4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = src[4 * c + q];
    uint4 q0, q1;
    uint32_t sc = 0;
    if constexpr (Q) {
      float f[32];
#pragma unroll
      for (int q = 0; q < 4; ++q) unpack_bf16x8(v[q], f + 8 * q);
      sc = mx_quantize32(f, q0, q1);
    }
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) {
      if (s[k] < 0) continue;
      uint4* dst = reinterpret_cast<uint4*>(xp + (int64_t)s[k] * H) + 4 * c;
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = v[q];
      if constexpr (Q) {
        uint4* dq = reinterpret_cast<uint4*>(xq + (int64_t)s[k] * H) + 2 * c;
        dq[0] = q0;
        dq[1] = q1;
        xs[(int64_t)s[k] * (H / 32) + c] = (uint8_t)sc;
      }
    }
  }
}

// MXFP8 quantisation of bf16 rows along their length: payload [rows][cols] E4M3 and
// scales [rows][cols/32] E8M0.  Rows at or beyond *row_limit (when given) are skipped:
// the routed buffers hold offsets[E] valid rows.  One thread per 32-element block.
__global__ __launch_bounds__(kRowThreads) void k_quantize_rows(
    const uint16_t* __restrict__ in, int64_t rows, int cols, const int32_t* __restrict__ row_limit,
    uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  const int64_t nb = (int64_t)cols / 32;
  const int64_t lim = row_limit ? (int64_t)*row_limit : rows;
  const int64_t total = (lim < rows ? lim : rows) * nb;
  for (int64_t b = (int64_t)blockIdx.x * kRowThreads + threadIdx.x; b < total;
       b += (int64_t)gridDim.x * kRowThreads) {
    const int64_t r = b / nb, c = b - r * nb;
    const uint4* src = reinterpret_cast<const uint4*>(in + r * cols) + 4 * c;
    float f[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) unpack_bf16x8(src[i], f + 8 * i);
    uint4 q0, q1;
    const uint32_t s = mx_quantize32(f, q0, q1);
    uint4* dq = reinterpret_cast<uint4*>(q + r * cols) + 2 * c;
    dq[0] = q0;
    dq[1] = q1;
    sc[r * nb + c] = (uint8_t)s;
  }
}

// out[t] = y[shared_row0 + t] + sum_k w_tk * y[slot_of[t,k]], in float, fixed k order,
// one rounding to bf16.
__global__ __launch_bounds__(kRowThreads) void k_combine(
    const uint16_t* __restrict__ y, int64_t shared_row0, int H, int K,
    const int32_t* __restrict__ slot_of, const float* __restrict__ rw, uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  int s[kMaxTopk];
  load_slots(slot_of, t, K, s);
  float w[kMaxTopk];
#pragma unroll
  for (int k = 0; k < kMaxTopk; ++k) w[k] = (s[k] >= 0) ? rw[(int64_t)t * K + k] : 0.0f;
  const uint4* ys = reinterpret_cast<const uint4*>(y + (shared_row0 + t) * (int64_t)H);
  for (int c = threadIdx.x; c < H / 8; c += kRowThreads) {
    const uint4 v = ys[c];
    float a[8] = {lo_bf(v.x), hi_bf(v.x), lo_bf(v.y), hi_bf(v.y),
                  lo_bf(v.z), hi_bf(v.z), lo_bf(v.w), hi_bf(v.w)};
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) {
      if (s[k] < 0) continue;
      const uint4 r = reinterpret_cast<const uint4*>(y + (int64_t)s[k] * H)[c];
      a[0] += w[k] * lo_bf(r.x); a[1] += w[k] * hi_bf(r.x);
      a[2] += w[k] * lo_bf(r.y); a[3] += w[k] * hi_bf(r.y);
      a[4] += w[k] * lo_bf(r.z); a[5] += w[k] * hi_bf(r.z);
      a[6] += w[k] * lo_bf(r.w); a[7] += w[k] * hi_bf(r.w);
    }
    uint4 o;
    o.x = pack_bf2(a[0], a[1]); o.y = pack_bf2(a[2], a[3]);
    o.z = pack_bf2(a[4], a[5]); o.w = pack_bf2(a[6], a[7]);
    reinterpret_cast<uint4*>(out + (int64_t)t * H)[c] = o;
  }
}

// Backward gather: dyw[slot] = w_tk * dy[t] (the router weight folded into the
// routed expert's upstream gradient), and the router-probability gradient
// dprobs[t, e_tk] = dy[t] . y[slot] (y is the unweighted expert output), written
// into the dense [T][E] row with zeros off the map.  The dot products are
// reduced per thread in a fixed order and then by a fixed LDS tree.  With Q,
// w_tk * dy[t] is also quantised to MXFP8 along H (the A operand of the
// scaled-FP8 data-gradient GEMM).  One thread per 32-element block.
template <bool Q>
__global__ __launch_bounds__(kRowThreads) void k_gather_dy_dprob(
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ y, int H, int E, int K,
    const int32_t* __restrict__ slot_of, const int32_t* __restrict__ top,
    const float* __restrict__ rw, uint16_t* __restrict__ dyw, float* __restrict__ dprobs,
    uint8_t* __restrict__ dyq, uint8_t* __restrict__ dys) {
  __shared__ float red[kMaxTopk][kRowThreads];
  const int t = blockIdx.x;
  int s[kMaxTopk];
  load_slots(slot_of, t, K, s);
  float w[kMaxTopk], part[kMaxTopk];
#pragma unroll
  for (int k = 0; k < kMaxTopk; ++k) {
    w[k] = (s[k] >= 0) ? rw[(int64_t)t * K + k] : 0.0f;
    part[k] = 0.0f;
  }
  const uint4* src = reinterpret_cast<const uint4*>(dy + (int64_t)t * H);
  for (int c = threadIdx.x; c < H / 32; c += kRowThreads) {
    float g[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) unpack_bf16x8(src[4 * c + q], g + 8 * q);
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) {
      if (s[k] < 0) continue;
      const uint4* yr = reinterpret_cast<const uint4*>(y + (int64_t)s[k] * H) + 4 * c;
      float d = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float yv[8];
        unpack_bf16x8(yr[q], yv);
#pragma unroll
        for (int i = 0; i < 8; ++i) d += g[8 * q + i] * yv[i];
      }
      part[k] += d;
      float wg[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) wg[i] = w[k] * g[i];
      uint4* dst = reinterpret_cast<uint4*>(dyw + (int64_t)s[k] * H) + 4 * c;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dst[q] = make_uint4(pack_bf2(wg[8 * q], wg[8 * q + 1]), pack_bf2(wg[8 * q + 2], wg[8 * q + 3]),
                            pack_bf2(wg[8 * q + 4], wg[8 * q + 5]), pack_bf2(wg[8 * q + 6], wg[8 * q + 7]));
      if constexpr (Q) {
        uint4 q0, q1;
        const uint32_t sc = mx_quantize32(wg, q0, q1);
        uint4* dq = reinterpret_cast<uint4*>(dyq + (int64_t)s[k] * H) + 2 * c;
        dq[0] = q0;
        dq[1] = q1;
        dys[(int64_t)s[k] * (H / 32) + c] = (uint8_t)sc;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxTopk; ++k) red[k][threadIdx.x] = part[k];
  __syncthreads();
  for (int d = kRowThreads / 2; d > 0; d >>= 1) {
    if (threadIdx.x < d) {
#pragma unroll
      for (int k = 0; k < kMaxTopk; ++k) red[k][threadIdx.x] += red[k][threadIdx.x + d];
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < E; e += kRowThreads) {
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k)
      if (k < K && s[k] >= 0 && top[(int64_t)t * K + k] == e) v = red[k][0];
    dprobs[(int64_t)t * E + e] = v;
  }
}

// dx[t] = dxp[shared_row0 + t] + sum_k dxp[slot_of[t,k]] (float, fixed order, one rounding).
__global__ __launch_bounds__(kRowThreads) void k_dx_combine(
    const uint16_t* __restrict__ dxp, int64_t shared_row0, int H, int K,
    const int32_t* __restrict__ slot_of, uint16_t* __restrict__ dx) {
  const int t = blockIdx.x;
  int s[kMaxTopk];
  load_slots(slot_of, t, K, s);
  const uint4* src = reinterpret_cast<const uint4*>(dxp + (shared_row0 + t) * (int64_t)H);
  for (int c = threadIdx.x; c < H / 8; c += kRowThreads) {
    const uint4 v = src[c];
    float a[8] = {lo_bf(v.x), hi_bf(v.x), lo_bf(v.y), hi_bf(v.y),
                  lo_bf(v.z), hi_bf(v.z), lo_bf(v.w), hi_bf(v.w)};
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) {
      if (s[k] < 0) continue;
      const uint4 r = reinterpret_cast<const uint4*>(dxp + (int64_t)s[k] * H)[c];
      a[0] += lo_bf(r.x); a[1] += hi_bf(r.x); a[2] += lo_bf(r.y); a[3] += hi_bf(r.y);
      a[4] += lo_bf(r.z); a[5] += hi_bf(r.z); a[6] += lo_bf(r.w); a[7] += hi_bf(r.w);
    }
    uint4 o;
    o.x = pack_bf2(a[0], a[1]); o.y = pack_bf2(a[2], a[3]);
    o.z = pack_bf2(a[4], a[5]); o.w = pack_bf2(a[6], a[7]);
    reinterpret_cast<uint4*>(dx + (int64_t)t * H)[c] = o;
  }
}

}  // namespace moe
