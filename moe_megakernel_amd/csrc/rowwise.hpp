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
__global__ __launch_bounds__(kRowThreads) void k_gather_rows(
    const uint16_t* __restrict__ x, int H, int K, const int32_t* __restrict__ slot_of,
    uint16_t* __restrict__ xp) {
  const int t = blockIdx.x;
  int s[kMaxTopk];
  load_slots(slot_of, t, K, s);
  const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)t * H);
  for (int c = threadIdx.x; c < H / 8; c += kRowThreads) {
    const uint4 v = src[c];
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k)
      if (s[k] >= 0) reinterpret_cast<uint4*>(xp + (int64_t)s[k] * H)[c] = v;
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
// reduced per thread in a fixed order and then by a fixed LDS tree.
__global__ __launch_bounds__(kRowThreads) void k_gather_dy_dprob(
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ y, int H, int E, int K,
    const int32_t* __restrict__ slot_of, const int32_t* __restrict__ top,
    const float* __restrict__ rw, uint16_t* __restrict__ dyw, float* __restrict__ dprobs) {
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
  for (int c = threadIdx.x; c < H / 8; c += kRowThreads) {
    const uint4 v = src[c];
    const float g[8] = {lo_bf(v.x), hi_bf(v.x), lo_bf(v.y), hi_bf(v.y),
                        lo_bf(v.z), hi_bf(v.z), lo_bf(v.w), hi_bf(v.w)};
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) {
      if (s[k] < 0) continue;
      const uint4 r = reinterpret_cast<const uint4*>(y + (int64_t)s[k] * H)[c];
      const float yv[8] = {lo_bf(r.x), hi_bf(r.x), lo_bf(r.y), hi_bf(r.y),
                           lo_bf(r.z), hi_bf(r.z), lo_bf(r.w), hi_bf(r.w)};
      float d = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) d += g[q] * yv[q];
      part[k] += d;
      uint4 o;
      o.x = pack_bf2(w[k] * g[0], w[k] * g[1]); o.y = pack_bf2(w[k] * g[2], w[k] * g[3]);
      o.z = pack_bf2(w[k] * g[4], w[k] * g[5]); o.w = pack_bf2(w[k] * g[6], w[k] * g[7]);
      reinterpret_cast<uint4*>(dyw + (int64_t)s[k] * H)[c] = o;
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
