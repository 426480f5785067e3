// Per-token row kernels: MXFP8 quantisation of rows, probability-weighted combine, the
// backward's weighted gather of dy fused with the router-probability gradient,
// and the data-gradient combine.  All are HBM-bound row copies/reductions: each
// thread moves 16-byte pieces (8 bf16) of a row, and the loads of two pieces are in
// flight together.  Every sum runs in a fixed order (no float atomics).  With MXFP8
// output, the 4 lanes holding one 32-element block agree on its E8M0 exponent through
// two cross-lane max steps (a row's piece c sits on lane c % 64 of its wave, and
// H is a multiple of 32, so a block's 4 pieces are 4 consecutive lanes).
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kRowThreads = 256;

__device__ __forceinline__ void load_slots(const int32_t* __restrict__ slot_of, int t, int K,
                                           int (&s)[kMaxTopk]) {
#pragma unroll
  for (int k = 0; k < kMaxTopk; ++k) s[k] = (k < K) ? slot_of[(int64_t)t * K + k] : -1;
}

// A 16-byte load marked non-temporal, for expert-output rows that the combines read
// exactly once.  Keeping them out of the way of the caches' replacement order took the
// two combines at 8192 tokens x H 7168 from 0.18 to 0.16 ms, and at 4096 x 4096 from
// 0.0365 to 0.035 ms (the other operands keep ordinary loads).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_once(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint4 pack_bf8(const float (&a)[8]) {
  uint4 o;
  o.x = pack_bf2(a[0], a[1]); o.y = pack_bf2(a[2], a[3]);
  o.z = pack_bf2(a[4], a[5]); o.w = pack_bf2(a[6], a[7]);
  return o;
}

// MXFP8 quantisation of bf16 rows along their length (the hidden states, the routed FC1
// input): payload [rows][cols] E4M3 and scales [rows][cols/32] E8M0.  One thread per
// 16-byte piece.  (h and dfc1 are quantised in the epilogues of the GEMMs that produce them.)
__global__ __launch_bounds__(kRowThreads) void k_quantize_rows(
    const uint16_t* __restrict__ in, int64_t rows, int cols, uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  const int64_t nc = (int64_t)cols / 8;
  const int64_t total = rows * nc;
  // the stride is a multiple of 4 pieces, so a block's 4 pieces stay on 4 adjacent lanes
  for (int64_t b = (int64_t)blockIdx.x * kRowThreads + threadIdx.x; b < total;
       b += (int64_t)gridDim.x * kRowThreads) {
    float f[8];
    unpack_bf16x8(reinterpret_cast<const uint4*>(in)[b], f);
    uint2 code;
    const uint32_t s = mx_quantize8(f, quad_max(absmax8(f)), code);
    reinterpret_cast<uint2*>(q)[b] = code;
    if ((b & 3) == 0) sc[b >> 2] = (uint8_t)s;
  }
}

// x[t] . g for the token's block (fixed order: pieces per thread, a wave butterfly, then
// the waves in order); every thread gets the result.
__device__ __forceinline__ float row_dot(const uint16_t* __restrict__ xr, const uint16_t* __restrict__ g, int H,
                                        float* red /* LDS [kRowThreads / 64] */) {
  const int nc = H / 8;
  float v = 0.0f;
  for (int c = threadIdx.x; c < nc; c += kRowThreads) {
    float a[8], b[8];
    unpack_bf16x8(reinterpret_cast<const uint4*>(xr)[c], a);
    unpack_bf16x8(reinterpret_cast<const uint4*>(g)[c], b);
#pragma unroll
    for (int i = 0; i < 8; ++i) v += a[i] * b[i];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float z = 0.0f;
#pragma unroll
  for (int q = 0; q < kRowThreads / 64; ++q) z += red[q];
  return z;
}

// Shared output gate score sigmoid(z) (one scalar per token).
__device__ __forceinline__ float gate_sigmoid(float z) { return 1.0f / (1.0f + expf(-z)); }

// out[t] = y[shared_row0 + t] + sum_k w_tk * y[slot_of[t,k]], in float, fixed k order,
// one rounding to bf16.  shared_row0 < 0: no shared row (the sum starts from zero).
// With the shared output gate (gw non-null) the shared row is scaled by
// sigmoid(x[t] . gw), which is also stored to gate_s[t] for the backward.
__global__ __launch_bounds__(kRowThreads) void k_combine(
    const uint16_t* __restrict__ y, int64_t shared_row0, int H, int K,
    const int32_t* __restrict__ slot_of, const float* __restrict__ rw, uint16_t* __restrict__ out,
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gw, float* __restrict__ gate_s) {
  __shared__ float red[kRowThreads / 64];
  const int t = blockIdx.x;
  float gscale = 1.0f;
  if (gw) {
    gscale = gate_sigmoid(row_dot(x + (int64_t)t * H, gw, H, red));
    if (threadIdx.x == 0) gate_s[t] = gscale;
  }
  int s[kMaxTopk];
  load_slots(slot_of, t, K, s);
  float w[kMaxTopk];
#pragma unroll
  for (int k = 0; k < kMaxTopk; ++k) w[k] = (s[k] >= 0) ? rw[(int64_t)t * K + k] : 0.0f;
  const uint4* ys = shared_row0 >= 0 ? reinterpret_cast<const uint4*>(y + (shared_row0 + t) * (int64_t)H) : nullptr;
  const int nc = H / 8;
  for (int c0 = threadIdx.x; c0 < nc; c0 += 2 * kRowThreads) {
    uint4 v[2], r[2][kMaxTopk];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = c0 + u * kRowThreads;
      if (c >= nc) break;
      v[u] = ys ? ys[c] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int k = 0; k < kMaxTopk; ++k)
        if (s[k] >= 0) r[u][k] = ld_once(reinterpret_cast<const uint4*>(y + (int64_t)s[k] * H) + c);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = c0 + u * kRowThreads;
      if (c >= nc) break;
      float a[8];
      unpack_bf16x8(v[u], a);
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] *= gscale;
#pragma unroll
      for (int k = 0; k < kMaxTopk; ++k) {
        if (s[k] < 0) continue;
        float b[8];
        unpack_bf16x8(r[u][k], b);
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] += w[k] * b[i];
      }
      reinterpret_cast<uint4*>(out + (int64_t)t * H)[c] = pack_bf8(a);
    }
  }
}

// Backward gather: dyw[slot] = w_tk * dy[t] (the router weight folded into the
// routed expert's upstream gradient), and the router-probability gradient
// dprobs[t, e_tk] = dy[t] . y[slot] (y is the unweighted expert output), written
// into the dense [T][E] row with zeros off the map, or (dense = 0, routing given as the
// fixed-width table) into the [T][K] row of the table, 0 at -1 entries.  With the shared
// output gate (gate_s non-null): dys[t] = s_t dy[t] (the shared expert's upstream
// gradient) and dz[t] = s_t (1 - s_t) (dy[t] . y[shared_row0 + t]) (the gate logit's).
// The dot products are reduced per thread in a fixed order, then across each wave by a
// fixed butterfly, then across the waves in order.  With Q, the BF16 w_tk * dy[t] is also
// quantised to MXFP8 along H into dyq / dysc (the A operand of the scaled-FP8
// data-gradient GEMM), as every other FP8 GEMM input is quantised from its BF16 tensor.
// One block per token.
template <bool Q>
__global__ __launch_bounds__(kRowThreads) void k_gather_dy_dprob(
    const uint16_t* __restrict__ dy, const uint16_t* __restrict__ y, int H, int E, int K,
    const int32_t* __restrict__ slot_of, const int32_t* __restrict__ top,
    const float* __restrict__ rw, uint16_t* __restrict__ dyw, float* __restrict__ dprobs,
    uint8_t* __restrict__ dyq, uint8_t* __restrict__ dysc, int dense, int64_t shared_row0,
    const float* __restrict__ gate_s, float* __restrict__ dz, uint16_t* __restrict__ dys) {
  __shared__ float red[kRowThreads / 64][kMaxTopk + 1];
  __shared__ float dp[kMaxTopk + 1];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int s[kMaxTopk];
  load_slots(slot_of, t, K, s);
  float w[kMaxTopk], part[kMaxTopk];
#pragma unroll
  for (int k = 0; k < kMaxTopk; ++k) {
    w[k] = (s[k] >= 0) ? rw[(int64_t)t * K + k] : 0.0f;
    part[k] = 0.0f;
  }
  const bool gated = gate_s != nullptr;
  const float gs = gated ? gate_s[t] : 0.0f;
  const uint4* ysh = gated ? reinterpret_cast<const uint4*>(y + (shared_row0 + t) * (int64_t)H) : nullptr;
  float part_s = 0.0f;
  const uint4* src = reinterpret_cast<const uint4*>(dy + (int64_t)t * H);
  const int nc = H / 8;
  for (int c0 = threadIdx.x; c0 < nc; c0 += 2 * kRowThreads) {
    uint4 g4[2], y4[2][kMaxTopk];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = c0 + u * kRowThreads;
      if (c >= nc) break;
      g4[u] = src[c];
#pragma unroll
      for (int k = 0; k < kMaxTopk; ++k)
        if (s[k] >= 0) y4[u][k] = reinterpret_cast<const uint4*>(y + (int64_t)s[k] * H)[c];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = c0 + u * kRowThreads;
      if (c >= nc) break;
      float g[8];
      unpack_bf16x8(g4[u], g);
      if (gated) {
        float ys[8], sg[8];
        unpack_bf16x8(ysh[c], ys);
        float d = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          d += g[i] * ys[i];
          sg[i] = gs * g[i];
        }
        part_s += d;
        reinterpret_cast<uint4*>(dys + (int64_t)t * H)[c] = pack_bf8(sg);
      }
#pragma unroll
      for (int k = 0; k < kMaxTopk; ++k) {
        if (s[k] < 0) continue;
        float yv[8];
        unpack_bf16x8(y4[u][k], yv);
        float d = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) d += g[i] * yv[i];
        part[k] += d;
        float wg[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) wg[i] = w[k] * g[i];
        reinterpret_cast<uint4*>(dyw + (int64_t)s[k] * H)[c] = pack_bf8(wg);
        if constexpr (Q) {   // the MXFP8 codes of the BF16 values just stored
          float wb[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) wb[i] = bf2f(f2bf(wg[i]));
          uint2 q;
          const uint32_t sc = mx_quantize8(wb, quad_max(absmax8(wb)), q);
          reinterpret_cast<uint2*>(dyq + (int64_t)s[k] * H)[c] = q;
          if ((c & 3) == 0) dysc[(int64_t)s[k] * (H / 32) + (c >> 2)] = (uint8_t)sc;
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k <= kMaxTopk; ++k) {
    float v = k < kMaxTopk ? part[k] : part_s;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0) red[wv][k] = v;
  }
  __syncthreads();
  if (threadIdx.x <= kMaxTopk) {
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < kRowThreads / 64; ++q) v += red[q][threadIdx.x];
    dp[threadIdx.x] = v;
  }
  __syncthreads();
  if (gated && threadIdx.x == 0) dz[t] = gs * (1.0f - gs) * dp[kMaxTopk];
  if (!dense) {   // a route with no slot accumulated nothing: dp[k] = 0 there
    if (threadIdx.x < K) dprobs[(int64_t)t * K + threadIdx.x] = dp[threadIdx.x];
    return;
  }
  for (int e = threadIdx.x; e < E; e += kRowThreads) {
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k)
      if (k < K && s[k] >= 0 && top[(int64_t)t * K + k] == e) v = dp[k];
    dprobs[(int64_t)t * E + e] = v;
  }
}

// dx[t] = dxp[shared_row0 + t] + sum_k dxp[slot_of[t,k]] (float, fixed order, one rounding);
// shared_row0 < 0: no shared row.  With the shared output gate, + dz[t] gw (the gate
// logit's contribution).
__global__ __launch_bounds__(kRowThreads) void k_dx_combine(
    const uint16_t* __restrict__ dxp, int64_t shared_row0, int H, int K,
    const int32_t* __restrict__ slot_of, uint16_t* __restrict__ dx,
    const uint16_t* __restrict__ gw, const float* __restrict__ dz) {
  const int t = blockIdx.x;
  int s[kMaxTopk];
  load_slots(slot_of, t, K, s);
  const uint4* src =
      shared_row0 >= 0 ? reinterpret_cast<const uint4*>(dxp + (shared_row0 + t) * (int64_t)H) : nullptr;
  const float dzt = gw ? dz[t] : 0.0f;
  const int nc = H / 8;
  for (int c0 = threadIdx.x; c0 < nc; c0 += 2 * kRowThreads) {
    uint4 v[2], r[2][kMaxTopk];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = c0 + u * kRowThreads;
      if (c >= nc) break;
      v[u] = src ? src[c] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int k = 0; k < kMaxTopk; ++k)
        if (s[k] >= 0) r[u][k] = ld_once(reinterpret_cast<const uint4*>(dxp + (int64_t)s[k] * H) + c);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = c0 + u * kRowThreads;
      if (c >= nc) break;
      float a[8];
      unpack_bf16x8(v[u], a);
#pragma unroll
      for (int k = 0; k < kMaxTopk; ++k) {
        if (s[k] < 0) continue;
        float b[8];
        unpack_bf16x8(r[u][k], b);
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] += b[i];
      }
      if (gw) {
        float gv[8];
        unpack_bf16x8(reinterpret_cast<const uint4*>(gw)[c], gv);
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] += dzt * gv[i];
      }
      reinterpret_cast<uint4*>(dx + (int64_t)t * H)[c] = pack_bf8(a);
    }
  }
}

// Gradient of the shared output gate's weight: main_grad_g += sum_t dz[t] x[t], in two
// fixed-order passes.  Pass 1: block (column group b of 512, token chunk q) sums its
// columns over the chunk's tokens: lane l owns columns 512 b + 8 l .. + 7 (one 16-byte
// piece per row), wave v takes tokens q*TC + v, + 4, ... four at a time (their loads in
// flight together, added in token order), and the 4 waves are added in order.
constexpr int kGateChunks = 64;
__global__ __launch_bounds__(256) void k_gate_wgrad_partial(
    const uint16_t* __restrict__ x, const float* __restrict__ dz, int T, int H, float* __restrict__ part) {
  __shared__ float red[4][64][9];   // [wave][lane][8 columns] (+1 pad)
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c8 = blockIdx.x * 64 + lane;              // 16-byte piece of the row
  const bool in = 8 * c8 < H;
  const int tc = (T + kGateChunks - 1) / kGateChunks;
  const int t0 = blockIdx.y * tc, t1 = min(T, t0 + tc);
  float acc[8] = {};
  if (in) {
    int t = t0 + wv;
    for (; t + 12 < t1; t += 16) {
      uint4 v[4];
      float z[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[u] = reinterpret_cast<const uint4*>(x + (int64_t)(t + 4 * u) * H)[c8];
        z[u] = dz[t + 4 * u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float a[8];
        unpack_bf16x8(v[u], a);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += z[u] * a[i];
      }
    }
    for (; t < t1; t += 4) {
      float a[8];
      unpack_bf16x8(reinterpret_cast<const uint4*>(x + (int64_t)t * H)[c8], a);
      const float z = dz[t];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += z * a[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[wv][lane][i] = acc[i];
  __syncthreads();
  if (wv == 0 && in) {
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = ((red[0][lane][i] + red[1][lane][i]) + red[2][lane][i]) + red[3][lane][i];
    float* dst = part + (int64_t)blockIdx.y * H + 8 * c8;
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = o[i];
  }
}

// Pass 2: chunks added in order, then the main_grad update (FP32, or BF16 with the
// contribution rounded to BF16 first, as for the other weights).
__global__ __launch_bounds__(256) void k_gate_wgrad_final(const float* __restrict__ part, int H,
                                                           uint8_t* __restrict__ mg, int bf16_mg) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= H) return;
  float v = 0.0f;
  for (int q = 0; q < kGateChunks; ++q) v += part[(int64_t)q * H + col];
  if (bf16_mg) {
    uint16_t* m = reinterpret_cast<uint16_t*>(mg);
    m[col] = f2bf(bf2f(m[col]) + bf2f(f2bf(v)));
  } else {
    float* m = reinterpret_cast<float*>(mg);
    m[col] = m[col] + v;
  }
}

}  // namespace moe
