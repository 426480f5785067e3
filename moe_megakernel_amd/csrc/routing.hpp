// Routing-map compaction, per-expert histogram + scan, and stable ranking
// into expert-contiguous slots.
//
// Compaction (Megatron-LM PR #6572, Design > Authoritative routing maps): each
// row of the dense [T][E] routing map becomes K expert IDs in ascending order,
// -1 for a missing route, with the router probability gathered at each listed
// route (0 at -1).  Dispatch on one GPU is a permutation: routes are grouped by
// expert, and inside an expert's segment ordered by ascending token, which makes
// the permutation unique.
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kRouteChunk = 256;   // tokens per block (4 waves of 64)

// Kernel 1: one thread per token.  Writes the fixed-width table and the
// per-chunk expert histogram (integer LDS atomics: the counts do not depend
// on the order of the additions).
__global__ __launch_bounds__(256) void k_route_compact(
    const uint8_t* __restrict__ rmap, const float* __restrict__ probs, int T, int E, int K,
    int32_t* __restrict__ top, float* __restrict__ rw, int32_t* __restrict__ chunk_counts,
    int32_t* __restrict__ chunk_status) {
  __shared__ int cnt[kMaxExperts + 1];
  __shared__ int overflow;
  if (threadIdx.x == 0) overflow = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int t = blockIdx.x * kRouteChunk + threadIdx.x;
  if (t < T) {
    const uint8_t* row = rmap + (int64_t)t * E;
    const float* prow = probs + (int64_t)t * E;
    int n = 0;
    auto take = [&](int e) {
      if (n < K) {
        top[(int64_t)t * K + n] = e;
        rw[(int64_t)t * K + n] = prow[e];     // probs are read only where the map is set
        atomicAdd(&cnt[e], 1);
      }
      ++n;
    };
    if ((E & 15) == 0 && ((reinterpret_cast<uintptr_t>(row) & 15) == 0)) {
      // the whole row (E <= 256 bytes) is loaded with independent 16-byte loads first
      uint4 r16[16];
      const uint4* src = reinterpret_cast<const uint4*>(row);
#pragma unroll
      for (int q = 0; q < 16; ++q) r16[q] = (q < (E >> 4)) ? src[q] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const uint32_t w4[4] = {r16[q].x, r16[q].y, r16[q].z, r16[q].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t v = w4[d];
          if (!v) continue;
#pragma unroll
          for (int b = 0; b < 4; ++b)
            if ((v >> (8 * b)) & 0xffu) take(16 * q + 4 * d + b);
        }
      }
    } else {
      for (int e = 0; e < E; ++e)
        if (row[e]) take(e);
    }
    for (int k = n; k < K; ++k) {
      top[(int64_t)t * K + k] = -1;
      rw[(int64_t)t * K + k] = 0.0f;
    }
    if (n > K) overflow = 1;     // benign race: every writer stores the same value
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
  if (threadIdx.x == 0) chunk_status[blockIdx.x] = overflow ? 7 /* MOE_ERR_ROUTE_OVERFLOW */ : 0;
}

// Kernel 2: one block of 256 threads.  Per expert: running sum over chunks
// (chunk base offsets) -> counts; exclusive scan over experts -> offsets;
// and the prefix over groups of ceil(rows / BM) used by the token-dim GEMMs
// (group E is the shared expert with T rows when present).  Also folds the
// per-chunk overflow flags into the status word.
__global__ __launch_bounds__(256) void k_route_scan(
    const int32_t* __restrict__ chunk_counts, int nchunks, int E, int T, int has_shared, int BM,
    int32_t* __restrict__ chunk_base, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ tile_prefix, const int32_t* __restrict__ chunk_status,
    int32_t* __restrict__ status) {
  __shared__ int s[256];
  __shared__ int u[256];
  __shared__ int flag;
  const int e = threadIdx.x;
  if (e == 0) flag = 0;
  __syncthreads();
  for (int c = e; c < nchunks; c += 256)
    if (chunk_status[c]) flag = chunk_status[c];
  int total = 0;
  if (e < E) {
    for (int c = 0; c < nchunks; ++c) {
      const int v = chunk_counts[(int64_t)c * E + e];
      chunk_base[(int64_t)c * E + e] = total;
      total += v;
    }
    counts[e] = total;
  }
  const int groups = E + (has_shared ? 1 : 0);
  int rows = (e < E) ? total : ((e == E && has_shared) ? T : 0);
  s[e] = (e < E) ? total : 0;
  u[e] = (e < groups) ? (rows + BM - 1) / BM : 0;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {      // inclusive Hillis-Steele scans
    const int a = (e >= d) ? s[e - d] : 0;
    const int b = (e >= d) ? u[e - d] : 0;
    __syncthreads();
    s[e] += a;
    u[e] += b;
    __syncthreads();
  }
  if (e == 0) { offsets[0] = 0; tile_prefix[0] = 0; *status = flag; }
  if (e < E) offsets[e + 1] = s[e];
  if (e < groups) tile_prefix[e + 1] = u[e];
}

// Kernel 3: one thread per token.  Rank of each route inside its expert's
// segment = routes of earlier chunks (chunk_base) + earlier waves of this
// chunk + earlier lanes of this wave (ballot prefix), all by ascending token.
__global__ __launch_bounds__(256) void k_route_rank(
    const int32_t* __restrict__ top, const float* __restrict__ rw, int T, int E, int K,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot_of, int32_t* __restrict__ slot_token, float* __restrict__ slot_w) {
  __shared__ int wcnt[4][kMaxExperts + 1];
  const int t = blockIdx.x * kRouteChunk + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int my[kMaxTopk];
  int pre[kMaxTopk];
#pragma unroll
  for (int k = 0; k < kMaxTopk; ++k) {
    my[k] = (t < T && k < K) ? top[(int64_t)t * K + k] : -1;
    pre[k] = 0;
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int e = 0; e < E; ++e) {
    bool pred = false;
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k) pred |= (my[k] == e);
    const uint64_t mask = __ballot(pred);
    const int p = __popcll(mask & lt);
#pragma unroll
    for (int k = 0; k < kMaxTopk; ++k)
      if (my[k] == e) pre[k] = p;
    if (lane == 0) wcnt[w][e] = __popcll(mask);
  }
  __syncthreads();
  if (t >= T) return;
#pragma unroll
  for (int k = 0; k < kMaxTopk; ++k) {
    if (k >= K) break;
    const int e = my[k];
    if (e < 0) {
      slot_of[(int64_t)t * K + k] = -1;
      continue;
    }
    int r = chunk_base[(int64_t)blockIdx.x * E + e] + pre[k];
    for (int v = 0; v < w; ++v) r += wcnt[v][e];
    const int s = offsets[e] + r;
    slot_of[(int64_t)t * K + k] = s;
    slot_token[s] = t * K + k;
    slot_w[s] = rw[(int64_t)t * K + k];
  }
}

}  // namespace moe
