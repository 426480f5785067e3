// Routing-map compaction, per-expert histogram + scan, and stable ranking
// into expert-contiguous slots.
//
// Compaction (Megatron-LM PR #6572, Design > Authoritative routing maps): each
// row of the dense [T][E] routing map becomes K expert IDs in ascending order,
// -1 for a missing route, with the router probability gathered at each listed
// route (0 at -1).  Dispatch on one GPU is a permutation: routes are grouped by
// expert, and inside an expert's segment ordered by ascending token, which makes
// the permutation unique.
//
// Work is split into chunks of kRouteChunk tokens: compaction writes each chunk's
// expert histogram, one scan turns the histograms into per-chunk bases and the
// expert offsets, and ranking places each route at offsets[e] + chunk base + its
// rank among the chunk's earlier routes to e.
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kRouteChunk = 32;       // tokens per chunk (one compaction block)
constexpr int kRouteTokPerWave = 8;   // compaction: tokens per wave (4 waves per block)

// Kernel 1: one wave per 8 tokens, a token's row read by the whole wave (lane l looks
// at experts 4l .. 4l + 3).  Positions in the ascending ID list come from per-byte
// ballots; the chunk histogram is built with integer LDS atomics (the counts do not
// depend on the order of the additions).
__global__ __launch_bounds__(256) void k_route_compact(
    const uint8_t* __restrict__ rmap, const float* __restrict__ probs, int T, int E, int K,
    int32_t* __restrict__ top, float* __restrict__ rw, int32_t* __restrict__ chunk_counts,
    int32_t* __restrict__ chunk_status) {
  __shared__ int cnt[kMaxExperts + 1];
  __shared__ int overflow;
  if (threadIdx.x == 0) overflow = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t0 = blockIdx.x * kRouteChunk + w * kRouteTokPerWave;
  const int e0 = 4 * lane;
  const bool word = (E & 3) == 0;   // rows are then 4-byte aligned
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // all map words of the wave's tokens first (independent loads)
  uint32_t m[kRouteTokPerWave];
#pragma unroll
  for (int i = 0; i < kRouteTokPerWave; ++i) {
    const int t = t0 + i;
    uint32_t bits = 0;
    if (t < T && e0 < E) {
      const uint8_t* row = rmap + (int64_t)t * E + e0;
      if (word) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(row);
#pragma unroll
        for (int j = 0; j < 4; ++j) bits |= ((v >> (8 * j)) & 0xffu) ? (1u << j) : 0u;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (e0 + j < E && row[j]) bits |= 1u << j;
      }
    }
    m[i] = bits;
  }
  // positions, then the probability loads of every listed route, then the stores
  int pos[kRouteTokPerWave], n[kRouteTokPerWave];
  float pr[kRouteTokPerWave][4];
#pragma unroll
  for (int i = 0; i < kRouteTokPerWave; ++i) {
    int before = 0, total = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint64_t b = __ballot((m[i] >> j) & 1u);
      before += __popcll(b & lt);
      total += __popcll(b);
    }
    pos[i] = before;
    n[i] = total;
    const int t = t0 + i;
    int p = before;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pr[i][j] = 0.0f;
      if ((m[i] >> j) & 1u) {
        if (p < K) pr[i][j] = probs[(int64_t)t * E + e0 + j];   // read only where the map is set
        ++p;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kRouteTokPerWave; ++i) {
    const int t = t0 + i;
    if (t >= T) break;
    int p = pos[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if ((m[i] >> j) & 1u) {
        if (p < K) {
          top[(int64_t)t * K + p] = e0 + j;
          rw[(int64_t)t * K + p] = pr[i][j];
          atomicAdd(&cnt[e0 + j], 1);
        }
        ++p;
      }
    }
    if (lane >= n[i] && lane < K) {
      top[(int64_t)t * K + lane] = -1;
      rw[(int64_t)t * K + lane] = 0.0f;
    }
    if (lane == 0 && n[i] > K) overflow = 1;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) chunk_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
  if (threadIdx.x == 0) chunk_status[blockIdx.x] = overflow ? 7 /* MOE_ERR_ROUTE_OVERFLOW */ : 0;
}

// Kernel 1 for a router that already produced the fixed-width table (the form the
// runtime consumes: Megatron Core API docs, mok.runtime, _MoKAutograd.forward takes
// router_weights and top_experts): validation and the chunk histogram in one pass.
// Thread (i, k) for the chunk's token i and route k.  An ID outside [-1, E) or an ID a
// row lists twice marks the chunk invalid and is stored as -1 (weight 0), so every later
// kernel sees an in-range table; the status word reports the error.
__global__ __launch_bounds__(kRouteChunk * kMaxTopk) void k_route_table(
    const int32_t* __restrict__ top_in, const float* __restrict__ rw_in, int T, int E, int K,
    int32_t* __restrict__ top, float* __restrict__ rw, int32_t* __restrict__ chunk_counts,
    int32_t* __restrict__ chunk_status) {
  __shared__ int cnt[kMaxExperts + 1];
  __shared__ int tab[kRouteChunk * kMaxTopk];
  __shared__ int bad;
  const int tid = threadIdx.x;
  if (tid == 0) bad = 0;
  for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
  const int64_t base = (int64_t)blockIdx.x * kRouteChunk * K;
  const int n = min(kRouteChunk, T - (int)blockIdx.x * kRouteChunk) * K;
  const int e = tid < n ? top_in[base + tid] : -1;
  tab[tid] = e;
  __syncthreads();
  if (tid < n) {
    const int k = tid % K;
    bool ok = e >= 0 && e < E;
    bool err = e < -1 || e >= E;
    for (int q = tid - k; q < tid; ++q)   // earlier routes of the same token
      if (ok && tab[q] == e) { ok = false; err = true; }
    top[base + tid] = ok ? e : -1;
    rw[base + tid] = ok ? rw_in[base + tid] : 0.0f;
    if (ok) atomicAdd(&cnt[e], 1);
    if (err) bad = 1;
  }
  __syncthreads();
  for (int x = tid; x < E; x += blockDim.x) chunk_counts[(int64_t)blockIdx.x * E + x] = cnt[x];
  if (tid == 0) chunk_status[blockIdx.x] = bad ? 9 /* MOE_ERR_ROUTE_INVALID */ : 0;
}

// Kernel 2: one block of 1024 threads.  Thread (s, e) owns expert e's chunks of segment
// s (segments of ceil(nchunks / S) consecutive chunks, S = 1024 / 256 = 4 or more): it
// sums them, the segment sums are scanned in LDS, and a second pass over the segment
// writes each chunk's base (routes to e in earlier chunks).  Then counts, the exclusive
// scan over experts (offsets), and the prefix over groups of ceil(rows / BM) used by the
// token-dimension GEMMs (group E is the shared expert with T rows when present).  Also
// folds the per-chunk overflow flags into the status word.
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void k_route_scan(
    const int32_t* __restrict__ chunk_counts, int nchunks, int E, int T, int has_shared, int BM,
    int32_t* __restrict__ chunk_base, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ tile_prefix, const int32_t* __restrict__ chunk_status,
    int32_t* __restrict__ status) {
  __shared__ int seg[kScanThreads];
  __shared__ int s_tot[256];
  __shared__ int s_til[256];
  __shared__ int flag;
  const int tid = threadIdx.x;
  int ep = 1;
  while (ep < E) ep <<= 1;                       // experts padded to a power of two (<= 256)
  const int S = kScanThreads / ep;               // segments per expert
  const int e = tid % ep, s = tid / ep;
  const int L = (nchunks + S - 1) / S;
  const int c0 = s * L, c1 = min(c0 + L, nchunks);
  if (tid == 0) flag = 0;
  __syncthreads();
  for (int c = tid; c < nchunks; c += kScanThreads)
    if (chunk_status[c]) flag = chunk_status[c];
  int sum = 0;
  if (e < E) {
#pragma unroll 8
    for (int c = c0; c < c1; ++c) sum += chunk_counts[(int64_t)c * E + e];
  }
  seg[tid] = sum;
  __syncthreads();
  int run = 0;
  for (int q = 0; q < s; ++q) run += seg[q * ep + e];
  if (e < E) {
    for (int c = c0; c < c1; ++c) {
      const int v = chunk_counts[(int64_t)c * E + e];
      chunk_base[(int64_t)c * E + e] = run;
      run += v;
    }
    if (s == S - 1) counts[e] = run;
  }
  // totals per expert -> offsets and tile prefix (first 256 threads)
  if (s == S - 1 && e < E) s_tot[e] = run;
  __syncthreads();
  if (tid < 256) {
    const int groups = E + (has_shared ? 1 : 0);
    const int total = tid < E ? s_tot[tid] : 0;
    const int rows = tid < E ? total : ((tid == E && has_shared) ? T : 0);
    s_tot[tid] = total;
    s_til[tid] = tid < groups ? (rows + BM - 1) / BM : 0;
  }
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {      // inclusive Hillis-Steele scans
    int a = 0, b = 0;
    if (tid < 256 && tid >= d) { a = s_tot[tid - d]; b = s_til[tid - d]; }
    __syncthreads();
    if (tid < 256) { s_tot[tid] += a; s_til[tid] += b; }
    __syncthreads();
  }
  if (tid == 0) { offsets[0] = 0; tile_prefix[0] = 0; *status = flag; }
  const int groups = E + (has_shared ? 1 : 0);
  if (tid < E) offsets[tid + 1] = s_tot[tid];
  if (tid < groups) tile_prefix[tid + 1] = s_til[tid];
}

// Kernel 3: one block per chunk, thread (i, k) for the chunk's token i and route k.  Its
// rank inside expert e's segment = chunk base + the routes to e of the chunk's earlier
// tokens (a token lists an expert at most once), counted against the chunk's table in LDS.
__global__ __launch_bounds__(kRouteChunk * kMaxTopk) void k_route_rank(
    const int32_t* __restrict__ top, const float* __restrict__ rw, int T, int E, int K,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot_of, int32_t* __restrict__ slot_token, int32_t* __restrict__ slot_t,
    float* __restrict__ slot_w) {
  __shared__ int tab[kRouteChunk * kMaxTopk];
  const int tid = threadIdx.x;
  const int tb = blockIdx.x * kRouteChunk;
  const int n = min(kRouteChunk, T - tb) * K;   // routes of this chunk
  const int e = tid < n ? top[(int64_t)tb * K + tid] : -1;
  tab[tid] = e;
  __syncthreads();
  if (tid >= n) return;
  const int i = tid / K;
  if (e < 0) {
    slot_of[(int64_t)tb * K + tid] = -1;
    return;
  }
  int r = chunk_base[(int64_t)blockIdx.x * E + e];
  for (int q = 0; q < i * K; ++q) r += (tab[q] == e) ? 1 : 0;
  const int s = offsets[e] + r;
  slot_of[(int64_t)tb * K + tid] = s;
  slot_token[s] = tb * K + tid;
  slot_t[s] = tb + i;   // the token alone: the x row the GEMMs read for this slot
  slot_w[s] = rw[(int64_t)tb * K + tid];
}

}  // namespace moe
