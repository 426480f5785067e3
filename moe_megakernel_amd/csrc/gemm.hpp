// Grouped BF16 GEMMs on gfx950 MFMA (v_mfma_f32_32x32x16_bf16) for the MoE
// layer: one launch covers every routed expert's row group plus the shared
// expert's group.
//
// Tile: 128 x 128 output, K step 64, 256 threads = 4 waves in a 2 x 2 grid,
// each wave a 64 x 64 sub-tile of 2 x 2 MFMA blocks (32 x 32, fp32 accumulate).
// Operands are staged through LDS, double buffered, always stored K-contiguous
// ([row][k], 144-byte padded rows) so every MFMA fragment is one 16-byte LDS
// read.  Waves 0-1 load the A tile, waves 2-3 the B tile, each thread 8 x 16 B
// per stage.  An operand whose source is K-contiguous is copied as 16-byte row
// chunks; one whose source is contiguous along M/N (weights in the data-gradient
// GEMMs, activations in the weight-gradient GEMMs) is loaded as 8 x 8 element
// blocks and transposed in registers on its way into LDS.
#pragma once
#include "common.hpp"

namespace moe {
namespace gemm {

constexpr int BM = 128, BN = 128, BK = 64, NT = 256;
constexpr int LDS_LD = BK + 8;                 // bf16 per LDS row: 144 B keeps 16-B reads conflict free
constexpr int TILE = 128 * LDS_LD;             // elements per operand tile
constexpr int LDS_ELEMS = 2 * 2 * TILE;        // [stage][A|B]

__device__ __forceinline__ uint32_t half16(const uint4& v, int i) {
  const uint32_t w = (i >> 1) == 0 ? v.x : (i >> 1) == 1 ? v.y : (i >> 1) == 2 ? v.z : v.w;
  return (i & 1) ? (w >> 16) : (w & 0xffffu);
}

// K-contiguous source: thread th (0..127) owns rows th/8 + 16 i, 16-byte chunk th%8.
__device__ __forceinline__ void load_kc(const uint16_t* const (&rp)[8], int k0, int kdim, int th, uint4 (&v)[8]) {
  const int kk = k0 + (th & 7) * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = (rp[i] != nullptr && kk < kdim) ? *reinterpret_cast<const uint4*>(rp[i] + kk) : make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ void store_kc(uint16_t* dst, int th, const uint4 (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<uint4*>(dst + ((th >> 3) + 16 * i) * LDS_LD + (th & 7) * 8) = v[i];
}

// Row-contiguous source (element (r, k) at f(k)[r]): thread th owns the 8 x 8 block
// k = k0 + 8 (th%8) + 0..7, r = 8 (th/8) + 0..7.
template <class F>
__device__ __forceinline__ void load_rc(const F& f, int k0, int kdim, int th, uint4 (&v)[8]) {
  const int kb = k0 + (th & 7) * 8;
  const int r8 = (th >> 3) * 8;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const uint16_t* p = (kb + kk < kdim) ? f(kb + kk) : nullptr;
    v[kk] = p ? *reinterpret_cast<const uint4*>(p + r8) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void store_rc(uint16_t* dst, int th, const uint4 (&v)[8]) {
  const int kg = th & 7, rg = th >> 3;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint4 o;
    o.x = half16(v[0], i) | (half16(v[1], i) << 16);
    o.y = half16(v[2], i) | (half16(v[3], i) << 16);
    o.z = half16(v[4], i) | (half16(v[5], i) << 16);
    o.w = half16(v[6], i) | (half16(v[7], i) << 16);
    *reinterpret_cast<uint4*>(dst + (rg * 8 + i) * LDS_LD + kg * 8) = o;
  }
}

// acc[i][j] += A_tile (128 x kdim) * B_tile^T (128 x kdim) for this wave's 64 x 64 block.
// For a K-contiguous operand, fa / fb map a tile row to its row pointer (nullptr: zero row);
// for a row-contiguous operand they map k to the pointer of element (k, tile row 0).
template <bool A_KC, bool B_KC, class FA, class FB>
__device__ __forceinline__ void tile_mma(f32x16_t (&acc)[2][2], int kdim, const FA& fa, const FB& fb,
                                         uint16_t* smem, bool wave_active) {
  const int tid = threadIdx.x;
  const bool loadA = tid < 128;
  const int th = tid & 127;
  const int lane = tid & 63, wid = tid >> 6, wm = wid >> 1, wn = wid & 1;

  const uint16_t* rp[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    rp[i] = nullptr;
    const int r = (th >> 3) + 16 * i;
    if constexpr (A_KC) { if (loadA) rp[i] = fa(r); }
    if constexpr (B_KC) { if (!loadA) rp[i] = fb(r); }
  }
  uint4 v[8];
  auto gload = [&](int k0) {
    if (loadA) {
      if constexpr (A_KC) load_kc(rp, k0, kdim, th, v); else load_rc(fa, k0, kdim, th, v);
    } else {
      if constexpr (B_KC) load_kc(rp, k0, kdim, th, v); else load_rc(fb, k0, kdim, th, v);
    }
  };
  auto sstore = [&](int stage) {
    uint16_t* dst = smem + stage * 2 * TILE + (loadA ? 0 : TILE);
    if (loadA) {
      if constexpr (A_KC) store_kc(dst, th, v); else store_rc(dst, th, v);
    } else {
      if constexpr (B_KC) store_kc(dst, th, v); else store_rc(dst, th, v);
    }
  };
  auto compute = [&](int stage) {
    if (!wave_active) return;
    const uint16_t* As = smem + stage * 2 * TILE;
    const uint16_t* Bs = As + TILE;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * 64 + i * 32 + (lane & 31)) * LDS_LD + ks * 16 + (lane >> 5) * 8);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * 64 + j * 32 + (lane & 31)) * LDS_LD + ks * 16 + (lane >> 5) * 8);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  const int nk = (kdim + BK - 1) / BK;
  if (nk <= 0) return;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    compute(cur);
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }
}


// ---------------------------------------------------------------------------------
// MXFP8 tile: v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands.  Per 64-wide K step,
// lane (r, g) (r = lane % 32, g = lane / 32) holds the 16 codes K = 16g .. 16g+15 in its
// first four registers and K = 32+16g .. 32+16g+15 in the last four, and its scale
// register carries the E8M0 scale of row / column r for the 32-element K block g (a
// layout measured on the hardware: the scale of lane group g covers the first halves of
// both groups' K ranges, so each group takes a 16-code slice from each 32-block).  Same LDS data layout as the
// BF16 tile (144-byte rows; a stage holds K = 128 codes), plus a scale tile per operand
// stored [row][4 blocks].  A is always K-contiguous (quantised activations); B is either
// a rowwise weight ([N][K] codes, scales [N][K/32]) or a columnwise one ([K][N] codes,
// scales [K/32][N]) loaded as 8 x 16 byte blocks and transposed with byte permutes.
// ---------------------------------------------------------------------------------
constexpr int BK8 = 128;

__device__ __forceinline__ void tr4x4_bytes(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                            uint32_t& b0, uint32_t& b1, uint32_t& b2, uint32_t& b3) {
  const uint32_t t0 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);   // a00 a10 a01 a11
  const uint32_t t1 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);   // a02 a12 a03 a13
  const uint32_t t2 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);   // a20 a30 a21 a31
  const uint32_t t3 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);   // a22 a32 a23 a33
  b0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);                  // a00 a10 a20 a30
  b1 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  b2 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  b3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

// Thread th owns k = 8 (th%16) + 0..7 and n = 16 (th/16) + 0..15 of a [K][N] byte source.
__device__ __forceinline__ void store_rc8(uint8_t* dst, int th, const uint4 (&v)[8]) {
  const int kg = th & 15, ng = th >> 4;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t lo[4], hi[4];
    tr4x4_bytes(word_of(v[0], w), word_of(v[1], w), word_of(v[2], w), word_of(v[3], w), lo[0], lo[1], lo[2], lo[3]);
    tr4x4_bytes(word_of(v[4], w), word_of(v[5], w), word_of(v[6], w), word_of(v[7], w), hi[0], hi[1], hi[2], hi[3]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint2*>(dst + (ng * 16 + 4 * w + j) * (LDS_LD * 2) + kg * 8) = make_uint2(lo[j], hi[j]);
  }
}

// fa(r): A row r codes (nullptr: zero row); fas(r): its scale row.  B_KC: fb(r), fbs(r) the
// same for B rows.  !B_KC: fb(k) -> codes of element (k, n0); fbs(kb) -> scale (kb, n0).
template <bool B_KC, class FA, class FAS, class FB, class FBS>
__device__ __forceinline__ void tile_mma_fp8(f32x16_t (&acc)[2][2], int kdim, const FA& fa, const FAS& fas,
                                             const FB& fb, const FBS& fbs, uint16_t* smem, uint8_t* ssc,
                                             bool wave_active) {
  const int tid = threadIdx.x;
  const bool loadA = tid < 128;
  const int th = tid & 127;
  const int lane = tid & 63, wid = tid >> 6, wm = wid >> 1, wn = wid & 1;

  const uint8_t* rp[8];
  const uint8_t* sp_row = nullptr;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = (th >> 3) + 16 * i;
    rp[i] = loadA ? fa(r) : nullptr;
    if constexpr (B_KC) { if (!loadA) rp[i] = fb(r); }
  }
  if (loadA) sp_row = fas(th);
  if constexpr (B_KC) { if (!loadA) sp_row = fbs(th); }

  uint4 v[8];
  uint32_t sv = 0;
  auto gload = [&](int k0) {
    if (loadA || B_KC) {
      const int kk = k0 + (th & 7) * 16;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = rp[i] ? *reinterpret_cast<const uint4*>(rp[i] + kk) : make_uint4(0, 0, 0, 0);
      sv = sp_row ? *reinterpret_cast<const uint32_t*>(sp_row + k0 / 32) : 0u;
    } else {
      if constexpr (!B_KC) {
        const int kb = k0 + (th & 15) * 8;
        const int n16 = (th >> 4) * 16;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const uint8_t* p = (kb + kk < kdim) ? fb(kb + kk) : nullptr;
          v[kk] = p ? *reinterpret_cast<const uint4*>(p + n16) : make_uint4(0, 0, 0, 0);
        }
        const uint8_t* q = fbs(k0 / 32 + (th >> 5));
        sv = *reinterpret_cast<const uint32_t*>(q + (th & 31) * 4);
      }
    }
  };
  auto sstore = [&](int stage) {
    uint8_t* dst = reinterpret_cast<uint8_t*>(smem + stage * 2 * TILE + (loadA ? 0 : TILE));
    uint8_t* sdst = ssc + stage * 1024 + (loadA ? 0 : 512);
    if (loadA || B_KC) {
      store_kc(reinterpret_cast<uint16_t*>(dst), th, v);
      *reinterpret_cast<uint32_t*>(sdst + th * 4) = sv;
    } else {
      store_rc8(dst, th, v);
      const int kb = th >> 5, n4 = (th & 31) * 4;
#pragma unroll
      for (int j = 0; j < 4; ++j) sdst[(n4 + j) * 4 + kb] = (uint8_t)(sv >> (8 * j));
    }
  };
  auto compute = [&](int stage) {
    if (!wave_active) return;
    const uint8_t* As = reinterpret_cast<const uint8_t*>(smem + stage * 2 * TILE);
    const uint8_t* Bs = As + TILE * 2;
    const uint8_t* sA = ssc + stage * 1024;
    const uint8_t* sB = sA + 512;
#pragma unroll
    for (int ks = 0; ks < BK8 / 64; ++ks) {
      i32x8_t a[2], b[2];
      int sa[2], sb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + (lane & 31);
        const uint8_t* p = As + r * (LDS_LD * 2) + ks * 64 + (lane >> 5) * 16;
        const uint4 u0 = *reinterpret_cast<const uint4*>(p);
        const uint4 u1 = *reinterpret_cast<const uint4*>(p + 32);
        a[i] = i32x8_t{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
        sa[i] = sA[r * 4 + ks * 2 + (lane >> 5)];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = wn * 64 + j * 32 + (lane & 31);
        const uint8_t* p = Bs + c * (LDS_LD * 2) + ks * 64 + (lane >> 5) * 16;
        const uint4 u0 = *reinterpret_cast<const uint4*>(p);
        const uint4 u1 = *reinterpret_cast<const uint4*>(p + 32);
        b[j] = i32x8_t{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
        sb[j] = sB[c * 4 + ks * 2 + (lane >> 5)];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
    }
  };

  const int nk = (kdim + BK8 - 1) / BK8;
  if (nk <= 0) return;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK8);
    compute(cur);
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }
}

// Position of accumulator element r of block (i, j) inside the 128 x 128 tile
// (32x32 MFMA result layout: lane holds column lane%32, rows 8 (r/4) + 4 (lane/32) + r%4).
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * 64 + j * 32 + (lane & 31); }

// ---------------------------------------------------------------------------------
// Token-dimension grouped tiles: group g < E is routed expert g with counts[g] rows
// starting at offsets[g] of the permuted buffers; group E is the shared expert with
// T rows.  tile_prefix[g] = sum of ceil(rows / BM) over groups before g.  Linear
// tiles (m-tile major, n-tile minor) are split into 8 contiguous chunks, chunk x
// run by the blocks with blockIdx % 8 == x (the blocks one XCD receives), so the
// n-tiles that share an A row panel run on one L2.
// ---------------------------------------------------------------------------------
struct TokTile {
  int g, m0, rows, nt;
  bool ok;
};

__device__ __forceinline__ TokTile map_tok_tile(const int32_t* __restrict__ tile_prefix, int groups, int ntn,
                                                int E, const int32_t* __restrict__ counts, int T, int* sp) {
  for (int i = threadIdx.x; i <= groups; i += NT) sp[i] = tile_prefix[i];
  __syncthreads();
  TokTile tt;
  const int total = sp[groups] * ntn;
  const int c = (total + 7) >> 3;
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int L = x * c + j;
  tt.ok = (j < c) && (L < total);
  if (!tt.ok) return tt;
  const int mt = L / ntn;
  tt.nt = L - mt * ntn;
  int lo = 0, hi = groups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sp[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  tt.g = lo;
  tt.m0 = (mt - sp[lo]) * BM;
  const int n = (lo < E) ? counts[lo] : T;
  tt.rows = min(BM, n - tt.m0);
  return tt;
}

struct TokArgs {
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* tile_prefix;
  int T, E, groups;           // groups = E + 1 (shared expert last)
  int64_t shared_row0;        // first row of the shared expert in the routed+shared buffers
};

// MXFP8 operands of the routed tiles of a token-dim GEMM (unused for BF16 routed weights).
struct MxOperands {
  const uint8_t* aq;     // routed A codes [rows][K]
  const uint8_t* as;     // routed A scales [rows][K/32]
  MxRef b0, b1;          // routed B: rowwise (forward) or columnwise (data gradient) copies
};

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[2][2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};
}

// FC1 + SwiGLU: [a | b] = A W1^T with gate rows -> a, up rows -> b; writes a, b
// (bf16, [rows][2I]: a at column j, b at I + j) and h = silu(a) * b (bf16, [rows][I]).
// The B tile interleaves 32 gate rows and 32 up rows so each lane holds a and b of
// the same output element.  MX: routed tiles take E4M3 x and rowwise E4M3 weights.
struct Fc1Args {
  TokArgs t;
  const uint16_t* xp;   // routed A [S][H]
  const uint16_t* x;    // shared A [T][H]
  MatRef wg, wu, sg, su;
  MxOperands mx;        // b0 = gate, b1 = up
  uint16_t* ab;
  uint16_t* h;
  int H, I;
};

template <bool MX>
__global__ __launch_bounds__(NT, 2) void k_fc1_swiglu(Fc1Args p) {
  __shared__ __align__(16) uint16_t smem[LDS_ELEMS];
  __shared__ __align__(16) uint8_t ssc[MX ? 2048 : 16];
  __shared__ int sp[kMaxExperts + 2];
  const TokTile tt = map_tok_tile(p.t.tile_prefix, p.t.groups, p.I / 64, p.t.E, p.t.counts, p.t.T, sp);
  if (!tt.ok) return;
  const bool shared = tt.g == p.t.E;
  const int e = shared ? 0 : tt.g;
  const int64_t arow0 = shared ? tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int H = p.H;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, wm = wid >> 1, wn = wid & 1;
  auto brow = [&](int rr) { return tt.nt * 64 + ((rr >> 5) >> 1) * 32 + (rr & 31); };
  f32x16_t acc[2][2];
  zero_acc(acc);
  if (MX && !shared) {
    const uint8_t* aq = p.mx.aq;
    const uint8_t* as = p.mx.as;
    const int rows = tt.rows;
    auto fa = [&](int r) -> const uint8_t* { return r < rows ? aq + (arow0 + r) * H : nullptr; };
    auto fas = [&](int r) -> const uint8_t* { return r < rows ? as + (arow0 + r) * (H / 32) : nullptr; };
    auto fb = [&](int rr) -> const uint8_t* { return (((rr >> 5) & 1) ? p.mx.b1 : p.mx.b0).data.row(e, brow(rr)); };
    auto fbs = [&](int rr) -> const uint8_t* { return (((rr >> 5) & 1) ? p.mx.b1 : p.mx.b0).scale.row(e, brow(rr)); };
    tile_mma_fp8<true>(acc, H, fa, fas, fb, fbs, smem, ssc, wm * 64 < tt.rows);
  } else {
    const uint16_t* abase = shared ? p.x : p.xp;
    auto fa = [&](int r) -> const uint16_t* { return r < tt.rows ? abase + (arow0 + r) * H : nullptr; };
    const uint8_t* gb = shared ? p.sg.row(0, 0) : p.wg.row(e, 0);
    const uint8_t* ub = shared ? p.su.row(0, 0) : p.wu.row(e, 0);
    const int64_t gld = shared ? p.sg.ld_bytes : p.wg.ld_bytes;
    const int64_t uld = shared ? p.su.ld_bytes : p.wu.ld_bytes;
    auto fb = [&](int rr) -> const uint16_t* {
      const int jj = brow(rr);
      return reinterpret_cast<const uint16_t*>(((rr >> 5) & 1) ? ub + (int64_t)jj * uld : gb + (int64_t)jj * gld);
    };
    tile_mma<true, true>(acc, H, fa, fb, smem, wm * 64 < tt.rows);
  }

  const int64_t crow0 = shared ? p.t.shared_row0 + tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int I = p.I;
  const int jj = tt.nt * 64 + wn * 32 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = acc_row(wm, i, r, lane);
      if (row >= tt.rows) continue;
      const float a = acc[i][0][r], b = acc[i][1][r];
      const int64_t R = crow0 + row;
      p.ab[R * 2 * I + jj] = (uint16_t)f2bf(a);
      p.ab[R * 2 * I + I + jj] = (uint16_t)f2bf(b);
      p.h[R * I + jj] = (uint16_t)f2bf(a * sigmoidf_(a) * b);
    }
}

// Plain token-dim GEMM with bf16 store: C[rows][N] = A[rows][K] * B, where B is either
// K-contiguous rows of a weight [N][K] (forward FC2: y = h W2^T) or row-contiguous
// (data-gradient FC1: dx = dfc1 W1, W1 [2I][H] split into gate rows and up rows).
// MX: routed tiles take E4M3 A codes and the rowwise (B_KC) or columnwise (!B_KC)
// E4M3 weight copies.
struct PlainArgs {
  TokArgs t;
  const uint16_t* a_r;   // routed A rows (indexed by offsets[g] + m)
  const uint16_t* a_s;   // shared A rows
  int64_t a_s_row0;      // first shared row inside a_s
  MatRef w0, w1, s0, s1; // weights: B_KC: w0 rows; !B_KC: k < ksplit from w0, else w1
  MxOperands mx;
  int ksplit;
  uint16_t* c;           // [rows][N] (routed rows at offsets, shared at shared_row0)
  int N, K;
};

template <bool B_KC, bool MX>
__global__ __launch_bounds__(NT, 2) void k_gemm_plain(PlainArgs p) {
  __shared__ __align__(16) uint16_t smem[LDS_ELEMS];
  __shared__ __align__(16) uint8_t ssc[MX ? 2048 : 16];
  __shared__ int sp[kMaxExperts + 2];
  const TokTile tt = map_tok_tile(p.t.tile_prefix, p.t.groups, p.N / BN, p.t.E, p.t.counts, p.t.T, sp);
  if (!tt.ok) return;
  const bool shared = tt.g == p.t.E;
  const int e = shared ? 0 : tt.g;
  const int64_t arow0 = shared ? p.a_s_row0 + tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int K = p.K;
  const int n0 = tt.nt * BN;
  const int ksplit = p.ksplit;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, wm = wid >> 1, wn = wid & 1;
  f32x16_t acc[2][2];
  zero_acc(acc);
  if (MX && !shared) {
    const uint8_t* aq = p.mx.aq;
    const uint8_t* as = p.mx.as;
    const int rows = tt.rows;
    auto fa = [&](int r) -> const uint8_t* { return r < rows ? aq + (arow0 + r) * K : nullptr; };
    auto fas = [&](int r) -> const uint8_t* { return r < rows ? as + (arow0 + r) * (K / 32) : nullptr; };
    if constexpr (B_KC) {
      auto fb = [&](int r) -> const uint8_t* { return p.mx.b0.data.row(e, n0 + r); };
      auto fbs = [&](int r) -> const uint8_t* { return p.mx.b0.scale.row(e, n0 + r); };
      tile_mma_fp8<true>(acc, K, fa, fas, fb, fbs, smem, ssc, wm * 64 < tt.rows);
    } else {
      const int kbsplit = ksplit / 32;
      auto fb = [&](int q) -> const uint8_t* {
        return (q < ksplit ? p.mx.b0.data.row(e, q) : p.mx.b1.data.row(e, q - ksplit)) + n0;
      };
      auto fbs = [&](int kb) -> const uint8_t* {
        return (kb < kbsplit ? p.mx.b0.scale.row(e, kb) : p.mx.b1.scale.row(e, kb - kbsplit)) + n0;
      };
      tile_mma_fp8<false>(acc, K, fa, fas, fb, fbs, smem, ssc, wm * 64 < tt.rows);
    }
  } else {
    const uint16_t* abase = shared ? p.a_s : p.a_r;
    auto fa = [&](int r) -> const uint16_t* { return r < tt.rows ? abase + (arow0 + r) * K : nullptr; };
    // per-tile base rows of the two weight parts, so the loaders only add row offsets
    const uint8_t* b0 = shared ? p.s0.row(0, 0) : p.w0.row(e, 0);
    const uint8_t* b1 = shared ? p.s1.row(0, 0) : p.w1.row(e, 0);
    const int64_t ld0 = shared ? p.s0.ld_bytes : p.w0.ld_bytes;
    const int64_t ld1 = shared ? p.s1.ld_bytes : p.w1.ld_bytes;
    auto fb = [&](int q) -> const uint16_t* {
      if constexpr (B_KC) {
        return reinterpret_cast<const uint16_t*>(b0 + (int64_t)(n0 + q) * ld0);
      } else {
        const uint8_t* rowp = (q < ksplit) ? b0 + (int64_t)q * ld0 : b1 + (int64_t)(q - ksplit) * ld1;
        return reinterpret_cast<const uint16_t*>(rowp) + n0;
      }
    };
    tile_mma<true, B_KC>(acc, K, fa, fb, smem, wm * 64 < tt.rows);
  }

  const int64_t crow0 = shared ? p.t.shared_row0 + tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int N = p.N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row(wm, i, r, lane);
        if (row >= tt.rows) continue;
        p.c[(crow0 + row) * N + n0 + acc_col(wn, j, lane)] = (uint16_t)f2bf(acc[i][j][r]);
      }
}

// Data gradient of FC2 fused with the SwiGLU backward: gh = dyw W2 (contracting over H,
// W2 [H][I] row-contiguous), then with the saved a, b:
//   da = gh * b * silu'(a),  db = gh * silu(a)  -> dfc1 [rows][2I] (da at j, db at I + j).
// MX: routed tiles take E4M3 dyw and the columnwise E4M3 copy of W2.
struct DgradSwigluArgs {
  TokArgs t;
  const uint16_t* a_r;   // routed dyw rows [S][H]
  const uint16_t* a_s;   // shared dy rows [T][H]
  MatRef wd, sd;
  MxOperands mx;         // b0 = columnwise W2
  const uint16_t* ab;
  uint16_t* dfc1;
  int H, I;
};

template <bool MX>
__global__ __launch_bounds__(NT, 2) void k_dgrad_swiglu(DgradSwigluArgs p) {
  __shared__ __align__(16) uint16_t smem[LDS_ELEMS];
  __shared__ __align__(16) uint8_t ssc[MX ? 2048 : 16];
  __shared__ int sp[kMaxExperts + 2];
  const TokTile tt = map_tok_tile(p.t.tile_prefix, p.t.groups, p.I / BN, p.t.E, p.t.counts, p.t.T, sp);
  if (!tt.ok) return;
  const bool shared = tt.g == p.t.E;
  const int e = shared ? 0 : tt.g;
  const int64_t arow0 = shared ? tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int H = p.H, I = p.I;
  const int n0 = tt.nt * BN;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, wm = wid >> 1, wn = wid & 1;
  f32x16_t acc[2][2];
  zero_acc(acc);
  if (MX && !shared) {
    const uint8_t* aq = p.mx.aq;
    const uint8_t* as = p.mx.as;
    const int rows = tt.rows;
    auto fa = [&](int r) -> const uint8_t* { return r < rows ? aq + (arow0 + r) * H : nullptr; };
    auto fas = [&](int r) -> const uint8_t* { return r < rows ? as + (arow0 + r) * (H / 32) : nullptr; };
    auto fb = [&](int k) -> const uint8_t* { return p.mx.b0.data.row(e, k) + n0; };
    auto fbs = [&](int kb) -> const uint8_t* { return p.mx.b0.scale.row(e, kb) + n0; };
    tile_mma_fp8<false>(acc, H, fa, fas, fb, fbs, smem, ssc, wm * 64 < tt.rows);
  } else {
    const uint16_t* abase = shared ? p.a_s : p.a_r;
    auto fa = [&](int r) -> const uint16_t* { return r < tt.rows ? abase + (arow0 + r) * H : nullptr; };
    const uint8_t* wb = shared ? p.sd.row(0, 0) : p.wd.row(e, 0);
    const int64_t wld = shared ? p.sd.ld_bytes : p.wd.ld_bytes;
    auto fb = [&](int k) -> const uint16_t* { return reinterpret_cast<const uint16_t*>(wb + (int64_t)k * wld) + n0; };
    tile_mma<true, false>(acc, H, fa, fb, smem, wm * 64 < tt.rows);
  }

  const int64_t crow0 = shared ? p.t.shared_row0 + tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row(wm, i, r, lane);
        if (row >= tt.rows) continue;
        const int n = n0 + acc_col(wn, j, lane);
        const int64_t R = (crow0 + row) * 2 * (int64_t)I;
        const float a = bf2f(p.ab[R + n]);
        const float b = bf2f(p.ab[R + I + n]);
        const float gh = acc[i][j][r];
        const float sg = sigmoidf_(a);
        const float da = gh * b * (sg * (1.0f + a * (1.0f - sg)));
        const float db = gh * (a * sg);
        p.dfc1[R + n] = (uint16_t)f2bf(da);
        p.dfc1[R + I + n] = (uint16_t)f2bf(db);
      }
}

// ---------------------------------------------------------------------------------
// Weight gradients: main_grad[e] (M x N, FP32) += A^T B over the expert's token rows
// (both operands row-contiguous along M / N; K = the group's tokens).  Each output
// tile has exactly one owner: it loads its main_grad tile into the accumulators,
// runs the full token loop, and stores once (no split-K, no atomics).  Shared-expert
// tiles come first in launch order (their K is all T tokens); routed tiles follow,
// chunked per XCD like the token-dim GEMMs.
// ---------------------------------------------------------------------------------
struct WgradArgs {
  const int32_t* counts;
  const int32_t* offsets;
  int T, E, has_shared;
  const uint16_t* a_r; const uint16_t* a_s; int64_t lda; int64_t a_s_row0;
  const uint16_t* b_r; const uint16_t* b_s; int64_t ldb; int64_t b_s_row0;
  GradRef g_lo, g_hi, s_lo, s_hi;   // output rows m < msplit -> *_lo, others -> *_hi (row - msplit)
  int msplit;
  int M, N;
};

__global__ __launch_bounds__(NT, 2) void k_wgrad(WgradArgs p) {
  __shared__ __align__(16) uint16_t smem[LDS_ELEMS];
  const int mtn = p.M / BM, ntn = p.N / BN, per = mtn * ntn;
  const int nshared = p.has_shared ? per : 0;
  int g, tile;
  if ((int)blockIdx.x < nshared) {
    g = p.E;
    tile = blockIdx.x;
  } else {
    const int b = blockIdx.x - nshared;
    const int total = p.E * per;
    const int c = (total + 7) >> 3;
    const int x = b & 7, j = b >> 3;
    const int L = x * c + j;
    if (j >= c || L >= total) return;
    g = L / per;
    tile = L - g * per;
  }
  const bool shared = g == p.E;
  const int e = shared ? 0 : g;
  const int kdim = shared ? p.T : p.counts[g];
  if (kdim == 0) return;
  const int m0 = (tile / ntn) * BM, n0 = (tile % ntn) * BN;
  const int64_t ar0 = shared ? p.a_s_row0 : (int64_t)p.offsets[g];
  const int64_t br0 = shared ? p.b_s_row0 : (int64_t)p.offsets[g];
  const uint16_t* A = (shared ? p.a_s : p.a_r) + m0;
  const uint16_t* B = (shared ? p.b_s : p.b_r) + n0;
  const int64_t lda = p.lda, ldb = p.ldb;
  auto fa = [&](int k) -> const uint16_t* { return A + (ar0 + k) * lda; };
  auto fb = [&](int k) -> const uint16_t* { return B + (br0 + k) * ldb; };

  const GradRef& lo = shared ? p.s_lo : p.g_lo;
  const GradRef& hi = shared ? p.s_hi : p.g_hi;
  float* cb = (m0 < p.msplit) ? lo.row(e, m0) : hi.row(e, m0 - p.msplit);
  const int64_t ldc = (m0 < p.msplit) ? lo.ld : hi.ld;
  cb += n0;

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, wm = wid >> 1, wn = wid & 1;
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = cb[acc_row(wm, i, r, lane) * ldc + acc_col(wn, j, lane)];

  tile_mma<false, false>(acc, kdim, fa, fb, smem, true);

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) cb[acc_row(wm, i, r, lane) * ldc + acc_col(wn, j, lane)] = acc[i][j][r];
}

}  // namespace gemm
}  // namespace moe
