// Grouped GEMMs of the MoE layer on gfx950 matrix cores.  One launch covers
// every routed expert's row group plus the shared expert's group.
//
// Tile: TM (M) x 128 (N) per workgroup of 256 threads = 4 waves in a WM x WN
// grid, each wave a block of MI x NJ MFMA 32x32 accumulators (fp32).  Several
// workgroups share a CU, so one workgroup's global loads overlap another's
// MFMAs; a wave whose rows are all past the group's last row skips its MFMAs.
//
// K is staged 64 bytes at a time (32 bf16 or 64 E4M3 codes) through two LDS
// stages with 80-byte padded rows ([row][k], so every fragment read is one
// 16-byte ds_read), with PFD register stages of global loads in flight.
// Operands whose source is K-contiguous are copied as 16-byte chunks; operands
// whose source is contiguous along M / N (weights in the data-gradient GEMMs,
// activations in the weight-gradient GEMMs) are loaded as 4 x 8 (bf16) or
// 4 x 16 (bytes) blocks and transposed in registers on the way into LDS.
//
// BF16: v_mfma_f32_32x32x16_bf16.  MXFP8: v_mfma_scale_f32_32x32x64_f8f6f4
// with one E8M0 scale per lane (row or column, 32-code K block).
#pragma once
#include "common.hpp"

namespace moe {
namespace gemm {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

#ifndef MOE_TILE_BM
#define MOE_TILE_BM 128
#endif
#ifndef MOE_TILE_BMW
#define MOE_TILE_BMW 128
#endif
#ifndef MOE_TILE_WM
#define MOE_TILE_WM 2
#endif
#ifndef MOE_TILE_PFD
#define MOE_TILE_PFD 1
#endif
#ifndef MOE_TILE_MINB
#define MOE_TILE_MINB 2
#endif
#ifndef MOE_TILE_MINB_DG
#define MOE_TILE_MINB_DG 3
#endif
#ifndef MOE_TILE_MINB_W
#define MOE_TILE_MINB_W MOE_TILE_MINB
#endif
#ifndef MOE_TILE_KBYTES
#define MOE_TILE_KBYTES 128
#endif
constexpr int BN = 128, NT = 256;
constexpr int BM = MOE_TILE_BM;                 // token rows per tile (token-dim GEMMs)
constexpr int BMW = MOE_TILE_BMW;               // weight rows per tile (weight gradients)
constexpr int WM = MOE_TILE_WM;                 // waves along M (WN = 4 / WM along N)
constexpr int PFD = MOE_TILE_PFD;               // register stages of prefetch
constexpr int MINB = MOE_TILE_MINB;             // workgroups per CU the register budget targets:
constexpr int MINB_DG = MOE_TILE_MINB_DG;       //   forward, data-gradient and weight-gradient GEMMs
constexpr int MINB_W = MOE_TILE_MINB_W;
constexpr int KBYTES = MOE_TILE_KBYTES;         // K bytes per stage (64 or 128)
constexpr int ROW = KBYTES + 16;                // LDS row stride (bytes): 80 or 144
constexpr int CPR = KBYTES / 16;                // 16-byte chunks per row per stage
constexpr int SBK = KBYTES / 32;                // E8M0 blocks per row per MXFP8 stage
#ifndef MOE_TILE_RK
#define MOE_TILE_RK 4
#endif
constexpr int RK = MOE_TILE_RK;                 // k rows per row-contiguous bf16 block (4 or 8)

template <int TM>
struct Cfg {
  static constexpr int WN = 4 / WM;
  static constexpr int B_OFF = TM * ROW;                 // B tile offset inside a stage
  static constexpr int STAGE = (TM + BN) * ROW;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static constexpr int SC_B = TM * SBK;                  // scale tile: A [TM][SBK] then B [128][SBK]
  static constexpr int SC_STAGE = (TM + BN) * SBK;
  static constexpr int WMR = TM / WM;                    // rows per wave
  static constexpr int WNC = BN / WN;                    // columns per wave
  static constexpr int MI = WMR / 32, NJ = WNC / 32;     // 32x32 blocks per wave
  static constexpr int AKC = TM * CPR / 256;             // A K-contiguous chunks per thread
  static constexpr int BKC = BN * CPR / 256;             // B K-contiguous chunks per thread
  static constexpr int KG16 = KBYTES / 2 / RK;           // RK-element k groups per stage (bf16)
  static constexpr int NA_RC = KG16 * (TM / 8);          // A row-contiguous blocks (bf16)
  static constexpr int NB_RC = KG16 * (BN / 8);          // B row-contiguous blocks (bf16)
  static constexpr int KG8 = KBYTES / 4;                 // 4-code k groups per stage (bytes)
  static constexpr int NB_RC8 = KG8 * (BN / 16);         // B row-contiguous blocks (bytes)
};

template <int TM>
using Acc = f32x16_t[Cfg<TM>::MI][Cfg<TM>::NJ];

// 4 x 4 byte transpose: b_j = [a0.byte j, a1.byte j, a2.byte j, a3.byte j].
__device__ __forceinline__ void tr4x4_bytes(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                            uint32_t& b0, uint32_t& b1, uint32_t& b2, uint32_t& b3) {
  const uint32_t t0 = __builtin_amdgcn_perm(a1, a0, 0x05010400u);   // a00 a10 a01 a11
  const uint32_t t1 = __builtin_amdgcn_perm(a1, a0, 0x07030602u);   // a02 a12 a03 a13
  const uint32_t t2 = __builtin_amdgcn_perm(a3, a2, 0x05010400u);   // a20 a30 a21 a31
  const uint32_t t3 = __builtin_amdgcn_perm(a3, a2, 0x07030602u);   // a22 a32 a23 a33
  b0 = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  b1 = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  b2 = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  b3 = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// RK rows (k) x 8 bf16 (r) -> LDS rows r0 + i, 2 RK bytes (RK k values) at byte offset kb.
template <int NK>
__device__ __forceinline__ void store_tr_bf16(uint8_t* tile, int r0, int kb, const u32x4_t (&v)[NK]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int wi = i >> 1, sh = (i & 1) * 16;
    uint32_t o[NK / 2];
#pragma unroll
    for (int q = 0; q < NK / 2; ++q)
      o[q] = ((v[2 * q][wi] >> sh) & 0xffffu) | (((v[2 * q + 1][wi] >> sh) & 0xffffu) << 16);
    if constexpr (NK == 8)
      *reinterpret_cast<u32x4_t*>(tile + (r0 + i) * ROW + kb) = u32x4_t{o[0], o[1], o[2], o[3]};
    else
      *reinterpret_cast<uint2*>(tile + (r0 + i) * ROW + kb) = make_uint2(o[0], o[1]);
  }
}

// 4 rows (k) x 16 codes (r) -> LDS rows r0 + 0..15, 4 bytes (4 k) at byte offset kb.
__device__ __forceinline__ void store_tr_u8(uint8_t* tile, int r0, int kb, const u32x4_t (&v)[4]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t b[4];
    tr4x4_bytes(v[0][w], v[1][w], v[2][w], v[3][w], b[0], b[1], b[2], b[3]);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(tile + (r0 + 4 * w + j) * ROW + kb) = b[j];
  }
}

// ---------------------------------------------------------------------------------
// Operand descriptions handed to the tile loop.
//  KC (K-contiguous): fa / fb(r) -> pointer to tile row r at K = 0 (callers clamp rows
//                     past the end to a valid row; result rows they feed are never stored).
//  RC (row-contiguous): fa / fb(k) -> pointer to element (k, tile row 0); only called for
//                     k < kdim (for bf16), rows k >= kdim are zero-filled (the token tail
//                     of the weight gradients).
//  Scales (MXFP8): fas / fbs(r) -> E8M0 row of tile row r (K-contiguous operand), or for a
//                  row-contiguous B: fbs(kb) -> E8M0 byte of (K block kb, tile column 0).
// ---------------------------------------------------------------------------------
enum Mode { KC = 0, RC = 1 };

// Global loads of one K stage held in registers until they are written to LDS.
// Thread mapping.  KC: chunk t % CPR of rows t / CPR + (256 / CPR) i.  RC bf16: block
// (kg = t % KG16, rg = t / KG16) of 4 k x 8 rows, on threads [0, NA_RC) for A and
// [256 - NB_RC, 256) for B.  RC bytes (B): block (kg = u % KG8, rg = u / KG8) of 4 k x 16.
template <int TM>
struct Staged {
  u32x4_t ka[Cfg<TM>::AKC];  // A KC chunks
  u32x4_t kb[Cfg<TM>::BKC];  // B KC chunks
  u32x4_t ra[RK];            // A RC block (RK k rows)
  u32x4_t rb[RK];            // B RC block (RK k rows of bf16; 4 of codes)
  uint32_t sa, sb;           // MXFP8 scale bytes (SBK per row; B RC: 4 columns of one block)
};

// acc[i][j] (wave rows wm*WMR + 32 i, columns wn*WNC + 32 j) += A[TM x K] * B[128 x K]^T.
// arows: for a row-contiguous A, the tile rows that exist (a multiple of 8); the 8-row
// blocks past it are zero-filled instead of loaded.
template <int TM, int AM, int BMODE, bool FP8, class FA, class FB, class FAS, class FBS>
__device__ __forceinline__ void tile_mma(Acc<TM>& acc, int kdim, const FA& fa, const FB& fb, const FAS& fas,
                                         const FBS& fbs, uint8_t* lds, uint8_t* sc, bool wave_active,
                                         int arows = TM) {
  using C = Cfg<TM>;
  static_assert(!(FP8 && AM == RC), "MXFP8 A operands are K-contiguous");
  static_assert(TM == 128 || TM == 256, "tile rows");
  static_assert(AM == KC || C::NA_RC <= NT, "row-contiguous A blocks must fit the workgroup");
  static_assert(BMODE == KC || (FP8 ? C::NB_RC8 : C::NB_RC) <= NT, "row-contiguous B blocks must fit");
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, wm = w / C::WN, wn = w % C::WN;
  constexpr int EB = FP8 ? 1 : 2;                 // bytes per element
  constexpr int KST = KBYTES / EB;                // K elements per stage

  constexpr int RSTEP = NT / CPR;                 // rows between a thread's KC chunks
  const int kc = t % CPR, kr = t / CPR;           // KC chunk and first row
  const uint8_t* rpa[C::AKC];
  const uint8_t* rpb[C::BKC];
  const uint8_t* spa = nullptr;      // A scale row of tile row t (t < TM)
  const uint8_t* spb = nullptr;      // B scale row of tile row t (t < 128, KC B)
#pragma unroll
  for (int i = 0; i < C::AKC; ++i) rpa[i] = nullptr;
#pragma unroll
  for (int i = 0; i < C::BKC; ++i) rpb[i] = nullptr;
  if constexpr (AM == KC) {
#pragma unroll
    for (int i = 0; i < C::AKC; ++i) rpa[i] = reinterpret_cast<const uint8_t*>(fa(kr + RSTEP * i));
    if constexpr (FP8) spa = (t < TM) ? fas(t) : nullptr;
  }
  if constexpr (BMODE == KC) {
#pragma unroll
    for (int i = 0; i < C::BKC; ++i) rpb[i] = reinterpret_cast<const uint8_t*>(fb(kr + RSTEP * i));
    if constexpr (FP8) spb = (t < BN) ? fbs(t) : nullptr;
  }
  // A RC blocks on threads [0, NA_RC); blocks past arows are zero-filled.
  const int akg = t % C::KG16, arg = t / C::KG16;
  const bool rcA = (AM == RC) && t < C::NA_RC && arg * 8 < arows;
  const bool rcAz = (AM == RC) && t < C::NA_RC && !rcA;
  // B RC blocks on the last NB_RC (bf16) or NB_RC8 (bytes) threads.
  const int u = t - (NT - (FP8 ? C::NB_RC8 : C::NB_RC));
  const bool rcB = (BMODE == RC) && u >= 0;
  const int bkg = FP8 ? u % C::KG8 : u % C::KG16, brg = FP8 ? u / C::KG8 : u / C::KG16;

  auto gload = [&](int k0, Staged<TM>& g) __attribute__((always_inline)) {   // k0 in elements
    const int kbyte = k0 * EB;
    if constexpr (AM == KC) {
#pragma unroll
      for (int i = 0; i < C::AKC; ++i) g.ka[i] = *reinterpret_cast<const u32x4_t*>(rpa[i] + kbyte + kc * 16);
      if constexpr (FP8) {
        if (t < TM) {
          if constexpr (SBK == 2) g.sa = *reinterpret_cast<const uint16_t*>(spa + k0 / 32);
          else g.sa = *reinterpret_cast<const uint32_t*>(spa + k0 / 32);
        }
      }
    } else {
      if (rcA) {
        const int kb = k0 + akg * RK, m8 = arg * 8;
#pragma unroll
        for (int q = 0; q < RK; ++q)
          g.ra[q] = (kb + q < kdim)
                        ? *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint8_t*>(fa(kb + q)) + m8 * EB)
                        : u32x4_t{0, 0, 0, 0};
      }
    }
    if constexpr (BMODE == KC) {
#pragma unroll
      for (int i = 0; i < C::BKC; ++i) g.kb[i] = *reinterpret_cast<const u32x4_t*>(rpb[i] + kbyte + kc * 16);
      if constexpr (FP8) {
        if (t < BN) {
          if constexpr (SBK == 2) g.sb = *reinterpret_cast<const uint16_t*>(spb + k0 / 32);
          else g.sb = *reinterpret_cast<const uint32_t*>(spb + k0 / 32);
        }
      }
    } else {
      if (rcB) {
        if constexpr (FP8) {
          const int kb = k0 + bkg * 4, n16 = brg * 16;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            g.rb[q] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint8_t*>(fb(kb + q)) + n16);
          // column scales: SBK blocks x 128 columns, 4 columns per thread on the first 32*SBK threads
          if (u < 32 * SBK)
            g.sb = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(fbs(k0 / 32 + (u >> 5))) +
                                                      (u & 31) * 4);
        } else {
          const int kb = k0 + bkg * RK, n8 = brg * 8;
#pragma unroll
          for (int q = 0; q < RK; ++q)
            g.rb[q] = (kb + q < kdim)
                          ? *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint8_t*>(fb(kb + q)) + n8 * 2)
                          : u32x4_t{0, 0, 0, 0};
        }
      }
    }
  };
  auto sstore = [&](int s, const Staged<TM>& g) __attribute__((always_inline)) {
    uint8_t* As = lds + s * C::STAGE;
    uint8_t* Bs = As + C::B_OFF;
    if constexpr (AM == KC) {
#pragma unroll
      for (int i = 0; i < C::AKC; ++i)
        *reinterpret_cast<u32x4_t*>(As + (kr + RSTEP * i) * ROW + kc * 16) = g.ka[i];
      if constexpr (FP8) {
        if (t < TM) {
          if constexpr (SBK == 2) *reinterpret_cast<uint16_t*>(sc + s * C::SC_STAGE + t * SBK) = (uint16_t)g.sa;
          else *reinterpret_cast<uint32_t*>(sc + s * C::SC_STAGE + t * SBK) = g.sa;
        }
      }
    } else {
      if (rcA) {
        store_tr_bf16<RK>(As, arg * 8, akg * 2 * RK, g.ra);
      } else if (rcAz) {
        u32x4_t z[RK];
#pragma unroll
        for (int q = 0; q < RK; ++q) z[q] = u32x4_t{0, 0, 0, 0};
        store_tr_bf16<RK>(As, arg * 8, akg * 2 * RK, z);
      }
    }
    if constexpr (BMODE == KC) {
#pragma unroll
      for (int i = 0; i < C::BKC; ++i) *reinterpret_cast<u32x4_t*>(Bs + (kr + RSTEP * i) * ROW + kc * 16) = g.kb[i];
      if constexpr (FP8) {
        if (t < BN) {
          if constexpr (SBK == 2) *reinterpret_cast<uint16_t*>(sc + s * C::SC_STAGE + C::SC_B + t * SBK) = (uint16_t)g.sb;
          else *reinterpret_cast<uint32_t*>(sc + s * C::SC_STAGE + C::SC_B + t * SBK) = g.sb;
        }
      }
    } else {
      if (rcB) {
        if constexpr (FP8) {
          const u32x4_t r4[4] = {g.rb[0], g.rb[1], g.rb[2], g.rb[3]};
          store_tr_u8(Bs, brg * 16, bkg * 4, r4);
          if (u < 32 * SBK) {
            const int kb = u >> 5, n4 = (u & 31) * 4;
            uint8_t* sB = sc + s * C::SC_STAGE + C::SC_B;
#pragma unroll
            for (int j = 0; j < 4; ++j) sB[(n4 + j) * SBK + kb] = (uint8_t)(g.sb >> (8 * j));
          }
        } else {
          store_tr_bf16<RK>(Bs, brg * 8, bkg * 2 * RK, g.rb);
        }
      }
    }
  };
  auto compute = [&](int s) __attribute__((always_inline)) {
    if (!wave_active) return;
    const uint8_t* As = lds + s * C::STAGE;
    const uint8_t* Bs = As + C::B_OFF;
    if constexpr (!FP8) {
#pragma unroll
      for (int ks = 0; ks < KBYTES / 32; ++ks) {
        bf16x8_t a[C::MI], b[C::NJ];
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
          a[i] = *reinterpret_cast<const bf16x8_t*>(As + (wm * C::WMR + i * 32 + (lane & 31)) * ROW + ks * 32 +
                                                    (lane >> 5) * 16);
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
          b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * C::WNC + j * 32 + (lane & 31)) * ROW + ks * 32 +
                                                    (lane >> 5) * 16);
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
          for (int j = 0; j < C::NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    } else {
      // Per 64-code K step, lane (r, g) holds codes 16g..16g+15 and 32+16g..32+16g+15 and
      // carries the scale of 32-code block g (the scaled MFMA's measured lane layout).
      const uint8_t* sA = sc + s * C::SC_STAGE;
      const uint8_t* sB = sA + C::SC_B;
#pragma unroll
      for (int ks = 0; ks < KBYTES / 64; ++ks) {
        i32x8_t a[C::MI], b[C::NJ];
        int sa[C::MI], sb[C::NJ];
#pragma unroll
        for (int i = 0; i < C::MI; ++i) {
          const int r = wm * C::WMR + i * 32 + (lane & 31);
          const uint8_t* p = As + r * ROW + ks * 64 + (lane >> 5) * 16;
          const u32x4_t u0 = *reinterpret_cast<const u32x4_t*>(p);
          const u32x4_t u1 = *reinterpret_cast<const u32x4_t*>(p + 32);
          a[i] = i32x8_t{(int)u0[0], (int)u0[1], (int)u0[2], (int)u0[3], (int)u1[0], (int)u1[1], (int)u1[2], (int)u1[3]};
          sa[i] = sA[r * SBK + ks * 2 + (lane >> 5)];
        }
#pragma unroll
        for (int j = 0; j < C::NJ; ++j) {
          const int c = wn * C::WNC + j * 32 + (lane & 31);
          const uint8_t* p = Bs + c * ROW + ks * 64 + (lane >> 5) * 16;
          const u32x4_t u0 = *reinterpret_cast<const u32x4_t*>(p);
          const u32x4_t u1 = *reinterpret_cast<const u32x4_t*>(p + 32);
          b[j] = i32x8_t{(int)u0[0], (int)u0[1], (int)u0[2], (int)u0[3], (int)u1[0], (int)u1[1], (int)u1[2], (int)u1[3]};
          sb[j] = sB[c * SBK + ks * 2 + (lane >> 5)];
        }
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
          for (int j = 0; j < C::NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
      }
    }
  };

  const int nk = (kdim + KST - 1) / KST;
  if (nk <= 0) return;
  Staged<TM> buf[PFD];
#pragma unroll
  for (int q = 0; q < PFD; ++q)
    if (q < nk) gload(q * KST, buf[q]);
  sstore(0, buf[0]);
  __syncthreads();
  for (int k0 = 0; k0 < nk; k0 += PFD) {
#pragma unroll
    for (int q = 0; q < PFD; ++q) {
      const int kt = k0 + q;          // buf[q] held stage kt, already in LDS: reuse it for kt + PFD
      if (kt < nk) {
        if (kt + PFD < nk) gload((kt + PFD) * KST, buf[q]);
        compute(kt & 1);
        if (kt + 1 < nk) sstore((kt + 1) & 1, buf[(q + 1) % PFD]);
        __syncthreads();
      }
    }
  }
}

// Accumulator element r of block (i, j): 32x32 MFMA result layout, lane holds column
// lane % 32 and rows 8 (r / 4) + 4 (lane / 32) + r % 4 of its block.
template <int TM>
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * Cfg<TM>::WMR + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
template <int TM>
__device__ __forceinline__ int acc_col(int wn, int j, int lane) {
  return wn * Cfg<TM>::WNC + j * 32 + (lane & 31);
}

template <int TM>
__device__ __forceinline__ void zero_acc(Acc<TM>& acc) {
#pragma unroll
  for (int i = 0; i < Cfg<TM>::MI; ++i)
#pragma unroll
    for (int j = 0; j < Cfg<TM>::NJ; ++j) acc[i][j] = f32x16_t{};
}

struct NoScale {
  __device__ const uint8_t* operator()(int) const { return nullptr; }
};

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

using TC = Cfg<BM>;

// FC1 + SwiGLU: [a | b] = A W1^T with gate rows -> a, up rows -> b; writes a, b
// (bf16, [rows][2I]: a at column j, b at I + j) and h = silu(a) * b (bf16, [rows][I]).
// The B tile interleaves 32 gate rows and 32 up rows, so a wave's accumulator blocks
// 2p (gate) and 2p + 1 (up) hold a and b of the same output elements in each lane.
// MX: routed tiles take E4M3 x and rowwise E4M3 weights.
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
__global__ __launch_bounds__(NT, MINB) void k_fc1_swiglu(Fc1Args p) {
  __shared__ __align__(16) uint8_t lds[TC::LDS_BYTES];
  __shared__ __align__(16) uint8_t sc[MX ? 2 * TC::SC_STAGE : 16];
  __shared__ int sp[kMaxExperts + 2];
  const TokTile tt = map_tok_tile(p.t.tile_prefix, p.t.groups, p.I / 64, p.t.E, p.t.counts, p.t.T, sp);
  if (!tt.ok) return;
  const bool shared = tt.g == p.t.E;
  const int e = shared ? 0 : tt.g;
  const int64_t arow0 = shared ? tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int H = p.H, last = tt.rows - 1;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w / TC::WN, wn = w % TC::WN;
  auto brow = [&](int rr) { return tt.nt * 64 + (rr >> 6) * 32 + (rr & 31); };   // logical column
  Acc<BM> acc;
  zero_acc<BM>(acc);
  const bool active = wm * TC::WMR < tt.rows;
  if (MX && !shared) {
    auto fa = [&](int r) { return p.mx.aq + (arow0 + min(r, last)) * H; };
    auto fas = [&](int r) { return p.mx.as + (arow0 + min(r, last)) * (H / 32); };
    auto fb = [&](int rr) { return (((rr >> 5) & 1) ? p.mx.b1 : p.mx.b0).data.row(e, brow(rr)); };
    auto fbs = [&](int rr) { return (((rr >> 5) & 1) ? p.mx.b1 : p.mx.b0).scale.row(e, brow(rr)); };
    tile_mma<BM, KC, KC, true>(acc, H, fa, fb, fas, fbs, lds, sc, active);
  } else {
    const uint16_t* abase = shared ? p.x : p.xp;
    auto fa = [&](int r) { return abase + (arow0 + min(r, last)) * H; };
    const uint8_t* gb = shared ? p.sg.row(0, 0) : p.wg.row(e, 0);
    const uint8_t* ub = shared ? p.su.row(0, 0) : p.wu.row(e, 0);
    const int64_t gld = shared ? p.sg.ld_bytes : p.wg.ld_bytes;
    const int64_t uld = shared ? p.su.ld_bytes : p.wu.ld_bytes;
    auto fb = [&](int rr) {
      const int jj = brow(rr);
      return ((rr >> 5) & 1) ? ub + (int64_t)jj * uld : gb + (int64_t)jj * gld;
    };
    tile_mma<BM, KC, KC, false>(acc, H, fa, fb, NoScale{}, NoScale{}, lds, sc, active);
  }

  const int64_t crow0 = shared ? p.t.shared_row0 + tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int I = p.I;
#pragma unroll
  for (int jp = 0; jp < TC::NJ / 2; ++jp) {
    const int jj = tt.nt * 64 + (wn * TC::NJ / 2 + jp) * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < TC::MI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row<BM>(wm, i, r, lane);
        if (row >= tt.rows) continue;
        const float a = acc[i][2 * jp][r], b = acc[i][2 * jp + 1][r];
        const int64_t R = crow0 + row;
        p.ab[R * 2 * I + jj] = (uint16_t)f2bf(a);
        p.ab[R * 2 * I + I + jj] = (uint16_t)f2bf(b);
        p.h[R * I + jj] = (uint16_t)f2bf(a * sigmoidf_(a) * b);
      }
  }
}

// Plain token-dim GEMM with bf16 store: C[rows][N] = A[rows][K] * B, where B is either
// K-contiguous rows of a weight [N][K] (forward FC2: y = h W2^T) or row-contiguous
// (data-gradient FC1: dx = dfc1 W1, W1 [2I][H] split into gate rows and up rows).
// MX: routed tiles take E4M3 A codes and the rowwise (KC) or columnwise (RC)
// E4M3 weight copies.
struct PlainArgs {
  TokArgs t;
  const uint16_t* a_r;   // routed A rows (indexed by offsets[g] + m)
  const uint16_t* a_s;   // shared A rows
  int64_t a_s_row0;      // first shared row inside a_s
  MatRef w0, w1, s0, s1; // weights: KC: w0 rows; RC: k < ksplit from w0, else w1
  MxOperands mx;
  int ksplit;
  uint16_t* c;           // [rows][N] (routed rows at offsets, shared at shared_row0)
  int N, K;
};

template <int BMODE, bool MX>
__global__ __launch_bounds__(NT, BMODE == KC ? MINB : MINB_DG) void k_gemm_plain(PlainArgs p) {
  __shared__ __align__(16) uint8_t lds[TC::LDS_BYTES];
  __shared__ __align__(16) uint8_t sc[MX ? 2 * TC::SC_STAGE : 16];
  __shared__ int sp[kMaxExperts + 2];
  const TokTile tt = map_tok_tile(p.t.tile_prefix, p.t.groups, p.N / BN, p.t.E, p.t.counts, p.t.T, sp);
  if (!tt.ok) return;
  const bool shared = tt.g == p.t.E;
  const int e = shared ? 0 : tt.g;
  const int64_t arow0 = shared ? p.a_s_row0 + tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int K = p.K, last = tt.rows - 1;
  const int n0 = tt.nt * BN;
  const int ksplit = p.ksplit;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w / TC::WN, wn = w % TC::WN;
  Acc<BM> acc;
  zero_acc<BM>(acc);
  const bool active = wm * TC::WMR < tt.rows;
  if (MX && !shared) {
    auto fa = [&](int r) { return p.mx.aq + (arow0 + min(r, last)) * K; };
    auto fas = [&](int r) { return p.mx.as + (arow0 + min(r, last)) * (K / 32); };
    if constexpr (BMODE == KC) {
      auto fb = [&](int r) { return p.mx.b0.data.row(e, n0 + r); };
      auto fbs = [&](int r) { return p.mx.b0.scale.row(e, n0 + r); };
      tile_mma<BM, KC, KC, true>(acc, K, fa, fb, fas, fbs, lds, sc, active);
    } else {
      const int kbsplit = ksplit / 32;
      auto fb = [&](int q) { return (q < ksplit ? p.mx.b0.data.row(e, q) : p.mx.b1.data.row(e, q - ksplit)) + n0; };
      auto fbs = [&](int kb) {
        return (kb < kbsplit ? p.mx.b0.scale.row(e, kb) : p.mx.b1.scale.row(e, kb - kbsplit)) + n0;
      };
      tile_mma<BM, KC, RC, true>(acc, K, fa, fb, fas, fbs, lds, sc, active);
    }
  } else {
    const uint16_t* abase = shared ? p.a_s : p.a_r;
    auto fa = [&](int r) { return abase + (arow0 + min(r, last)) * K; };
    // per-tile base rows of the two weight parts, so the loaders only add row offsets
    const uint8_t* b0 = shared ? p.s0.row(0, 0) : p.w0.row(e, 0);
    const uint8_t* b1 = shared ? p.s1.row(0, 0) : p.w1.row(e, 0);
    const int64_t ld0 = shared ? p.s0.ld_bytes : p.w0.ld_bytes;
    const int64_t ld1 = shared ? p.s1.ld_bytes : p.w1.ld_bytes;
    if constexpr (BMODE == KC) {
      auto fb = [&](int q) { return b0 + (int64_t)(n0 + q) * ld0; };
      tile_mma<BM, KC, KC, false>(acc, K, fa, fb, NoScale{}, NoScale{}, lds, sc, active);
    } else {
      auto fb = [&](int q) {
        return ((q < ksplit) ? b0 + (int64_t)q * ld0 : b1 + (int64_t)(q - ksplit) * ld1) + 2 * n0;
      };
      tile_mma<BM, KC, RC, false>(acc, K, fa, fb, NoScale{}, NoScale{}, lds, sc, active);
    }
  }

  const int64_t crow0 = shared ? p.t.shared_row0 + tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int N = p.N;
#pragma unroll
  for (int i = 0; i < TC::MI; ++i)
#pragma unroll
    for (int j = 0; j < TC::NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row<BM>(wm, i, r, lane);
        if (row >= tt.rows) continue;
        p.c[(crow0 + row) * N + n0 + acc_col<BM>(wn, j, lane)] = (uint16_t)f2bf(acc[i][j][r]);
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
__global__ __launch_bounds__(NT, MINB_DG) void k_dgrad_swiglu(DgradSwigluArgs p) {
  __shared__ __align__(16) uint8_t lds[TC::LDS_BYTES];
  __shared__ __align__(16) uint8_t sc[MX ? 2 * TC::SC_STAGE : 16];
  __shared__ int sp[kMaxExperts + 2];
  const TokTile tt = map_tok_tile(p.t.tile_prefix, p.t.groups, p.I / BN, p.t.E, p.t.counts, p.t.T, sp);
  if (!tt.ok) return;
  const bool shared = tt.g == p.t.E;
  const int e = shared ? 0 : tt.g;
  const int64_t arow0 = shared ? tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int H = p.H, I = p.I, last = tt.rows - 1;
  const int n0 = tt.nt * BN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w / TC::WN, wn = w % TC::WN;
  Acc<BM> acc;
  zero_acc<BM>(acc);
  const bool active = wm * TC::WMR < tt.rows;
  if (MX && !shared) {
    auto fa = [&](int r) { return p.mx.aq + (arow0 + min(r, last)) * H; };
    auto fas = [&](int r) { return p.mx.as + (arow0 + min(r, last)) * (H / 32); };
    auto fb = [&](int k) { return p.mx.b0.data.row(e, k) + n0; };
    auto fbs = [&](int kb) { return p.mx.b0.scale.row(e, kb) + n0; };
    tile_mma<BM, KC, RC, true>(acc, H, fa, fb, fas, fbs, lds, sc, active);
  } else {
    const uint16_t* abase = shared ? p.a_s : p.a_r;
    auto fa = [&](int r) { return abase + (arow0 + min(r, last)) * H; };
    const uint8_t* wb = shared ? p.sd.row(0, 0) : p.wd.row(e, 0);
    const int64_t wld = shared ? p.sd.ld_bytes : p.wd.ld_bytes;
    auto fb = [&](int k) { return wb + (int64_t)k * wld + 2 * n0; };
    tile_mma<BM, KC, RC, false>(acc, H, fa, fb, NoScale{}, NoScale{}, lds, sc, active);
  }

  const int64_t crow0 = shared ? p.t.shared_row0 + tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
#pragma unroll
  for (int i = 0; i < TC::MI; ++i)
#pragma unroll
    for (int j = 0; j < TC::NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row<BM>(wm, i, r, lane);
        if (row >= tt.rows) continue;
        const int n = n0 + acc_col<BM>(wn, j, lane);
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
// (both operands row-contiguous along M / N; K = the group's tokens).  M is made of
// `parts` row ranges of `mpart` rows each (FC1: gate then up, FC2: one part), each
// tiled by BMW with a masked tail, so no tile straddles two main_grad buffers.  Each
// output tile has exactly one owner: it loads its main_grad tile into the
// accumulators, runs the full token loop, and stores once (no split-K, no atomics).
// Shared-expert tiles come first in launch order (their K is all T tokens); routed
// tiles follow, chunked per XCD like the token-dim GEMMs.
// ---------------------------------------------------------------------------------
struct WgradArgs {
  const int32_t* counts;
  const int32_t* offsets;
  int T, E, has_shared;
  const uint16_t* a_r; const uint16_t* a_s; int64_t lda; int64_t a_s_row0;
  const uint16_t* b_r; const uint16_t* b_s; int64_t ldb; int64_t b_s_row0;
  GradRef g_lo, g_hi, s_lo, s_hi;   // part 0 -> *_lo, part 1 -> *_hi
  int parts, mpart;                 // M = parts * mpart; A column of part p row m: p * mpart + m
  int N;
};

__host__ __device__ inline int wgrad_tiles_per_group(int parts, int mpart, int N) {
  return parts * ((mpart + BMW - 1) / BMW) * (N / BN);
}

using WC = Cfg<BMW>;

// FC is 1 or 2 (which projection's gradient); it only names the kernel symbol apart.
template <int FC>
__global__ __launch_bounds__(NT, MINB_W) void k_wgrad(WgradArgs p) {
  __shared__ __align__(16) uint8_t lds[WC::LDS_BYTES];
  const int mtp = (p.mpart + BMW - 1) / BMW, ntn = p.N / BN;
  const int per = p.parts * mtp * ntn;
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
  const int part = tile / (mtp * ntn);
  const int rem = tile - part * mtp * ntn;
  // Supertile order: blocks of sm x sn tiles run consecutively, so the sm A-row slices and
  // sn B-column slices they share are re-read from L2 while the main_grad stream flows past.
  const int sm = (mtp % 4 == 0) ? 4 : ((mtp % 2 == 0) ? 2 : 1);
  const int sn = (ntn % 8 == 0) ? 8 : ((ntn % 4 == 0) ? 4 : ((ntn % 2 == 0) ? 2 : 1));
  const int sblk = rem / (sm * sn), sin = rem - sblk * sm * sn;
  const int sbn = ntn / sn;
  const int mt = (sblk / sbn) * sm + sin / sn, nt = (sblk % sbn) * sn + sin % sn;
  const int m0 = mt * BMW, n0 = nt * BN;
  const int mrows = min(BMW, p.mpart - m0);
  const int64_t ar0 = shared ? p.a_s_row0 : (int64_t)p.offsets[g];
  const int64_t br0 = shared ? p.b_s_row0 : (int64_t)p.offsets[g];
  const uint16_t* A = (shared ? p.a_s : p.a_r) + (int64_t)part * p.mpart + m0;
  const uint16_t* B = (shared ? p.b_s : p.b_r) + n0;
  const int64_t lda = p.lda, ldb = p.ldb;
  auto fa = [&](int k) { return A + (ar0 + k) * lda; };
  auto fb = [&](int k) { return B + (br0 + k) * ldb; };

  const GradRef& G = part == 0 ? (shared ? p.s_lo : p.g_lo) : (shared ? p.s_hi : p.g_hi);
  float* cb = G.row(e, m0) + n0;
  const int64_t ldc = G.ld;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w / WC::WN, wn = w % WC::WN;
  Acc<BMW> acc;
  if (mrows == BMW) {   // full tile: unmasked main_grad read-modify-write
#pragma unroll
    for (int i = 0; i < WC::MI; ++i)
#pragma unroll
      for (int j = 0; j < WC::NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = cb[acc_row<BMW>(wm, i, r, lane) * ldc + acc_col<BMW>(wn, j, lane)];
    tile_mma<BMW, RC, RC, false>(acc, kdim, fa, fb, NoScale{}, NoScale{}, lds, nullptr, true, BMW);
#pragma unroll
    for (int i = 0; i < WC::MI; ++i)
#pragma unroll
      for (int j = 0; j < WC::NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) cb[acc_row<BMW>(wm, i, r, lane) * ldc + acc_col<BMW>(wn, j, lane)] = acc[i][j][r];
    return;
  }
  const bool active = wm * WC::WMR < mrows;
  zero_acc<BMW>(acc);
  if (active) {
#pragma unroll
    for (int i = 0; i < WC::MI; ++i)
#pragma unroll
      for (int j = 0; j < WC::NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = acc_row<BMW>(wm, i, r, lane);
          if (row < mrows) acc[i][j][r] = cb[row * ldc + acc_col<BMW>(wn, j, lane)];
        }
  }

  tile_mma<BMW, RC, RC, false>(acc, kdim, fa, fb, NoScale{}, NoScale{}, lds, nullptr, active, mrows);

  if (!active) return;
#pragma unroll
  for (int i = 0; i < WC::MI; ++i)
#pragma unroll
    for (int j = 0; j < WC::NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row<BMW>(wm, i, r, lane);
        if (row < mrows) cb[row * ldc + acc_col<BMW>(wn, j, lane)] = acc[i][j][r];
      }
}

}  // namespace gemm
}  // namespace moe
