// Grouped GEMMs of the MoE layer on gfx950 matrix cores.  One launch covers
// every routed expert's row group plus the shared expert's group.
//
// Tile: TM (M) x TN (N) per workgroup of NWM x NWN waves, each wave a block of
// MI x NJ MFMA 32x32 accumulators (fp32).  A wave whose rows all lie past the
// group's last row skips its MFMAs.
//
// Operand movement: every K stage (128 bytes of K per row: 64 bf16 or 128 E4M3)
// is copied global -> LDS by the load unit itself (global_load_lds_dwordx4: one
// wave instruction moves 64 x 16 bytes into 1 KB of LDS), so no registers hold
// staged data and NS stages can be in flight.  LDS tiles are unpadded; 16-byte
// chunks are XOR-swizzled by row so that both the DMA writes and the fragment
// reads are free of bank conflicts.  An operand is stored as it lies in memory:
//   K-contiguous ("KC", rows of a [rows][K] matrix): tile [rows][128 B],
//       fragments read with ds_read_b128;
//   row-contiguous ("RC", k-th row holds the tile's M / N run): tile
//       [k][T * elem bytes], fragments read transposed with ds_read_b64_tr_b16
//       (bf16) or ds_read_b64_tr_b8 (E4M3).
// Row-contiguous k rows past the end of K are loaded from a zero page, so the
// weight-gradient token tail contributes exactly zero.  With PF > 0 every wave also
// touches each 128-byte line of the stage PF steps past the newest DMA'd one with a
// 4-byte LDS DMA into a scratch word, pulling the lines into L2 ahead of their DMA
// (nothing lands in registers, so a late return cannot clobber one).
//
// BF16: v_mfma_f32_32x32x16_bf16.  MXFP8: v_mfma_scale_f32_32x32x64_f8f6f4
// with one E8M0 scale per lane (row or column, 32-code K block).
#pragma once
#include <type_traits>

#include "common.hpp"

namespace moe {
namespace gemm {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
// global-memory views, so that main_grad's accesses compile to global (not flat)
// instructions: a flat access counts against the LDS wait counter too, and would hold up
// every LDS wait behind the outstanding main_grad loads
typedef __attribute__((address_space(1))) f32x4_t glb_f32x4;
typedef __attribute__((address_space(1))) u32x2_t glb_u32x2;
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;


template <int TM_, int TN_, int NWM_, int NWN_, int NS_, int MINB_, int PF_ = 0, int KB_ = 128, int NSB_ = 0,
          int SCG_ = 8>
struct Tile {
  static constexpr int TM = TM_, TN = TN_, NWM = NWM_, NWN = NWN_, NS = NS_, MINB = MINB_;
  static constexpr int PF = PF_;   // L2 prefetch distance in stages past the newest DMA stage (0: off)
  static constexpr int KB = KB_;   // K bytes per row per stage: 128, or 64 (BF16 only)
  // Stages of the B operand in LDS: NS, or (NS = 2) three, so the B DMAs run one stage
  // further ahead than the A DMAs.  The two operands have separate rings, A first.
  static constexpr int NSB = NSB_ ? NSB_ : NS;
  static constexpr int NW = NWM * NWN, NTH = 64 * NW;
  static constexpr int WMR = TM / NWM, WNC = TN / NWN;   // rows / columns per wave
  static constexpr int MI = WMR / 32, NJ = WNC / 32;     // 32x32 blocks per wave
  static constexpr int A_BYTES = TM * KB, B_BYTES = TN * KB;
  static constexpr int A_DMA = A_BYTES / 1024 / NW;      // 1 KB DMA instructions per wave per stage
  static constexpr int B_DMA = B_BYTES / 1024 / NW;
  // MXFP8 scales (one E8M0 byte per 32 codes; a stage of 128 codes has 4 per row).  The
  // K-contiguous scale rows (A, and B in KC mode) are staged SCG stages at a time, 4 SCG
  // bytes per row, in two group buffers: fetching a row's scales once per group instead
  // of once per stage cuts the L2 requests of these rows by SCG.  B in RC mode ([K/32][TN]
  // bytes, contiguous along N) keeps one [4][TN] block per stage in an NS-deep ring.
  static constexpr int SCG = SCG_;                        // stages per scale group: 8 or 4
  static constexpr int SCG_A = TM * 4 * SCG, SCG_B = TN * 4 * SCG;   // group buffer parts
  static constexpr int SC_RCB = 4 * TN;                   // RC B scales of one stage
  static constexpr int LDS = NS * A_BYTES + NSB * B_BYTES;
  static constexpr int SC_KC = 2 * (SCG_A + SCG_B);       // scale LDS with a K-contiguous B
  static constexpr int SC_LDS = SC_KC + NS * SC_RCB;      // ... with a row-contiguous B
  static_assert(SCG == 8 || SCG == 4, "scale group of 8 or 4 stages");
  // L2 prefetch: one dword per 128-byte line of a stage (TM + TN lines), PF_N per wave
  static constexpr int PF_N = PF ? (TM + TN + NTH - 1) / NTH : 0;
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "DMA split");
  static_assert(WMR % 32 == 0 && WNC % 32 == 0 && NS >= 2, "tile shape");
  static_assert(KB == 128 || (KB == 64 && PF == 0), "64-byte stages take no L2 prefetch");
  static_assert(NSB == NS || (NSB == 3 && NS == 2 && PF == 0), "B ring one stage deeper than A");
};

template <class TL>
using Acc = f32x16_t[TL::MI][TL::NJ];

// Zero page: the source of row-contiguous k rows past the end of K.  Internal linkage:
// each translation unit that launches kernels holds its own copy.
static __device__ __align__(16) uint4 g_zero_page[64];

__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}

// LDS DMA: lane l's 16 (or 4) bytes at gptr land at LDS byte m0v + 16 l (or 4 l); m0v
// is the same for the whole wave.  The asm keeps the compiler from inserting its own
// full vmcnt waits before every LDS read; the pipeline below waits on exact counts.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t m0v) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(m0v);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gptr), "s"(m)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* gptr, uint32_t m0v) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(m0v);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(gptr), "s"(m)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Swizzles (16-byte chunk index XOR a function of the row), chosen so that the 16 or
// 32 lanes one LDS cycle serves touch 64 distinct banks:
//  KC, rows of KB = 128 or 64 bytes: ds_read_b128 of 16 consecutive rows, same chunk.
template <int KB>
__device__ __forceinline__ int swz_kc(int r) { return KB == 128 ? (r >> 1) & 7 : (r >> 2) & 3; }
//  RC bf16 (rows of 256 or 512 bytes): tr16 reads 4 k rows x 4 chunks.
__device__ __forceinline__ int swz_rc16(int k) { return (k & 3) << 2; }
//  RC E4M3 (rows of RB = 128 or 256 bytes): tr8 reads 8 k rows x 2 chunks.
template <int RB>
__device__ __forceinline__ int swz_rc8(int k) { return RB == 128 ? ((k >> 1) & 3) << 1 : (k & 7) << 1; }

enum Mode { KC = 0, RC = 1 };

struct NoScale {
  __device__ const uint8_t* operator()(int) const { return nullptr; }
};

// ---------------------------------------------------------------------------------
// acc[i][j] (wave rows wm*WMR + 32 i, columns wn*WNC + 32 j) += A[TM x K] * B[TN x K]^T.
//  KC operand: fa(r) / fb(r) -> bytes of tile row r at K = 0 (callers clamp rows past
//              the end to a valid row; the result rows they feed are never stored).
//              A rows at or past acols are loaded from the zero page instead.
//  RC operand: fa(k) / fb(k) -> bytes of element (k, tile row 0); called for k < kdim.
//              acols / bcols: tile rows of a row-contiguous A / B that exist (a multiple
//              of 8); the 16-byte pieces past them come from the zero page instead.
//  MXFP8 scales: fas(r) / fbs(r) -> E8M0 row of tile row r (KC operand), or for a
//              row-contiguous B, fbs(kb) -> E8M0 byte of (K block kb, tile column 0).
// ---------------------------------------------------------------------------------
template <class TL, int AM, int BMODE, bool FP8, bool BMAP = false, class FA, class FB, class FAS, class FBS>
__device__ __forceinline__ void tile_mma(Acc<TL>& acc, int kdim, const FA& fa, const FB& fb, const FAS& fas,
                                         const FBS& fbs, uint8_t* lds, uint8_t* sc, bool wave_active,
                                         int acols = TL::TM, uint8_t* pf_lds = nullptr, int bcols = TL::TN,
                                         const int32_t* bmap = nullptr, int32_t* map_lds = nullptr) {
  static_assert(!(FP8 && AM == RC), "MXFP8 A operands are K-contiguous");
  static_assert(!FP8 || TL::KB == 128, "MXFP8 stages are 128 codes (4 scale blocks)");
  constexpr int KB = TL::KB;
  constexpr int EB = FP8 ? 1 : 2;        // bytes per element
  constexpr int KST = KB / EB;           // K elements per stage
  constexpr int RBA = TL::TM * EB, RBB = TL::TN * EB;   // RC row bytes
  // the RC swizzles permute 16 chunks (bf16) or 8/16 chunks (E4M3) inside a row
  static_assert(AM != RC || (FP8 ? (RBA == 128 || RBA == 256) : (RBA == 256 || RBA == 512)), "RC A row bytes");
  static_assert(BMODE != RC || (FP8 ? (RBB == 128 || RBB == 256) : (RBB == 256 || RBB == 512)), "RC B row bytes");
  // loads per stage per wave (the waits below use it only for NS >= 3, which MXFP8 tiles
  // do not take: their scale DMAs vary per stage)
  constexpr int LPS = TL::A_DMA + TL::B_DMA + TL::PF_N;
  static_assert(!FP8 || TL::NS == 2, "MXFP8 tiles use two stages");
  // BMAP: a row-contiguous B whose k-th row is source row bmap[k] (bmap null: row k).
  // Stage j's KST map entries go to map_lds[(j % MS) * 64 ..], MS = 2 NS - 2 slots, DMA'd
  // by wave 0 as the last load of stage j - (NS - 1)'s group (maps 0 .. NS - 2 before the
  // ring starts).  Stage j is issued at step j - (NS - 1), after that step's wait has
  // drained stage j - (NS - 1)'s group and its barrier, so the map has landed and is
  // visible.  The prologue's NS - 1 stage issues write maps NS - 1 .. 2 NS - 3 while other
  // waves may still read maps 0 .. NS - 2 (no barrier between them), hence 2 NS - 2 slots;
  // in the ring, step kt writes map kt + 2 NS - 2 over map kt, which the issue of step
  // kt - NS + 1 read, before this step's barrier.
  constexpr int MS = 2 * TL::NS - 2;
  static_assert(!BMAP || (BMODE == RC && !FP8 && TL::KB / 2 <= 64), "row-mapped B");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w / TL::NWN, wn = w % TL::NWN;
  const uint32_t lds0 = lds_off(lds);
  const uint32_t scg0 = FP8 ? lds_off(sc) : 0u;                    // group buffer 0
  const uint32_t scr0 = scg0 + 2 * (TL::SCG_A + TL::SCG_B);          // RC B ring
  const uint8_t* zp = reinterpret_cast<const uint8_t*>(g_zero_page) + 16 * lane;
  const int nk = (kdim + KST - 1) / KST;

  // ---- per-lane DMA sources.  Slot i of this wave fills 1 KB block w * X_DMA + i.
  const uint8_t* pa[TL::A_DMA];
  const uint8_t* pb[TL::B_DMA];
  int ka[TL::A_DMA], kb[TL::B_DMA];       // RC: k row within the stage
  int ca[TL::A_DMA], cb[TL::B_DMA];       // RC: byte offset inside the tile row
#pragma unroll
  for (int i = 0; i < TL::A_DMA; ++i) {
    const int off = (w * TL::A_DMA + i) * 1024 + 16 * lane;
    if constexpr (AM == KC) {
      const int r = off / KB, c = ((off % KB) >> 4) ^ swz_kc<KB>(r);
      pa[i] = r < acols ? reinterpret_cast<const uint8_t*>(fa(r)) + 16 * c : nullptr;   // nullptr: zero page
      ka[i] = ca[i] = 0;
    } else {
      const int k = off / RBA, c = ((off % RBA) >> 4) ^ swz_rc16(k);
      pa[i] = nullptr;
      ka[i] = 16 * c < acols * EB ? k : (1 << 30);   // columns past acols: never loaded
      ca[i] = 16 * c;
    }
  }
#pragma unroll
  for (int i = 0; i < TL::B_DMA; ++i) {
    const int off = (w * TL::B_DMA + i) * 1024 + 16 * lane;
    if constexpr (BMODE == KC) {
      const int r = off / KB, c = ((off % KB) >> 4) ^ swz_kc<KB>(r);
      pb[i] = reinterpret_cast<const uint8_t*>(fb(r)) + 16 * c;
      kb[i] = cb[i] = 0;
    } else {
      const int k = off / RBB;
      const int c = ((off % RBB) >> 4) ^ (FP8 ? swz_rc8<RBB>(k) : swz_rc16(k));
      pb[i] = nullptr;
      kb[i] = 16 * c < bcols * EB ? k : (1 << 30);   // columns past bcols: never loaded
      cb[i] = 16 * c;
    }
  }
  // MXFP8 scale groups.  Dword DMA instruction q of a group covers RPI = 64 / SCG scale
  // rows x SCG stages: A rows RPI q.. for q < GA, then (KC B) B rows.  Lane l loads row
  // RPI q' + l / SCG at group stage (l % SCG) ^ (q' % SCG) to byte 4 l of the
  // instruction's 256-byte block, so row R's stage s sits at byte 4 SCG R +
  // 4 (s ^ (R / RPI % SCG)) and 32 consecutive rows read at one stage hit 32 different
  // banks.  Stages past K come from the zero page.  A group is issued in SCG pieces,
  // piece p with the data of the group before's stage p + 1.
  constexpr int RPI = 64 / TL::SCG;
  constexpr int GA = TL::TM / RPI, GB = (BMODE == KC) ? TL::TN / RPI : 0;
  constexpr int GPP = (GA + GB) / TL::SCG;   // instructions per piece
  static_assert(!FP8 || (TL::TM % RPI == 0 && TL::TN % RPI == 0 && (GA + GB) % TL::SCG == 0), "scale group split");
  auto scale_piece = [&](int G, int piece) __attribute__((always_inline)) {
    if constexpr (FP8) {
      const uint32_t gbase = scg0 + (G & 1) * (TL::SCG_A + TL::SCG_B);
      for (int q = piece * GPP + w; q < (piece + 1) * GPP; q += TL::NW) {
        const bool isa = q < GA;
        const int qq = isa ? q : q - GA;
        const int R = RPI * qq + lane / TL::SCG;
        const int kt = G * TL::SCG + ((lane % TL::SCG) ^ (qq % TL::SCG));
        const uint8_t* src = reinterpret_cast<const uint8_t*>(g_zero_page) + 4 * lane;
        if (kt < nk) {
          if (isa) {
            src = reinterpret_cast<const uint8_t*>(fas(R)) + 4 * kt;
          } else {
            if constexpr (BMODE == KC) src = reinterpret_cast<const uint8_t*>(fbs(R)) + 4 * kt;
          }
        }
        dma4(src, gbase + (isa ? 0 : TL::SCG_A) + qq * 256);
      }
    }
  };

  // L2 prefetch sources: line p * NTH + 64 w + lane of a stage; lines < TM belong to A.
  const uint32_t pfm0 = TL::PF ? lds_off(pf_lds) : 0u;
  auto pf_issue = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < TL::PF_N; ++p) {
      const int line = p * TL::NTH + 64 * w + lane;
      const uint8_t* src = reinterpret_cast<const uint8_t*>(g_zero_page) + 4 * lane;
      if (line < TL::TM) {
        if constexpr (AM == KC) {
          if (line < acols) src = reinterpret_cast<const uint8_t*>(fa(line)) + kt * 128;
        } else {
          const int k = kt * KST + line / (RBA / 128);
          if (k < kdim && 128 * (line % (RBA / 128)) < acols * EB)
            src = reinterpret_cast<const uint8_t*>(fa(k)) + 128 * (line % (RBA / 128));
        }
      } else if (line < TL::TM + TL::TN) {
        const int lb = line - TL::TM;
        if constexpr (BMODE == KC) {
          src = reinterpret_cast<const uint8_t*>(fb(lb)) + kt * 128;
        } else {
          const int k = kt * KST + lb / (RBB / 128);
          if (k < kdim && 128 * (lb % (RBB / 128)) < bcols * EB)
            src = reinterpret_cast<const uint8_t*>(fb(k)) + 128 * (lb % (RBB / 128));
        }
      }
      dma4(src, pfm0);
    }
  };

  const uint32_t map0 = BMAP ? lds_off(map_lds) : 0u;
  auto map_issue = [&](int kt) __attribute__((always_inline)) {
    if (w == 0) {
      const int k = kt * KST + lane;
      const uint8_t* src = reinterpret_cast<const uint8_t*>(g_zero_page) + 4 * lane;
      if (lane < KST && k < kdim) src = reinterpret_cast<const uint8_t*>(bmap + k);
      dma4(src, map0 + (kt % MS) * 256);
    }
  };

  // stage kt's A tile sits in A slot kt % NS, its B tile in B slot kt % NSB
  auto issue_a = [&](int kt) __attribute__((always_inline)) {
    const uint32_t sa = lds0 + (kt % TL::NS) * TL::A_BYTES;
    const int k0 = kt * KST;
#pragma unroll
    for (int i = 0; i < TL::A_DMA; ++i) {
      const uint32_t m0v = sa + (w * TL::A_DMA + i) * 1024;
      if constexpr (AM == KC) {
        dma16(pa[i] ? pa[i] + kt * KB : zp, m0v);
      } else {
        const int k = k0 + ka[i];
        dma16(k < kdim ? reinterpret_cast<const uint8_t*>(fa(k)) + ca[i] : zp, m0v);
      }
    }
  };
  auto issue_b = [&](int kt) __attribute__((always_inline)) {
    const uint32_t sb = lds0 + TL::NS * TL::A_BYTES + (kt % TL::NSB) * TL::B_BYTES;
    const int k0 = kt * KST;
#pragma unroll
    for (int i = 0; i < TL::B_DMA; ++i) {
      const uint32_t m0v = sb + (w * TL::B_DMA + i) * 1024;
      if constexpr (BMODE == KC) {
        dma16(pb[i] + kt * KB, m0v);
      } else {
        const int k = k0 + kb[i];
        int row = k;
        if constexpr (BMAP) {
          if (bmap) row = map_lds[(kt % MS) * 64 + kb[i]];
        }
        dma16(k < kdim ? reinterpret_cast<const uint8_t*>(fb(row)) + cb[i] : zp, m0v);
      }
    }
  };
  // the MXFP8 scale loads that go out with stage kt
  auto issue_sc = [&](int kt) __attribute__((always_inline)) {
    const int slot = kt % TL::NS;
    if constexpr (FP8) {
      if constexpr (BMODE == RC) {   // this stage's [4][TN] block of B scales
        for (int q = w; q < TL::SC_RCB / 256; q += TL::NW) {
          const int idx = q * 64 + lane;   // bytes 4 idx .. 4 idx + 3
          const int kblk = (4 * idx) / TL::TN, col = (4 * idx) % TL::TN;
          dma4(col < bcols ? reinterpret_cast<const uint8_t*>(fbs(kt * 4 + kblk)) + col
                           : reinterpret_cast<const uint8_t*>(g_zero_page) + 4 * lane,
               scr0 + slot * TL::SC_RCB + q * 256);
        }
      }
      if (kt == 0) {
        for (int piece = 0; piece < TL::SCG; ++piece) scale_piece(0, piece);
      } else {
        const int G = (kt - 1) / TL::SCG + 1;
        if (G * TL::SCG < nk) scale_piece(G, (kt - 1) % TL::SCG);
      }
    }
  };
  // one whole stage (equal rings): A, B, then the stage's map, scale and prefetch loads
  auto issue = [&](int kt) __attribute__((always_inline)) {
    issue_a(kt);
    issue_b(kt);
    if constexpr (BMAP) {
      if (bmap) map_issue(kt + TL::NS - 1);
    }
    issue_sc(kt);
    if constexpr (TL::PF > 0) pf_issue(min(kt + TL::PF, nk - 1));
  };

  // ---- fragment reads and MFMAs of one stage
  auto compute = [&](int kt) __attribute__((always_inline)) {
    const int slot = kt % TL::NS;
    const uint8_t* As = lds + slot * TL::A_BYTES;
    const uint8_t* Bs = lds + TL::NS * TL::A_BYTES + (kt % TL::NSB) * TL::B_BYTES;
    const int g = lane >> 5, grp = lane >> 4, j16 = lane & 15;
    // Small wave tiles read all fragments of the stage first, so the LDS reads of later K
    // steps overlap the MFMAs of earlier ones; large ones (whose fragments would not fit
    // in registers beside the accumulators) read and multiply one K step at a time.
    if constexpr (!FP8) {
      constexpr int NKS = KB / 32;   // 16-element K steps per stage
      // (the row-mapped instantiation sits at its register cap: reading every fragment of
      // the stage ahead there spills; a three-stage ring reads one K step at a time too, so
      // that the weight gradients keep 128 VGPRs and two workgroups per CU)
      constexpr bool PRE = NKS * (TL::MI + TL::NJ) * 4 <= 64 && !BMAP && TL::NS < 3;
      bf16x8_t a[NKS][TL::MI], b[NKS][TL::NJ];
      auto load = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TL::MI; ++i) {
          if constexpr (AM == KC) {
            const int r = wm * TL::WMR + i * 32 + (lane & 31);
            a[ks][i] = *reinterpret_cast<const bf16x8_t*>(As + r * KB + (((2 * ks + g) ^ swz_kc<KB>(r)) << 4));
          } else {
            const int m0 = wm * TL::WMR + i * 32 + 16 * (grp & 1);
            i16x4_t h[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int k = 16 * ks + 8 * (grp >> 1) + 4 * hh + (j16 >> 2);
              const int byte = 2 * (m0 + 4 * (j16 & 3));
              h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_i16x4*)((lds_u8*)As + k * RBA + ((((byte >> 4) ^ swz_rc16(k)) << 4) | (byte & 15))));
            }
            a[ks][i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
          }
        }
#pragma unroll
        for (int j = 0; j < TL::NJ; ++j) {
          if constexpr (BMODE == KC) {
            const int r = wn * TL::WNC + j * 32 + (lane & 31);
            b[ks][j] = *reinterpret_cast<const bf16x8_t*>(Bs + r * KB + (((2 * ks + g) ^ swz_kc<KB>(r)) << 4));
          } else {
            const int n0 = wn * TL::WNC + j * 32 + 16 * (grp & 1);
            i16x4_t h[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int k = 16 * ks + 8 * (grp >> 1) + 4 * hh + (j16 >> 2);
              const int byte = 2 * (n0 + 4 * (j16 & 3));
              h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_i16x4*)((lds_u8*)Bs + k * RBB + ((((byte >> 4) ^ swz_rc16(k)) << 4) | (byte & 15))));
            }
            b[ks][j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
          }
        }
      };
      auto mma = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TL::MI; ++i)
#pragma unroll
          for (int j = 0; j < TL::NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks][i], b[ks][j], acc[i][j], 0, 0, 0);
      };
      if constexpr (PRE) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) load(ks);
        __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the MFMAs
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) mma(ks);
      } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          load(ks);
          mma(ks);
        }
      }
    } else {
      // Per 64-code K step, lane (r, g) holds codes 16g..16g+15 and 32+16g..32+16g+15 and
      // carries the scale of 32-code block g (the scaled MFMA's measured lane layout).
      const int gs = kt % TL::SCG;   // stage inside its scale group
      const uint8_t* sA = sc + ((kt / TL::SCG) & 1) * (TL::SCG_A + TL::SCG_B);
      const uint8_t* sB = sA + TL::SCG_A;
      const uint8_t* sR = sc + 2 * (TL::SCG_A + TL::SCG_B) + slot * TL::SC_RCB;
      auto gsc = [&](const uint8_t* base, int R, int ks) __attribute__((always_inline)) {
        return base[4 * TL::SCG * R + 4 * (gs ^ ((R / RPI) % TL::SCG)) + 2 * ks + g];
      };
      constexpr bool PRE = 2 * (TL::MI + TL::NJ) * 8 <= 64;
      i32x8_t a[2][TL::MI], b[2][TL::NJ];
      int sa[2][TL::MI], sb[2][TL::NJ];
      auto load = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TL::MI; ++i) {
          const int r = wm * TL::WMR + i * 32 + (lane & 31);
          const uint8_t* p = As + r * KB;
          const u32x4_t u0 = *reinterpret_cast<const u32x4_t*>(p + (((4 * ks + g) ^ swz_kc<KB>(r)) << 4));
          const u32x4_t u1 = *reinterpret_cast<const u32x4_t*>(p + (((4 * ks + g + 2) ^ swz_kc<KB>(r)) << 4));
          a[ks][i] = i32x8_t{(int)u0[0], (int)u0[1], (int)u0[2], (int)u0[3], (int)u1[0], (int)u1[1], (int)u1[2], (int)u1[3]};
          sa[ks][i] = gsc(sA, r, ks);
        }
#pragma unroll
        for (int j = 0; j < TL::NJ; ++j) {
          const int c = wn * TL::WNC + j * 32 + (lane & 31);
          if constexpr (BMODE == KC) {
            const uint8_t* p = Bs + c * KB;
            const u32x4_t u0 = *reinterpret_cast<const u32x4_t*>(p + (((4 * ks + g) ^ swz_kc<KB>(c)) << 4));
            const u32x4_t u1 = *reinterpret_cast<const u32x4_t*>(p + (((4 * ks + g + 2) ^ swz_kc<KB>(c)) << 4));
            b[ks][j] = i32x8_t{(int)u0[0], (int)u0[1], (int)u0[2], (int)u0[3], (int)u1[0], (int)u1[1], (int)u1[2], (int)u1[3]};
            sb[ks][j] = gsc(sB, c, ks);
          } else {
            const int n0 = wn * TL::WNC + j * 32 + 16 * (grp & 1);
            i32x2_t q[4];
#pragma unroll
            for (int hh = 0; hh < 4; ++hh) {
              const int k = 64 * ks + 16 * g + 8 * (hh & 1) + 32 * (hh >> 1) + (j16 >> 1);
              const int byte = n0 + 8 * (j16 & 1);
              q[hh] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                  (lds_i32x2*)((lds_u8*)Bs + k * RBB + ((((byte >> 4) ^ swz_rc8<RBB>(k)) << 4) | (byte & 15))));
            }
            b[ks][j] = i32x8_t{q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1], q[3][0], q[3][1]};
            sb[ks][j] = sR[(2 * ks + g) * TL::TN + c];
          }
        }
      };
      auto mma = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TL::MI; ++i)
#pragma unroll
          for (int j = 0; j < TL::NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[ks][i], b[ks][j], acc[i][j], 0, 0, 0,
                                                                         sa[ks][i], 0, sb[ks][j]);
      };
      if constexpr (PRE) {
        load(0);
        load(1);
        __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the MFMAs
        mma(0);
        mma(1);
      } else {
        load(0);
        mma(0);
        load(1);
        mma(1);
      }
    }
  };

  // ---- NS-stage pipeline, one barrier per stage.  At the top of step kt the wave's
  // DMAs of stage kt must have landed; those of the up to NS - 2 later stages may fly
  // (with PF, each stage's group of loads ends with its prefetch, which may fly too).
  // With the deeper B ring, step kt issues A(kt + 1) and then B(kt + 2), so B's loads
  // (the weight panel, the HBM-bound operand of the token GEMMs) get one more stage of
  // lead than A's.
  if constexpr (BMAP) {
    if (bmap && nk > 0) {
      for (int s = 0; s < TL::NS - 1; ++s) map_issue(s);
      wait_vm<0>();
      __syncthreads();
    }
  }
  // (MXFP8: a K-contiguous B only, so that every scale load goes out with its A stage)
  static_assert(TL::NSB == TL::NS || (!BMAP && (!FP8 || BMODE == KC)), "deeper B ring: token GEMMs");
  if constexpr (TL::NSB == TL::NS) {
#pragma unroll
    for (int s = 0; s < TL::NS - 1; ++s)
      if (s < nk) issue(s);
  } else {
    // B(0), A(0), B(1): at the top of step kt the newest loads are A(kt) (with the MXFP8
    // scale loads that go out with it) and then B(kt + 1)
    if (nk > 0) {
      issue_b(0);
      issue_a(0);
      issue_sc(0);
    }
    if (nk > 1) issue_b(1);
  }
  // Two copies of the loop, so that skipping the MFMAs of an idle wave is not a branch
  // inside it (a conditional update would make the accumulators flow through a join
  // and cost a copy of every accumulator register per stage).
  auto run = [&](auto act) __attribute__((always_inline)) {
    if constexpr (TL::NSB != TL::NS) {
      for (int kt = 0; kt < nk; ++kt) {
        // A(kt) and B(kt) must have landed; B(kt + 1), issued after A(kt), may fly
        if (kt + 1 < nk) wait_vm<TL::B_DMA>();
        else wait_vm<0>();
        __syncthreads();
        if (kt + 1 < nk) {
          issue_a(kt + 1);
          issue_sc(kt + 1);
        }
        if (kt + 2 < nk) issue_b(kt + 2);
        if constexpr (decltype(act)::value) compute(kt);
      }
    } else {
      for (int kt = 0; kt < nk; ++kt) {
        const int ahead = min(TL::NS - 2, nk - 1 - kt);
        constexpr int TAIL = TL::PF_N;   // the prefetch that follows stage kt's DMAs
        if constexpr (TL::NS >= 4) {
          if (ahead >= 2) wait_vm<2 * LPS + TAIL>();
          else if (ahead == 1) wait_vm<LPS + TAIL>();
          else wait_vm<TAIL>();
        } else if constexpr (TL::NS == 3) {
          if (ahead >= 1) wait_vm<LPS + TAIL>();
          else wait_vm<TAIL>();
        } else {
          wait_vm<TAIL>();
        }
        __syncthreads();
        if (kt + TL::NS - 1 < nk) issue(kt + TL::NS - 1);
        if constexpr (decltype(act)::value) compute(kt);
      }
    }
  };
  if (wave_active) run(std::true_type{});
  else run(std::false_type{});
}

// Accumulator element r of block (i, j): 32x32 MFMA result layout, lane holds column
// lane % 32 and rows 8 (r / 4) + 4 (lane / 32) + r % 4 of its block.
template <class TL>
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * TL::WMR + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
template <class TL>
__device__ __forceinline__ int acc_col(int wn, int j, int lane) {
  return wn * TL::WNC + j * 32 + (lane & 31);
}

template <class TL>
__device__ __forceinline__ void zero_acc(Acc<TL>& acc) {
#pragma unroll
  for (int i = 0; i < TL::MI; ++i)
#pragma unroll
    for (int j = 0; j < TL::NJ; ++j) acc[i][j] = f32x16_t{};
}

// ---------------------------------------------------------------------------------
// Token-dimension grouped tiles: group g < E is routed expert g with counts[g] rows
// starting at offsets[g] of the permuted buffers; group E, when present, is the
// shared expert with T rows.  tile_prefix[g] = sum of ceil(rows / BMT) over groups before g.
// The blocks with blockIdx % 8 == x (the blocks one XCD receives) run one contiguous eighth
// of the shared expert's linear tiles, then one contiguous eighth of the routed tiles.
// Splitting the two kinds separately keeps the XCDs' work equal when a shared tile is
// longer than a routed one (BF16 shared next to MXFP8 routed weights: twice the K stages),
// and the shared tiles start first.  The grid holds at least ceil(tiles / 8) + 1 blocks
// per XCD.  Inside a group the linear order walks bands of
// kBandM m-tiles, column by column (m fastest), so the tiles resident on one XCD at a
// time form a block of about kBandM m-tiles x (32 / kBandM) n-tiles: their A row panels
// and B column panels are fetched into that XCD's L2 once per pass instead of the whole
// weight being streamed again for every m-tile pair.  A group with one m-tile (at most
// BMT rows) is walked along n as before.
// ---------------------------------------------------------------------------------
#ifndef MOE_BAND_M
#define MOE_BAND_M 8
#endif
constexpr int kBandM = MOE_BAND_M;

struct TokTile {
  int g, m0, rows, nt;
  bool ok;
};

template <int BMT>
__device__ __forceinline__ TokTile map_tok_tile(const int32_t* __restrict__ tile_prefix, int groups, int ntn,
                                                int E, const int32_t* __restrict__ counts, int T, int* sp) {
  for (int i = threadIdx.x; i <= groups; i += blockDim.x) sp[i] = tile_prefix[i];
  __syncthreads();
  TokTile tt;
  const int rt = sp[min(E, groups)] * ntn;         // routed tiles
  const int st = sp[groups] * ntn - rt;            // shared tiles (0 without the shared expert)
  const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int s0 = (int)((int64_t)st * x / 8), ns = (int)((int64_t)st * (x + 1) / 8) - s0;
  const int r0 = (int)((int64_t)rt * x / 8), nr = (int)((int64_t)rt * (x + 1) / 8) - r0;
  tt.ok = j < ns + nr;
  if (!tt.ok) return tt;
  const int L = j < ns ? rt + s0 + j : r0 + (j - ns);
  const int mt = L / ntn;
  int lo = 0, hi = groups - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sp[mid] <= mt) lo = mid; else hi = mid - 1;
  }
  tt.g = lo;
  const int li = L - sp[lo] * ntn;                 // tile inside the group
  const int band = li / (kBandM * ntn);
  const int r = li - band * kBandM * ntn;
  const int h = min(kBandM, sp[lo + 1] - sp[lo] - band * kBandM);   // m-tiles in this band
  tt.nt = r / h;
  tt.m0 = (band * kBandM + r % h) * BMT;
  const int n = (lo < E) ? counts[lo] : T;
  tt.rows = min(BMT, n - tt.m0);
  return tt;
}

struct TokArgs {
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* tile_prefix;
  int T, E, groups;           // E, or E + 1 with the shared expert (last group)
  int64_t shared_row0;        // first row of the shared expert in the routed+shared buffers
};

// MXFP8 operands of the routed tiles of a token-dim GEMM (unused for BF16 routed weights).
struct MxOperands {
  const uint8_t* aq;     // routed A codes [rows][K] (FC1: one row per token)
  const uint8_t* as;     // routed A scales [rows][K/32]
  MxRef b0, b1;          // routed B: rowwise (forward) or columnwise (data gradient) copies
};

// Tile shapes per kernel: TM, TN, waves along M, waves along N, LDS stages, the
// workgroups per CU the register budget targets, L2 prefetch distance, K bytes per
// stage, LDS stages of the B operand (default: as many as A).  BF16 and MXFP8 routed
// weights take separate shapes; within one of the two, every token-dimension GEMM has
// the same M tile (the routing scan builds one tile prefix for it).
// BF16 FC1, FC2 and FC2 data gradient: the weight panel gets a third LDS stage (at 4096
// tokens over 96 experts each panel is read once, from HBM, and the extra stage of lead
// hides more of its latency: 3-4% per kernel there, 1-3% slower with 2731 tokens per
// expert, where the panels are L2 hits).
#ifndef MOE_TL_FC1
#define MOE_TL_FC1 192, 256, 2, 4, 2, 1, 0, 128, 3
#endif
#ifndef MOE_TL_FC2
#define MOE_TL_FC2 192, 256, 2, 4, 2, 1, 0, 128, 3
#endif
#ifndef MOE_TL_DG2
#define MOE_TL_DG2 192, 256, 2, 4, 2, 1, 0, 128, 3
#endif
#ifndef MOE_TL_DG1
#define MOE_TL_DG1 192, 256, 2, 4, 2, 1
#endif
// MXFP8 FC1: the weight panel in three stages too, which fits beside the scale staging
// with scale groups of 4 stages (158 KB of LDS): fc1 0.5% faster at the 4096-token layer,
// 2% at the 8192-token one.  (Groups of 4 alone cost 0.3%; FC2 with the deeper ring ran
// 1-1.5% slower at the larger layers and keeps two stages.)
#ifndef MOE_TL_FC1_MX
#define MOE_TL_FC1_MX 192, 256, 2, 4, 2, 1, 0, 128, 3, 4
#endif
#ifndef MOE_TL_FC2_MX
#define MOE_TL_FC2_MX 192, 256, 2, 4, 2, 1
#endif
#ifndef MOE_TL_DG2_MX
#define MOE_TL_DG2_MX 192, 256, 2, 4, 2, 1, 1
#endif
#ifndef MOE_TL_DG1_MX
#define MOE_TL_DG1_MX 192, 256, 2, 4, 2, 1, 1
#endif
#ifndef MOE_TL_WG
#define MOE_TL_WG 128, 256, 2, 4, 2, 2, 0, 64
#endif
// FP32 main_grad, short token loops (few tokens per expert): a third 64-byte stage.  Two
// 72 KB workgroups still share a CU; 3-5% faster at 171 tokens per expert, where the
// main_grad stream binds, 3-5% slower at 768 or 2731, hence only there.
#ifndef MOE_TL_WG_SHORT
#define MOE_TL_WG_SHORT 128, 256, 2, 4, 3, 2, 0, 64
#endif
#ifndef MOE_TL_WG16
#define MOE_TL_WG16 128, 128, 2, 2, 2, 4, 0, 64
#endif
// BF16, many tokens per expert: two 4-wave workgroups per CU on 192 x 128 tiles (the same
// 96 x 64 wave tiles, two 128-byte stages, exactly 80 KB of LDS each).  Where the tiles
// are MFMA-bound, one workgroup's barrier and DMA waits and its epilogue overlap the other
// workgroup's multiplies (EP16 share: fc1 -8%, dgrad_fc2 -4%); where the weight panels
// stream from HBM they lose the three-stage weight ring (4096-token layer: fc1 +3%,
// dgrad_fc2 +9%), so the library takes them above kWideSlots slots per expert.
#ifndef MOE_TL_WIDE
#define MOE_TL_WIDE 192, 128, 2, 2, 2, 2, 0, 128
#endif
template <bool MX> struct Shapes;
template <> struct Shapes<false> {
  using FC1 = Tile<MOE_TL_FC1>; using FC2 = Tile<MOE_TL_FC2>;
  using DG2 = Tile<MOE_TL_DG2>; using DG1 = Tile<MOE_TL_DG1>;
};
template <> struct Shapes<true> {
  using FC1 = Tile<MOE_TL_FC1_MX>; using FC2 = Tile<MOE_TL_FC2_MX>;
  using DG2 = Tile<MOE_TL_DG2_MX>; using DG1 = Tile<MOE_TL_DG1_MX>;
};
struct ShapesWide {
  using FC1 = Tile<MOE_TL_WIDE>; using FC2 = Tile<MOE_TL_WIDE>;
  using DG2 = Tile<MOE_TL_WIDE>; using DG1 = Tile<MOE_TL_WIDE>;
};
// the shapes of one launch: MXFP8, BF16, or BF16 with many tokens per expert (WIDE)
template <bool MX, bool WIDE>
using ShapesOf = typename std::conditional<WIDE, ShapesWide, Shapes<MX>>::type;
// weight gradients: FP32 main_grad (MG16 = false; SHORT: the short-token-loop shape)
// and BF16 main_grad (true; half the read-modify-write bytes per tile, so smaller tiles at
// higher occupancy win there)
template <bool MG16, bool SHORT = false>
using TL_WG = typename std::conditional<
    MG16, Tile<MOE_TL_WG16>, typename std::conditional<SHORT, Tile<MOE_TL_WG_SHORT>, Tile<MOE_TL_WG>>::type>::type;
template <bool MX>
constexpr int bm_of() { return Shapes<MX>::FC1::TM; }
static_assert(Shapes<false>::FC2::TM == bm_of<false>() && Shapes<false>::DG2::TM == bm_of<false>() &&
              Shapes<false>::DG1::TM == bm_of<false>(), "BF16 token-dimension tiles share their M tile");
static_assert(Shapes<true>::FC2::TM == bm_of<true>() && Shapes<true>::DG2::TM == bm_of<true>() &&
              Shapes<true>::DG1::TM == bm_of<true>(), "MXFP8 token-dimension tiles share their M tile");
static_assert(ShapesWide::FC1::TM == bm_of<false>(), "both BF16 shape sets share the M tile");

template <class TL>
__device__ __forceinline__ int wave_m() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) / TL::NWN; }
template <class TL>
__device__ __forceinline__ int wave_n() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) % TL::NWN; }

// Token-dimension epilogue through LDS.  After the K loop the stage buffers are free: the
// accumulators of one wave row (WMR tile rows x TN columns, fp32) are parked there per
// round, then every thread takes pieces of 8 consecutive output columns of a row, so the
// epilogue's global loads and stores move 16 bytes per lane instead of 2.  LDS row r holds
// 16-byte chunk c at c ^ 8 ((r >> 2) & 1): the two row groups a wave writes at once fall
// in disjoint banks.
//  PAIR = false: f(tile_row, col, v) with v = tile columns col .. col + 7;
//  PAIR = true (FC1's interleaved gate/up tile: columns 64 k .. 64 k + 31 are gate
//  columns 32 k .. 32 k + 31 and the next 32 the matching up columns): f(tile_row, lc, g, u)
//  with g, u = gate and up values of the tile's logical columns lc .. lc + 7.
template <class TL, bool PAIR, class F>
__device__ __forceinline__ void tok_epilogue(const Acc<TL>& acc, uint8_t* lds, int rows, int ncols, const F& f) {
  constexpr int PPR = PAIR ? TL::TN / 16 : TL::TN / 8;   // pieces per row
  constexpr int PPT = TL::WMR * PPR / TL::NTH;           // pieces per thread per round
  static_assert(TL::WMR * TL::TN * 4 <= TL::LDS && (TL::WMR * PPR) % TL::NTH == 0, "epilogue round");
  float* ct = reinterpret_cast<float*>(lds);
  const int t = threadIdx.x, lane = t & 63, wm = wave_m<TL>(), wn = wave_n<TL>();
  auto sw = [](int r) { return ((r >> 2) & 1) << 3; };
  auto get8 = [&](const float* rowp, int r, int c0, float* v) __attribute__((always_inline)) {
    const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(rowp + (((c0 >> 2) ^ sw(r)) << 2));
    const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(rowp + ((((c0 >> 2) + 1) ^ sw(r)) << 2));
#pragma unroll
    for (int k = 0; k < 4; ++k) { v[k] = x0[k]; v[4 + k] = x1[k]; }
  };
#pragma unroll
  for (int q = 0; q < TL::NWM; ++q) {
    if (q * TL::WMR >= rows) break;
    __syncthreads();   // the LDS is free (K loop or the previous round done)
    if (wm == q) {
#pragma unroll
      for (int i = 0; i < TL::MI; ++i)
#pragma unroll
        for (int j = 0; j < TL::NJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            const int col = acc_col<TL>(wn, j, lane);
            ct[row * TL::TN + (((col >> 2) ^ sw(row)) << 2) + (col & 3)] = acc[i][j][r];
          }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int pi = u * TL::NTH + t, row = pi / PPR, pc = pi % PPR;
      const int trow = q * TL::WMR + row;
      const float* rowp = ct + row * TL::TN;
      if constexpr (PAIR) {
        const int lc = 8 * pc, c0 = (lc >> 5) * 64 + (lc & 31);
        if (trow < rows) {
          float g[8], v[8];
          get8(rowp, row, c0, g);
          get8(rowp, row, c0 + 32, v);
          f(trow, lc, g, v);
        }
      } else {
        const int col = 8 * pc;
        if (trow < rows && col < ncols) {
          float v[8];
          get8(rowp, row, col, v);
          f(trow, col, v);
        }
      }
    }
  }
}

// FC1 + SwiGLU: [a | b] = A W1^T with gate rows -> a, up rows -> b; writes a, b
// (bf16, [rows][2I]: a at column j, b at I + j) and h = silu(a) * b (bf16, [rows][I]).
// The B tile interleaves 32 gate rows and 32 up rows, so a wave's accumulator blocks
// 2p (gate) and 2p + 1 (up) hold a and b of the same output elements in each lane.
// MX: routed tiles take E4M3 x and rowwise E4M3 weights.
struct Fc1Args {
  TokArgs t;
  const int32_t* slot_t;   // token of each routed slot
  const uint16_t* x;       // A [T][H]: routed rows through slot_t, shared rows directly
  MatRef wg, wu, sg, su;
  MxOperands mx;        // b0 = gate, b1 = up
  uint16_t* ab;
  uint16_t* h;
  uint8_t* hq;   // MXFP8 routed tiles: E4M3 codes [rows][I] and E8M0 scales [rows][I/32] of the
  uint8_t* hs;   // BF16 h just stored (blocks of 32 along I), the FC2 input
  int H, I;
  float limit;   // SwiGLU clamp: h = silu(min(a, L)) clamp(b, -L, L) for L > 0, decided on
                 // the FP32 accumulator; a clamped input is stored as +-infinity in ab, which
                 // tells the backward it was clamped
};

template <bool MX, bool WIDE = false>
__global__ __launch_bounds__((ShapesOf<MX, WIDE>::FC1::NTH), (ShapesOf<MX, WIDE>::FC1::MINB)) void k_fc1_swiglu(
    Fc1Args p) {
  using TL = typename ShapesOf<MX, WIDE>::FC1;
  static_assert(TL::WNC % 64 == 0 && TL::TN <= 256, "gate/up pairs per wave; 2I is a multiple of TN");
  // BF16: the tile map's scratch and the token list live in the second A stage, which the
  // K loop first writes after its first barrier, when both are dead (the token rows are
  // in the DMA sources by then); MXFP8 reads the token list for its scale rows all along
  constexpr int XTRA = MX ? 4 * (kMaxExperts + 2) + 4 * TL::TM : 0;
  static_assert(MX || TL::A_BYTES >= 4 * (kMaxExperts + 2 + TL::TM), "map scratch in an A stage");
  __shared__ __align__(16) uint8_t lds[TL::LDS + (TL::PF ? 256 : 0) + (MX ? TL::SC_KC : 0) + XTRA];
  uint8_t* pfb = lds + TL::LDS;
  uint8_t* sc = pfb + (TL::PF ? 256 : 0);
  int* sp = reinterpret_cast<int*>(MX ? sc + (MX ? TL::SC_KC : 0) : lds + TL::A_BYTES);
  int* tok = sp + (kMaxExperts + 2);   // token (x row) of each tile row
  const TokTile tt = map_tok_tile<TL::TM>(p.t.tile_prefix, p.t.groups, 2 * p.I / TL::TN, p.t.E, p.t.counts, p.t.T, sp);
  if (!tt.ok) return;
  const bool shared = tt.g == p.t.E;
  const int e = shared ? 0 : tt.g;
  const int64_t arow0 = shared ? tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int H = p.H, last = tt.rows - 1;
  for (int i = threadIdx.x; i < tt.rows; i += TL::NTH)
    tok[i] = shared ? tt.m0 + i : p.slot_t[arow0 + i];
  __syncthreads();
  const int wm = wave_m<TL>();
  auto brow = [&](int rr) { return tt.nt * (TL::TN / 2) + (rr >> 6) * 32 + (rr & 31); };   // logical column
  Acc<TL> acc;
  zero_acc<TL>(acc);
  const bool active = wm * TL::WMR < tt.rows;
  bool done = false;
  if constexpr (MX) {
    if (!shared) {
      auto fa = [&](int r) { return p.mx.aq + (int64_t)tok[min(r, last)] * H; };
      auto fas = [&](int r) { return p.mx.as + (int64_t)tok[min(r, last)] * (H / 32); };
      // per-tile bases of the gate and up weights and scales
      const uint8_t* gd = p.mx.b0.data.row(e, 0);
      const uint8_t* ud = p.mx.b1.data.row(e, 0);
      const uint8_t* gs = p.mx.b0.scale.row(e, 0);
      const uint8_t* us = p.mx.b1.scale.row(e, 0);
      const int64_t gdl = p.mx.b0.data.ld_bytes, udl = p.mx.b1.data.ld_bytes;
      const int64_t gsl = p.mx.b0.scale.ld_bytes, usl = p.mx.b1.scale.ld_bytes;
      auto fb = [&](int rr) { return ((rr >> 5) & 1) ? ud + brow(rr) * udl : gd + brow(rr) * gdl; };
      auto fbs = [&](int rr) { return ((rr >> 5) & 1) ? us + brow(rr) * usl : gs + brow(rr) * gsl; };
      tile_mma<TL, KC, KC, true>(acc, H, fa, fb, fas, fbs, lds, sc, active, tt.rows, pfb);
      done = true;
    }
  }
  if (!done) {
    auto fa = [&](int r) { return p.x + (int64_t)tok[min(r, last)] * H; };
    const uint8_t* gb = shared ? p.sg.row(0, 0) : p.wg.row(e, 0);
    const uint8_t* ub = shared ? p.su.row(0, 0) : p.wu.row(e, 0);
    const int64_t gld = shared ? p.sg.ld_bytes : p.wg.ld_bytes;
    const int64_t uld = shared ? p.su.ld_bytes : p.wu.ld_bytes;
    auto fb = [&](int rr) {
      const int jj = brow(rr);
      return ((rr >> 5) & 1) ? ub + (int64_t)jj * uld : gb + (int64_t)jj * gld;
    };
    tile_mma<TL, KC, KC, false>(acc, H, fa, fb, NoScale{}, NoScale{}, lds, sc, active, tt.rows, pfb);
  }

  const int64_t crow0 = shared ? p.t.shared_row0 + tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int I = p.I;
  const float L = p.limit;
  // two copies of the epilogue, so that a layer without a clamp runs none of its selects
  auto epilogue = [&](auto clamp) __attribute__((always_inline)) {
    constexpr bool CL = decltype(clamp)::value;
    tok_epilogue<TL, true>(acc, lds, tt.rows, TL::TN, [&](int row, int lc, const float* ga, const float* ub) {
      const int jj = tt.nt * (TL::TN / 2) + lc;
      const int64_t R = crow0 + row;
      uint32_t aw[4], bw[4], hw[4];
#pragma unroll
      for (int k = 0; k < 8; k += 2) {
        float hv[2], as[2], bs[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float a = ga[k + e], b = ub[k + e];
          // the clamp is decided here, on the FP32 accumulator; a clamped input is stored as
          // +-infinity, so the backward reads the decision instead of taking it again on a
          // rounded value
          const bool a_hi = CL && a > L;
          const bool b_out = CL && fabsf(b) > L;
          const float ac = a_hi ? L : a;
          const float bc = b_out ? copysignf(L, b) : b;
          hv[e] = ac * sigmoidf_(ac) * bc;
          as[e] = a_hi ? __builtin_inff() : a;
          bs[e] = b_out ? copysignf(__builtin_inff(), b) : b;
        }
        aw[k / 2] = pack_bf2(as[0], as[1]);
        bw[k / 2] = pack_bf2(bs[0], bs[1]);
        hw[k / 2] = pack_bf2(hv[0], hv[1]);
      }
      *reinterpret_cast<uint4*>(p.ab + R * 2 * I + jj) = make_uint4(aw[0], aw[1], aw[2], aw[3]);
      *reinterpret_cast<uint4*>(p.ab + R * 2 * I + I + jj) = make_uint4(bw[0], bw[1], bw[2], bw[3]);
      *reinterpret_cast<uint4*>(p.h + R * I + jj) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      if constexpr (MX) {
        if (!shared) {   // the routed FC2 input: MXFP8 codes of the BF16 h of these 8 columns; the
                         // 4 lanes holding one 32-column block are adjacent (8 columns per lane)
          float hb[8];
#pragma unroll
          for (int k = 0; k < 4; ++k) { hb[2 * k] = lo_bf(hw[k]); hb[2 * k + 1] = hi_bf(hw[k]); }
          uint2 q;
          const uint32_t sc = mx_quantize8(hb, quad_max(absmax8(hb)), q);
          *reinterpret_cast<uint2*>(p.hq + R * I + jj) = q;
          if ((jj & 31) == 0) p.hs[R * (I / 32) + jj / 32] = (uint8_t)sc;
        }
      }
    });
  };
  if (L > 0.0f) epilogue(std::true_type{});
  else epilogue(std::false_type{});
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
  int ksplit;            // a multiple of 128, so no K stage straddles the two parts
  uint16_t* c;           // [rows][N] (routed rows at offsets, shared at shared_row0)
  int N, K;
};

template <int BMODE, bool MX, bool WIDE = false>
using TL_PLAIN =
    typename std::conditional<BMODE == KC, typename ShapesOf<MX, WIDE>::FC2, typename ShapesOf<MX, WIDE>::DG1>::type;

template <int BMODE, bool MX, bool WIDE = false>
__global__ __launch_bounds__((TL_PLAIN<BMODE, MX, WIDE>::NTH), (TL_PLAIN<BMODE, MX, WIDE>::MINB)) void k_gemm_plain(
    PlainArgs p) {
  using TL = TL_PLAIN<BMODE, MX, WIDE>;
  constexpr int XTRA = MX ? 4 * (kMaxExperts + 2) : 0;   // BF16: the map scratch in the second A stage
  constexpr int SCB = BMODE == KC ? TL::SC_KC : TL::SC_LDS;   // MXFP8 scale staging
  __shared__ __align__(16) uint8_t lds[TL::LDS + (TL::PF ? 256 : 0) + (MX ? SCB : 0) + XTRA];
  uint8_t* pfb = lds + TL::LDS;
  uint8_t* sc = pfb + (TL::PF ? 256 : 0);
  int* sp = reinterpret_cast<int*>(MX ? sc + (MX ? SCB : 0) : lds + TL::A_BYTES);
  const TokTile tt = map_tok_tile<TL::TM>(p.t.tile_prefix, p.t.groups, (p.N + TL::TN - 1) / TL::TN, p.t.E, p.t.counts,
                                          p.t.T, sp);
  if (!tt.ok) return;
  const bool shared = tt.g == p.t.E;
  const int e = shared ? 0 : tt.g;
  const int64_t arow0 = shared ? p.a_s_row0 + tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int K = p.K, last = tt.rows - 1;
  const int n0 = tt.nt * TL::TN;
  const int ncols = min(TL::TN, p.N - n0);   // the last N tile may be partial (a multiple of 128)
  const int nlast = ncols - 1;
  const int ksplit = p.ksplit;
  const int wm = wave_m<TL>();
  Acc<TL> acc;
  zero_acc<TL>(acc);
  const bool active = wm * TL::WMR < tt.rows;
  bool done = false;
  if constexpr (MX) if (!shared) {
    done = true;
    auto fa = [&](int r) { return p.mx.aq + (arow0 + min(r, last)) * K; };
    auto fas = [&](int r) { return p.mx.as + (arow0 + min(r, last)) * (K / 32); };
    if constexpr (BMODE == KC) {
      const uint8_t* d0 = p.mx.b0.data.row(e, n0);     // per-tile bases
      const uint8_t* s0 = p.mx.b0.scale.row(e, n0);
      const int64_t dl = p.mx.b0.data.ld_bytes, sl = p.mx.b0.scale.ld_bytes;
      auto fb = [&](int r) { return d0 + min(r, nlast) * dl; };
      auto fbs = [&](int r) { return s0 + min(r, nlast) * sl; };
      tile_mma<TL, KC, KC, true>(acc, K, fa, fb, fas, fbs, lds, sc, active, tt.rows, pfb);
    } else {
      const int kbsplit = ksplit / 32;
      // per-tile bases of the two weight parts, so the loaders only add row offsets
      const uint8_t* d0 = p.mx.b0.data.row(e, 0) + n0;
      const uint8_t* d1 = p.mx.b1.data.row(e, 0) + n0;
      const uint8_t* s0 = p.mx.b0.scale.row(e, 0) + n0;
      const uint8_t* s1 = p.mx.b1.scale.row(e, 0) + n0;
      const int64_t dl0 = p.mx.b0.data.ld_bytes, dl1 = p.mx.b1.data.ld_bytes;
      const int64_t sl0 = p.mx.b0.scale.ld_bytes, sl1 = p.mx.b1.scale.ld_bytes;
      auto fb = [&](int q) { return q < ksplit ? d0 + (int64_t)q * dl0 : d1 + (int64_t)(q - ksplit) * dl1; };
      auto fbs = [&](int kb) { return kb < kbsplit ? s0 + (int64_t)kb * sl0 : s1 + (int64_t)(kb - kbsplit) * sl1; };
      tile_mma<TL, KC, RC, true>(acc, K, fa, fb, fas, fbs, lds, sc, active, tt.rows, pfb, ncols);
    }
  }
  if (!done) {
    const uint16_t* abase = shared ? p.a_s : p.a_r;
    auto fa = [&](int r) { return abase + (arow0 + min(r, last)) * K; };
    // per-tile base rows of the two weight parts, so the loaders only add row offsets
    const uint8_t* b0 = shared ? p.s0.row(0, 0) : p.w0.row(e, 0);
    const uint8_t* b1 = shared ? p.s1.row(0, 0) : p.w1.row(e, 0);
    const int64_t ld0 = shared ? p.s0.ld_bytes : p.w0.ld_bytes;
    const int64_t ld1 = shared ? p.s1.ld_bytes : p.w1.ld_bytes;
    if constexpr (BMODE == KC) {
      auto fb = [&](int q) { return b0 + (int64_t)(n0 + min(q, nlast)) * ld0; };
      tile_mma<TL, KC, KC, false>(acc, K, fa, fb, NoScale{}, NoScale{}, lds, sc, active, tt.rows, pfb);
    } else {
      auto fb = [&](int q) {
        return ((q < ksplit) ? b0 + (int64_t)q * ld0 : b1 + (int64_t)(q - ksplit) * ld1) + 2 * n0;
      };
      tile_mma<TL, KC, RC, false>(acc, K, fa, fb, NoScale{}, NoScale{}, lds, sc, active, tt.rows, pfb, ncols);
    }
  }

  const int64_t crow0 = shared ? p.t.shared_row0 + tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int N = p.N;
  tok_epilogue<TL, false>(acc, lds, tt.rows, ncols, [&](int row, int col, const float* v) {
    *reinterpret_cast<uint4*>(p.c + (crow0 + row) * N + n0 + col) =
        make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
  });
}

// Data gradient of FC2 fused with the SwiGLU backward: gh = dyw W2 (contracting over H,
// W2 [H][I] row-contiguous), then with the saved a, b:
//   da = gh * b * silu'(a),  db = gh * silu(a)  -> dfc1 [rows][2I] (da at j, db at I + j)
//   (with the clamp: a and b clamped first, and zero gradient through a clamped input;
//   the forward stored each clamped input as +-infinity).
// MX: routed tiles take E4M3 dyw and the columnwise E4M3 copy of W2.
struct DgradSwigluArgs {
  TokArgs t;
  const uint16_t* a_r;   // routed dyw rows [S][H]
  const uint16_t* a_s;   // shared dy rows [T][H]
  MatRef wd, sd;
  MxOperands mx;         // b0 = columnwise W2
  const uint16_t* ab;
  uint16_t* dfc1;
  uint8_t* dfq;  // MXFP8 routed tiles: E4M3 codes [rows][2I] and E8M0 scales [rows][2I/32] of the
  uint8_t* dfs;  // BF16 dfc1 just stored (blocks of 32 along 2I), the FC1 data-gradient input
  int H, I;
  float limit;   // SwiGLU clamp limit (0: none); no gradient flows through a clamped input,
                 // which the forward stored as +-infinity
};

template <bool MX, bool WIDE = false>
__global__ __launch_bounds__((ShapesOf<MX, WIDE>::DG2::NTH), (ShapesOf<MX, WIDE>::DG2::MINB)) void k_dgrad_swiglu(
    DgradSwigluArgs p) {
  using TL = typename ShapesOf<MX, WIDE>::DG2;
  constexpr int XTRA = MX ? 4 * (kMaxExperts + 2) : 0;   // BF16: the map scratch in the second A stage
  __shared__ __align__(16) uint8_t lds[TL::LDS + (TL::PF ? 256 : 0) + (MX ? TL::SC_LDS : 0) + XTRA];
  uint8_t* pfb = lds + TL::LDS;
  uint8_t* sc = pfb + (TL::PF ? 256 : 0);
  int* sp = reinterpret_cast<int*>(MX ? sc + (MX ? TL::SC_LDS : 0) : lds + TL::A_BYTES);
  const TokTile tt = map_tok_tile<TL::TM>(p.t.tile_prefix, p.t.groups, (p.I + TL::TN - 1) / TL::TN, p.t.E, p.t.counts,
                                          p.t.T, sp);
  if (!tt.ok) return;
  const bool shared = tt.g == p.t.E;
  const int e = shared ? 0 : tt.g;
  const int64_t arow0 = shared ? tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const int H = p.H, I = p.I, last = tt.rows - 1;
  const int n0 = tt.nt * TL::TN;
  const int ncols = min(TL::TN, I - n0);   // the last N tile may be partial (a multiple of 128)
  const int wm = wave_m<TL>();
  Acc<TL> acc;
  zero_acc<TL>(acc);
  const bool active = wm * TL::WMR < tt.rows;
  bool done = false;
  if constexpr (MX) if (!shared) {
    done = true;
    auto fa = [&](int r) { return p.mx.aq + (arow0 + min(r, last)) * H; };
    auto fas = [&](int r) { return p.mx.as + (arow0 + min(r, last)) * (H / 32); };
    const uint8_t* d0 = p.mx.b0.data.row(e, 0) + n0;     // per-tile bases
    const uint8_t* s0 = p.mx.b0.scale.row(e, 0) + n0;
    const int64_t dl = p.mx.b0.data.ld_bytes, sl = p.mx.b0.scale.ld_bytes;
    auto fb = [&](int k) { return d0 + (int64_t)k * dl; };
    auto fbs = [&](int kb) { return s0 + (int64_t)kb * sl; };
    tile_mma<TL, KC, RC, true>(acc, H, fa, fb, fas, fbs, lds, sc, active, tt.rows, pfb, ncols);
  }
  if (!done) {
    const uint16_t* abase = shared ? p.a_s : p.a_r;
    auto fa = [&](int r) { return abase + (arow0 + min(r, last)) * H; };
    const uint8_t* wb = shared ? p.sd.row(0, 0) : p.wd.row(e, 0);
    const int64_t wld = shared ? p.sd.ld_bytes : p.wd.ld_bytes;
    auto fb = [&](int k) { return wb + (int64_t)k * wld + 2 * n0; };
    tile_mma<TL, KC, RC, false>(acc, H, fa, fb, NoScale{}, NoScale{}, lds, sc, active, tt.rows, pfb, ncols);
  }

  const int64_t crow0 = shared ? p.t.shared_row0 + tt.m0 : (int64_t)p.t.offsets[tt.g] + tt.m0;
  const float L = p.limit;
  auto epilogue = [&](auto clamp) __attribute__((always_inline)) {   // as in the FC1 kernel
    constexpr bool CL = decltype(clamp)::value;
    tok_epilogue<TL, false>(acc, lds, tt.rows, ncols, [&](int row, int col, const float* gv) {
      const int n = n0 + col;
      const int64_t R = (crow0 + row) * 2 * (int64_t)I;
      float av[8], bv[8];
      unpack_bf16x8(*reinterpret_cast<const uint4*>(p.ab + R + n), av);   // the stored BF16 a, b
      unpack_bf16x8(*reinterpret_cast<const uint4*>(p.ab + R + I + n), bv);
      float da[8], db[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float a = av[k], b = bv[k], gh = gv[k];
        // the forward's clamp decisions: a clamped input was stored as +-infinity
        const bool a_hi = CL && a == __builtin_inff();
        const bool b_out = CL && __builtin_isinf(b);
        const float ac = a_hi ? L : a;
        const float bc = b_out ? copysignf(L, b) : b;
        const float sg = sigmoidf_(ac);
        da[k] = a_hi ? 0.0f : gh * bc * (sg * (1.0f + ac * (1.0f - sg)));
        db[k] = b_out ? 0.0f : gh * (ac * sg);
      }
      const uint4 dav = make_uint4(pack_bf2(da[0], da[1]), pack_bf2(da[2], da[3]), pack_bf2(da[4], da[5]),
                                   pack_bf2(da[6], da[7]));
      const uint4 dbv = make_uint4(pack_bf2(db[0], db[1]), pack_bf2(db[2], db[3]), pack_bf2(db[4], db[5]),
                                   pack_bf2(db[6], db[7]));
      *reinterpret_cast<uint4*>(p.dfc1 + R + n) = dav;
      *reinterpret_cast<uint4*>(p.dfc1 + R + I + n) = dbv;
      if constexpr (MX) {
        if (!shared) {   // the routed FC1 data-gradient input: MXFP8 codes of the BF16 da and db
                         // (the 4 lanes holding one 32-column block are adjacent)
          float fa[8], fb[8];
          unpack_bf16x8(dav, fa);
          unpack_bf16x8(dbv, fb);
          uint2 qa, qb;
          const uint32_t sa = mx_quantize8(fa, quad_max(absmax8(fa)), qa);
          const uint32_t sb = mx_quantize8(fb, quad_max(absmax8(fb)), qb);
          *reinterpret_cast<uint2*>(p.dfq + R + n) = qa;
          *reinterpret_cast<uint2*>(p.dfq + R + I + n) = qb;
          if ((n & 31) == 0) {
            p.dfs[R / 32 + n / 32] = (uint8_t)sa;
            p.dfs[R / 32 + (I + n) / 32] = (uint8_t)sb;
          }
        }
      }
    });
  };
  if (L > 0.0f) epilogue(std::true_type{});
  else epilogue(std::false_type{});
}

// ---------------------------------------------------------------------------------
// Weight gradients: main_grad[e] (M x N, FP32) += A^T B over the expert's token rows
// (both operands row-contiguous along M / N; K = the group's tokens).  M is made of
// `parts` row ranges of `mpart` rows each (FC1: gate then up, FC2: one part), each
// tiled by TM with a masked tail, so no tile straddles two main_grad buffers.  Each
// output tile has exactly one owner: it runs the full token loop and then adds its
// result to main_grad once (no split-K, no atomics).
// Shared-expert tiles (when has_shared) come first in launch order (their K is all T
// tokens); routed tiles follow, chunked per XCD like the token-dim GEMMs.
// ---------------------------------------------------------------------------------
struct WgradArgs {
  const int32_t* counts;
  const int32_t* offsets;
  int T, E, has_shared;
  const uint16_t* a_r; const uint16_t* a_s; int64_t lda; int64_t a_s_row0;
  const uint16_t* b_r; const uint16_t* b_s; int64_t ldb; int64_t b_s_row0;
  const int32_t* b_map;   // routed B row k of the group = b_r row b_map[offsets[g] + k]
                          //   (null: row offsets[g] + k)
  GradRef g_lo, g_hi, s_lo, s_hi;   // part 0 -> *_lo, part 1 -> *_hi
  int parts, mpart;                 // M = parts * mpart; A column of part p row m: p * mpart + m
  int N;
};

template <bool MG16, bool SHORT>
__host__ __device__ inline int wgrad_tiles_per_group(int parts, int mpart, int N) {
  using TL = TL_WG<MG16, SHORT>;
  return parts * ((mpart + TL::TM - 1) / TL::TM) * ((N + TL::TN - 1) / TL::TN);
}

// FC is 1 or 2 (which projection's gradient); it only names the kernel symbol apart.
// MG16: BF16 main_grad (the contribution is rounded to BF16, then added with one BF16
// rounding), else FP32.
template <int FC, bool MG16, bool SHORT>
__global__ __launch_bounds__((TL_WG<MG16, SHORT>::NTH), (TL_WG<MG16, SHORT>::MINB)) void k_wgrad(WgradArgs p) {
  using TL = TL_WG<MG16, SHORT>;
  __shared__ __align__(16) uint8_t lds[TL::LDS];
  __shared__ __align__(16) uint8_t pfb[TL::PF ? 256 : 4];
  __shared__ __align__(16) int32_t bmap_lds[FC == 1 ? 64 * (2 * TL::NS - 2) : 4];   // the map ring
  const int mtp = (p.mpart + TL::TM - 1) / TL::TM, ntn = (p.N + TL::TN - 1) / TL::TN;
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
  const int m0 = mt * TL::TM, n0 = nt * TL::TN;
  const int ncols = min(TL::TN, p.N - n0);   // the last N tile may be partial (a multiple of 128)
  const int mrows = min(TL::TM, p.mpart - m0);
  const int64_t ar0 = shared ? p.a_s_row0 : (int64_t)p.offsets[g];
  const int64_t br0 = shared ? p.b_s_row0 : (int64_t)p.offsets[g];
  const uint16_t* A = (shared ? p.a_s : p.a_r) + (int64_t)part * p.mpart + m0;
  const int64_t lda = p.lda, ldb = p.ldb;
  const int32_t* bmap = (!shared && p.b_map) ? p.b_map + br0 : nullptr;
  const uint16_t* B = (shared ? p.b_s : p.b_r) + n0 + (bmap ? 0 : br0 * ldb);
  auto fa = [&](int k) { return A + (ar0 + k) * lda; };
  auto fb = [&](int row) { return B + (int64_t)row * ldb; };

  constexpr int ES = MG16 ? 2 : 4;   // main_grad element bytes
  const GradRef& G = part == 0 ? (shared ? p.s_lo : p.g_lo) : (shared ? p.s_hi : p.g_hi);
  uint8_t* cb = G.row<ES>(e, m0) + (int64_t)n0 * ES;
  const int64_t ldc = G.ld * ES;   // bytes

  const int lane = threadIdx.x & 63, wm = wave_m<TL>(), wn = wave_n<TL>();
  Acc<TL> acc;
  zero_acc<TL>(acc);
  const bool active = wm * TL::WMR < mrows;
  tile_mma<TL, RC, RC, false, FC == 1>(acc, kdim, fa, fb, NoScale{}, NoScale{}, lds, nullptr, active, mrows, pfb,
                                        ncols, bmap, bmap_lds);

  // main_grad += acc, one slice of SR rows per round: the waves of the wave row holding
  // them park those accumulators in LDS, then every thread adds pieces of 4 elements of
  // whole rows to main_grad (coalesced row reads and writes).  The main_grad loads of a
  // round are issued before its LDS traffic.  main_grad is read and written once per
  // step, so its loads and stores are non-temporal: the stream does not evict the token
  // operands that neighbouring tiles re-read from L2.  LDS slice [SR][TN] fp32; 16-byte
  // chunk c of row r sits at c ^ 8 ((r >> 2) & 1), so the two row groups a wave writes at
  // once use disjoint banks.
  constexpr int CPRW = TL::TN / 4;                       // 16-byte chunks per row
  // rows per round: a wave row, or (when its slice does not fit the LDS) the largest
  // multiple of 32 rows that does
  constexpr int SR = (TL::WMR * TL::TN * 4 <= TL::LDS) ? TL::WMR : 32 * (TL::LDS / (32 * TL::TN * 4));
  constexpr int NR = TL::TM / SR;                        // rounds
  constexpr int CPT = SR * CPRW / TL::NTH;               // chunks per thread per round
  static_assert(SR >= 32 && TL::WMR % SR == 0 && (SR * CPRW) % TL::NTH == 0, "epilogue slice");
  float* ct = reinterpret_cast<float*>(lds);
  const int t = threadIdx.x;
  auto sw = [](int r) { return ((r >> 2) & 1) << 3; };
#pragma unroll
  for (int q = 0; q < NR; ++q) {
    const int r0 = q * SR;                               // first tile row of the round
    const int rd = r0 / TL::WMR, ib = (r0 % TL::WMR) / 32;   // its wave row and first 32-row block
    f32x4_t mg[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = u * TL::NTH + t, row = c / CPRW, cc = c % CPRW;
      const int grow = r0 + row;
      const uint8_t* src = cb + grow * ldc + cc * 4 * ES;
      const bool in = grow < mrows && 4 * cc < ncols;
      if constexpr (MG16) {
        const u32x2_t v = in ? __builtin_nontemporal_load(((const glb_u32x2*)(src))) : u32x2_t{};
        mg[u] = f32x4_t{lo_bf(v[0]), hi_bf(v[0]), lo_bf(v[1]), hi_bf(v[1])};
      } else {
        mg[u] = in ? __builtin_nontemporal_load(((const glb_f32x4*)(src))) : f32x4_t{};
      }
    }
    __syncthreads();   // the LDS slice is free (K loop or previous round done)
    if (wm == rd) {
#pragma unroll
      for (int i = 0; i < TL::MI; ++i) {
        if (i < ib || i >= ib + SR / 32) continue;
#pragma unroll
        for (int j = 0; j < TL::NJ; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = (i - ib) * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            const int col = acc_col<TL>(wn, j, lane);
            ct[row * TL::TN + (((col >> 2) ^ sw(row)) << 2) + (col & 3)] = acc[i][j][r];
          }
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = u * TL::NTH + t, row = c / CPRW, cc = c % CPRW;
      const int grow = r0 + row;
      if (grow < mrows && 4 * cc < ncols) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(ct + row * TL::TN + ((cc ^ sw(row)) << 2));
        uint8_t* dst = cb + grow * ldc + cc * 4 * ES;
        if constexpr (MG16) {
          // contribution rounded to BF16, then main_grad + it rounded to BF16 (the float
          // sum of two BF16 values rounds to the same BF16 as their exact sum)
          f32x4_t r;
#pragma unroll
          for (int k = 0; k < 4; ++k) r[k] = mg[u][k] + bf2f(f2bf(v[k]));
          __builtin_nontemporal_store(u32x2_t{pack_bf2(r[0], r[1]), pack_bf2(r[2], r[3])}, ((glb_u32x2*)(dst)));
        } else {
          __builtin_nontemporal_store(mg[u] + v, ((glb_f32x4*)(dst)));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Launchers, defined in translation units of their own (gemm_tok.hip: the token-dimension
// GEMMs; gemm_wgrad.hip: the weight gradients), so that each family can take its own
// instruction-scheduling strategy.
// ---------------------------------------------------------------------------------
template <bool MX, bool WIDE>
void launch_fc1(dim3 grid, hipStream_t st, const Fc1Args& a);
template <int BMODE, bool MX, bool WIDE>
void launch_plain(dim3 grid, hipStream_t st, const PlainArgs& a);
template <bool MX, bool WIDE>
void launch_dgrad_swiglu(dim3 grid, hipStream_t st, const DgradSwigluArgs& a);
template <int FC, bool MG16, bool SHORT>
void launch_wgrad(dim3 grid, hipStream_t st, const WgradArgs& a);

}  // namespace gemm
}  // namespace moe
