// LDS-DMA main kernel with full-line A rows (gfx950).
//
// The same tile as dma_kernel.hpp (one workgroup per 256 x 256 tile, 32-k
// steps, MFMA 32x32x16, counted waits and raw barriers), with two changes:
// how A reaches LDS, and a ping-pong schedule of the two wave groups.  There, a 32-k step of a
// K-contiguous A row is 64 bytes, so each global_load_lds_dwordx4 touches
// sixteen half-used 128-byte lines, and the load path's cost follows the
// number of lines touched rather than the bytes moved.  Here A is staged 64 k
// at a time in 128-byte LDS rows ("super-steps"): one DMA instruction covers
// eight whole lines, half as many per byte.
//
// LDS: three A super-slots of 256 x 64 (32 KiB each) and four B stages of
// 32 x 256 (16 KiB each), 160 KiB in all.  In k-step t = 2u + h a wave
// issues half h of A super-step u + 2 and all of its B k-step t + 3, so
// every step issues the same four instructions and "all but this step's" is
// one fixed vmcnt.
//
// Schedule: the two halves of the workgroup (one wave of each per SIMD)
// alternate between a memory phase (LDS fragment reads, DMA issue) and a
// compute phase (MFMAs), one phase apart, so the matrix core of a SIMD is fed
// by one wave while the other loads.  Phases end at workgroup barriers; the
// loop states which barrier frees or publishes which slot.
//
// A slot layout: row r at r * 128 bytes; its octet c (k 8c .. 8c+7 of the
// super-step) in 16-byte slot c ^ f8(r), with f8(r) = (r ^ (r >> 3)) & 7, so
// that 8 consecutive rows, and 16 consecutive rows of one parity, reading
// the same octet hit distinct 16-byte bank groups.
//
// A ragged remainder of fewer than 64 k (an odd number of full 32-k steps
// and/or a K tail) is filled by masked register loads with zero fill after
// the pipelined loop.
//
// C leaves through the LDS, free after the last step: rounded to the output
// format, staged per wave and read back row by row, so that each store
// instruction writes whole 256-byte rows (store_tile_staged).  Split
// launches write their fp32 partials straight from the accumulators.
//
// Issue economy: a wave's memory phase is short of issue slots, not of
// bandwidth, so the loop keeps its bookkeeping cheap.  LDS slot indices
// rotate in 32-bit scalar registers, and the DMA uses the SGPR-base form of
// global_load_lds_dwordx4 (a uniform 64-bit base advanced once per step, a
// fixed 32-bit offset per lane), which takes no per-instruction 64-bit vector
// adds.  Lane offsets span at most 255 rows of an operand, so the host sends
// operands whose row stride exceeds 2^23 elements to another tile.
#pragma once

#include <type_traits>

#include "dma_kernel.hpp"

namespace gemmf16 {

template <int WAVES_M_ = 4, int WAVES_N_ = 2>
struct DmaA128Cfg {
  static constexpr int BM = 256, BN = 256, BK = 32;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, NW = WAVES_M * WAVES_N;
  static constexpr int NT = 64 * NW;
  static constexpr int MI = 32, KI = 16, KS = BK / KI;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_SLOT = BM * 64 * 2, A_SLOTS = 3;     // 32 KiB per 64-k super-step
  static constexpr int B_STAGE = BN * BK * 2, B_STAGES = 4;   // 16 KiB per 32-k step
  static constexpr int B_BASE = A_SLOTS * A_SLOT;
  static constexpr int LDS = B_BASE + B_STAGES * B_STAGE;
  static constexpr int DMA_A = A_SLOT / 1024 / NW;            // per wave per super-step
  static constexpr int DMA_B = B_STAGE / 1024 / NW;           // per wave per step
  static constexpr int DMA_PER_STEP = DMA_A / 2 + DMA_B;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert((DMA_A == 4 || DMA_A == 8) && DMA_A * NW * 1024 == A_SLOT, "DMA split (A)");
  static_assert(DMA_B * NW * 1024 == B_STAGE, "DMA split (B)");
  static_assert(FN * FM >= 4, "DMA placement");
};

__device__ __forceinline__ int f8(int r) { return (r ^ (r >> 3)) & 7; }

// global_load_lds_dwordx4 in its SGPR-base form: a uniform 64-bit base and a
// 32-bit per-lane byte offset, so a step's DMA needs no 64-bit VALU address
// arithmetic.  As in dma16_batch, the instruction offset (1024 j for the j-th
// instruction of a batch) is added to both addresses; the per-lane offsets
// carry the matching -1024 j.
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(((uint64_t)hi << 32) | lo);
}

template <int NI>
__device__ __forceinline__ void dma16s_batch(const uint32_t* off, const char* base, uint32_t lds) {
  static_assert(NI == 2 || NI == 4, "batch size");
  if constexpr (NI == 4) {
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %5\n\t"
        "global_load_lds_dwordx4 %2, %5 offset:1024\n\t"
        "global_load_lds_dwordx4 %3, %5 offset:2048\n\t"
        "global_load_lds_dwordx4 %4, %5 offset:3072"
        :
        : "s"(lds), "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(base)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %3\n\t"
        "global_load_lds_dwordx4 %2, %3 offset:1024"
        :
        : "s"(lds), "v"(off[0]), "v"(off[1]), "s"(base)
        : "memory", "m0");
  }
}

// Bytes below a source's base that its offsets start from, so that the
// biased offsets (down to -3072) stay non-negative.
constexpr int kSBias = 4096;

// Per-lane sources of this wave's NI A instructions of a super-step:
// instruction i covers rows (NI w + i) * 8 .. +8; lane l -> row +l/8, 16-byte
// slot l%8 -> octet (l%8) ^ f8(row).  Rows past M read the last valid row.
template <int NI>
struct ASourceS {
  const char* base;  // byte address of (row r0, k kb) less kSBias
  uint32_t off[NI];
  int64_t step;      // bytes per 64-k super-step

  __device__ __forceinline__ void init(const uint16_t* A, int64_t s_r, int64_t s_k, int64_t R_tot,
                                       int64_t r0, int64_t kb, int wave, int lane) {
    base = uniform_ptr((const char*)(A + r0 * s_r + kb * s_k) - kSBias);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (NI * wave + i) * 8 + lane / 8;
      const int c = (lane % 8) ^ f8(r);
      int64_t rr = r0 + r;
      if (rr > R_tot - 1) rr = R_tot - 1;
      off[i] = (uint32_t)(((rr - r0) * s_r + 8 * c * s_k) * 2 + kSBias - 1024 * (i % (NI / 2)));
    }
    step = (int64_t)128 * s_k;
  }
  template <int H>
  __device__ __forceinline__ void issue_half(uint32_t lds, int64_t u) {
    dma16s_batch<NI / 2>(&off[H * (NI / 2)], base + u * step, lds);
  }
  // Same, from a super-step base the caller advances (base + u * step).
  template <int H>
  __device__ __forceinline__ void issue_half_at(uint32_t lds, const char* b) {
    dma16s_batch<NI / 2>(&off[H * (NI / 2)], b, lds);
  }
  __device__ __forceinline__ const uint16_t* ptr(int i, int64_t u) const {
    return (const uint16_t*)(base + u * step + off[i] + 1024 * (i % (NI / 2)));
  }
  __device__ __forceinline__ void fill_masked(char* slot, int wave, int lane, int64_t u, int64_t kb,
                                              int64_t k_end, int64_t s_k) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (NI * wave + i) * 8 + lane / 8;
      const int c = (lane % 8) ^ f8(r);
      const int64_t kk = kb + u * 64 + 8 * c;
      const int64_t d = k_end - kk;
      const int nk = d < 0 ? 0 : (d < 8 ? (int)d : 8);
      const u32x4 v = load_partial8(ptr(i, nk > 0 ? u : 0), s_k, nk);
      *reinterpret_cast<u32x4*>(slot + (NI * wave + i) * 1024 + lane * 16) = v;
    }
  }
};

// DmaSource in SGPR-base form (same rows, slots and clamping).
template <int NI, bool KMAJOR>
struct BSourceS {
  const char* base;  // byte address of (row r0, k kb) less kSBias
  uint32_t off[NI];
  int64_t step;      // bytes per 32-k step

  __device__ __forceinline__ void init(const uint16_t* B, int64_t s_r, int64_t s_k, int64_t R_tot,
                                       int64_t r0, int64_t kb, int wave, int lane) {
    base = uniform_ptr((const char*)(B + r0 * s_r + kb * s_k) - kSBias);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      int64_t e;
      if constexpr (KMAJOR) {
        const int r = (NI * wave + i) * 16 + lane / 4;
        const int c = (lane % 4) ^ fa(r);
        int64_t rr = r0 + r;
        if (rr > R_tot - 1) rr = R_tot - 1;
        e = (rr - r0) * s_r + 8 * c * s_k;
      } else {
        const int k = (NI * wave + i) * 2 + lane / 32;
        const int slot = lane % 32;
        const int b = (slot / 2) ^ hb(k);
        int64_t n = r0 + b * 16 + (slot % 2) * 8;
        if (n > R_tot - 8) n = R_tot - 8;
        e = (n - r0) * s_r + k * s_k;
      }
      off[i] = (uint32_t)(e * 2 + kSBias - 1024 * i);
    }
    step = (int64_t)64 * s_k;
  }
  __device__ __forceinline__ void issue_batch(uint32_t lds_wave, int64_t t) {
    dma16s_batch<NI>(off, base + t * step, lds_wave);
  }
  // Same, from a step base the caller advances (base + t * step).
  __device__ __forceinline__ void issue_batch_at(uint32_t lds_wave, const char* b) {
    dma16s_batch<NI>(off, b, lds_wave);
  }
  __device__ __forceinline__ void fill_masked(char* lds_op, int wave, int lane, int64_t t,
                                              int64_t kb, int64_t k_end, int64_t s_k) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint16_t* q = (const uint16_t*)(base + t * step + off[i] + 1024 * i);
      u32x4 v;
      if constexpr (KMAJOR) {
        const int r = (NI * wave + i) * 16 + lane / 4;
        const int c = (lane % 4) ^ fa(r);
        const int64_t kk = kb + t * 32 + 8 * c;
        const int64_t d = k_end - kk;
        const int nk = d < 0 ? 0 : (d < 8 ? (int)d : 8);
        v = load_partial8(q, s_k, nk);
      } else {
        const int k = (NI * wave + i) * 2 + lane / 32;
        const bool ok = kb + t * 32 + k < k_end;
        v = ok ? *reinterpret_cast<const u32x4*>(q) : zero4();
      }
      *reinterpret_cast<u32x4*>(lds_op + (NI * wave + i) * 1024 + lane * 16) = v;
    }
  }
};

// B pre-packed into the LDS image of its K-major stages (see
// gemm_f16_pack_b): 256-column panels of ceil(K/32) 16 KiB blocks, zero
// padded past N and K, so every DMA instruction reads 1 KiB of consecutive
// bytes and the K tail needs no masks.  s_r is the panel stride in elements.
template <int NI>
struct PackedBSource {
  const char* base;  // byte address of this tile's first block less kSBias
  uint32_t off[NI];  // all equal: 1 KiB per instruction is the batch offset
  static constexpr int64_t step = 16384;  // bytes per 32-k block

  __device__ __forceinline__ void init(const uint16_t* B, int64_t s_r, int64_t, int64_t,
                                       int64_t r0, int64_t kb, int wave, int lane) {
    base = uniform_ptr((const char*)(B + (r0 / 256) * s_r + (kb / 32) * 8192) - kSBias);
#pragma unroll
    for (int i = 0; i < NI; ++i) off[i] = (uint32_t)(NI * wave * 1024 + lane * 16 + kSBias);
  }

  __device__ __forceinline__ void issue_batch(uint32_t lds_wave, int64_t t) {
    dma16s_batch<NI>(off, base + t * step, lds_wave);
  }
  __device__ __forceinline__ void issue_batch_at(uint32_t lds_wave, const char* b) {
    dma16s_batch<NI>(off, b, lds_wave);
  }

  // The block of step t as it lies (its K tail is already zero).
  __device__ __forceinline__ void fill_masked(char* lds_op, int wave, int lane, int64_t t, int64_t,
                                              int64_t, int64_t) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      *reinterpret_cast<u32x4*>(lds_op + (NI * wave + i) * 1024 + lane * 16) =
          *reinterpret_cast<const u32x4*>(base + t * step + off[i] + 1024 * i);
  }
};

// One fragment of k-substep ks of the 32-k step in half H of a super-step:
// piece q < FM is A fragment q, piece FM + i is B fragment i.  B stages are
// laid out as in dma_kernel.hpp: N-major 512-byte k-rows, or, for a
// K-contiguous B (BKMAJOR), 64-byte n-rows like its A tiles.
template <class CF, int H, bool BKMAJOR>
__device__ __forceinline__ void read_piece_a128(DmaFrags<CF>& f, const char* ta, const char* tb,
                                                int ks, int wm, int wn, int lane, int q) {
  const int lr = lane % 32, lo = lane / 32;
  if (q < CF::FM) {
    const int c = 4 * H + 2 * ks + lo;
    const int r = wm * CF::WTM + q * 32 + lr;
    f.fb_[q] = *reinterpret_cast<const f16x8*>(ta + r * 128 + ((c ^ f8(r)) * 16));
  } else if constexpr (BKMAJOR) {
    const int cb = ks * 2 + lo;
    const int r = wn * CF::WTN + (q - CF::FM) * 32 + lr;
    f.fa_[q - CF::FM] = *reinterpret_cast<const f16x8*>(tb + r * 64 + ((cb ^ fa(r)) * 16));
  } else {
    const int g = lane / 16, s = lane % 16;
    const int kr = ks * 16 + 8 * (g / 2) + s / 4;
    const int n = wn * CF::WTN + (q - CF::FM) * 32 + 16 * (g % 2);
    const char* p0 = tb + kr * 512 + (((n >> 4) ^ hb(kr)) * 32) + 8 * (s % 4);
    f.fa_[q - CF::FM] = read_tr_pair(p0, p0 + 4 * 512);
  }
}

template <class CF, int H, bool BKMAJOR>
__device__ __forceinline__ void read_frags_a128(DmaFrags<CF>& f, const char* ta, const char* tb,
                                                int ks, int wm, int wn, int lane) {
#pragma unroll
  for (int q = 0; q < CF::FM + CF::FN; ++q) read_piece_a128<CF, H, BKMAJOR>(f, ta, tb, ks, wm, wn, lane, q);
}

// The MFMAs of `cur` with the reads of `nxt` (k-substep ks, super-step half
// H) placed one fragment after each of MFMAs 1 .. FM + FN, so the reads
// issue in the shadow of matrix work.  The first MFMA goes alone: with the
// reads one MFMA later the 131072 x 2048 x 7168 product ran 0.3-2.7% faster
// on three machines and 8192^3 moved -0.6 to +1.6% (same bits).  `nxt` may
// be the registers of a fragment set consumed earlier in program order.
// EDGE: a wave of an edge tile skips the MFMAs of the 32 x 32 blocks i >= fnv
// or j >= fmv, whose outputs are never stored (the kernel skips only blocks
// wholly past M: fnv = FN, see there).  fnv and fmv are uniform over the wave.
template <class CF, int H, bool BKMAJOR, int DT, bool EDGE>
__device__ __forceinline__ void mma_and_read(const DmaFrags<CF>& cur, DmaFrags<CF>& nxt,
                                             f32x16 (&acc)[CF::FN][CF::FM], const char* ta,
                                             const char* tb, int ks, int wm, int wn, int lane,
                                             int fnv, int fmv) {
  static_assert(CF::FM + CF::FN < CF::FN * CF::FM, "one read per MFMA at most");
#pragma unroll
  for (int q = 0; q < CF::FN * CF::FM; ++q) {
    const int i = q / CF::FM, j = q % CF::FM;
    if (!EDGE || (i < fnv && j < fmv)) acc[i][j] = mfma<32, DT>(cur.fa_[i], cur.fb_[j], acc[i][j]);
    if (q >= 1 && q <= CF::FM + CF::FN) read_piece_a128<CF, H, BKMAJOR>(nxt, ta, tb, ks, wm, wn, lane, q - 1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// MFMAs Q0 .. Q1-1 (in the order q = i FM + j) of the fragments f.
template <class CF, int DT, bool EDGE, int Q0 = 0, int Q1 = CF::FN * CF::FM>
__device__ __forceinline__ void mma_frags_a128(const DmaFrags<CF>& f, f32x16 (&acc)[CF::FN][CF::FM],
                                               int fnv, int fmv) {
#pragma unroll
  for (int q = Q0; q < Q1; ++q) {
    const int i = q / CF::FM, j = q % CF::FM;
    if (!EDGE || (i < fnv && j < fmv)) acc[i][j] = mfma<32, DT>(f.fa_[i], f.fb_[j], acc[i][j]);
  }
}

// Exchange of lanes 32..63 of x with lanes 0..31 of y (v_permlane32_swap).
__device__ __forceinline__ void swap_lane_halves(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}

template <int DT>
__device__ __forceinline__ uint32_t pack_out2(float lo, float hi) {
  return (uint32_t)cvt_out<DT>(lo) | ((uint32_t)cvt_out<DT>(hi) << 16);
}

// Eight consecutive outputs v (binary16 pairs, lowest column first) to dst,
// with the widest stores dst's alignment allows: one 16-byte store, two of
// 8, four of 4, or, 2 bytes past a 4-byte boundary, 2 + 3 x 4 + 2 bytes.
__device__ __forceinline__ void store8_any(uint16_t* dst, u32x4 v) {
  const uintptr_t ad = (uintptr_t)dst;
  if ((ad & 15u) == 0) {
    *reinterpret_cast<u32x4*>(dst) = v;
  } else if ((ad & 7u) == 0) {
    reinterpret_cast<u32x2*>(dst)[0] = u32x2{v[0], v[1]};
    reinterpret_cast<u32x2*>(dst)[1] = u32x2{v[2], v[3]};
  } else if ((ad & 3u) == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) reinterpret_cast<uint32_t*>(dst)[q] = v[q];
  } else {
    dst[0] = (uint16_t)v[0];
    uint32_t* d = reinterpret_cast<uint32_t*>(dst + 1);
#pragma unroll
    for (int q = 0; q < 3; ++q) d[q] = __builtin_amdgcn_alignbit(v[q + 1], v[q], 16);
    dst[7] = (uint16_t)(v[3] >> 16);
  }
}

// Output of a tile staged through LDS, so that each store instruction
// writes four whole rows of the wave's 64 x 128 block (256 bytes each) rather
// than 8 bytes into each of 32 rows.  Stored straight from the accumulators,
// the L1 and L2 take one request per row piece, and on 256 CUs finishing
// their tiles together that burst cost about 10 us per 256 x 256 tile (5%
// of the 131072 x 2048 x 7168 product); staged, it costs about half of that.
// Rows past M are not stored; nor are the columns past N of an 8-column chunk
// that crosses N.  With C 16-byte aligned and ldc % 8 == 0 every chunk is one
// 16-byte store; otherwise each chunk takes the widest stores its address
// allows (the 16 lanes of one row share that choice).
//
// In a 32 x 32 block lane l holds, per group g of 4 registers, columns
// 8 g + 4 (l / 32) .. + 3 of row l % 32.  Packed to binary16 pairs, one lane
// swap across the two wave halves gives lane l < 32 columns 16 p .. 16 p + 7
// of groups 2 p, 2 p + 1 and lane l + 32 columns 16 p + 8 .. 16 p + 15: one
// 16-byte chunk each.  A wave writes its chunks into its own 16 KiB of LDS
// (rows of 256 bytes, chunk c of row r at position c ^ (r % 16), so that
// both the writes of 32 rows and the reads of 4 whole rows fall on distinct
// banks) and reads them back row by row.  The caller has made the LDS free.
template <class CF, int DT>
__device__ __forceinline__ void store_tile_staged(const KArgs& a, const f32x16 (&acc)[CF::FN][CF::FM],
                                                  char* smem, int64_t m0, int64_t n0, int wave, int wm,
                                                  int wn, int lane) {
  static_assert(CF::WTN == 128, "16 chunks of 16 bytes per wave row");
  static_assert(CF::NW * CF::WTM * CF::WTN * 2 <= CF::LDS, "staging space");
  const int lr = lane % 32, h = lane >> 5;
  char* const stage = smem + wave * (CF::WTM * CF::WTN * 2);
#pragma unroll
  for (int i = 0; i < CF::FN; ++i)
#pragma unroll
    for (int j = 0; j < CF::FM; ++j)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        uint32_t x0 = pack_out2<DT>(acc[i][j][8 * p], acc[i][j][8 * p + 1]);
        uint32_t x1 = pack_out2<DT>(acc[i][j][8 * p + 2], acc[i][j][8 * p + 3]);
        uint32_t y0 = pack_out2<DT>(acc[i][j][8 * p + 4], acc[i][j][8 * p + 5]);
        uint32_t y1 = pack_out2<DT>(acc[i][j][8 * p + 6], acc[i][j][8 * p + 7]);
        swap_lane_halves(x0, y0);
        swap_lane_halves(x1, y1);
        const int r = j * 32 + lr, c = 4 * i + 2 * p + h;
        *reinterpret_cast<u32x4*>(stage + r * 256 + ((c ^ (r & 15)) << 4)) = u32x4{x0, x1, y0, y1};
      }
  uint16_t* const cw = a.C + (m0 + wm * CF::WTM) * a.ldc + n0 + wn * CF::WTN;
  // Rows and columns of this wave's block that lie inside C (clamped).
  const int64_t mr = a.M - (m0 + wm * CF::WTM), nc = a.N - (n0 + wn * CF::WTN);
  const int rows = mr < 0 ? 0 : (mr > CF::WTM ? CF::WTM : (int)mr);
  const int cols = nc < 0 ? 0 : (nc > CF::WTN ? CF::WTN : (int)nc);
  if (((uintptr_t)a.C & 15u) == 0 && (a.ldc & 7) == 0) {
#pragma unroll
    for (int it = 0; it < CF::WTM / 4; ++it) {
      const int r = 4 * it + lane / 16, c = lane % 16;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * 256 + ((c ^ (r & 15)) << 4));
      if (r < rows && 8 * c + 8 <= cols) *reinterpret_cast<u32x4*>(cw + (int64_t)r * a.ldc + c * 8) = v;
    }
  } else {
    for (int it = 0; it < CF::WTM / 4; ++it) {
      const int r = 4 * it + lane / 16, c = lane % 16;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * 256 + ((c ^ (r & 15)) << 4));
      const int nv = cols - 8 * c;
      uint16_t* const dst = cw + (int64_t)r * a.ldc + c * 8;
      if (r < rows && nv >= 8) {
        store8_any(dst, v);
      } else if (r < rows && nv > 0) {
#pragma unroll
        for (int e = 0; e < 7; ++e)
          if (e < nv) dst[e] = (uint16_t)(v[e / 2] >> (16 * (e % 2)));
      }
    }
  }
}

// fp32 partials of the wave's 64 x 128 block to base (its element (0, 0); row
// stride ld floats; rows x cols of it inside the target), staged through
// LDS in two passes of 32 rows so that each store instruction writes two
// whole 512-byte rows rather than 32 bytes into each of 32 rows.  In a
// 32 x 32 block lane l holds, per group g, the 4 floats of columns
// 8 g + 4 (l / 32) .. + 3 of row l % 32: one 16-byte chunk, chunk
// 8 i + 2 g + l / 32 of its 512-byte row, placed at c ^ (r % 32) (distinct
// banks for the 32 rows written and for the rows read back).  With ld % 4 == 0
// and a 16-byte aligned base every whole chunk is one 16-byte store; other
// chunks store element by element.  The caller has made the LDS free.
template <class CF>
__device__ __forceinline__ void store_partial_staged(float* base, int64_t ld, int rows, int cols,
                                                     const f32x16 (&acc)[CF::FN][CF::FM], char* smem,
                                                     int wave, int lane) {
  static_assert(CF::WTN == 128 && CF::WTM == 64, "32 chunks of 16 bytes per row, two passes");
  static_assert(CF::NW * 32 * CF::WTN * 4 <= CF::LDS, "staging space");
  float* const stage = reinterpret_cast<float*>(smem + wave * (32 * CF::WTN * 4));
  const int lr = lane % 32, h = lane >> 5;
  const bool vec = (ld & 3) == 0 && ((uintptr_t)base & 15u) == 0;
#pragma unroll
  for (int j = 0; j < CF::FM; ++j) {
#pragma unroll
    for (int i = 0; i < CF::FN; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 8 * i + 2 * g + h;
        *reinterpret_cast<f32x4*>(stage + lr * 128 + ((c ^ lr) << 2)) =
            f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
      }
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int r = 2 * it + lane / 32, c = lane % 32;
      const f32x4 v = *reinterpret_cast<const f32x4*>(stage + r * 128 + ((c ^ r) << 2));
      const int row = 32 * j + r, nv = cols - 4 * c;
      float* const dst = base + (int64_t)row * ld + 4 * c;
      if (row < rows && nv >= 4 && vec) {
        *reinterpret_cast<f32x4*>(dst) = v;
      } else if (row < rows && nv > 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < nv) dst[e] = v[e];
      }
    }
  }
}

// K-contiguous A; N-contiguous B, or K-contiguous B with BKMAJOR.
// BPACK: B comes pre-packed (PackedBSource; read as a K-major B).
template <class CF, bool BKMAJOR, bool PARTIAL, bool GROUPED = false, int DT = DT_F16,
          bool BPACK = false>
__global__ __launch_bounds__(CF::NT) void gemm_dma_a128_kernel(KArgs a) {
  static_assert(!BPACK || BKMAJOR, "packed B stages are K-major");
  static_assert(!(PARTIAL && GROUPED), "grouped launches are never split");
  __shared__ __attribute__((aligned(1024))) char smem[CF::LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;

  const int64_t T = a.GM * a.GN;
  int64_t w = blockIdx.x;
  int64_t split = 0;
  if constexpr (PARTIAL) {
    if (a.sk_tiles > 0) {            // stream-K tail: see KArgs
      split = w / a.sk_tiles;
      w = a.sk_first + (w - split * a.sk_tiles);
    } else {
      split_tile_of(blockIdx.x, T, a.split_xcd, split, w);
    }
  }
  int64_t pm, pn;
  if constexpr (GROUPED) {
    if (!group_tile(a, w, pm, pn)) return;   // uniform per workgroup, before any barrier
  } else {
    raster_tile(w, a.GM, a.GN, a.panel, pm, pn);
  }
  const int64_t m0 = pm * CF::BM, n0 = pn * CF::BN;
  const int64_t kb = split * a.k_split;
  const int64_t ke = (kb + a.k_split < a.K) ? kb + a.k_split : a.K;
  // 32-row blocks of this wave's sub-tile that hold any output (all of them
  // except in the last tile row).  Blocks past N are computed anyway: a tile
  // of the last column that skipped them would finish early, the tiles of its
  // row (which share their A panel in L2 while they run in step) would drift
  // apart, and A would be fetched again.  Computing them was 6.5% faster on
  // 262181 x 1061 x 8192 (37 live columns of 256 in the last tile column),
  // 8.4% on 131072 x 1061 x 7168 and 2.2% on 131072 x 2080 x 7168.
  const int64_t mrem = a.M - (m0 + wm * CF::WTM);
  const int fnv = CF::FN;
  const int fmv = mrem <= 0 ? 0 : (mrem >= CF::WTM ? CF::FM : (int)((mrem + 31) / 32));
  const bool edge = fmv < CF::FM;

  ASourceS<CF::DMA_A> sa;
  std::conditional_t<BPACK, PackedBSource<CF::DMA_B>, BSourceS<CF::DMA_B, BKMAJOR>> sb;
  sa.init(a.A, a.lda_m, a.lda_k, a.M, m0, kb, wave, lane);
  sb.init(a.B, a.ldb_n, a.ldb_k, a.N, n0, kb, wave, lane);

  f32x16 acc[CF::FN][CF::FM];
#pragma unroll
  for (int i = 0; i < CF::FN; ++i)
#pragma unroll
    for (int j = 0; j < CF::FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto slot_a = [&](int64_t u) { return smem + (int)(u % CF::A_SLOTS) * CF::A_SLOT; };
  auto stage_b = [&](int64_t t) { return smem + CF::B_BASE + (int)(t % CF::B_STAGES) * CF::B_STAGE; };
  auto lds_a = [&](int64_t u, int h) {
    return __builtin_amdgcn_readfirstlane(lds_addr(slot_a(u)) + (CF::DMA_A * wave + (CF::DMA_A / 2) * h) * 1024);
  };
  auto lds_b = [&](int64_t t) {
    return __builtin_amdgcn_readfirstlane(lds_addr(stage_b(t)) + CF::DMA_B * wave * 1024);
  };

  const int64_t nsup = (ke - kb) / 64;     // whole 64-k super-steps
  const int64_t nfull2 = 2 * nsup;         // 32-k steps they hold
  const int64_t rem = (ke - kb) - 64 * nsup;
  DmaFrags<CF> f0, f1;

  if (nsup > 0) {
    // Two groups of waves take turns on the matrix cores.  Waves w and
    // w + NW/2 share a SIMD; group 0 is waves 0 .. NW/2-1 (tile rows 0..127),
    // group 1 the rest.  Each 32-k step t of a group has a memory phase M(t)
    // (second k-substep fragments of step t, this wave's DMA of step t + 3)
    // and a compute phase C(t) (the 16 MFMAs of step t, with the first
    // k-substep fragments of step t + 1 read under the second eight).
    // Group 1 runs one phase behind group 0, so while one wave of a SIMD
    // issues MFMAs the other issues its loads.  Every phase ends at a
    // workgroup barrier; barrier b ends phase b - 1 of group 0 and phase
    // b - 2 of group 1 (group 1 passes barrier 1 before its first phase).
    //
    // Invariants (D = 3 steps of prefetch, 4 B stages, 3 A super-slots):
    //  - a wave's reads are complete when it leaves its memory phase
    //    (lgkmcnt 0), so what group 1 reads of step t, in C(t-1) and M(t),
    //    is free after barrier 2t + 2.  That barrier precedes group 0's
    //    M(t + 1), the first phase to issue a DMA into that B stage (step
    //    t + 4) or, when t ends a super-step, into that A super-slot;
    //  - a wave leaves C(t) with only M(t)'s DMA outstanding (vmcnt), so
    //    step t + 2 and its super-step have landed, for every wave, before
    //    barrier 2t + 3, which precedes the first read of them (group 0's
    //    C(t + 1)).
    const bool g1 = wave >= CF::NW / 2;
    const int64_t u1 = nsup > 1 ? 1 : 0;
    sa.template issue_half<0>(lds_a(0, 0), 0);
    sa.template issue_half<1>(lds_a(0, 1), 0);
    sb.issue_batch(lds_b(0), 0);
    sb.issue_batch(lds_b(1), 1);
    sa.template issue_half<0>(lds_a(1, 0), u1);
    sa.template issue_half<1>(lds_a(1, 1), u1);
    sb.issue_batch(lds_b(2), nfull2 > 2 ? 2 : nfull2 - 1);
    wait_vmcnt<CF::DMA_A + CF::DMA_B>();   // A(0), B(0) and B(1) landed
    wg_barrier();
    read_frags_a128<CF, 0, BKMAJOR>(f0, slot_a(0), stage_b(0), 0, wm, wn, lane);
    if (g1) wg_barrier();

    // One step: H is the step's half of its super-step u, whose A super-slot
    // is iu (i1, i2: those of u + 1 and u + 2); the DMA of step t + 3 carries
    // half H of super-step u + 2 (clamped to the last one).  Slot indices
    // rotate in 32-bit registers: a 64-bit modulo per step costs more issue
    // slots than the memory phase has to spare.
    const int ns = (int)nsup, nf2 = 2 * ns;
    auto sl_a = [&](int i) { return smem + i * CF::A_SLOT; };
    auto st_b = [&](int t) { return smem + CF::B_BASE + (t & (CF::B_STAGES - 1)) * CF::B_STAGE; };
    const uint32_t la0 = __builtin_amdgcn_readfirstlane(lds_addr(smem) + CF::DMA_A * wave * 1024);
    const uint32_t lb0 =
        __builtin_amdgcn_readfirstlane(lds_addr(smem) + CF::B_BASE + CF::DMA_B * wave * 1024);
    // DMA source bases of super-step u + 2 and step t + 3 (each clamped to
    // the last one), advanced in place rather than multiplied out.
    const char* pa = sa.base + (int64_t)(ns > 2 ? 2 : ns - 1) * sa.step;
    const char* pb = sb.base + (int64_t)(nf2 > 3 ? 3 : nf2 - 1) * sb.step;
    auto step = [&](auto h_tag, auto e_tag, int iu, int i1, int i2, int t) {
      constexpr int H = decltype(h_tag)::value;
      constexpr bool EDGE = decltype(e_tag)::value;
      // M(t)
      read_frags_a128<CF, H, BKMAJOR>(f1, sl_a(iu), st_b(t), 1, wm, wn, lane);
      sa.template issue_half_at<H>(la0 + i2 * CF::A_SLOT + (CF::DMA_A / 2) * H * 1024, pa);
      sb.issue_batch_at(lb0 + ((t + 3) & (CF::B_STAGES - 1)) * CF::B_STAGE, pb);
      if (t + 4 < nf2) pb += sb.step;
      wait_lgkmcnt0();
      __builtin_amdgcn_sched_barrier(0);
      // The first MFMA of C(t) goes ahead of the barrier (its operands are
      // registers already loaded; MFMAs touch no LDS), so the matrix core
      // has work queued across the hand-off: +2% on the 131072 x 2048 x 7168
      // product, unchanged on 8192^3.  Through C(t) the wave runs at raised
      // issue priority, so its MFMAs go first when the partner wave of its
      // SIMD (in its memory phase) is also ready: +2% on the same product.
      __builtin_amdgcn_s_setprio(1);
      mma_frags_a128<CF, DT, EDGE, 0, 1>(f0, acc, fnv, fmv);
      wg_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // C(t); the reads for step t + 1 fetch unused bytes of free slots on
      // the last step.
      mma_frags_a128<CF, DT, EDGE, 1>(f0, acc, fnv, fmv);
      __builtin_amdgcn_sched_barrier(0);
      mma_and_read<CF, 1 - H, BKMAJOR, DT, EDGE>(f1, f0, acc, sl_a(H ? i1 : iu), st_b(t + 1), 0,
                                                 wm, wn, lane, fnv, fmv);
      wait_vmcnt<CF::DMA_PER_STEP>();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      wg_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // Both loops pass the same barriers; the edge one skips empty blocks.
    auto run = [&](auto e_tag) {
      static_assert(CF::A_SLOTS == 3, "slot rotation");
      int iu = 0;
      for (int u = 0; u < ns; ++u) {
        const int i1 = iu == 2 ? 0 : iu + 1, i2 = iu == 0 ? 2 : iu - 1;
        step(std::integral_constant<int, 0>{}, e_tag, iu, i1, i2, 2 * u);
        step(std::integral_constant<int, 1>{}, e_tag, iu, i1, i2, 2 * u + 1);
        if (u + 3 < ns) pa += sa.step;
        iu = i1;
      }
    };
    if (edge)
      run(std::true_type{});
    else
      run(std::false_type{});
    if (!g1) wg_barrier();   // pairs with group 1's extra first barrier
    wait_vmcnt<0>();         // no LDS transfer may still be in flight past this point
  }
  if (rem > 0) {
    // Remainder (< 64 k): masked fill of A super-slot nsup and B stages of
    // steps nfull2 and nfull2 + 1, all free after the last barrier.
    sa.fill_masked(slot_a(nsup), wave, lane, nsup, kb, ke, a.lda_k);
    sb.fill_masked(stage_b(nfull2), wave, lane, nfull2, kb, ke, a.ldb_k);
    if (rem > 32) sb.fill_masked(stage_b(nfull2 + 1), wave, lane, nfull2 + 1, kb, ke, a.ldb_k);
    __syncthreads();
    read_frags_a128<CF, 0, BKMAJOR>(f0, slot_a(nsup), stage_b(nfull2), 0, wm, wn, lane);
    read_frags_a128<CF, 0, BKMAJOR>(f1, slot_a(nsup), stage_b(nfull2), 1, wm, wn, lane);
    mma_frags_a128<CF, DT, true>(f0, acc, fnv, fmv);
    mma_frags_a128<CF, DT, true>(f1, acc, fnv, fmv);
    if (rem > 32) {
      read_frags_a128<CF, 1, BKMAJOR>(f0, slot_a(nsup), stage_b(nfull2 + 1), 0, wm, wn, lane);
      read_frags_a128<CF, 1, BKMAJOR>(f1, slot_a(nsup), stage_b(nfull2 + 1), 1, wm, wn, lane);
      mma_frags_a128<CF, DT, true>(f0, acc, fnv, fmv);
      mma_frags_a128<CF, DT, true>(f1, acc, fnv, fmv);
    }
  }

  if constexpr (!PARTIAL) {
    wait_lgkmcnt0();   // this wave's last LDS reads have returned,
    wg_barrier();      // and every other wave's: the LDS is free
    store_tile_staged<CF, DT>(a, acc, smem, m0, n0, wave, wm, wn, lane);
  } else {
    // fp32 partials, staged through LDS: a stream-K tail tile to its dense
    // slot (the whole tile, edges included), a split K range to W[split].
    wait_lgkmcnt0();
    wg_barrier();
    if (a.sk_tiles > 0) {
      float* const slot = a.W + (int64_t)blockIdx.x * (CF::BM * CF::BN);
      store_partial_staged<CF>(slot + (wm * CF::WTM) * CF::BN + wn * CF::WTN, CF::BN, CF::WTM, CF::WTN,
                               acc, smem, wave, lane);
    } else {
      const int64_t mr = a.M - (m0 + wm * CF::WTM), nc = a.N - (n0 + wn * CF::WTN);
      const int rows = mr < 0 ? 0 : (mr > CF::WTM ? CF::WTM : (int)mr);
      const int cols = nc < 0 ? 0 : (nc > CF::WTN ? CF::WTN : (int)nc);
      store_partial_staged<CF>(a.W + (split * a.M + m0 + wm * CF::WTM) * a.N + n0 + wn * CF::WTN, a.N,
                               rows, cols, acc, smem, wave, lane);
    }
  }
}

}  // namespace gemmf16
