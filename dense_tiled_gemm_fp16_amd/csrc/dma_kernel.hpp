// The large-tile main kernel with direct global -> LDS loads (gfx950).
//
// Same method as tile_kernel.hpp -- one workgroup per BM x BN output tile,
// fp32 accumulation over K in BK steps, one store per output (Triton article,
// "parallelise over outputs, keep K in the accumulator") -- with a deeper
// software pipeline (TileLang tutorial ch. 14, rung 3; tiling tutorial,
// section 06) built from two gfx950 instructions:
//
//   global_load_lds_dwordx4  each lane moves 16 bytes from global memory
//                            straight into LDS at (wave base + 16 * lane): no
//                            staging registers, no LDS write instructions.
//   ds_read_b64_tr_b16       a transposing LDS read: in each group of 16
//                            lanes, lane j receives element (j % 4) of the
//                            8-byte load of source lane 4q + j/4 as its
//                            element q.  When source lane s reads row
//                            k0 + s/4, columns n0 + 4(s%4).. of an N-major
//                            tile, lane j gets 4 consecutive k of column
//                            n0 + j: the MFMA operand layout, read directly
//                            from a B tile stored the way it lies in memory.
//
// Pipeline: STAGES LDS stages of one BK step each.  Step t+STAGES-1 is issued
// while step t is multiplied; at the end of step t each wave waits until its
// own loads of step t+2 have landed (s_waitcnt vmcnt), then one barrier makes
// them visible to all waves.  Step t+1 is therefore complete during step t,
// and its first operand fragments are read before the barrier, so the MFMA
// pipe does not wait for LDS after it.  A plain __syncthreads would force
// vmcnt(0) and drain every stage in flight, so the raw s_barrier is used with
// explicit, counted waits.
//
// LDS layouts (16-byte slots permuted with XOR so the MFMA operand reads hit
// distinct banks; the permutation is applied on the global side, since a DMA
// lane's LDS slot is fixed by its lane id):
//   A (and K-contiguous B): [rows][BK] row-major, 64 bytes per row; octet c of
//     row r sits in slot c ^ fa(r).
//   N-contiguous B: [BK][BN] row-major, 2 BN bytes per k-row; the 32-byte
//     block b of row k sits at block b ^ hb(k).
//
// Edges: rows past M (A) or N (B) are loaded from the last valid row and the
// outputs they feed are never stored.  A ragged last K step (K or the split
// end not a multiple of BK) is filled by masked register loads with zero fill
// instead of DMA.
#pragma once

#include "tile_kernel.hpp"

namespace gemmf16 {

template <int STAGES_, int WAVES_M_ = 2, int WAVES_N_ = 2, int BM_ = 256, int BN_ = 256>
struct DmaCfg {
  static constexpr int BM = BM_, BN = BN_, BK = 32, STAGES = STAGES_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, NW = WAVES_M * WAVES_N;
  static constexpr int NT = 64 * NW;
  static constexpr int MI = 32, KI = 16, KS = BK / KI;   // 2 MFMA k-steps per stage
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;   // 16 KiB each
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDS = STAGES * STAGE;
  static constexpr int DMA_A = A_BYTES / 1024 / NW;   // DMA instructions per wave per stage
  static constexpr int DMA_B = B_BYTES / 1024 / NW;
  static constexpr int DMA_PER_STAGE = DMA_A + DMA_B;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(DMA_A * NW * 1024 == A_BYTES && DMA_B * NW * 1024 == B_BYTES, "DMA split");
  static_assert(FN * FM >= 4, "DMA placement");
  static_assert(BN == 128 || BN == 256, "N-major B k-rows of 256 or 512 bytes");
};

// octet slot permutation of the 64-byte rows: distinct banks for 8 and for 16
// consecutive rows reading the same octet
__device__ __forceinline__ int fa(int r) { return ((r >> 2) ^ (((r >> 1) & 1) << 1)) & 3; }
// 32-byte block permutation of the 512-byte k-rows of an N-major tile
__device__ __forceinline__ int hb(int k) { return ((2 * (k & 3)) ^ (((k >> 1) ^ k) & 1)) & 7; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// All of this wave's LDS reads have returned their data.
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef short s16x4 __attribute__((__vector_size__(8)));
// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One global_load_lds_dwordx4: lane l's 16 bytes at g land at LDS byte
// address lds + 16 * l.  Issued through inline asm so the compiler does not
// insert its own vmcnt(0) before every LDS read it cannot prove disjoint from
// the transfer; completion is awaited explicitly with wait_vmcnt.
__device__ __forceinline__ void dma16(const uint16_t* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(g)
               : "memory", "m0");
}

// NI consecutive 1 KiB DMA slots with a single m0: the instruction offset is
// added to both the global and the LDS address, so the source pointer of
// slot i is biased by -1024*i bytes (-512 elements) and the offset restores
// it.  One m0 write per batch instead of one per instruction keeps the wave
// from stalling on m0 rewrites between MFMAs.
template <int NI>
__device__ __forceinline__ void dma16_batch(const uint16_t* const* p, int64_t off, uint32_t lds) {
  static_assert(NI == 1 || NI == 2 || NI == 4, "batch size");
  if constexpr (NI == 4) {
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "global_load_lds_dwordx4 %2, off offset:1024\n\t"
        "global_load_lds_dwordx4 %3, off offset:2048\n\t"
        "global_load_lds_dwordx4 %4, off offset:3072"
        :
        : "s"(lds), "v"(p[0] + off), "v"(p[1] + off - 512), "v"(p[2] + off - 1024),
          "v"(p[3] + off - 1536)
        : "memory", "m0");
  } else if constexpr (NI == 2) {
    asm volatile(
        "s_mov_b32 m0, %0\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "global_load_lds_dwordx4 %2, off offset:1024"
        :
        : "s"(lds), "v"(p[0] + off), "v"(p[1] + off - 512)
        : "memory", "m0");
  } else {
    dma16(p[0] + off, lds);
  }
}

__device__ __forceinline__ f16x8 read_tr_pair(const char* p0, const char* p1) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p1));
  const f16x4 l = __builtin_bit_cast(f16x4, lo), h = __builtin_bit_cast(f16x4, hi);
  return f16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
}

// Per-lane source pointers of one operand's DMA instructions, advanced by one
// BK step at a time.
//   KMAJOR: a K-contiguous operand (A, or B given as a transposed view):
//     instruction i of wave w covers rows (4w + i) * 16 .. +16 of the tile;
//     lane l -> row +l/4, slot l%4 -> octet (l%4) ^ fa(row).
//   else (N-contiguous B, k-rows of BN columns): instruction i of wave w
//     covers the 1024 / (2 BN) k-rows from (NI w + i) * 1024 / (2 BN); lane l
//     -> k-row + l / SPR, 16-byte slot l % SPR (SPR = BN / 8 slots per
//     k-row) -> 32-byte block (slot/2) ^ hb(k), half slot%2.
template <int NI, bool KMAJOR, int BN = 256>
struct DmaSource {
  static constexpr int SPR = BN / 8, KPI = 64 / SPR;   // slots per k-row, k-rows per instruction
  const uint16_t* p[NI];
  int64_t step;  // elements per BK step

  __device__ __forceinline__ void init(const uint16_t* base, int64_t s_r, int64_t s_k,
                                       int64_t R_tot, int64_t r0, int64_t kb, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (KMAJOR) {
        const int r = (NI * wave + i) * 16 + lane / 4;
        const int c = (lane % 4) ^ fa(r);
        int64_t rr = r0 + r;
        if (rr > R_tot - 1) rr = R_tot - 1;
        p[i] = base + rr * s_r + (kb + 8 * c) * s_k;
      } else {
        const int k = (NI * wave + i) * KPI + lane / SPR;
        const int slot = lane % SPR;
        const int b = (slot / 2) ^ hb(k);
        int64_t n = r0 + b * 16 + (slot % 2) * 8;
        if (n > R_tot - 8) n = R_tot - 8;   // whole chunk past N: any valid chunk
        p[i] = base + n * s_r + (kb + k) * s_k;
      }
    }
    step = (int64_t)32 * s_k;
  }

  // All of this wave's DMA instructions of the step `t` BK-steps past kb,
  // into the operand area whose first slot for this wave is at lds_wave.
  __device__ __forceinline__ void issue_batch(uint32_t lds_wave, int64_t t) {
    dma16_batch<NI>(p, t * step, lds_wave);
  }

  // Same, from a pointer to the operand area of a stage.
  __device__ __forceinline__ void issue(const char* lds_op, int wave, int64_t t) {
    issue_batch(__builtin_amdgcn_readfirstlane(lds_addr(lds_op) + NI * wave * 1024), t);
  }

  // Masked register fill of a ragged step (k < k_end kept, zero fill), into
  // the same LDS slots the DMA would write.
  __device__ __forceinline__ void fill_masked(char* lds_op, int wave, int lane, int64_t t,
                                              int64_t kb, int64_t k_end, int64_t s_k) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint16_t* q = p[i] + t * step;
      u32x4 v;
      if constexpr (KMAJOR) {
        const int r = (NI * wave + i) * 16 + lane / 4;
        const int c = (lane % 4) ^ fa(r);
        const int64_t kk = kb + t * 32 + 8 * c;
        const int64_t d = k_end - kk;
        const int nk = d < 0 ? 0 : (d < 8 ? (int)d : 8);
        v = load_partial8(q, s_k, nk);
      } else {
        const int k = (NI * wave + i) * KPI + lane / SPR;
        const bool ok = kb + t * 32 + k < k_end;
        v = ok ? *reinterpret_cast<const u32x4*>(q) : zero4();
      }
      *reinterpret_cast<u32x4*>(lds_op + (NI * wave + i) * 1024 + lane * 16) = v;
    }
  }
};

template <class CF>
struct DmaFrags {
  f16x8 fa_[CF::FN];  // from the B tile: MFMA first operand (rows = n)
  f16x8 fb_[CF::FM];  // from the A tile: MFMA second operand (cols = m)
};

// Operand fragments of k-step ks of a stage.
template <class CF, bool BKMAJOR>
__device__ __forceinline__ void read_frags(DmaFrags<CF>& f, const char* ta, const char* tb, int ks,
                                           int wm, int wn, int lane) {
  const int lr = lane % 32, lo = lane / 32;   // row in block, k-octet
  const int c = ks * 2 + lo;
#pragma unroll
  for (int j = 0; j < CF::FM; ++j) {
    const int r = wm * CF::WTM + j * 32 + lr;
    f.fb_[j] = *reinterpret_cast<const f16x8*>(ta + r * 64 + ((c ^ fa(r)) * 16));
  }
  if constexpr (BKMAJOR) {
#pragma unroll
    for (int i = 0; i < CF::FN; ++i) {
      const int r = wn * CF::WTN + i * 32 + lr;
      f.fa_[i] = *reinterpret_cast<const f16x8*>(tb + r * 64 + ((c ^ fa(r)) * 16));
    }
  } else {
    // 16-lane group g: columns +16*(g%2), k-octet g/2; source lane s reads
    // k-row 8*octet + s/4 (+4 for the second half), columns 4*(s%4)..+3.
    constexpr int ROWB = 2 * CF::BN;   // bytes per k-row
    const int g = lane / 16, s = lane % 16;
    const int kr = ks * 16 + 8 * (g / 2) + s / 4;
#pragma unroll
    for (int i = 0; i < CF::FN; ++i) {
      const int n = wn * CF::WTN + i * 32 + 16 * (g % 2);
      const char* p0 = tb + kr * ROWB + (((n >> 4) ^ hb(kr)) * 32) + 8 * (s % 4);
      f.fa_[i] = read_tr_pair(p0, p0 + 4 * ROWB);
    }
  }
}

// The MFMAs of one k-step with this wave's DMA batches of the step
// STAGES-1 ahead placed a quarter and three quarters of the way through, so
// their address and m0 setup issue in the shadow of matrix work.
template <class CF, int DT, class SA, class SB>
__device__ __forceinline__ void mma_frags_dma(const DmaFrags<CF>& f, f32x16 (&acc)[CF::FN][CF::FM],
                                              SA& sa, SB& sb, uint32_t la, uint32_t lb,
                                              int64_t t) {
  constexpr int NQ = CF::FN * CF::FM;
#pragma unroll
  for (int i = 0; i < CF::FN; ++i)
#pragma unroll
    for (int j = 0; j < CF::FM; ++j) {
      acc[i][j] = mfma<32, DT>(f.fa_[i], f.fb_[j], acc[i][j]);
      const int q = i * CF::FM + j;
      if (q == NQ / 4 - 1) sa.issue_batch(la, t);
      if (q == 3 * NQ / 4 - 1) sb.issue_batch(lb, t);
    }
}

template <class CF, int DT = DT_F16>
__device__ __forceinline__ void mma_frags(const DmaFrags<CF>& f, f32x16 (&acc)[CF::FN][CF::FM]) {
#pragma unroll
  for (int i = 0; i < CF::FN; ++i)
#pragma unroll
    for (int j = 0; j < CF::FM; ++j) acc[i][j] = mfma<32, DT>(f.fa_[i], f.fb_[j], acc[i][j]);
}

// FP8 operands (F8 = 2 fmt_a + fmt_b, 0 E4M3 and 1 E5M2): a stage of the
// 16-bit layout then holds 64 k of bytes, and the fragments of its two
// k-substeps (chunks lo and 2 + lo of a row for lane half lo) together are
// the 32 bytes one v_mfma_f32_32x32x64_f8f6f4 takes per lane.  That
// instruction pairs byte b of one operand with byte b of the other, so a k
// order that A and B share gives the step's whole product.  The DMA batches
// of the step STAGES-1 ahead sit after the first and the third MFMA.
__device__ __forceinline__ i32x8 cat16(const f16x8& x, const f16x8& y) {
  const u32x4 a = __builtin_bit_cast(u32x4, x), b = __builtin_bit_cast(u32x4, y);
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

template <class CF, int F8, bool WITH_DMA, class SA, class SB>
__device__ __forceinline__ void mma_frags_f8(const DmaFrags<CF>& f0, const DmaFrags<CF>& f1,
                                             f32x16 (&acc)[CF::FN][CF::FM], SA& sa, SB& sb, uint32_t la,
                                             uint32_t lb, int64_t t) {
  constexpr int NQ = CF::FN * CF::FM;
#pragma unroll
  for (int i = 0; i < CF::FN; ++i)
#pragma unroll
    for (int j = 0; j < CF::FM; ++j) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat16(f0.fa_[i], f1.fa_[i]),
                                                                  cat16(f0.fb_[j], f1.fb_[j]), acc[i][j],
                                                                  F8 % 2, F8 / 2, 0, 0, 0, 0);
      if constexpr (WITH_DMA) {
        const int q = i * CF::FM + j;
        if (q == NQ / 4 - 1) sa.issue_batch(la, t);
        if (q == 3 * NQ / 4 - 1) sb.issue_batch(lb, t);
      }
    }
}

// DT: DT_F16 or DT_BF16 operands and output.  F8 >= 0: FP8 A and
// K-contiguous B (formats F8 / 2, F8 % 2; strides and K in bytes, K even,
// row strides even), binary16 out: the operands are read as byte pairs, so a
// stage holds 64 k.
template <class CF, bool BKMAJOR, bool PARTIAL, int DT = DT_F16, int F8 = -1>
__global__ __launch_bounds__(CF::NT) void gemm_dma_kernel(KArgs a) {
  static_assert(F8 < 0 || (BKMAJOR && DT == DT_F16), "FP8: K-contiguous B, binary16 out");
  __shared__ __attribute__((aligned(1024))) char smem[CF::LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;

  const int64_t T = a.GM * a.GN;
  int64_t w = blockIdx.x;
  int64_t split = 0;
  if constexpr (PARTIAL) split_tile_of(blockIdx.x, T, a.split_xcd, split, w);
  int64_t pm, pn;
  raster_tile(w, a.GM, a.GN, a.panel, pm, pn);
  const int64_t m0 = pm * CF::BM, n0 = pn * CF::BN;
  // FP8: byte offsets and strides halved into 16-bit pair units.
  constexpr int SH = F8 >= 0 ? 1 : 0;
  const int64_t kb8 = split * a.k_split;
  const int64_t kb = kb8 >> SH;
  const int64_t ke = ((kb8 + a.k_split < a.K) ? kb8 + a.k_split : a.K) >> SH;

  DmaSource<CF::DMA_A, true> sa;
  DmaSource<CF::DMA_B, BKMAJOR, CF::BN> sb;
  sa.init(a.A, a.lda_m >> SH, a.lda_k, a.M, m0, kb, wave, lane);
  sb.init(a.B, a.ldb_n >> SH, a.ldb_k, a.N, n0, kb, wave, lane);

  f32x16 acc[CF::FN][CF::FM];
#pragma unroll
  for (int i = 0; i < CF::FN; ++i)
#pragma unroll
    for (int j = 0; j < CF::FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto stage_a = [&](int64_t t) { return smem + (int)(t % CF::STAGES) * CF::STAGE; };
  auto stage_b = [&](int64_t t) { return smem + (int)(t % CF::STAGES) * CF::STAGE + CF::A_BYTES; };

  const int64_t nfull = (ke - kb) / CF::BK;
  const bool tail = (ke - kb) % CF::BK != 0;
  DmaFrags<CF> f0, f1;

  if (nfull > 0) {
    // Prologue: steps 0 .. STAGES-2 in flight (clamped to the last full step
    // when there are fewer), steps 0 and 1 complete.
    for (int64_t t = 0; t < CF::STAGES - 1; ++t) {
      const int64_t tt = t < nfull ? t : nfull - 1;
      sa.issue(stage_a(t), wave, tt);
      sb.issue(stage_b(t), wave, tt);
    }
    wait_vmcnt<CF::DMA_PER_STAGE * (CF::STAGES - 3)>();
    wg_barrier();
    read_frags<CF, BKMAJOR>(f0, stage_a(0), stage_b(0), 0, wm, wn, lane);

    // Steady state, branch-free.  Phases are fenced with sched_barrier so
    // each batch of LDS reads is issued a whole k-step (16 MFMAs) before its
    // use.  In the last STAGES-1 steps the DMA re-loads the last full step
    // into the stage of step t-1, which no wave reads any more.
    for (int64_t t = 0; t < nfull; ++t) {
      const int64_t ahead = t + CF::STAGES - 1;
      const int64_t tt = ahead < nfull ? ahead : nfull - 1;
      const uint32_t la =
          __builtin_amdgcn_readfirstlane(lds_addr(stage_a(ahead)) + CF::DMA_A * wave * 1024);
      const uint32_t lb =
          __builtin_amdgcn_readfirstlane(lds_addr(stage_b(ahead)) + CF::DMA_B * wave * 1024);
      read_frags<CF, BKMAJOR>(f1, stage_a(t), stage_b(t), 1, wm, wn, lane);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (F8 >= 0) {
        mma_frags_f8<CF, F8, true>(f0, f1, acc, sa, sb, la, lb, tt);
        __builtin_amdgcn_sched_barrier(0);
        read_frags<CF, BKMAJOR>(f0, stage_a(t + 1), stage_b(t + 1), 0, wm, wn, lane);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        mma_frags_dma<CF, DT>(f0, acc, sa, sb, la, lb, tt);
        __builtin_amdgcn_sched_barrier(0);
        // First fragments of step t+1 (complete since the last barrier).  On
        // the last step this reads a stale stage and the values go unused.
        read_frags<CF, BKMAJOR>(f0, stage_a(t + 1), stage_b(t + 1), 0, wm, wn, lane);
        __builtin_amdgcn_sched_barrier(0);
        mma_frags<CF, DT>(f1, acc);
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_vmcnt<CF::DMA_PER_STAGE * (CF::STAGES - 3)>();   // step t+2 landed
      wg_barrier();
    }
    wait_vmcnt<0>();   // no LDS transfer may still be in flight past this point
  }
  if (tail) {
    // Ragged last step: masked fill of stage nfull % STAGES (free: every read
    // of earlier steps finished before the last barrier).
    sa.fill_masked(stage_a(nfull), wave, lane, nfull, kb, ke, a.lda_k);
    sb.fill_masked(stage_b(nfull), wave, lane, nfull, kb, ke, a.ldb_k);
    __syncthreads();
    read_frags<CF, BKMAJOR>(f0, stage_a(nfull), stage_b(nfull), 0, wm, wn, lane);
    read_frags<CF, BKMAJOR>(f1, stage_a(nfull), stage_b(nfull), 1, wm, wn, lane);
    if constexpr (F8 >= 0) {
      mma_frags_f8<CF, F8, false>(f0, f1, acc, sa, sb, 0, 0, 0);
    } else {
      mma_frags<CF, DT>(f0, acc);
      mma_frags<CF, DT>(f1, acc);
    }
  }

  // Epilogue: the same C^T-block layout as the register-staged kernel.
  const int lr = lane % 32;
#pragma unroll
  for (int i = 0; i < CF::FN; ++i)
#pragma unroll
    for (int j = 0; j < CF::FM; ++j) {
      const int64_t m = m0 + wm * CF::WTM + j * 32 + lr;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + wn * CF::WTN + i * 32 + 8 * g + 4 * (lane >> 5);
        const float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1];
        const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
        if constexpr (PARTIAL)
          store4_f32(a, split, m, n, v0, v1, v2, v3);
        else
          store4_out<DT>(a, m, n, v0, v1, v2, v3);
      }
    }
}

}  // namespace gemmf16
