// FP8 main kernel (gfx950): C = A.B with OCP FP8 operands (E4M3 or E5M2, per
// operand), fp32 accumulation and binary16 output.
//
// TileLang tutorial ch. 14, section 5 (lower precision) keeps the GEMM
// skeleton and changes the matrix instruction and the K step.  Here the
// skeleton is the full-line-A LDS-DMA kernel of dma_a128_kernel.hpp, byte
// for byte: one workgroup per 256 x 256 tile, 8 waves of 64 x 128, three A
// super-slots of 256 rows x 128 bytes and four B stages of 256 rows x 64
// bytes, the same DMA instructions, barriers and ping-pong phases.  What a
// byte holds changes: a super-step is 128 k and a step 64 k, and each 32 x 32
// block of a step is one v_mfma_f32_32x32x64_f8f6f4 (formats as immediates).
//
// A is K-contiguous (A [M, K] row-major).  B is K-contiguous (given as
// [N, K] rows, i.e. a transposed view), when the DMA moves pairs of bytes
// with the 16-bit helpers (views with half the row stride), or, in the BN
// kernels, N-contiguous (B [K, N] row-major): 64 k-rows of 256 bytes per
// stage, read back with the 8-bit transposing LDS read (read_b_f8_n).  A lane's 32 operand bytes are
// k = 32 g .. 32 g + 31 of the step for lane group g = lane / 32, for A and B
// alike: the matrix instruction pairs byte b of the A operand with byte b of
// the B operand, so any assignment of k to bytes that both operands share is
// the product.
//
// K tails (under 128 k after the whole super-steps) are filled byte by byte
// with zero fill after the pipelined loop.
#pragma once

#include <type_traits>

#include "dma_a128_kernel.hpp"

namespace gemmf16 {


enum F8Format { F8_E4M3 = 0, F8_E5M2 = 1 };

struct F8Cfg {
  static constexpr int BM = 256, BN = 256, BK = 64;   // BK in FP8 elements (bytes)
  static constexpr int WAVES_M = 4, WAVES_N = 2, NW = 8, NT = 512;
  static constexpr int WTM = 64, WTN = 128, FM = 2, FN = 4;
  static constexpr int A_SLOT = BM * 128, A_SLOTS = 3;      // 32 KiB per 128-k super-step
  static constexpr int B_STAGE = BN * BK, B_STAGES = 4;     // 16 KiB per 64-k step
  static constexpr int B_BASE = A_SLOTS * A_SLOT;
  static constexpr int LDS = B_BASE + B_STAGES * B_STAGE;
  static constexpr int DMA_A = A_SLOT / 1024 / NW;          // 4 per wave per super-step
  static constexpr int DMA_B = B_STAGE / 1024 / NW;         // 2 per wave per step
  static constexpr int DMA_PER_STEP = DMA_A / 2 + DMA_B;
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

struct F8Frags {
  i32x8 fa_[F8Cfg::FN];   // B blocks (first MFMA operand, rows = n)
  i32x8 fb_[F8Cfg::FM];   // A blocks (second operand, rows = m)
};

__device__ __forceinline__ i32x8 join8(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// A block j of the step in half H of a super-step: row r, 16-byte chunks
// 4H + 2g and 4H + 2g + 1 of its 128-byte row (swizzled by f8).
__device__ __forceinline__ i32x8 read_a_f8(const char* ta, int H, int j, int wm, int lane) {
  const int r = wm * F8Cfg::WTM + j * 32 + lane % 32, c = 4 * H + 2 * (lane / 32);
  const char* row = ta + r * 128;
  return join8(*reinterpret_cast<const u32x4*>(row + ((c ^ f8(r)) * 16)),
               *reinterpret_cast<const u32x4*>(row + (((c + 1) ^ f8(r)) * 16)));
}

// B block i of a step: n-row r, chunks 2g and 2g + 1 of its 64-byte row
// (swizzled by fa, as the 16-bit K-major B stages).
__device__ __forceinline__ i32x8 read_b_f8(const char* tb, int i, int wn, int lane) {
  const int r = wn * F8Cfg::WTN + i * 32 + lane % 32, c = 2 * (lane / 32);
  const char* row = tb + r * 64;
  return join8(*reinterpret_cast<const u32x4*>(row + ((c ^ fa(r)) * 16)),
               *reinterpret_cast<const u32x4*>(row + (((c + 1) ^ fa(r)) * 16)));
}

// N-contiguous B (B [K, N] row-major, BN kernels).  A stage is 64 k-rows of
// 256 bytes; the 16-byte chunk of columns 16c .. 16c+15 of k-row k sits at
// chunk c ^ h8(k), so that the transposing reads of 8 consecutive k-rows hit
// 16 distinct chunks (all 64 banks) per half wave.
__device__ __forceinline__ int h8(int k) { return 2 * (k & 7); }

// Per-lane sources of this wave's NI DMA instructions of an N-major B step:
// instruction i covers k-rows (NI w + i) * 4 .. +4, lane l -> k-row +l/16,
// LDS chunk l%16 <- global column chunk (l%16) ^ h8(k-row).  A chunk wholly
// past N reads any valid chunk (N is a multiple of 16).  SGPR-base form as
// ASourceS; B is addressed in bytes.
template <int NI>
struct BSourceN8 {
  const char* base;  // byte address of (k kb, column n0) less kSBias
  uint32_t off[NI];
  int64_t step;      // bytes per 64-k step

  __device__ __forceinline__ void init(const void* B, int64_t ldb_k, int64_t N, int64_t n0,
                                       int64_t kb, int wave, int lane) {
    base = uniform_ptr((const char*)B + kb * ldb_k + n0 - kSBias);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int k = (NI * wave + i) * 4 + lane / 16;
      int64_t n = n0 + 16 * ((lane % 16) ^ h8(k));
      if (n > N - 16) n = N - 16;
      off[i] = (uint32_t)(k * ldb_k + (n - n0) + kSBias - 1024 * i);
    }
    step = 64 * ldb_k;
  }
  __device__ __forceinline__ void issue_batch(uint32_t lds_wave, int64_t t) {
    dma16s_batch<NI>(off, base + t * step, lds_wave);
  }
  __device__ __forceinline__ void issue_batch_at(uint32_t lds_wave, const char* b) {
    dma16s_batch<NI>(off, b, lds_wave);
  }
  // Step t past kb with k-rows at or past k_end zero (the K tail).
  __device__ __forceinline__ void fill_masked(char* lds_op, int wave, int lane, int64_t t, int64_t kb,
                                              int64_t k_end) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int k = (NI * wave + i) * 4 + lane / 16;
      const bool ok = kb + t * 64 + k < k_end;
      const char* q = base + t * step + off[i] + 1024 * i;
      *reinterpret_cast<u32x4*>(lds_op + (NI * wave + i) * 1024 + lane * 16) =
          ok ? *reinterpret_cast<const u32x4*>(q) : zero4();
    }
  }
};

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ i32x2 read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}

// B block i of an N-major stage with ds_read_b64_tr_b8: in each group of 16
// lanes, lane j receives byte j%8 of the 8-byte reads of source lanes
// 2q + j/8 (q = 0..7) as its bytes q.  Source lane s of group G reads k-row
// 32 (G/2) + 8r + s/2, columns 16 (G%2) + 8 (s%2) .. +8 of the block, so lane
// l receives column l%32, k-rows 32 (l/32) + 8r .. +8 in read r: its 32 bytes
// are k = 32 g .. 32 g + 31 in order, as read_a_f8 delivers A.
__device__ __forceinline__ i32x8 read_b_f8_n(const char* tb, int i, int wn, int lane) {
  const int G = lane / 16, s = lane % 16;
  const int nb = wn * F8Cfg::WTN + i * 32 + 16 * (G & 1);
  const int kr = 32 * (G >> 1) + (s >> 1);                // h8 is the same for kr + 8r
  const char* p = tb + kr * 256 + (((nb >> 4) ^ h8(kr)) * 16) + 8 * (s & 1);
  const i32x2 r0 = read_tr8(p), r1 = read_tr8(p + 8 * 256), r2 = read_tr8(p + 16 * 256),
              r3 = read_tr8(p + 24 * 256);
  return i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

template <bool BN>
__device__ __forceinline__ i32x8 read_b_any(const char* tb, int i, int wn, int lane) {
  if constexpr (BN)
    return read_b_f8_n(tb, i, wn, lane);
  else
    return read_b_f8(tb, i, wn, lane);
}

template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma_f8(const i32x8& b, const i32x8& a, const f32x16& c) {
  // First operand: the B block (format FB); second: the A block (format FA);
  // unit scales.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, FB, FA, 0, 0, 0, 0);
}

template <int FA, int FB, bool EDGE>
__device__ __forceinline__ void mma_f8(const F8Frags& f, f32x16 (&acc)[F8Cfg::FN][F8Cfg::FM], int i0,
                                       int i1, int fnv, int fmv) {
#pragma unroll
  for (int i = i0; i < i1; ++i)
#pragma unroll
    for (int j = 0; j < F8Cfg::FM; ++j)
      if (!EDGE || (i < fnv && j < fmv)) acc[i][j] = mfma_f8<FA, FB>(f.fa_[i], f.fb_[j], acc[i][j]);
}

// Byte-masked fill of one LDS row chunk: bytes k .. k+15 of a K-contiguous
// row at p (k < k_end kept, zero fill).
__device__ __forceinline__ u32x4 load_bytes16(const uint8_t* p, int64_t k, int64_t k_end) {
  const int64_t d = k_end - k;
  if (d >= 16) return *reinterpret_cast<const u32x4*>(p + k);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  for (int e = 0; e < 16; ++e)
    if (e < d) w[e / 4] |= (uint32_t)p[k + e] << (8 * (e % 4));
  return u32x4{w[0], w[1], w[2], w[3]};
}

// K-contiguous FP8 A and B; formats FA / FB; fp32 partials when PARTIAL.
// BN: B N-contiguous (B [K, N] row-major) instead of K-contiguous.
// BPACK: B pre-packed by the 16-bit packing pass over its byte pairs (the
// 16 KiB blocks are then the LDS images of this kernel's K-major 64-k B
// stages; ldb_n is the panel stride in byte pairs).
// GROUPED: one launch over the groups of a grouped product (group_tile).
template <int FA, int FB, bool PARTIAL, bool BN = false, bool BPACK = false, bool GROUPED = false>
__global__ __launch_bounds__(F8Cfg::NT) void gemm_f8_kernel(KArgs a) {
  using CF = F8Cfg;
  static_assert(!(BN && BPACK), "packed B stages are K-major");
  static_assert(!(GROUPED && (PARTIAL || BPACK)), "grouped launches are never split or packed");
  __shared__ __attribute__((aligned(1024))) char smem[CF::LDS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;

  const int64_t T = a.GM * a.GN;
  int64_t w = blockIdx.x;
  int64_t split = 0;
  if constexpr (PARTIAL) {
    if (a.sk_tiles > 0) {            // stream-K tail (see KArgs)
      split = w / a.sk_tiles;
      w = a.sk_first + (w - split * a.sk_tiles);
    } else {
      split_tile_of(blockIdx.x, T, a.split_xcd, split, w);
    }
  }
  int64_t pm, pn;
  if constexpr (GROUPED) {
    if (!group_tile<1>(a, w, pm, pn)) return;   // uniform per workgroup, before any barrier
  } else {
    raster_tile(w, a.GM, a.GN, a.panel, pm, pn);
  }
  const int64_t m0 = pm * CF::BM, n0 = pn * CF::BN;
  const int64_t kb = split * a.k_split;   // bytes; a multiple of 128
  const int64_t ke = (kb + a.k_split < a.K) ? kb + a.k_split : a.K;
  // Only blocks wholly past M are skipped; blocks past N are computed so the
  // tiles of one row stay in step (as in the 16-bit kernel).
  const int64_t mrem = a.M - (m0 + wm * CF::WTM);
  const int fnv = CF::FN;
  const int fmv = mrem <= 0 ? 0 : (mrem >= CF::WTM ? CF::FM : (int)((mrem + 31) / 32));
  const bool edge = fmv < CF::FM;

  // Byte-pair views for the DMA: strides and K offsets halve.
  ASourceS<CF::DMA_A> sa;
  std::conditional_t<BPACK, PackedBSource<CF::DMA_B>,
                     std::conditional_t<BN, BSourceN8<CF::DMA_B>, BSourceS<CF::DMA_B, true>>> sb;
  sa.init(a.A, a.lda_m / 2, 1, a.M, m0, kb / 2, wave, lane);
  if constexpr (BN)
    sb.init(a.B, a.ldb_k, a.N, n0, kb, wave, lane);
  else if constexpr (BPACK)
    sb.init(a.B, a.ldb_n, 1, a.N, n0, kb / 2, wave, lane);
  else
    sb.init(a.B, a.ldb_n / 2, 1, a.N, n0, kb / 2, wave, lane);

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

  const int64_t nsup = (ke - kb) / 128;    // whole 128-k super-steps
  const int64_t nfull2 = 2 * nsup;         // 64-k steps they hold
  const int64_t rem = (ke - kb) - 128 * nsup;
  F8Frags f;

  if (nsup > 0) {
    // The schedule and its invariants are those of gemm_dma_a128_kernel: two
    // wave groups one phase apart; M(t) reads the A blocks and B blocks 2, 3
    // of step t and issues this wave's DMA of step t + 3; C(t) runs the step's
    // 8 MFMAs and reads B blocks 0, 1 of step t + 1 under the last four.
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
    f.fa_[0] = read_b_any<BN>(stage_b(0), 0, wn, lane);
    f.fa_[1] = read_b_any<BN>(stage_b(0), 1, wn, lane);
    if (g1) wg_barrier();

    // Slot indices rotate in 32-bit registers, as in the fp16 kernel.
    const int ns = (int)nsup, nf2 = 2 * ns;
    auto sl_a = [&](int i) { return smem + i * CF::A_SLOT; };
    auto st_b = [&](int t) { return smem + CF::B_BASE + (t & (CF::B_STAGES - 1)) * CF::B_STAGE; };
    const uint32_t la0 = __builtin_amdgcn_readfirstlane(lds_addr(smem) + CF::DMA_A * wave * 1024);
    const uint32_t lb0 =
        __builtin_amdgcn_readfirstlane(lds_addr(smem) + CF::B_BASE + CF::DMA_B * wave * 1024);
    const char* pa = sa.base + (int64_t)(ns > 2 ? 2 : ns - 1) * sa.step;
    const char* pb = sb.base + (int64_t)(nf2 > 3 ? 3 : nf2 - 1) * sb.step;
    auto step = [&](auto h_tag, auto e_tag, int iu, int i2, int t) {
      constexpr int H = decltype(h_tag)::value;
      constexpr bool EDGE = decltype(e_tag)::value;
      // M(t)
      f.fb_[0] = read_a_f8(sl_a(iu), H, 0, wm, lane);
      f.fb_[1] = read_a_f8(sl_a(iu), H, 1, wm, lane);
      f.fa_[2] = read_b_any<BN>(st_b(t), 2, wn, lane);
      f.fa_[3] = read_b_any<BN>(st_b(t), 3, wn, lane);
      sa.template issue_half_at<H>(la0 + i2 * CF::A_SLOT + (CF::DMA_A / 2) * H * 1024, pa);
      sb.issue_batch_at(lb0 + ((t + 3) & (CF::B_STAGES - 1)) * CF::B_STAGE, pb);
      if (t + 4 < nf2) pb += sb.step;
      wait_lgkmcnt0();
      __builtin_amdgcn_sched_barrier(0);
      // C(t), at raised issue priority and with its first MFMA ahead of the
      // barrier, as in the fp16 kernel; on the last step the reads fetch
      // unused bytes of a free stage.
      __builtin_amdgcn_s_setprio(1);
      if (!EDGE || (0 < fnv && 0 < fmv)) acc[0][0] = mfma_f8<FA, FB>(f.fa_[0], f.fb_[0], acc[0][0]);
      wg_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (!EDGE || (0 < fnv && 1 < fmv)) acc[0][1] = mfma_f8<FA, FB>(f.fa_[0], f.fb_[1], acc[0][1]);
      mma_f8<FA, FB, EDGE>(f, acc, 1, 2, fnv, fmv);
      __builtin_amdgcn_sched_barrier(0);
      const char* nb = st_b(t + 1);
#pragma unroll
      for (int i = 2; i < CF::FN; ++i)
#pragma unroll
        for (int j = 0; j < CF::FM; ++j) {
          if (!EDGE || (i < fnv && j < fmv)) acc[i][j] = mfma_f8<FA, FB>(f.fa_[i], f.fb_[j], acc[i][j]);
          if (j == 0) f.fa_[i - 2] = read_b_any<BN>(nb, i - 2, wn, lane);
          __builtin_amdgcn_sched_barrier(0);
        }
      wait_vmcnt<CF::DMA_PER_STEP>();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      wg_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    auto run = [&](auto e_tag) {
      static_assert(CF::A_SLOTS == 3, "slot rotation");
      int iu = 0;
      for (int u = 0; u < ns; ++u) {
        const int i1 = iu == 2 ? 0 : iu + 1, i2 = iu == 0 ? 2 : iu - 1;
        step(std::integral_constant<int, 0>{}, e_tag, iu, i2, 2 * u);
        step(std::integral_constant<int, 1>{}, e_tag, iu, i2, 2 * u + 1);
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
    // Tail of under 128 k: byte-masked fill of A super-slot nsup and B stages
    // nfull2 (and nfull2 + 1), all free after the last barrier; rows past M
    // or N read the last valid row.
    const uint8_t* A8 = reinterpret_cast<const uint8_t*>(a.A);
    [[maybe_unused]] const uint8_t* B8 = reinterpret_cast<const uint8_t*>(a.B);
    const int64_t k0 = kb + 128 * nsup;
    char* sl = slot_a(nsup);
    for (int cell = tid; cell < CF::BM * 8; cell += CF::NT) {
      const int r = cell / 8, c = cell % 8;
      int64_t rr = m0 + r;
      if (rr > a.M - 1) rr = a.M - 1;
      *reinterpret_cast<u32x4*>(sl + r * 128 + ((c ^ f8(r)) * 16)) =
          load_bytes16(A8 + rr * a.lda_m, k0 + 16 * c, ke);
    }
    for (int s = 0; s < (rem > 64 ? 2 : 1); ++s) {
      char* st = stage_b(nfull2 + s);
      if constexpr (BN) {
        sb.fill_masked(st, wave, lane, nfull2 + s, kb, ke);
      } else if constexpr (BPACK) {
        sb.fill_masked(st, wave, lane, nfull2 + s, kb, ke, 0);   // zero past K already
      } else {
        for (int cell = tid; cell < CF::BN * 4; cell += CF::NT) {
          const int r = cell / 4, c = cell % 4;
          int64_t rr = n0 + r;
          if (rr > a.N - 1) rr = a.N - 1;
          *reinterpret_cast<u32x4*>(st + r * 64 + ((c ^ fa(r)) * 16)) =
              load_bytes16(B8 + rr * a.ldb_n, k0 + 64 * s + 16 * c, ke);
        }
      }
    }
    __syncthreads();
    for (int s = 0; s < (rem > 64 ? 2 : 1); ++s) {
#pragma unroll
      for (int i = 0; i < CF::FN; ++i) f.fa_[i] = read_b_any<BN>(stage_b(nfull2 + s), i, wn, lane);
#pragma unroll
      for (int j = 0; j < CF::FM; ++j) f.fb_[j] = read_a_f8(slot_a(nsup), s, j, wm, lane);
      mma_f8<FA, FB, true>(f, acc, 0, CF::FN, fnv, fmv);
    }
  }

  if constexpr (!PARTIAL) {
    // Staged through LDS, as in the 16-bit kernel.
    wait_lgkmcnt0();
    wg_barrier();
    store_tile_staged<CF, DT_F16>(a, acc, smem, m0, n0, wave, wm, wn, lane);
  } else {
    // fp32 partials staged through LDS, as in the 16-bit kernel.
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
