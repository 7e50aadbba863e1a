// Decode-shaped product (M <= 64) with N-contiguous B (gfx950).
//
// With a few rows of A the whole of B is streamed once to serve them, so the
// product is bound by HBM bandwidth, not by matrix throughput (the tiling
// tutorial, section 04: at M = 1 the weight reads dominate; the TileLang
// tutorial ch. 14, pitfall 1: pipelining a memory-bound GEMM only takes
// on-chip space).  Everything here serves the B stream: every 16-byte load of
// a wave covers whole 128-byte lines, each wave issues all the loads of its
// share before any arithmetic, and there is no LDS staging of B.
//
// Work split: workgroup (nb, s) owns the 128 columns [128 nb, 128 nb + 128)
// and the K range [s KR, (s+1) KR), cut into units of 32 k.  Its 4 waves
// take the units round-robin.  In a unit, lane (g, c) (g = lane / 16,
// c = lane % 16) loads the 8 rows 8g .. 8g+7 of the 8 columns 8c .. 8c+7
// (one 16-byte vector per row; one load instruction of the wave covers 4
// rows x 256 bytes), then transposes the 8 x 8 halves in registers into 8
// k-octets, one per column 8c + f.  Those are exactly the B operands of
// v_mfma_f32_16x16x32_f16 in which lane (g, c) supplies "column" c and
// k-octet g: MFMA f multiplies the rows of A by the 16 columns {8c + f}.
// The A operand is one 16-byte load of 8 consecutive k per lane (row
// 16 fa + c of A); rows past M are zero, so M = 1 costs the same as M = 16
// (the matrix cores are idle here anyway).  Lane (g, c) ends with outputs
// (16 fa + 4g + r, 8c + f), r < 4, f < 8: 8 consecutive columns per row.
//
// B stored as [N, K] rows (K-contiguous, BK): lane (g, c) loads, for each
// group f of 16 columns, the 8 k of octet g of column 16 f + c, one 16-byte
// vector that is already the B operand of the MFMA (no transpose), and ends
// with outputs (16 fa + 4g + r, 16 f + c).  One load instruction of the wave
// covers 16 columns x 64 bytes.
//
// The 4 waves' sums are added through LDS in ascending wave order; with one
// K range the workgroup writes C (round to nearest even), with several it
// writes fp32 partials P[s][m][n] that splitk_reduce sums in ascending s in
// a second launch.  There is no in-kernel "last workgroup sums" step: it
// needs a device-scope release per workgroup, an L2 writeback on gfx950,
// which costs more than the second launch.  K is masked per row with zero
// fill (never wrapped); N is masked per column; addresses are int64.
#pragma once

#include "tile_kernel.hpp"

namespace gemmf16 {

struct DecArgs {
  const uint16_t* A;
  int64_t lda_m, lda_k;
  const uint16_t* B;
  int64_t ldb_k;       // N-contiguous B (ldb_n == 1): 16-byte aligned, ldb_k % 8 == 0
  int64_t ldb_n;       // K-contiguous B (ldb_k == 1, BK kernels): 16-byte aligned, ldb_n % 8 == 0
  uint16_t* C;
  int64_t ldc;
  float* P;            // partials [S][M][N] (S > 1 only)
  int64_t M, N, K;
  int64_t kr;          // rows per K range, a multiple of 32
  int32_t GN, S;
  int32_t a_vec;       // A K-contiguous with 16-byte aligned rows: vector A loads
  int32_t c_vec;       // C 16-byte aligned with ldc % 8 == 0: vector C stores
};

constexpr int kDecCols = 128;  // columns per workgroup
constexpr int kDecUnit = 32;   // k per unit (one MFMA k-step)
// Waves per workgroup (the block is 64 * kDecWaves threads).  Four, with
// one workgroup per compute unit, ran fastest: 8 waves took 10.3 us per M = 1
// call against 10.0, and two workgroups per compute unit (K ranges of 224,
// registers for only one of them at a time) 14.1.
constexpr int kDecWaves = 4;
// Units per wave whose loads are in flight together.  With one wave per
// SIMD a wave may hold 512 registers, so 64 rows of A (128 accumulators per
// lane) keep four units as well: 420 registers, no spills, 17.3 us per
// M = 64 call against 18.6 with two units.
template <int MT>
constexpr int dec_upw() { return 4; }

// FP8 operands (F8 = 2 fmt_a + fmt_b, 0 E4M3 and 1 E5M2 per operand): the
// bytes are widened to binary16, which holds every E4M3 and E5M2 value
// exactly, and the same fp16 MFMAs run on them (a product of two binary16
// values is exact in fp32, so the sums are those of FP8 products).  The
// packed convert of gfx950 takes a byte pair of a word's low or high half;
// it is written out here because the builtin's vector result lost its second
// element (the compiler copied the first into it).  All 256 codes of both
// formats, NaNs included, convert to the binary16 values of the OCP formats.
template <int FMT>
__device__ __forceinline__ uint32_t f8pair_to_f16(uint32_t w, bool hi) {
  uint32_t r;
  if constexpr (FMT == 0) {
    if (hi)
      asm("v_cvt_scalef32_pk_f16_fp8 %0, %1, 1.0 op_sel:[1,0,0]" : "=v"(r) : "v"(w));
    else
      asm("v_cvt_scalef32_pk_f16_fp8 %0, %1, 1.0" : "=v"(r) : "v"(w));
  } else {
    if (hi)
      asm("v_cvt_scalef32_pk_f16_bf8 %0, %1, 1.0 op_sel:[1,0,0]" : "=v"(r) : "v"(w));
    else
      asm("v_cvt_scalef32_pk_f16_bf8 %0, %1, 1.0" : "=v"(r) : "v"(w));
  }
  return r;
}

// 8 FP8 bytes (two words, byte j = element j) as 8 binary16 values.
template <int FMT>
__device__ __forceinline__ u32x4 f8x8_to_f16(uint32_t lo, uint32_t hi) {
  return u32x4{f8pair_to_f16<FMT>(lo, false), f8pair_to_f16<FMT>(lo, true), f8pair_to_f16<FMT>(hi, false),
               f8pair_to_f16<FMT>(hi, true)};
}

// 8 FP8 bytes from p with element stride s (bytes), the first n of them
// (zero past), packed as two words.
__device__ __forceinline__ void load_partial8_b(const uint8_t* p, int64_t s, int n, uint32_t& lo, uint32_t& hi) {
  uint32_t b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = e < n ? (uint32_t)p[e * s] : 0u;
  lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
  hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
}

// 8 consecutive k of A row m from k0, zero past M or at/after ke.
__device__ __forceinline__ u32x4 dec_load_a(const DecArgs& a, int64_t m, int64_t k0, int64_t ke) {
  if (m >= a.M || k0 >= ke) return zero4();
  const uint16_t* p = a.A + m * a.lda_m + k0 * a.lda_k;
  const int nk = (ke - k0 >= 8) ? 8 : (int)(ke - k0);
  if (a.a_vec && nk == 8) return *reinterpret_cast<const u32x4*>(p);
  return load_partial8(p, a.lda_k, nk);
}

// The same for FP8 A of format FMT (strides in bytes), widened to binary16.
template <int FMT>
__device__ __forceinline__ u32x4 dec_load_a8(const DecArgs& a, int64_t m, int64_t k0, int64_t ke) {
  if (m >= a.M || k0 >= ke) return zero4();
  const uint8_t* p = reinterpret_cast<const uint8_t*>(a.A) + m * a.lda_m + k0 * a.lda_k;
  const int nk = (ke - k0 >= 8) ? 8 : (int)(ke - k0);
  uint32_t lo, hi;
  if (a.a_vec && nk == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    lo = v.x;
    hi = v.y;
  } else {
    load_partial8_b(p, a.lda_k, nk, lo, hi);
  }
  return f8x8_to_f16<FMT>(lo, hi);
}

// The k loop of one wave over its units (u = w, w + 4, ...) of [kb, ke).
// FULL: every unit lies inside the range and the 8 columns of every lane
// are inside N, so the B loads carry no masks and no branches; otherwise
// each load is masked on its own.  AVEC (with FULL): A rows are 16-byte
// vectors, read unmasked (rows past M from row 0, then zeroed); without it
// A is read element by element (M <= 64 rows, a small share of the bytes),
// so an A with unaligned rows (K odd, say) keeps B's full-width loads.
// F8 >= 0: FP8 A and B (formats F8 / 2 and F8 % 2), loaded as 8-byte
// vectors and widened to binary16: N-contiguous B as 8 columns of a k-row
// per lane (a wave's load instruction still covers 4 rows x 128 bytes,
// whole lines; bcol then points at bytes), K-contiguous B as 8 k of one
// column (16 columns x 32 bytes per instruction).
template <int MT, int DT, bool FULL, bool BK, bool AVEC = FULL, int F8 = -1>
__device__ __forceinline__ void dec_units(const DecArgs& a, f32x4 (&acc)[MT / 16][8], int w, int g, int c,
                                          int64_t kb, int64_t ke, const uint16_t* bcol, int nvalid,
                                          int64_t n0) {
  constexpr int FA = MT / 16;
  constexpr int FMA_ = F8 < 0 ? 0 : F8 / 2, FMB = F8 < 0 ? 0 : F8 % 2;
  const uint8_t* bcol8 = reinterpret_cast<const uint8_t*>(bcol);
  constexpr int UPW = dec_upw<MT>();
  const int64_t units = (ke - kb + kDecUnit - 1) / kDecUnit;
  for (int64_t u0 = w; u0 < units; u0 += kDecWaves * UPW) {
    // All loads of UPW units first (A, then B), arithmetic after.  A unit
    // past the range end is read from the last unit (cache hits) and its
    // operands replaced by zeros, so the code has no branch and the waits
    // before each unit's arithmetic count only the loads issued before it.
    u32x4 av[UPW][FA], bv[UPW][8];
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      const int64_t u = u0 + (int64_t)kDecWaves * i;
      const bool live = u < units;
      const int64_t k0 = kb + (live ? u : units - 1) * kDecUnit + 8 * g;
#pragma unroll
      for (int fa = 0; fa < FA; ++fa) {
        const int64_t m = 16 * fa + c;
        if constexpr (F8 >= 0) {
          if constexpr (FULL && AVEC) {
            const u32x2 x = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(a.A) +
                                                            (m < a.M ? m : 0) * a.lda_m + k0);
            av[i][fa] = (live && m < a.M) ? f8x8_to_f16<FMA_>(x[0], x[1]) : zero4();
          } else {
            av[i][fa] = live ? dec_load_a8<FMA_>(a, m, k0, ke) : zero4();
          }
        } else if constexpr (FULL && AVEC) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(a.A + (m < a.M ? m : 0) * a.lda_m + k0);
          av[i][fa] = (live && m < a.M) ? x : zero4();
        } else {
          av[i][fa] = live ? dec_load_a(a, m, k0, ke) : zero4();
        }
      }
    }
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      const int64_t u = u0 + (int64_t)kDecWaves * i;
      const bool live = u < units;
      const int64_t k0 = kb + (live ? u : units - 1) * kDecUnit + 8 * g;
      if constexpr (BK && F8 >= 0) {
        // FP8 [N, K] rows: 8 bytes of column 16 f + c, k0 .. k0 + 7.
#pragma unroll
        for (int f = 0; f < 8; ++f) {
          const int64_t n = n0 + 16 * f + c;
          const uint8_t* q = reinterpret_cast<const uint8_t*>(a.B) + n * a.ldb_n + k0;
          uint32_t lo, hi;
          if constexpr (FULL) {
            const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(q));
            lo = x[0];
            hi = x[1];
          } else {
            const int64_t d = ke - k0;
            const int nk = (live && n < a.N) ? (d < 0 ? 0 : (d < 8 ? (int)d : 8)) : 0;
            if (nk == 8) {
              const u32x2 x = *reinterpret_cast<const u32x2*>(q);
              lo = x[0];
              hi = x[1];
            } else {
              load_partial8_b(q, 1, nk, lo, hi);
            }
          }
          bv[i][f] = f8x8_to_f16<FMB>(lo, hi);
        }
      } else if constexpr (BK) {
        // Column 16 f + c of the strip, k0 .. k0 + 7; columns past N read
        // zeros (FULL: the whole strip is inside N).
#pragma unroll
        for (int f = 0; f < 8; ++f) {
          const int64_t n = n0 + 16 * f + c;
          const uint16_t* q = a.B + n * a.ldb_n + k0;
          if constexpr (FULL) {
            if constexpr (MT <= 32)
              bv[i][f] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q));
            else
              bv[i][f] = *reinterpret_cast<const u32x4*>(q);
          } else {
            const int64_t d = ke - k0;
            const int nk = d < 0 ? 0 : (d < 8 ? (int)d : 8);
            bv[i][f] = (live && n < a.N && nk > 0)
                           ? (nk == 8 ? *reinterpret_cast<const u32x4*>(q) : load_partial8(q, 1, nk))
                           : zero4();
          }
        }
      } else if constexpr (F8 >= 0) {
        // FP8 rows: 8 bytes per lane and k-row, masked as the 16-bit rows
        // below (N % 16 == 0, so a lane's 8 columns are all inside N or all
        // past it).
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x2* q = reinterpret_cast<const u32x2*>(bcol8 + (k0 + j) * a.ldb_k);
          u32x2 x;
          if constexpr (FULL) {
            if constexpr (MT <= 32)
              x = __builtin_nontemporal_load(q);
            else
              x = *q;
            bv[i][j] = f8x8_to_f16<FMB>(x[0], x[1]);
          } else {
            if (live && nvalid == 8 && k0 + j < ke) {
              x = *q;
              bv[i][j] = f8x8_to_f16<FMB>(x[0], x[1]);
            } else {
              bv[i][j] = zero4();
            }
          }
        }
      } else if constexpr (FULL) {
        // (a dead unit's A operand is zero, so its B rows need no mask).
        // B is read once: non-temporal loads keep it from displacing what
        // the caches hold (M = 1: 10.6 -> 10.1 us per call); with 64 rows
        // of A, whose re-reads by every strip come from L2, plain loads
        // were faster (16.2 against 18.0 us).
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x4* q = reinterpret_cast<const u32x4*>(bcol + (k0 + j) * a.ldb_k);
          if constexpr (MT <= 32)
            bv[i][j] = __builtin_nontemporal_load(q);
          else
            bv[i][j] = *q;
        }
      } else {
        // Whole 8-column chunks load as one vector: the decode plan takes
        // only 16-byte aligned B rows with ldb_k % 8 == 0 (and [N, K] rows
        // with ldb_n % 8 == 0), so such a chunk is 16-byte aligned.  A
        // ragged last K range with element loads ran 4x slower than the other
        // ranges and held the whole launch (1 x 2048 x 7170: 22.2 us of
        // kernel time, now 8.0-8.8, against 5.4 for K = 7168).
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint16_t* q = bcol + (k0 + j) * a.ldb_k;
          bv[i][j] = (live && nvalid > 0 && k0 + j < ke)
                         ? (nvalid == 8 ? *reinterpret_cast<const u32x4*>(q) : load_partial8(q, 1, nvalid))
                         : zero4();
        }
      }
    }
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      u32x4 bt[8];
      if constexpr (BK) {
#pragma unroll
        for (int f = 0; f < 8; ++f) bt[f] = bv[i][f];
      } else {
        transpose8x8(bv[i], bt);
      }
#pragma unroll
      for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int fa = 0; fa < FA; ++fa)
          acc[fa][f] = mfma<16, DT>(__builtin_bit_cast(f16x8, av[i][fa]), __builtin_bit_cast(f16x8, bt[f]),
                                    acc[fa][f]);
    }
  }
}

// F8 >= 0: FP8 A and B of formats (F8 / 2, F8 % 2), binary16 out (DT =
// DT_F16); an N-contiguous B strip is then 128 bytes wide per k-row.
template <int MT, int DT, bool BK = false, int F8 = -1>
__global__ __launch_bounds__(64 * kDecWaves) void decode_kernel(DecArgs a) {
  static_assert(MT % 16 == 0 && MT <= 64, "16, 32, 48 or 64 rows of A");
  static_assert(F8 < 0 || DT == DT_F16, "FP8: binary16 out");
  constexpr int FA = MT / 16;
  __shared__ __attribute__((aligned(16))) float red[kDecWaves][16][16][8];   // [wave][m][c][f]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int g = lane >> 4, c = lane & 15;
  const int64_t nb = blockIdx.x % a.GN, s = blockIdx.x / a.GN;
  const int64_t kb = s * a.kr;
  const int64_t ke = (kb + a.kr < a.K) ? kb + a.kr : a.K;
  const int64_t n0 = nb * kDecCols + c * 8;   // N-contiguous B: this lane's 8 columns
  const int nvalid = (n0 + 8 <= a.N) ? 8 : (n0 < a.N ? (int)(a.N - n0) : 0);
  const uint16_t* bcol = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(a.B) +
                                                          (nvalid > 0 ? n0 : 0) * (F8 >= 0 ? 1 : 2));
  const int64_t sn0 = nb * kDecCols;            // the strip's first column

  f32x4 acc[FA][8];
#pragma unroll
  for (int i = 0; i < FA; ++i)
#pragma unroll
    for (int f = 0; f < 8; ++f) acc[i][f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Uniform per workgroup: whole strip inside N and whole units (and, for
  // A's vector loads, 16-byte A rows): A rows that are not 16-byte aligned
  // keep the unmasked B loads (1 x 2048 x 7168 with rows of 7170 halves:
  // 5.5 us of kernel time, as for aligned rows).
  const bool full = (nb + 1) * kDecCols <= a.N && (ke - kb) % kDecUnit == 0;
  if (full && a.a_vec)
    dec_units<MT, DT, true, BK, true, F8>(a, acc, w, g, c, kb, ke, bcol, nvalid, sn0);
  else if (full)
    dec_units<MT, DT, true, BK, false, F8>(a, acc, w, g, c, kb, ke, bcol, nvalid, sn0);
  else
    dec_units<MT, DT, false, BK, false, F8>(a, acc, w, g, c, kb, ke, bcol, nvalid, sn0);

  // Sum the waves in ascending order, 16 rows of A at a time; thread t < 256
  // then owns row t / 16 and the 8 columns 8 (t % 16) .. + 7 of the block.
  const int tm = (tid >> 4) & 15, tc = tid & 15;
  const bool summer = tid < 256;
  const int64_t col = nb * kDecCols + tc * 8;
  const int cvalid = (col + 8 <= a.N) ? 8 : (col < a.N ? (int)(a.N - col) : 0);
#pragma unroll
  for (int fa = 0; fa < FA; ++fa) {
    if (16 * fa >= a.M) break;   // uniform across the workgroup
    if (fa > 0) __syncthreads();  // red is free
    // red[w][m] holds the strip's 128 columns in order (the view [c][f] is
    // column 8 c + f); K-contiguous B leaves lane c with columns 16 f + c.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* dst = &red[w][4 * g + r][0][0];
      if constexpr (BK) {
#pragma unroll
        for (int f = 0; f < 8; ++f) dst[16 * f + c] = acc[fa][f][r];
      } else {
        *reinterpret_cast<f32x4*>(dst + 8 * c) = f32x4{acc[fa][0][r], acc[fa][1][r], acc[fa][2][r], acc[fa][3][r]};
        *reinterpret_cast<f32x4*>(dst + 8 * c + 4) =
            f32x4{acc[fa][4][r], acc[fa][5][r], acc[fa][6][r], acc[fa][7][r]};
      }
    }
    __syncthreads();
    const int64_t m = 16 * fa + tm;
    if (summer && m < a.M && cvalid > 0) {
      float t[8];
#pragma unroll
      for (int f = 0; f < 8; ++f) t[f] = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kDecWaves; ++ww) {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(&red[ww][tm][tc][0]);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(&red[ww][tm][tc][4]);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          t[f] += lo[f];
          t[f + 4] += hi[f];
        }
      }
      if (a.S == 1) {
        uint16_t* o = a.C + m * a.ldc + col;
        if (a.c_vec && cvalid == 8) {
          uint32_t h[4];
#pragma unroll
          for (int d = 0; d < 4; ++d)
            h[d] = (uint32_t)cvt_out<DT>(t[2 * d]) | ((uint32_t)cvt_out<DT>(t[2 * d + 1]) << 16);
          *reinterpret_cast<u32x4*>(o) = u32x4{h[0], h[1], h[2], h[3]};
        } else {
#pragma unroll
          for (int f = 0; f < 8; ++f)
            if (f < cvalid) o[f] = cvt_out<DT>(t[f]);
        }
      } else {
        float* o = a.P + (s * a.M + m) * a.N + col;
        if ((a.N & 3) == 0 && cvalid == 8) {
          *reinterpret_cast<f32x4*>(o) = f32x4{t[0], t[1], t[2], t[3]};
          *reinterpret_cast<f32x4*>(o + 4) = f32x4{t[4], t[5], t[6], t[7]};
        } else {
#pragma unroll
          for (int f = 0; f < 8; ++f)
            if (f < cvalid) o[f] = t[f];
        }
      }
    }
  }
}

}  // namespace gemmf16
