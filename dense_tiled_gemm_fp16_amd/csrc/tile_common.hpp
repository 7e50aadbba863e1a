// Device-side building blocks shared by the GEMM kernels (gfx950 / CDNA4).
//
// Operand tiles in LDS.  Both operands are staged in one format: an operand
// tile has R "rows" (output rows m for A, output columns n for B) and BK
// reduction indices.  It is stored as 16-byte cells, one cell = 8 consecutive
// k of one row (a "k-octet"), because that is exactly what one lane feeds a
// v_mfma_f32_{32x32x16,16x16x32}_f16 per operand.  Cell (r, c) of octet c
// lives at
//     cell index  c * R + (r ^ swz(r, c)),   swz(r, c) = (c ^ (r >> 3)) & 7
// The XOR keeps r inside its aligned group of 8, so the MFMA read pattern
// (lanes = 8 consecutive rows of one octet) touches 8 distinct 16-byte bank
// groups, and so do the two write patterns: a K-contiguous copy (one row, 8
// octets per 8 lanes) and an M/N-contiguous copy (8 rows spaced 8 apart, one
// octet).  This is the bank-conflict-avoiding shared-memory swizzle of the
// TileLang tutorial (ch. 14, rung 4), re-derived for the gfx950 LDS.
//
// Operand load paths (global -> registers -> LDS), picked per operand on the
// host from its strides and alignment:
//   KVEC   stride along k is 1, row stride a multiple of 8, base 16-byte
//          aligned: one 16-byte global load is one cell.
//   RVEC   stride along the row dimension is 1 (A M-contiguous, B
//          N-contiguous), k stride a multiple of 8, base aligned: a thread
//          loads 8 k-rows x 8 rows as eight 16-byte vectors and transposes
//          the 8x8 block of halves in registers into 8 cells.
//   GATHER anything else: element-wise 2-byte loads, each masked.
// Every path masks on both axes with zero fill (Triton article, section
// "three dimensions that do not divide"): a row outside the view or a k at or
// beyond the range end contributes 0 and is never read; K is never wrapped.
// All address arithmetic is int64 (same article, section "addresses and
// bounds in one short kernel").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemmf16 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum LoadPath { PATH_GATHER = 0, PATH_KVEC = 1, PATH_RVEC = 2 };

// Element formats of A, B and C (accumulation is fp32 for both).  Loads and
// LDS staging move 16-bit elements whatever the format; only the MFMA, the
// VALU decode of inputs and the final conversion differ.
enum DType { DT_F16 = 0, DT_BF16 = 1 };
// Operand formats of a call: the two 16-bit formats, then the four pairs of
// FP8 formats (A, B) = (E4M3|E5M2, E4M3|E5M2) at DT_F8 + 2 * fmt_a + fmt_b
// (binary16 output).
constexpr int DT_F8 = 2, NDT = 6;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// fp32 -> output element, round to nearest even (v_cvt_f16_f32 /
// v_cvt_pk_bf16_f32 in the default rounding mode).
template <int DT>
__device__ __forceinline__ uint16_t cvt_out(float v) {
  if constexpr (DT == DT_F16)
    return __builtin_bit_cast(uint16_t, (_Float16)v);
  else
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Input element -> fp32 (exact for both formats).
template <int DT>
__device__ __forceinline__ float cvt_in(uint16_t h) {
  if constexpr (DT == DT_F16)
    return (float)__builtin_bit_cast(_Float16, h);
  else
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}

__device__ __forceinline__ int swz(int r, int c) { return (c ^ (r >> 3)) & 7; }

// Byte offset of cell (r, c) in an operand tile with R rows.
template <int R>
__device__ __forceinline__ int cell_off(int r, int c) {
  return (c * R + (r ^ swz(r, c))) * 16;
}

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// 8 halves starting at p, element i kept only if i < nvalid (0..8); others 0.
// Element-wise loads: used for ragged cells and the gather path.
__device__ __forceinline__ u32x4 load_partial8(const uint16_t* p, int64_t step, int nvalid) {
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (e < nvalid) ? (uint32_t)p[e * step] : 0u;
  return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// Transpose an 8x8 block of halves: in[e] holds row e (8 halves); returns
// out[j] = column j (8 halves, element e from in[e]).
__device__ __forceinline__ void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int d = j >> 1;
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = in[2 * p][d], hi = in[2 * p + 1][d];
      w[p] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    out[j] = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// One operand's global -> register -> LDS staging for an R x BK tile.
//   base  : operand base pointer
//   s_r   : element stride along the tile's rows (lda_m for A, ldb_n for B)
//   s_k   : element stride along k (lda_k for A, ldb_k for B)
//   R_tot : valid extent of the row dimension (M for A, N for B)
template <int R, int BK, int NT, int PATH>
struct OperandStage {
  static constexpr int OCT = BK / 8;
  static_assert(BK % 8 == 0 && R % 8 == 0, "tile shape");
  // KVEC / GATHER: cells, thread t takes cells t, t+NT, ...; octet fixed per thread.
  static constexpr int CELLS = R * OCT;
  static constexpr int CPT = (CELLS + NT - 1) / NT;
  static_assert(PATH == PATH_RVEC || NT % OCT == 0, "octet must be fixed per thread");
  // RVEC: units of 8 k x 8 rows.
  static constexpr int UNITS = OCT * (R / 8);
  static constexpr int UPT = (UNITS + NT - 1) / NT;
  static constexpr int NREG = (PATH == PATH_RVEC) ? UPT * 8 : CPT;

  u32x4 v[NREG];
  const uint16_t* base;
  int64_t s_r, s_k, R_tot, r0;
  int tid;

  __device__ __forceinline__ void init(const uint16_t* b, int64_t sr, int64_t sk, int64_t rtot,
                                       int64_t row0, int t) {
    base = b; s_r = sr; s_k = sk; R_tot = rtot; r0 = row0; tid = t;
  }

  // Load the tile's k range [k0, k0 + BK), clipped at k_end (exclusive).
  //   ROWMASK: some rows of the tile may lie outside [0, R_tot).  Such rows
  //            are read from the last valid row (an in-bounds address) and
  //            replaced by zeros, or skipped entirely on the RVEC path.
  //   KMASK:   the k range may end inside the tile (the last K step).
  // With neither flag the loads are straight-line code with no branches.
  template <bool ROWMASK, bool KMASK>
  __device__ __forceinline__ void load(int64_t k0, int64_t k_end) {
    if constexpr (PATH == PATH_RVEC) {
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int unit = tid + NT * u;
        if (UNITS % NT != 0 && unit >= UNITS) break;
        const int g = unit % (R / 8), c = unit / (R / 8);
        const int64_t rr = r0 + 8 * g;            // first row of the 8-row group
        const int64_t kk = k0 + 8 * c;            // first k of the octet
        int nk = 8;
        if constexpr (KMASK) {
          const int64_t d = k_end - kk;
          nk = d < 0 ? 0 : (d < 8 ? (int)d : 8);
        }
        int nr = 8;
        if constexpr (ROWMASK) {
          const int64_t d = R_tot - rr;
          nr = d < 0 ? 0 : (d < 8 ? (int)d : 8);
        }
        const uint16_t* p = base + (nr > 0 ? rr : 0) + (nk > 0 ? kk : 0) * s_k;
        if (!ROWMASK || nr == 8) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            v[u * 8 + e] = (!KMASK || e < nk) ? *reinterpret_cast<const u32x4*>(p + e * s_k) : zero4();
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            v[u * 8 + e] = (e < nk && nr > 0) ? load_partial8(p + e * s_k, 1, nr) : zero4();
        }
      }
    } else {
      const int c = tid % OCT;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int cell = tid + NT * i;
        if (CELLS % NT != 0 && cell >= CELLS) break;
        int64_t rr = r0 + cell / OCT;
        bool rv = true;
        if constexpr (ROWMASK) {
          rv = rr < R_tot;
          rr = rv ? rr : R_tot - 1;
        }
        const int64_t kk = k0 + 8 * c;
        int nk = 8;
        if constexpr (KMASK) {
          const int64_t d = k_end - kk;
          nk = d < 0 ? 0 : (d < 8 ? (int)d : 8);
        }
        const uint16_t* p = base + rr * s_r + (nk > 0 ? kk : 0) * s_k;
        u32x4 x;
        if constexpr (PATH == PATH_KVEC) {
          if (!KMASK || nk == 8)
            x = *reinterpret_cast<const u32x4*>(p);
          else
            x = load_partial8(p, 1, nk);
        } else {
          x = load_partial8(p, s_k, nk);
        }
        if constexpr (ROWMASK) x = rv ? x : zero4();
        v[i] = x;
      }
    }
  }

  __device__ __forceinline__ void store(char* lds) const {
    if constexpr (PATH == PATH_RVEC) {
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int unit = tid + NT * u;
        if (UNITS % NT != 0 && unit >= UNITS) break;
        const int g = unit % (R / 8), c = unit / (R / 8);
        u32x4 t[8];
        transpose8x8(&v[u * 8], t);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<u32x4*>(lds + cell_off<R>(8 * g + j, c)) = t[j];
      }
    } else {
      const int c = tid % OCT;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int cell = tid + NT * i;
        if (CELLS % NT != 0 && cell >= CELLS) break;
        *reinterpret_cast<u32x4*>(lds + cell_off<R>(cell / OCT, c)) = v[i];
      }
    }
  }
};

// Workgroup id -> output tile (pid_m, pid_n).
//
// Grouped ("panel") rasterisation as in the TileLang tutorial (ch. 14, rung 4,
// threadblock rasterisation for L2 reuse) and the Triton article (section
// "neighbouring programs share cache"): consecutive ids walk down a panel of
// `panel` tile-rows before moving to the next tile-column, so workgroups that
// run together share A row-panels and B column-panels in cache.  Panels run
// along the longer side of the tile grid (the direction rule of the TileLang
// tutorial, sections 1.5 and 6.1): with more tile-columns than tile-rows a
// panel is `panel` tile-columns wide and consecutive ids walk across it.
//
// XCD remap (gfx950-specific): the dispatcher hands consecutive workgroup ids
// to the 8 XCDs round-robin, and each XCD has its own L2.  Id w is first
// renumbered to (w % 8) * (T / 8) + w / 8, so each XCD receives one contiguous
// run of the panel order and its panels stay in its own L2.  Ids past the
// last multiple of 8 keep their place.
__device__ __forceinline__ void raster_tile(int64_t w, int64_t GM, int64_t GN, int panel,
                                            int64_t& pm, int64_t& pn) {
  const int64_t T = GM * GN;
  if (panel <= 0) {  // plain row-major order, no remap
    pm = w / GN;
    pn = w % GN;
    return;
  }
  const int64_t per = T / 8;
  if (w < per * 8) w = (w % 8) * per + w / 8;
  const bool by_cols = GN > GM;             // panels of tile-columns
  const int64_t R = by_cols ? GN : GM, X = by_cols ? GM : GN;
  const int64_t group_size = (int64_t)panel * X;
  const int64_t group = w / group_size;
  const int64_t first = group * panel;
  int64_t rows = R - first;
  if (rows > panel) rows = panel;
  const int64_t in_group = w - group * group_size;
  const int64_t r = first + in_group % rows, x = in_group / rows;
  pm = by_cols ? x : r;
  pn = by_cols ? r : x;
}

}  // namespace gemmf16
