// Host side of libgemmf16: argument validation, planning (kernel family,
// tile, K split, raster panel, operand load paths) and launches.  The C-ABI
// is declared and documented in include/gemm_f16.h.
//
// Validation mirrors the Triton article's wrapper (section "addresses and
// bounds in one short kernel"): shapes must be non-empty, strides positive,
// and the output must not share storage with the inputs (its ownership
// paragraph: one writer per output, no program may overwrite data another
// program still has to read).  Everything is checked before the first HIP
// call, so on any error nothing is enqueued and C is untouched.
//
// Kernel choice follows the TileLang tutorial's variant criteria (ch. 14,
// section 4.1: split K when the output tiles cannot fill the compute units
// and K is large) and the decode/prefill distinction of the tiling tutorial
// (section 04: with very few rows of A the product is a weight-streaming,
// bandwidth-bound problem).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/gemm_f16.h"
#include "decode_kernel.hpp"
#include "group_kernel.hpp"
#include "pack_kernel.hpp"
#include "reduce_kernel.hpp"
#include "tiles.hpp"

using namespace gemmf16;

// Workspace of gemm_f16_noalloc: one fixed array per GPU, loaded with the
// code object.  In host code `scratch` names a host-side stand-in, not device
// memory; its device address is taken once per device with
// hipGetSymbolAddress (with that device current, see scratch_address) and
// only that address is ever passed to kernels or used by host calls.
static __device__ __align__(256) unsigned char scratch[GEMM_F16_SCRATCH_BYTES];

namespace {

constexpr int kVersion = 100;  // 0.1.0

typedef void (*kfn_dec)(DecArgs);
typedef void (*kfn_reduce)(const float*, int, int64_t, int64_t, uint16_t*, int64_t, int);

const TileInfo& tile_info(int id) {
  // Unused ids (0, 9 to 12) hold an empty entry: no kernels, nt == 0.
  static const TileInfo table[TILE_MAX + 1] = {
      TileInfo{},        tile_info_t128(), tile_info_t64x32(),    tile_info_s16(),
      tile_info_s32(),   tile_info_s64(),  tile_info_t256(),      tile_info_dma128(),
      tile_info_dma64x128(), TileInfo{},   TileInfo{},            TileInfo{},
      TileInfo{},        tile_info_dma256w8b(), tile_info_dma256a128(), tile_info_f8()};
  return table[id];
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Device address of `scratch` on the current device, taken once per device.
int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GEMM_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GEMM_ERR_HIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return GEMM_OK;
}

// Compute units of the current device, cached per device.
int device_cus(int* cus) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GEMM_ERR_HIP;
  if (dev >= 0 && dev < 64) {
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return GEMM_OK;
    }
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
    return GEMM_ERR_HIP;
  if (dev >= 0 && dev < 64) cache[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return GEMM_OK;
}

// Largest element offset of a rows x cols view, or false on int64 overflow.
bool view_span(int64_t rows, int64_t cols, int64_t sr, int64_t sc, int64_t* out) {
  int64_t a, b, s;
  if (__builtin_mul_overflow(rows - 1, sr, &a) || __builtin_mul_overflow(cols - 1, sc, &b) ||
      __builtin_add_overflow(a, b, &s) || s > INT64_MAX / 2 - 1)
    return false;
  *out = s;
  return true;
}

bool ranges_overlap(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) {
  return a0 < b1 && b0 < a1;
}

int classify(const void* base, int64_t s_r, int64_t s_k) {
  const bool aligned = ((uintptr_t)base & 15u) == 0;
  if (aligned && s_k == 1 && s_r % 8 == 0) return PATH_KVEC;
  if (aligned && s_r == 1 && s_k % 8 == 0) return PATH_RVEC;
  return PATH_GATHER;
}

struct Plan {
  int variant, tile_id, split, panel, a_path, b_path, c_vec;
  int dec_mt;   // > 0: the decode kernel with this many rows of A (16, 32 or 64)
  int red_elem;   // split reduction: one thread per output (else per 4 outputs)
  int64_t GM, GN, grid, grid2, k_split;
  int64_t sk_tiles;  // STREAMK: tiles split over K after the whole waves
  bool pack;         // B is packed into the workspace first (see maybe_pack)
  size_t pack_bytes; // its size; stream-K partials follow it
  bool pack_a;       // A is realigned into the front of the workspace first
  size_t pack_a_bytes;   // its size (a multiple of 256); packed B and partials follow
  int64_t lda_p;     // row stride of the realigned A (K rounded up to 64)
  size_t ws;
};

struct Call {
  int dt;  // element format of A, B and C (DT_F16 or DT_BF16)
  const void *A, *B, *C;
  int64_t lda_m, lda_k, ldb_k, ldb_n, ldc, M, N, K;
  int64_t spanA, spanB, spanC;
};

int validate(const Call& c) {
  if (!c.A || !c.B || !c.C) return GEMM_ERR_NULL;
  if (c.M <= 0 || c.N <= 0 || c.K <= 0) return GEMM_ERR_SHAPE;
  if (c.lda_m <= 0 || c.lda_k <= 0 || c.ldb_k <= 0 || c.ldb_n <= 0) return GEMM_ERR_STRIDE;
  if (c.ldc < c.N) return GEMM_ERR_LDC;
  return GEMM_OK;
}

// Bytes per A and B element (C is always 16-bit).
uintptr_t in_bytes(const Call& c) { return c.dt >= DT_F8 ? 1 : 2; }

int spans(Call& c) {
  if (!view_span(c.M, c.K, c.lda_m, c.lda_k, &c.spanA) ||
      !view_span(c.K, c.N, c.ldb_k, c.ldb_n, &c.spanB) ||
      !view_span(c.M, c.N, c.ldc, 1, &c.spanC))
    return GEMM_ERR_SHAPE;
  const uintptr_t a0 = (uintptr_t)c.A, a1 = a0 + in_bytes(c) * (uintptr_t)(c.spanA + 1);
  const uintptr_t b0 = (uintptr_t)c.B, b1 = b0 + in_bytes(c) * (uintptr_t)(c.spanB + 1);
  const uintptr_t c0 = (uintptr_t)c.C, c1 = c0 + 2 * (uintptr_t)(c.spanC + 1);
  if (a1 < a0 || b1 < b0 || c1 < c0) return GEMM_ERR_SHAPE;
  if (ranges_overlap(c0, c1, a0, a1) || ranges_overlap(c0, c1, b0, b1)) return GEMM_ERR_ALIAS;
  return GEMM_OK;
}

int check_opts(const gemm_f16_opts* o) {
  if (!o) return GEMM_OK;
  if (o->variant < GEMM_VARIANT_AUTO || o->variant > GEMM_VARIANT_STREAMK) return GEMM_ERR_OPTS;
  if (o->split_k < 0 || o->split_k > 256) return GEMM_ERR_OPTS;
  if (!(o->panel == -1 || (o->panel >= 0 && o->panel <= 4096))) return GEMM_ERR_OPTS;
  if (o->tile < 0 || o->tile > TILE_MAX || (o->tile && tile_info(o->tile).nt == 0)) return GEMM_ERR_OPTS;
  return GEMM_OK;
}

// Choose split and derive the per-split K extent (a multiple of BK).
void set_split(Plan& p, int64_t K, int bk, int64_t split) {
  if (split < 1) split = 1;
  int64_t ks = cdiv(cdiv(K, split), bk) * bk;
  p.k_split = ks;
  p.split = (int)cdiv(K, ks);
}

// Workspace and reduction launch of a plan with p.split K ranges.  The
// reduction's shape depends on the output size only, so a forced plan needs
// no device query: small outputs (decode shapes) take one thread per output,
// whose loads of all K ranges are in flight together.
int plan_partials(const Call& c, Plan& p) {
  p.ws = 0;
  p.grid2 = 0;
  p.red_elem = 0;
  if (p.split <= 1) return GEMM_OK;
  int64_t mn, bytes;
  if (__builtin_mul_overflow(c.M, c.N, &mn) || __builtin_mul_overflow(mn, (int64_t)p.split, &bytes) ||
      __builtin_mul_overflow(bytes, (int64_t)4, &bytes) || bytes > INT64_MAX - 256)
    return GEMM_ERR_SHAPE;
  p.ws = (size_t)((bytes + 255) / 256 * 256);
  p.red_elem = mn <= (INT64_C(1) << 18) ? 1 : 0;
  int64_t g2 = p.red_elem ? cdiv(mn, 256) : cdiv(c.M * cdiv(c.N, 4), 256);
  if (g2 > 8192) g2 = 8192;
  p.grid2 = g2;
  return GEMM_OK;
}

bool has_format(const TileInfo& t, int dt) {
  if (dt < 0 || dt >= NDT) return false;
  for (int i = 0; i < 9; ++i)
    if (t.final_fn[dt][i]) return true;
  return false;
}

// Fewer 256x256 tiles than half a wave and a long K: every tile goes to the
// stream-K tail, cut into about cus / tiles K ranges, rather than to the
// 128x128 register-path tile (2048 x 2048 x 8192 ran 1.8x faster so; at
// K = 2048 the main plan was still ahead).
bool small_grid_streamk(const Call& c, int64_t t256, int cus) {
  return 2 * t256 < cus && c.K >= 3072 && c.M >= 256 && c.N >= 256;
}

int64_t max_stride(const Call& c) {
  return std::max(std::max(c.lda_m, c.lda_k), std::max(c.ldb_k, c.ldb_n));
}

// Whether a tile's kernels take this call's format and layout (needs
// p.a_path and p.b_path).
bool tile_takes(const TileInfo& t, const Call& c, const Plan& p) {
  // (FP8 on the 128-wide LDS-DMA tiles reads byte pairs: K even.)
  return t.final_fn[c.dt][p.a_path * 3 + p.b_path] != nullptr &&
         !(c.dt >= DT_F8 && t.id != TILE_F8 && c.K % 2 != 0) &&
         !(t.n_mult && p.b_path == PATH_RVEC && (c.N % t.n_mult != 0 || c.N < t.n_mult)) &&
         !(t.max_k && c.K > t.max_k) && !(t.max_ld && max_stride(c) > t.max_ld);
}

bool dma_tile_takes(const Call& c, const Plan& p) { return tile_takes(tile_info(TILE_DMA256A128), c, p); }

// Whether the 128x128 LDS-DMA tile reads the operands as they lie (fp16,
// K-contiguous A, B either way with N % 8 == 0 when N-contiguous).
bool dma128_reads(const Call& c) {
  Plan q{};
  q.a_path = classify(c.A, c.lda_m, c.lda_k);
  q.b_path = classify(c.B, c.ldb_n, c.ldb_k);
  return tile_takes(tile_info(TILE_DMA128), c, q);
}

constexpr int64_t kPackMinRows = 16384;   // automatic plans pack a K-contiguous B from this M on
constexpr int64_t kPackMinRowsGather = 1024;   // and a B the DMA tile cannot read from this M on
constexpr int32_t kBPathPacked = 3;       // a_path / b_path reported for a packed operand
constexpr int64_t kRealignMinN = 256;     // automatic plans realign an unreadable A from this N on,
constexpr int64_t kRealignMinWorkMC = INT64_C(1) << 33;   // an M-contiguous one from this M N K on
constexpr double kPackMinWork = 134217728.0;   // and pack or realign nothing below 2^27 M N K

bool worth_packing(const Call& c) { return (double)c.M * (double)c.N * (double)c.K >= kPackMinWork; }

// Realigned A: M rows of K rounded up to 64 elements (128-byte rows), the
// whole rounded up to 256 bytes.  0 when the size does not fit.
size_t realign_a_bytes(int64_t M, int64_t K) {
  const int64_t ldp = cdiv(K, 64) * 64;
  int64_t n;
  if (__builtin_mul_overflow(M, ldp, &n) || n > (INT64_MAX - 255) / 2 || cdiv(M, 64) * cdiv(ldp, 128) > INT32_MAX ||
      cdiv(M * cdiv(ldp, 1024), 4) > INT32_MAX)
    return 0;
  return (size_t)((2 * n + 255) / 256 * 256);
}

// The realigning launch: A [M, K] through its strides into Ap [M, ldp].
int launch_realign_a(const uint16_t* A, int64_t lda_m, int64_t lda_k, int64_t M, int64_t K, int64_t ldp,
                     uint16_t* Ap, hipStream_t stream) {
  if (lda_k == 1) {   // rows already K-contiguous: a straight copy into aligned rows
    int64_t nseg = cdiv(ldp, 1024);
    const int64_t blocks = cdiv(M * nseg, 4);
    void* args[] = {&A, &lda_m, &M, &K, &ldp, &nseg, &Ap};
    if (hipLaunchKernel((const void*)realign_a_rows_kernel, dim3((unsigned)blocks), dim3(256), args, 0,
                        stream) != hipSuccess)
      return GEMM_ERR_HIP;
    return GEMM_OK;
  }
  int64_t nbk = cdiv(ldp, 128);
  const int64_t blocks = cdiv(M, 64) * nbk;
  void* args[] = {&A, &lda_m, &lda_k, &M, &K, &ldp, &nbk, &Ap};
  if (hipLaunchKernel((const void*)realign_a_kernel, dim3((unsigned)blocks), dim3(256), args, 0, stream) !=
      hipSuccess)
    return GEMM_ERR_HIP;
  return GEMM_OK;
}

// Pre-packed B: ceil(N/256) panels of ceil(K/32) blocks of 16 KiB (see
// pack_b_kernel).  0 for shapes out of range or too large to count.
size_t packed_b_bytes(int64_t K, int64_t N) {
  if (K <= 0 || N <= 0 || K > (INT64_C(1) << 40) || N > (INT64_C(1) << 40)) return 0;
  int64_t blocks, bytes;
  if (__builtin_mul_overflow(cdiv(N, 256), cdiv(K, 32), &blocks) ||
      __builtin_mul_overflow(blocks, (int64_t)16384, &bytes))
    return 0;
  return (size_t)bytes;
}

// The packing launch: B [K, N] through its strides into Bp.
int launch_pack_b(const uint16_t* B, int64_t ldb_k, int64_t ldb_n, int64_t K, int64_t N, uint16_t* Bp,
                  hipStream_t stream) {
  int64_t S = cdiv(K, 32);
  int64_t slots = (int64_t)(packed_b_bytes(K, N) / 16);
  int kvec = (ldb_k == 1 && ((uintptr_t)B & 15u) == 0 && ldb_n % 8 == 0) ? 1 : 0;
  if (ldb_n == 1 && ldb_k != 1) {   // N-contiguous rows: transposed through LDS, one block per workgroup
    void* rargs[] = {&B, &ldb_k, &K, &N, &S, &Bp};
    if (hipLaunchKernel((const void*)pack_b_rows_kernel, dim3((unsigned)(slots / 1024)), dim3(256), rargs, 0,
                        stream) != hipSuccess)
      return GEMM_ERR_HIP;
    return GEMM_OK;
  }
  if (kvec) {   // K-contiguous aligned rows: a line per 8 threads, over pairs of blocks
    int64_t threads = cdiv(N, 256) * cdiv(S, 2) * 2048;
    void* largs[] = {&B, &ldb_n, &K, &N, &S, &threads, &Bp};
    if (hipLaunchKernel((const void*)pack_b_lines_kernel, dim3((unsigned)cdiv(threads, 256)), dim3(256), largs,
                        0, stream) != hipSuccess)
      return GEMM_ERR_HIP;
    return GEMM_OK;
  }
  void* args[] = {&B, &ldb_k, &ldb_n, &K, &N, &S, &slots, &Bp, &kvec};
  if (hipLaunchKernel((const void*)pack_b_kernel, dim3((unsigned)cdiv(slots, 256)), dim3(256), args, 0,
                      stream) != hipSuccess)
    return GEMM_ERR_HIP;
  return GEMM_OK;
}

// The FP8 packing launch: B [K, N] bytes through their strides into Bp.
int launch_pack_b8(const uint8_t* B, int64_t ldb_k, int64_t ldb_n, int64_t K, int64_t N, uint8_t* Bp,
                   hipStream_t stream) {
  int64_t S = cdiv(K, 64);
  int64_t slots = (int64_t)(packed_b_bytes(cdiv(K, 2), N) / 16);
  void* args[] = {&B, &ldb_k, &ldb_n, &K, &N, &S, &slots, &Bp};
  if (hipLaunchKernel((const void*)pack_b8_kernel, dim3((unsigned)cdiv(slots, 256)), dim3(256), args, 0,
                      stream) != hipSuccess)
    return GEMM_ERR_HIP;
  return GEMM_OK;
}

// The product launch on a packed B (main variant of the 256 x 256 tile, no
// split): A K-contiguous with 16-byte aligned rows at most max_ld apart.
int launch_packed_product(int dt, const void* A, int64_t lda_m, int64_t lda_k, const void* Bp, void* C,
                          int64_t ldc, int64_t M, int64_t N, int64_t K, int panel, hipStream_t stream) {
  const TileInfo& ti = tile_info(TILE_DMA256A128);
  KArgs a;
  a.A = (const uint16_t*)A;
  a.lda_m = lda_m;
  a.lda_k = lda_k;
  a.B = (const uint16_t*)Bp;
  a.ldb_k = 1;
  a.ldb_n = cdiv(K, 32) * 8192;   // elements per 256-column panel
  a.C = (uint16_t*)C;
  a.ldc = ldc;
  a.W = nullptr;
  a.M = M;
  a.N = N;
  a.K = K;
  a.k_split = K;
  a.GM = cdiv(M, ti.bm);
  a.GN = cdiv(N, ti.bn);
  a.panel = panel;
  a.c_vec = (((uintptr_t)C & 7u) == 0 && (ldc & 3) == 0) ? 1 : 0;
  a.g_off = nullptr;
  a.g_tiles = nullptr;
  a.ldb_g = 0;
  a.G = 0;
  a.sk_first = 0;
  a.sk_tiles = 0;
  a.split_xcd = 0;
  int64_t grid;
  if (__builtin_mul_overflow(a.GM, a.GN, &grid) || grid > INT32_MAX) return GEMM_ERR_SHAPE;
  void* args[] = {&a};
  if (hipLaunchKernel((const void*)ti.packed_fn[dt], dim3((unsigned)grid), dim3(ti.nt), args, 0,
                      stream) != hipSuccess)
    return GEMM_ERR_HIP;
  return GEMM_OK;
}

// K-contiguous B under the 256 x 256 tiles: their K-major stages take half
// a cache line per B row per DMA, about 5% slower than an N-contiguous B.
// With many row tiles over each B panel, one packing pass over B (the
// pre-packed layout, whole lines per DMA) costs less than that, so an
// automatic MAIN or STREAMK plan packs B into the front of the workspace
// (stream-K partials follow it) and runs the packed-B kernels.  The FP8
// kernel's K-major 64-k stages have the same half-line DMA; a K-contiguous
// FP8 B packs as 16-bit byte pairs (K even) or byte by byte.  (Its
// N-contiguous B, read with the transposing LDS read, is as fast as the
// packed stages, so the packing pass would only add time.)  A B the DMA
// cannot read at all (any_b) is packed for MAIN and STREAMK plans from 1024
// rows and for SPLITK plans on the 256 x 256 tile from 256 rows, their
// partials after it.
void maybe_pack(const Call& c, int variant, bool allow_pack, Plan& p, bool any_b) {
  const TileInfo& ti = tile_info(p.tile_id);
  const bool f8 = c.dt >= DT_F8;
  if (!allow_pack || variant != GEMM_VARIANT_AUTO || p.b_path != PATH_KVEC) return;
  const bool family = p.variant == GEMM_VARIANT_STREAMK || (p.variant == GEMM_VARIANT_MAIN && p.split == 1) ||
                      (p.variant == GEMM_VARIANT_SPLITK && any_b);
  const bool kernels = ti.packed_fn[c.dt] && ti.packed_partial_fn[c.dt];
  const bool tile = f8 || (p.tile_id == TILE_DMA256A128 && c.K <= ti.max_k);
  const int64_t min_rows = !any_b ? kPackMinRows : (p.variant == GEMM_VARIANT_SPLITK ? 256 : kPackMinRowsGather);
  if (!family || !kernels || !tile || c.M < min_rows) return;
  const size_t bytes = packed_b_bytes(f8 ? cdiv(c.K, 2) : c.K, c.N);
  if (bytes == 0 || p.ws > SIZE_MAX - bytes) return;
  p.pack = true;
  p.pack_bytes = bytes;
  p.ws += bytes;
}

// Adds the realigned A in front of the workspace (false if the sizes overflow).
bool add_realign(const Call& c, Plan& p) {
  const size_t bytes = realign_a_bytes(c.M, c.K);
  if (bytes == 0 || p.ws > SIZE_MAX - bytes) return false;
  p.pack_a = true;
  p.pack_a_bytes = bytes;
  p.lda_p = cdiv(c.K, 64) * 64;
  p.ws += bytes;
  return true;
}

// allow_pack: automatic plans may pack B; allow_realign: and realign A.
// cus_given > 0: plan for that many compute units instead of asking the
// current device.
int make_plan(const Call& c, const gemm_f16_opts* o, Plan& p, bool allow_pack = true,
              bool allow_realign = true, int cus_given = 0) {
  int rc = check_opts(o);
  if (rc) return rc;
  p.pack = false;
  p.pack_bytes = 0;
  p.pack_a = false;
  p.pack_a_bytes = 0;
  p.lda_p = 0;
  const int variant = o ? o->variant : GEMM_VARIANT_AUTO;
  const int want_split = o ? o->split_k : 0;
  const int want_panel = o ? o->panel : 0;
  const int want_tile = o ? o->tile : 0;

  int cus = cus_given;
  auto need_cus = [&]() -> int {
    if (cus > 0) return GEMM_OK;
    return device_cus(&cus);
  };

  // FP8 operands: K-contiguous A and B with 16-byte aligned rows, on the FP8
  // tile, in the main, split-K and stream-K families; with N-contiguous B
  // also the skinny family (the decode kernel).
  const bool f8 = c.dt >= DT_F8;
  if (f8) {
    // A K-contiguous; B K-contiguous ([N, K] rows) or N-contiguous ([K, N]
    // rows, N a multiple of 16); 16-byte aligned rows at most 2^24 bytes
    // apart (the DMA's 32-bit lane offsets span 255 rows).
    const bool b_k = c.ldb_k == 1, b_n = !b_k && c.ldb_n == 1;
    const int64_t ldb = b_k ? c.ldb_n : c.ldb_k;
    if (c.lda_k != 1 || c.lda_m % 16 != 0 || ((uintptr_t)c.A & 15u) || !(b_k || b_n) ||
        ldb % 16 != 0 || ((uintptr_t)c.B & 15u) || c.lda_m > (INT64_C(1) << 24) ||
        ldb > (INT64_C(1) << 24) || (b_n && c.N % 16 != 0))
      return GEMM_ERR_LAYOUT;
    // (The 128 x 128 and 64 x 128 LDS-DMA tiles also take FP8 with
    // K-contiguous B and K even; a forced one with another layout hands
    // over to the FP8 tile.)
    if ((variant == GEMM_VARIANT_SKINNY && (!(b_n || (b_k && c.M <= 16)) || want_tile)) ||
        variant == GEMM_VARIANT_TILE64X32 ||
        (want_tile && want_tile != TILE_F8 && want_tile != TILE_DMA128 && want_tile != TILE_DMA64X128))
      return GEMM_ERR_OPTS;
  }

  // A forced tile must have kernels for this format (checked before any
  // device query).
  if (want_tile && !has_format(tile_info(want_tile), c.dt)) return GEMM_ERR_OPTS;

  p.sk_tiles = 0;
  p.variant = variant;
  if (p.variant == GEMM_VARIANT_AUTO) {
    if ((rc = need_cus())) return rc;
    // FP8 with N-contiguous B streams through the decode kernel too, up to
    // 32 rows (N = 2048, K = 7168, per call in graphs of calls: M = 1, 16,
    // 32 in 8.9, 10.4, 12.7 us against 14.2, 14.8, 14.9 on the 256 x 256 FP8
    // tile split over K; M = 33 level, M = 48 and 64 behind: 16.3 and 19.1
    // against 15.5 and 15.8), and with B as [N, K] rows up to 16 rows (M = 1
    // and 16: 11.4 and 12.5 us against 14.8 and 15.2; N = 7168: 28.9 and
    // 32.6 against 64.0 and 64.3).
    if (c.M <= 64 && (!f8 || (c.ldb_n == 1 && c.M <= 32) || (c.ldb_k == 1 && c.M <= 16))) {
      p.variant = GEMM_VARIANT_SKINNY;
    } else {
      const int64_t T = cdiv(c.M, CfgT128::BM) * cdiv(c.N, CfgT128::BN);
      const int64_t mn = c.M > c.N ? c.M : c.N;
      // Split-K when the 128x128 tiles fill at most half the compute units.
      // On the 128x128 LDS-DMA tile from K >= 2048: below it the main plan
      // was ahead (1024^3: 13.6 us against 16.8 with 2 ranges; 768^2 x 1024
      // 13.4 against 15.3), from it on the split was (1024^2 x 2048: 18.5
      // against 23.7; 128 x 2048 x 2048 15.4 against 20.8; 96 x 8192 x 8192
      // 31.1 against 72.0; 1024 x 2048 x 2048 level).  For operands that
      // tile does not read, from K >= 2 max(M, N) and K >= 1024 (two K
      // ranges of at least 512 on the 256x256 tile).  FP8 on that tile from
      // K >= 4096: its main plans run further ahead (1024^2 x 2048: 10.6 us
      // on the 64 x 128 tile against 18.2 split; 1024^2 x 8192: 24.4 split
      // against 37.8).
      const bool dma = dma128_reads(c);
      const bool split = dma ? c.K >= (f8 ? 4096 : 2048) : (c.K >= 2 * mn && c.K >= 1024);
      p.variant = (2 * T <= cus && split) ? GEMM_VARIANT_SPLITK : GEMM_VARIANT_MAIN;
    }
  }

  // Option combinations that no plan accepts are rejected before any device
  // query.  bfloat16 is built for the 128x128, skinny and full-line-A tiles.
  if ((p.variant == GEMM_VARIANT_MAIN || p.variant == GEMM_VARIANT_TILE64X32) && want_split > 1)
    return GEMM_ERR_OPTS;
  if (c.dt != DT_F16 && p.variant == GEMM_VARIANT_TILE64X32) return GEMM_ERR_OPTS;
  if (p.variant == GEMM_VARIANT_SKINNY && c.M > 64) return GEMM_ERR_OPTS;

  p.a_path = f8 ? PATH_KVEC : classify(c.A, c.lda_m, c.lda_k);
  p.b_path = f8 ? (c.ldb_k == 1 ? PATH_KVEC : PATH_RVEC) : classify(c.B, c.ldb_n, c.ldb_k);
  // An A that the LDS-DMA tile cannot read (rows not on 16-byte boundaries,
  // or M-contiguous) would keep every plan on the 128x128 tile's element-wise
  // or transposing loads, at a half to a third of the rate.  An automatic
  // plan copies it first into K-contiguous 128-byte rows in the workspace
  // (one pass of 4MK bytes) and is planned as for that A.
  const bool realign = allow_realign && variant == GEMM_VARIANT_AUTO && !f8 &&
                       (p.variant == GEMM_VARIANT_MAIN || p.variant == GEMM_VARIANT_SPLITK) &&
                       p.a_path != PATH_KVEC && c.N >= kRealignMinN && worth_packing(c) &&
                       realign_a_bytes(c.M, c.K) != 0 &&
                       (p.a_path == PATH_GATHER || (double)c.M * c.N * c.K >= (double)kRealignMinWorkMC);
  if (realign) p.a_path = PATH_KVEC;
  // A B that the LDS-DMA tile cannot read directly (rows not 16-byte
  // aligned, or neither dimension contiguous) would take the element-wise
  // path on the 128x128 tile, at less than half the rate.  An automatic plan
  // with enough rows packs it instead (the packing pass reads any strides)
  // and is planned as for a K-contiguous B; if no packing plan comes of it,
  // the call is planned again with B's own path.
  // Split-K plans pack it from the 256x256 tile's M, N >= 256 on: with
  // K >> M the element-wise B loads cost far more than one pass over B
  // (512 x 514 x 65536: 215 us on the element-wise plan).
  const bool pack_any = allow_pack && variant == GEMM_VARIANT_AUTO && !f8 &&
                        ((p.variant == GEMM_VARIANT_MAIN && c.M >= kPackMinRowsGather) ||
                         (p.variant == GEMM_VARIANT_SPLITK && c.M >= 256 && c.N >= 256)) &&
                        worth_packing(c) && p.a_path == PATH_KVEC &&
                        (p.b_path == PATH_GATHER || (p.b_path == PATH_RVEC && c.N % 8 != 0));
  if (pack_any) p.b_path = PATH_KVEC;

  // Tile.
  switch (p.variant) {
    case GEMM_VARIANT_MAIN:
      if (want_tile) {
        p.tile_id = want_tile;
      } else {
        // The 128x128 LDS-DMA tile (fp16, K-contiguous A, B either way with
        // N % 8 == 0) up to 80 tiles of 256x256 (on 256 compute units): 1.3-1.4x
        // the 128x128 register tile (1536^3: 20.4 against 28.0 us) and ahead of
        // the 256x256 tile below a wave (2048^3: 28.2 against 38.1 us); from 81
        // tiles on the 256x256 tile leads (2304^3: 41.9 against 43.8; 3072^3:
        // 60.7 against 88.7).  A B to be packed (one the DMA cannot read) takes
        // the 256x256 tile, the one with packed-B kernels.  Few tiles with a
        // long K (K >= 4096, under three quarters of a wave of 128x128 tiles)
        // keep the stream-K plan of the 256x256 tile below (1536^2 x 8192:
        // 64.4 against 79.5 us), and so does any grid under half a wave with
        // K >= 8192 (2048^2 x 8192: 86.5 against 89.9; x 16384: 140.8 against
        // 166.4; 1792^2 x 8192: 74.1 against 86.2); with a shorter K the
        // 128x128 DMA tile is ahead of it (2048^2 x 4096: 49.0 against 56.1;
        // 2048^2 x 6144: 70.9 against 73.3; 1536^2 x 3072: 34.6 against 38.6).
        // Without that tile: 256x256 tiles from a quarter wave on when K is
        // not short, else the 128x128 register tile.  FP8 (B as [N, K] rows,
        // K even) takes the same rule with the FP8 tile as the 256x256 one
        // (per call: 1024^3 7.7 us against 13.6; 2048^3 14.9 against 21.1;
        // 2048^2 x 4096 28.4 against 41.6; 2560^3 level; 3072^3 51.1 against
        // 32.8 on the FP8 tile); other FP8 layouts run on the FP8 tile.
        if ((rc = need_cus())) return rc;
        const int64_t t256 = cdiv(c.M, 256) * cdiv(c.N, 256);
        const bool t14 = f8 || dma_tile_takes(c, p);
        const int big_tile = f8 ? TILE_F8 : TILE_DMA256A128;
        const bool t7 = tile_takes(tile_info(TILE_DMA128), c, p);
        const bool big = 16 * t256 >= 5 * (int64_t)cus;
        const bool sk_small = small_grid_streamk(c, t256, cus) && (16 * t256 < 3 * (int64_t)cus ? c.K >= 4096 : c.K >= 8192);
        const bool quarter = 4 * t256 >= cus && (c.K >= 2048 || 3 * t256 >= cus);
        const bool packed_b = pack_any && c.N >= 256;
        // Up to a quarter wave of 128x128 tiles, the 64x128 LDS-DMA tile
        // (same layouts), with twice the workgroups: 1024^3 in 12.5 us against
        // 13.5, 512^3 8.2 against 8.9, 256^3 6.3 against 7.0; from 1536^3 (144
        // tiles) on it falls behind (22.3 against 20.0).
        const int64_t t128 = cdiv(c.M, 128) * cdiv(c.N, 128);
        if (t14 && (packed_b || big || sk_small))
          p.tile_id = big_tile;
        else if (t7 && !big)
          p.tile_id = 4 * t128 <= (int64_t)cus ? TILE_DMA64X128 : TILE_DMA128;
        else if (f8)
          p.tile_id = TILE_F8;
        else
          p.tile_id = (2 * t256 >= cus || ((quarter || small_grid_streamk(c, t256, cus)) && t14))
                          ? TILE_DMA256A128 : TILE_T128;
      }
      break;
    case GEMM_VARIANT_SPLITK: {
      // The 128x128 LDS-DMA tile where it reads the operands (a realigned A
      // included; a B to be packed needs the 256x256 tile's packed-B
      // kernels) and its K ranges, one workgroup per compute unit, come to
      // at most 2048 k: 1024^2 x 4096 in 24.1 us against 30.5 on the 256x256
      // tile, 256^2 x 16384 16.5 against 22.9, 1024^2 x 8192 36.1 against
      // 40.7, and 128 x 4096 x 8192 23.7 against 31.0 on the 128x128
      // register tile.  Longer ranges repay the 256x256 tile's larger
      // partials (512^2 x 65536: 52.9 against 61.0; 768^2 x 32768: 58.9
      // against 70.4; 1024 x 2048 x 8192: 54.5 against 65.0).  Otherwise
      // the 256x256 full-line-A tile once the output holds a whole one (it
      // falls back to 128x128 for layouts it does not take).
      bool dma128 = false;
      if (!want_tile && !pack_any && tile_takes(tile_info(TILE_DMA128), c, p)) {
        if ((rc = need_cus())) return rc;
        const int64_t t128 = cdiv(c.M, 128) * cdiv(c.N, 128);
        const int64_t s7 = std::min<int64_t>((int64_t)cus / t128, c.K / 512);
        dma128 = c.M < 256 || c.N < 256 || (s7 >= 1 && c.K <= 2048 * s7);
      }
      if (want_tile)
        p.tile_id = want_tile;
      else if (dma128)
        p.tile_id = TILE_DMA128;
      else if (f8)
        p.tile_id = TILE_F8;
      else
        p.tile_id = (c.M >= 256 && c.N >= 256) ? TILE_DMA256A128 : TILE_T128;
      break;
    }
    case GEMM_VARIANT_STREAMK:
      if (want_tile && want_tile != (f8 ? TILE_F8 : TILE_DMA256A128)) return GEMM_ERR_OPTS;
      p.tile_id = f8 ? TILE_F8 : TILE_DMA256A128;
      break;
    case GEMM_VARIANT_TILE64X32:
      if (want_tile && want_tile != TILE_T64X32) return GEMM_ERR_OPTS;
      p.tile_id = TILE_T64X32;
      break;
    case GEMM_VARIANT_SKINNY:
      if (c.M > 64) return GEMM_ERR_OPTS;
      p.tile_id = want_tile ? want_tile : (c.M <= 16 ? TILE_S16 : (c.M <= 32 ? TILE_S32 : TILE_S64));
      break;
    default:
      return GEMM_ERR_OPTS;
  }
  // M <= 64 with N-contiguous B, or M <= 16 with K-contiguous B (16-byte
  // vectors): the decode kernel (128-column strips, one workgroup per strip
  // and K range, about one workgroup per compute unit, K ranges of at least
  // 128 k).  With K-contiguous B and 17..64 rows the skinny tiles were faster
  // (M = 32, 48, 64: 15.3, 17.4, 19.3 us per call against 16.6, 19.4, 20.9);
  // up to 16 rows the decode kernel (M = 1 and 16: 12.3 and 12.9 against
  // 13.4 and 13.5).
  p.dec_mt = 0;
  p.red_elem = 0;
  if (p.variant == GEMM_VARIANT_SKINNY && !want_tile && c.M <= 64 &&
      (p.b_path == PATH_RVEC || (p.b_path == PATH_KVEC && c.M <= 16))) {
    p.dec_mt = c.M <= 16 ? 16 : (c.M <= 32 ? 32 : 64);
    p.GM = 1;
    p.GN = cdiv(c.N, kDecCols);
    int64_t s = want_split;
    if (s == 0) {
      // As many K ranges as keep the workgroups within one per compute unit:
      // a second round for a few of them costs a whole extra pass (N = 7168,
      // K = 2048: 56 strips x 5 ranges = 280 workgroups took 14.2 us per
      // M = 1 call, x 4 ranges 10.6 us).
      if ((rc = need_cus())) return rc;
      s = cus / p.GN;
      if (s < 1) s = 1;
      if (s > cdiv(c.K, 4 * kDecUnit)) s = cdiv(c.K, 4 * kDecUnit);
    }
    p.k_split = cdiv(cdiv(c.K, s), kDecUnit) * kDecUnit;
    p.split = (int)cdiv(c.K, p.k_split);
    p.panel = -1;
    p.c_vec = (((uintptr_t)c.C & 15u) == 0 && (c.ldc & 7) == 0) ? 1 : 0;
    int64_t grid;
    if (__builtin_mul_overflow(p.GN, (int64_t)p.split, &grid) || grid > INT32_MAX)
      return GEMM_ERR_SHAPE;
    p.grid = grid;
    p.tile_id = TILE_S16;   // reported tile id of the skinny family
    return plan_partials(c, p);
  }

  // A tile whose kernels do not cover this operand layout hands over to its
  // fallback (the LDS-DMA tile needs K-contiguous A and, for N-contiguous B,
  // N a multiple of 8).
  for (;;) {
    const TileInfo& t = tile_info(p.tile_id);
    if (tile_takes(t, c, p)) break;
    // fp16 tiles hand over along their fallback chain; bfloat16 goes straight
    // to the 128x128 tile, which covers every layout in both formats.  A
    // chain that ends without a taker (a tile without this format) is an
    // option error, never a loop.
    const int next = c.dt == DT_F16 ? t.fallback : (c.dt == DT_BF16 ? TILE_T128 : TILE_F8);
    if (next <= 0 || next > TILE_MAX || next == p.tile_id) return GEMM_ERR_OPTS;
    p.tile_id = next;
  }
  const TileInfo& ti = tile_info(p.tile_id);
  p.GM = cdiv(c.M, ti.bm);
  p.GN = cdiv(c.N, ti.bn);
  const int64_t T = p.GM * p.GN;
  const bool sk_tile = p.tile_id == TILE_DMA256A128 || p.tile_id == TILE_F8;
  if (p.variant == GEMM_VARIANT_STREAMK && !sk_tile) return GEMM_ERR_OPTS;
  if (variant == GEMM_VARIANT_AUTO && p.variant == GEMM_VARIANT_MAIN && (!want_tile || f8) &&
      sk_tile && c.K >= 2048) {
    // A final wave at most half full goes to the stream-K tail (one 256x256
    // workgroup fits a compute unit, so a wave is `cus` tiles).
    if ((rc = need_cus())) return rc;
    const int64_t tail = T % cus;
    if ((T >= cus && tail > 0 && 2 * tail <= cus) || small_grid_streamk(c, T, cus))
      p.variant = GEMM_VARIANT_STREAMK;
  }
  if (p.variant == GEMM_VARIANT_STREAMK) {
    if ((rc = need_cus())) return rc;
    // Tail tiles: the partial last wave; when the tiles fill whole waves (a
    // forced plan), the last whole wave, or every tile if there is less.
    int64_t L = T % cus;
    if (L == 0) L = T < cus ? T : cus;
    int64_t s = want_split;
    if (s == 0) {
      s = cus / L;                                  // fill the idle compute units
      if (s > cdiv(c.K, 16 * ti.bk)) s = cdiv(c.K, 16 * ti.bk);   // at least 8 super-steps per range
      if (s > 64) s = 64;
      if (s < 1) s = 1;
    }
    set_split(p, c.K, 2 * ti.bk, s);   // whole super-steps per range
    p.sk_tiles = L;
    p.grid = T - L;
    p.grid2 = L * (ti.bm * ti.bn / 1024);
    p.panel = want_panel != 0 ? want_panel : 4;
    p.c_vec = (((uintptr_t)c.C & 7u) == 0 && (c.ldc & 3) == 0) ? 1 : 0;
    p.red_elem = 0;
    int64_t bytes;
    if (__builtin_mul_overflow(L * p.split, (int64_t)ti.bm * ti.bn * 4, &bytes) || bytes > INT64_MAX - 256)
      return GEMM_ERR_SHAPE;
    p.ws = (size_t)((bytes + 255) / 256 * 256);
    maybe_pack(c, variant, allow_pack, p, pack_any);
    if (pack_any && !p.pack) return make_plan(c, o, p, false, allow_realign, cus_given);
    if (realign && !add_realign(c, p)) return make_plan(c, o, p, allow_pack, false, cus_given);
    return GEMM_OK;
  }

  // K split.
  if (p.variant == GEMM_VARIANT_SPLITK || p.variant == GEMM_VARIANT_SKINNY) {
    int64_t s = want_split;
    if (s == 0) {
      if ((rc = need_cus())) return rc;
      // Workgroups per compute unit: two for split-K on 128x128 tiles; one
      // for skinny tiles, where every K range adds S x M x N x 4 bytes of
      // partials against the 2KN bytes of B (M = 32..64 ran fastest at one);
      // five eighths for the 256x256 tile, whose partials are 4x larger per
      // workgroup (512 x 512 x 65536: 51 us at 160 workgroups against 54 at
      // 128 and 57 at 256).  Split counts of 8 or more are rounded up to a
      // multiple of 8 so the launch can keep each K range's tiles on one XCD.
      // The 128x128 LDS-DMA tile: one workgroup per compute unit, rounded
      // down (1024^2 x 2048: 18.5 us with 4 ranges against 27.5 with 8;
      // 256 x 1024 x 4096: 16.3 with 8 against 19.4 with 16).
      const bool dma128 = p.tile_id == TILE_DMA128 && p.variant == GEMM_VARIANT_SPLITK;
      const int64_t per_cu8 = p.variant == GEMM_VARIANT_SKINNY ? 8 : (ti.bm >= 256 ? 5 : 16);
      s = dma128 ? cus / T : cdiv(per_cu8 * (int64_t)cus, 8 * T);
      // Two per compute unit while the K ranges stay at least 2048 k long
      // (M or N under 256): its 64 KiB ring lets two workgroups share a
      // compute unit, and over a long range the second hides the first
      // one's waits (1024^2 x 16384: 51.9 us with 8 ranges against 62.7
      // with 4; 1024^2 x 8192: 35.4 with 8, 36.1 with 4).
      if (dma128 && s >= 1 && c.K / s >= 4096) s *= 2;
      // On the LDS-DMA tiles, K ranges of at least 512 k: at smaller K more,
      // shorter ranges cost more in partials and per-workgroup start-up than
      // the extra compute units give (1024 x 1024 x 4096: 29.0 us with 8
      // ranges against 33.4 with 16 on the 256x256 tile; 1024 x 1024 x 2048:
      // 23.8 with 4).
      if (p.variant == GEMM_VARIANT_SPLITK && (ti.bm >= 256 || dma128) && s > c.K / 512)
        s = c.K / 512 > 1 ? c.K / 512 : 1;
      if (s < 1) s = 1;
      const int64_t max_by_k = cdiv(c.K, 2 * ti.bk);  // at least two K steps per split
      if (s >= 8) s = dma128 ? s / 8 * 8 : cdiv(s, 8) * 8;
      if (s > max_by_k) s = max_by_k;
      if (s > 64) s = 64;
    }
    set_split(p, c.K, f8 ? 2 * ti.bk : ti.bk, s);   // FP8: whole 128-k super-steps
  } else {
    if (want_split > 1) return GEMM_ERR_OPTS;
    set_split(p, c.K, ti.bk, 1);
  }

  // Raster.
  if (want_panel != 0)
    p.panel = want_panel;
  else
    p.panel = (p.variant == GEMM_VARIANT_MAIN || p.variant == GEMM_VARIANT_TILE64X32)
                  ? (ti.bm >= 256 ? 4 : 8)
                  : -1;

  p.c_vec = (((uintptr_t)c.C & 7u) == 0 && (c.ldc & 3) == 0) ? 1 : 0;

  int64_t grid;
  if (__builtin_mul_overflow(T, (int64_t)p.split, &grid) || grid > (INT64_C(1) << 32) / ti.nt - 1)
    return GEMM_ERR_SHAPE;
  p.grid = grid;
  if ((rc = plan_partials(c, p))) return rc;

  maybe_pack(c, variant, allow_pack, p, pack_any);
  if (pack_any && !p.pack) return make_plan(c, o, p, false, allow_realign, cus_given);
  if (realign && !add_realign(c, p)) return make_plan(c, o, p, allow_pack, false, cus_given);
  return GEMM_OK;
}

void fill_info(const Plan& p, gemm_f16_plan_info* info) {
  const TileInfo& ti = tile_info(p.tile_id);
  info->variant = p.variant;
  info->tile_m = p.dec_mt ? p.dec_mt : ti.bm;
  info->tile_n = p.dec_mt ? kDecCols : ti.bn;
  info->tile_k = p.dec_mt ? kDecUnit : ti.bk;
  info->split_k = p.split;
  info->panel = p.panel;
  info->a_path = p.pack_a ? kBPathPacked : p.a_path;
  info->b_path = p.pack ? kBPathPacked : p.b_path;
  info->tile_id = p.tile_id;
  info->grid = p.grid;
  info->grid2 = p.grid2;
  info->workspace_bytes = p.ws;
  info->sk_tiles = p.sk_tiles;
}

// Second launch of a split plan: sum the partials in ws into C.
int launch_reduce(const Call& c, const Plan& p, void* ws, hipStream_t stream) {
  if (p.split <= 1) return GEMM_OK;
  const float* W = (const float*)ws;
  int S = p.split;
  int64_t M = c.M, N = c.N, ldc = c.ldc;
  uint16_t* C = (uint16_t*)c.C;
  int cv = p.c_vec;
  kfn_reduce fn = c.dt != DT_BF16   // binary16 output for the fp16 and FP8 formats
      ? (p.red_elem ? splitk_reduce_elem<DT_F16> : splitk_reduce_quad<DT_F16>)
      : (p.red_elem ? splitk_reduce_elem<DT_BF16> : splitk_reduce_quad<DT_BF16>);
  void* rargs[] = {&W, &S, &M, &N, &C, &ldc, &cv};
  if (hipLaunchKernel((const void*)fn, dim3((unsigned)p.grid2), dim3(256), rargs, 0, stream) != hipSuccess)
    return GEMM_ERR_HIP;
  return GEMM_OK;
}

template <int MT>
kfn_dec pick_dec(int dt) {
  switch (dt) {
    case DT_F16: return decode_kernel<MT, DT_F16>;
    case DT_BF16: return decode_kernel<MT, DT_BF16>;
    case DT_F8 + 0: return decode_kernel<MT, DT_F16, false, 0>;
    case DT_F8 + 1: return decode_kernel<MT, DT_F16, false, 1>;
    case DT_F8 + 2: return decode_kernel<MT, DT_F16, false, 2>;
    default: return decode_kernel<MT, DT_F16, false, 3>;
  }
}
kfn_dec pick_dec_bk(int dt) {   // B as [N, K] rows, up to 16 rows of A
  switch (dt) {
    case DT_F16: return decode_kernel<16, DT_F16, true>;
    case DT_BF16: return decode_kernel<16, DT_BF16, true>;
    case DT_F8 + 0: return decode_kernel<16, DT_F16, true, 0>;
    case DT_F8 + 1: return decode_kernel<16, DT_F16, true, 1>;
    case DT_F8 + 2: return decode_kernel<16, DT_F16, true, 2>;
    default: return decode_kernel<16, DT_F16, true, 3>;
  }
}

int launch_decode(const Call& c, const Plan& p, void* ws, hipStream_t stream) {
  DecArgs d;
  d.A = (const uint16_t*)c.A;
  d.lda_m = c.lda_m;
  d.lda_k = c.lda_k;
  d.B = (const uint16_t*)c.B;
  d.ldb_k = c.ldb_k;
  d.ldb_n = c.ldb_n;
  d.C = (uint16_t*)c.C;
  d.ldc = c.ldc;
  d.P = (float*)ws;
  d.M = c.M;
  d.N = c.N;
  d.K = c.K;
  d.kr = p.k_split;
  d.GN = (int32_t)p.GN;
  d.S = p.split;
  d.a_vec = (c.lda_k == 1 && c.lda_m % 8 == 0 && ((uintptr_t)c.A & 15u) == 0) ? 1 : 0;
  d.c_vec = p.c_vec;
  kfn_dec fn = p.b_path == PATH_KVEC ? pick_dec_bk(c.dt)
               : p.dec_mt == 16       ? pick_dec<16>(c.dt)
               : p.dec_mt == 32       ? pick_dec<32>(c.dt)
                                      : pick_dec<64>(c.dt);
  void* args[] = {&d};
  if (hipLaunchKernel((const void*)fn, dim3((unsigned)p.grid), dim3(64 * kDecWaves), args, 0, stream) != hipSuccess)
    return GEMM_ERR_HIP;
  if (p.split > 1) {
    // The reduction writes C with 8-byte vectors (its own alignment rule).
    Plan q = p;
    q.c_vec = (((uintptr_t)c.C & 7u) == 0 && (c.ldc & 3) == 0) ? 1 : 0;
    return launch_reduce(c, q, ws, stream);
  }
  return GEMM_OK;
}

// Stream-K plan: whole waves of tiles (raster ids 0 .. grid-1) with the
// final kernel, the tail tiles' K ranges with the partial kernel into the
// workspace, then the fixed-order fix-up into C.
int launch_streamk(const Call& c, const Plan& p, KArgs a, kfn_t final_fn, kfn_t partial_fn, void* ws,
                   hipStream_t stream) {
  const TileInfo& ti = tile_info(p.tile_id);
  void* args[] = {&a};
  a.k_split = c.K;   // whole waves: every tile over all of K
  if (p.grid > 0 &&
      hipLaunchKernel((const void*)final_fn, dim3((unsigned)p.grid), dim3(ti.nt), args, 0, stream) != hipSuccess)
    return GEMM_ERR_HIP;
  a.k_split = p.k_split;
  a.W = (float*)ws;
  a.sk_first = p.grid;
  a.sk_tiles = p.sk_tiles;
  if (hipLaunchKernel((const void*)partial_fn, dim3((unsigned)(p.sk_tiles * p.split)), dim3(ti.nt), args, 0,
                      stream) != hipSuccess)
    return GEMM_ERR_HIP;
  const float* W = (const float*)ws;
  int S = p.split, panel = p.panel, bm = ti.bm, bn = ti.bn, cv = p.c_vec;
  int64_t L = p.sk_tiles, first = p.grid, GM = p.GM, GN = p.GN, M = c.M, N = c.N, ldc = c.ldc;
  uint16_t* C = (uint16_t*)c.C;
  void* fargs[] = {&W, &S, &L, &first, &GM, &GN, &panel, &bm, &bn, &M, &N, &C, &ldc, &cv};
  const void* fix = c.dt != DT_BF16 ? (const void*)sk_fixup<DT_F16> : (const void*)sk_fixup<DT_BF16>;
  if (hipLaunchKernel(fix, dim3((unsigned)p.grid2), dim3(256), fargs, 0, stream) != hipSuccess)
    return GEMM_ERR_HIP;
  return GEMM_OK;
}

int launch(const Call& c, const Plan& p, void* ws, hipStream_t stream) {
  if (p.dec_mt) return launch_decode(c, p, ws, stream);
  // Realigning plan: A into the front of the workspace.
  if (p.pack_a) {
    const int rc = launch_realign_a((const uint16_t*)c.A, c.lda_m, c.lda_k, c.M, c.K, p.lda_p,
                                    (uint16_t*)ws, stream);
    if (rc) return rc;
  }
  const void* const A = p.pack_a ? ws : c.A;
  if (p.pack_a) ws = (char*)ws + p.pack_a_bytes;
  // Packing plan: B into the workspace (K16: K in 16-bit units).
  const int64_t K16 = c.dt >= DT_F8 ? cdiv(c.K, 2) : c.K;
  if (p.pack) {
    int rc;
    if (c.dt < DT_F8)        // 16-bit B through its strides
      rc = launch_pack_b((const uint16_t*)c.B, c.ldb_k, c.ldb_n, c.K, c.N, (uint16_t*)ws, stream);
    else if (c.K % 2 == 0)   // K-contiguous FP8 rows as byte pairs
      rc = launch_pack_b((const uint16_t*)c.B, 1, c.ldb_n / 2, K16, c.N, (uint16_t*)ws, stream);
    else                     // odd K: byte by byte, zero past K
      rc = launch_pack_b8((const uint8_t*)c.B, c.ldb_k, c.ldb_n, c.K, c.N, (uint8_t*)ws, stream);
    if (rc) return rc;
  }
  const TileInfo& ti = tile_info(p.tile_id);
  KArgs a;
  a.A = (const uint16_t*)A;
  a.lda_m = p.pack_a ? p.lda_p : c.lda_m;
  a.lda_k = p.pack_a ? 1 : c.lda_k;
  a.B = (const uint16_t*)c.B;
  a.ldb_k = c.ldb_k;
  a.ldb_n = c.ldb_n;
  a.C = (uint16_t*)c.C;
  a.ldc = c.ldc;
  a.W = (float*)ws;
  a.M = c.M;
  a.N = c.N;
  a.K = c.K;
  a.k_split = p.k_split;
  a.GM = p.GM;
  a.GN = p.GN;
  a.panel = p.panel;
  a.c_vec = p.c_vec;
  a.g_off = nullptr;
  a.g_tiles = nullptr;
  a.ldb_g = 0;
  a.G = 0;
  a.sk_first = 0;
  a.sk_tiles = 0;
  a.split_xcd = 0;
  const int sel = p.a_path * 3 + p.b_path;
  kfn_t final_fn = ti.final_fn[c.dt][sel], partial_fn = ti.partial_fn[c.dt][sel];
  if (p.pack) {   // the packed B at the front of the workspace, partials after it
    a.B = (const uint16_t*)ws;
    a.ldb_k = 1;
    a.ldb_n = cdiv(K16, 32) * 8192;   // 16-bit units per 256-column panel
    final_fn = ti.packed_fn[c.dt];
    partial_fn = ti.packed_partial_fn[c.dt];
    ws = (char*)ws + p.pack_bytes;
    a.W = (float*)ws;
  }
  if (p.variant == GEMM_VARIANT_STREAMK) return launch_streamk(c, p, a, final_fn, partial_fn, ws, stream);
  kfn_t fn = (p.split > 1) ? partial_fn : final_fn;
  a.split_xcd = (p.split > 1 && p.split % 8 == 0) ? 1 : 0;
  void* args[] = {&a};
  if (hipLaunchKernel((const void*)fn, dim3((unsigned)p.grid), dim3(ti.nt), args, 0, stream) != hipSuccess)
    return GEMM_ERR_HIP;
  return launch_reduce(c, p, ws, stream);
}

int plan_impl(int dt, const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
              int64_t ldb_n, const void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
              const gemm_f16_opts* opts, gemm_f16_plan_info* info, int cus = 0) {
  Call c{dt, A, B, C, lda_m, lda_k, ldb_k, ldb_n, ldc, M, N, K, 0, 0, 0};
  int rc = validate(c);
  if (rc) return rc;
  if ((rc = spans(c))) return rc;
  Plan p;
  if ((rc = make_plan(c, opts, p, true, true, cus))) return rc;
  if (info) fill_info(p, info);
  return GEMM_OK;
}

int ex_impl(int dt, const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
            int64_t ldb_n, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream,
            void* workspace, size_t workspace_bytes, const gemm_f16_opts* opts) {
  Call c{dt, A, B, C, lda_m, lda_k, ldb_k, ldb_n, ldc, M, N, K, 0, 0, 0};
  int rc = validate(c);
  if (rc) return rc;
  if ((rc = spans(c))) return rc;
  Plan p;
  if ((rc = make_plan(c, opts, p))) return rc;
  // A packing plan runs only where the room is there: the library's own
  // allocation, or a caller workspace that holds the packed operands.
  if ((p.pack || p.pack_a) && workspace && workspace_bytes < p.ws &&
      (rc = make_plan(c, opts, p, false, false)))
    return rc;
  hipStream_t s = (hipStream_t)stream;
  if (p.ws == 0) return launch(c, p, nullptr, s);
  if (workspace) {
    if (workspace_bytes < p.ws || ((uintptr_t)workspace & 255u)) return GEMM_ERR_WORKSPACE;
    const uintptr_t w0 = (uintptr_t)workspace, w1 = w0 + p.ws;
    const uintptr_t a0 = (uintptr_t)A, a1 = a0 + in_bytes(c) * (uintptr_t)(c.spanA + 1);
    const uintptr_t b0 = (uintptr_t)B, b1 = b0 + in_bytes(c) * (uintptr_t)(c.spanB + 1);
    const uintptr_t c0 = (uintptr_t)C, c1 = c0 + 2 * (uintptr_t)(c.spanC + 1);
    if (ranges_overlap(w0, w1, a0, a1) || ranges_overlap(w0, w1, b0, b1) ||
        ranges_overlap(w0, w1, c0, c1))
      return GEMM_ERR_ALIAS;
    return launch(c, p, workspace, s);
  }
  void* ws = nullptr;
  if (hipMallocAsync(&ws, p.ws, s) != hipSuccess) return GEMM_ERR_HIP;
  rc = launch(c, p, ws, s);
  if (hipFreeAsync(ws, s) != hipSuccess && rc == GEMM_OK) rc = GEMM_ERR_HIP;
  return rc;
}

// The automatic fp16 plan without a packing pass, its workspace in scratch.
int noalloc_impl(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
                 int64_t ldb_n, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
  Call c{DT_F16, A, B, C, lda_m, lda_k, ldb_k, ldb_n, ldc, M, N, K, 0, 0, 0};
  int rc = validate(c);
  if (rc) return rc;
  if ((rc = spans(c))) return rc;
  Plan p;
  if ((rc = make_plan(c, nullptr, p, false, false))) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (p.ws == 0) return launch(c, p, nullptr, s);
  if (p.ws > GEMM_F16_SCRATCH_BYTES) return GEMM_ERR_SCRATCH;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return launch(c, p, ws, s);
}

size_t ws_impl(int dt, int64_t M, int64_t N, int64_t K, const gemm_f16_opts* opts) {
  // Shape-only plan on non-overlapping, aligned stand-in addresses.
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const int64_t Kp = (K + 15) / 16 * 16;   // FP8: K-contiguous A and B rows
  Call c = dt >= DT_F8 ? Call{dt, (const void*)0x100000000000ull, (const void*)0x200000000000ull,
                              (const void*)0x300000000000ull, Kp, 1, 1, Kp, N, M, N, K, 0, 0, 0}
                       : Call{dt, (const void*)0x100000000000ull, (const void*)0x200000000000ull,
                              (const void*)0x300000000000ull, K, 1, N, 1, N, M, N, K, 0, 0, 0};
  if (spans(c)) return 0;
  Plan p;
  if (make_plan(c, opts, p, false, false)) return 0;   // split workspaces only (see the packing plans)
  return p.ws;
}

// ---- grouped launches

constexpr int32_t kMaxGroups = 1 << 20;

size_t grouped_ws_bytes(int32_t G) { return (size_t)((16 * ((int64_t)G + 1) + 255) / 256 * 256); }

struct GroupCall {
  int dt;  // DT_F16 or DT_BF16
  const void *A, *B, *C;
  const int64_t* off;
  int64_t lda_m, lda_k, ldb_g, ldb_k, ldb_n, ldc, M, N, K;
  int32_t G;
  int64_t spanA, spanB, spanC;
};

int validate_grouped(GroupCall& c) {
  if (!c.A || !c.B || !c.C || !c.off) return GEMM_ERR_NULL;
  if (c.G < 1 || c.G > kMaxGroups || c.M <= 0 || c.N <= 0 || c.K <= 0) return GEMM_ERR_SHAPE;
  if (c.lda_m <= 0 || c.lda_k <= 0 || c.ldb_k <= 0 || c.ldb_n <= 0 || c.ldb_g < 0)
    return GEMM_ERR_STRIDE;
  if (c.ldc < c.N) return GEMM_ERR_LDC;
  int64_t sb, g_off;
  if (!view_span(c.M, c.K, c.lda_m, c.lda_k, &c.spanA) || !view_span(c.K, c.N, c.ldb_k, c.ldb_n, &sb) ||
      !view_span(c.M, c.N, c.ldc, 1, &c.spanC) ||
      __builtin_mul_overflow((int64_t)(c.G - 1), c.ldb_g, &g_off) ||
      __builtin_add_overflow(sb, g_off, &c.spanB) || c.spanB > INT64_MAX / 2 - 1)
    return GEMM_ERR_SHAPE;
  const uintptr_t eb = c.dt >= DT_F8 ? 1 : 2;   // bytes per A and B element
  const uintptr_t a0 = (uintptr_t)c.A, a1 = a0 + eb * (uintptr_t)(c.spanA + 1);
  const uintptr_t b0 = (uintptr_t)c.B, b1 = b0 + eb * (uintptr_t)(c.spanB + 1);
  const uintptr_t c0 = (uintptr_t)c.C, c1 = c0 + 2 * (uintptr_t)(c.spanC + 1);
  if (a1 < a0 || b1 < b0 || c1 < c0) return GEMM_ERR_SHAPE;
  if (ranges_overlap(c0, c1, a0, a1) || ranges_overlap(c0, c1, b0, b1)) return GEMM_ERR_ALIAS;
  if (c.dt >= DT_F8) {
    // The FP8 tile's layouts (as for gemm_f8_ex), and every group's B on a
    // 16-byte boundary.
    const bool b_k = c.ldb_k == 1, b_n = !b_k && c.ldb_n == 1;
    const int64_t ldb = b_k ? c.ldb_n : c.ldb_k;
    if (c.lda_k != 1 || c.lda_m % 16 != 0 || ((uintptr_t)c.A & 15u) || !(b_k || b_n) || ldb % 16 != 0 ||
        ((uintptr_t)c.B & 15u) || c.lda_m > (INT64_C(1) << 24) || ldb > (INT64_C(1) << 24) ||
        (b_n && c.N % 16 != 0) || c.ldb_g % 16 != 0)
      return GEMM_ERR_LAYOUT;
  }
  return GEMM_OK;
}

// The tile and kernel of a grouped launch: the full-line-A LDS-DMA tile when
// the groups average at least one of its 256-row tiles and the layouts suit
// it, the 128 x 128 register-path tile otherwise.  (The 128 x 128 LDS-DMA
// tile, ahead below a wave of tiles, fell behind it over the many waves of
// a grouped launch: G = 128 groups of 128 rows, N = 2048, K = 7168 in 948 us
// against 809.)
int grouped_plan(const GroupCall& c, int* tile_id, kfn_t* fn, int64_t* grid) {
  if (c.dt >= DT_F8) {   // the FP8 tile, whatever the group sizes
    const TileInfo& ti = tile_info(TILE_F8);
    *fn = ti.grouped_fn[c.dt][PATH_KVEC * 3 + (c.ldb_k == 1 ? PATH_KVEC : PATH_RVEC)];
    if (!*fn) return GEMM_ERR_OPTS;
    const int64_t GN = cdiv(c.N, ti.bn), rows = cdiv(c.M, ti.bm) + c.G;
    if (__builtin_mul_overflow(rows, GN, grid) || *grid > (INT64_C(1) << 31) - 1) return GEMM_ERR_SHAPE;
    *tile_id = TILE_F8;
    return GEMM_OK;
  }
  // Groups start at arbitrary rows, so an M-contiguous A (vectors along m)
  // would lose its alignment: it takes the element-wise path.
  int a_path = classify(c.A, c.lda_m, c.lda_k);
  if (a_path == PATH_RVEC) a_path = PATH_GATHER;
  const int b_path = classify(c.B, c.ldb_n, c.ldb_k);
  const bool ldb_g_ok = c.ldb_g % 8 == 0;   // every group's B keeps the 16-byte alignment
  int id = TILE_T128;
  const TileInfo& d = tile_info(TILE_DMA256A128);
  if (ldb_g_ok && c.M >= (int64_t)256 * c.G && d.grouped_fn[c.dt][a_path * 3 + b_path] &&
      !(b_path == PATH_RVEC && (c.N % d.n_mult != 0 || c.N < d.n_mult)) && !(c.K > d.max_k) &&
      !(std::max(std::max(c.lda_m, c.lda_k), std::max(c.ldb_k, c.ldb_n)) > d.max_ld))
    id = TILE_DMA256A128;
  const TileInfo& ti = tile_info(id);
  // Layout classes were taken on group 0's B; other groups share them only if
  // ldb_g keeps the alignment, else take the element-wise path for B.
  const int bp = ldb_g_ok ? b_path : PATH_GATHER;
  *fn = ti.grouped_fn[c.dt][a_path * 3 + bp];
  if (!*fn) return GEMM_ERR_OPTS;
  const int64_t GN = cdiv(c.N, ti.bn), rows = cdiv(c.M, ti.bm) + c.G;
  if (__builtin_mul_overflow(rows, GN, grid) || *grid > (INT64_C(1) << 31) - 1) return GEMM_ERR_SHAPE;
  *tile_id = id;
  return GEMM_OK;
}

int launch_grouped(const GroupCall& c, int tile_id, kfn_t fn, int64_t grid, void* ws, hipStream_t s) {
  const TileInfo& ti = tile_info(tile_id);
  int64_t* off = (int64_t*)ws;
  int64_t* tiles = off + (c.G + 1);
  {
    const int64_t* oin = c.off;
    int32_t G = c.G, BM = ti.bm;
    int64_t M = c.M;
    void* args[] = {&oin, &G, &M, &BM, &off, &tiles};
    if (hipLaunchKernel((const void*)group_setup, dim3(1), dim3(1024), args, 0, s) != hipSuccess)
      return GEMM_ERR_HIP;
  }
  KArgs a;
  a.A = (const uint16_t*)c.A;
  a.lda_m = c.lda_m;
  a.lda_k = c.lda_k;
  a.B = (const uint16_t*)c.B;
  a.ldb_k = c.ldb_k;
  a.ldb_n = c.ldb_n;
  a.C = (uint16_t*)c.C;
  a.ldc = c.ldc;
  a.W = nullptr;
  a.M = c.M;
  a.N = c.N;
  a.K = c.K;
  a.k_split = c.K;
  a.GM = cdiv(c.M, ti.bm) + c.G;
  a.GN = cdiv(c.N, ti.bn);
  a.panel = -1;
  a.c_vec = (((uintptr_t)c.C & 7u) == 0 && (c.ldc & 3) == 0) ? 1 : 0;
  a.g_off = off;
  a.g_tiles = tiles;
  a.ldb_g = c.ldb_g;
  a.G = c.G;
  a.sk_first = 0;
  a.sk_tiles = 0;
  a.split_xcd = 0;
  void* args[] = {&a};
  if (hipLaunchKernel((const void*)fn, dim3((unsigned)grid), dim3(ti.nt), args, 0, s) != hipSuccess)
    return GEMM_ERR_HIP;
  return GEMM_OK;
}

int grouped_impl(int dt, const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_g,
                 int64_t ldb_k, int64_t ldb_n, void* C, int64_t ldc, const int64_t* offsets, int32_t G,
                 int64_t M_total, int64_t N, int64_t K, void* stream, void* workspace,
                 size_t workspace_bytes) {
  GroupCall c{dt, A, B, C, offsets, lda_m, lda_k, ldb_g, ldb_k, ldb_n, ldc, M_total, N, K, G, 0, 0, 0};
  int rc = validate_grouped(c);
  if (rc) return rc;
  int tile_id = 0;
  kfn_t fn = nullptr;
  int64_t grid = 0;
  if ((rc = grouped_plan(c, &tile_id, &fn, &grid))) return rc;
  const size_t need = grouped_ws_bytes(G);
  hipStream_t s = (hipStream_t)stream;
  if (workspace) {
    if (workspace_bytes < need || ((uintptr_t)workspace & 255u)) return GEMM_ERR_WORKSPACE;
    const uintptr_t eb = dt >= DT_F8 ? 1 : 2;
    const uintptr_t w0 = (uintptr_t)workspace, w1 = w0 + need;
    const uintptr_t a0 = (uintptr_t)A, a1 = a0 + eb * (uintptr_t)(c.spanA + 1);
    const uintptr_t b0 = (uintptr_t)B, b1 = b0 + eb * (uintptr_t)(c.spanB + 1);
    const uintptr_t c0 = (uintptr_t)C, c1 = c0 + 2 * (uintptr_t)(c.spanC + 1);
    if (ranges_overlap(w0, w1, a0, a1) || ranges_overlap(w0, w1, b0, b1) ||
        ranges_overlap(w0, w1, c0, c1))
      return GEMM_ERR_ALIAS;
    return launch_grouped(c, tile_id, fn, grid, workspace, s);
  }
  void* ws = nullptr;
  if (hipMallocAsync(&ws, need, s) != hipSuccess) return GEMM_ERR_HIP;
  rc = launch_grouped(c, tile_id, fn, grid, ws, s);
  if (hipFreeAsync(ws, s) != hipSuccess && rc == GEMM_OK) rc = GEMM_ERR_HIP;
  return rc;
}

}  // namespace

extern "C" {

int gemm_f16_grouped(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_g,
                     int64_t ldb_k, int64_t ldb_n, void* C, int64_t ldc, const int64_t* offsets,
                     int32_t G, int64_t M_total, int64_t N, int64_t K, void* stream,
                     void* workspace, size_t workspace_bytes) {
  return grouped_impl(DT_F16, A, lda_m, lda_k, B, ldb_g, ldb_k, ldb_n, C, ldc, offsets, G, M_total, N, K,
                      stream, workspace, workspace_bytes);
}

int gemm_bf16_grouped(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_g,
                      int64_t ldb_k, int64_t ldb_n, void* C, int64_t ldc, const int64_t* offsets,
                      int32_t G, int64_t M_total, int64_t N, int64_t K, void* stream,
                      void* workspace, size_t workspace_bytes) {
  return grouped_impl(DT_BF16, A, lda_m, lda_k, B, ldb_g, ldb_k, ldb_n, C, ldc, offsets, G, M_total, N, K,
                      stream, workspace, workspace_bytes);
}

static int f8_dt(int32_t fmt_a, int32_t fmt_b);

int gemm_f8_grouped(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_g,
                    int64_t ldb_k, int64_t ldb_n, void* C, int64_t ldc, const int64_t* offsets,
                    int32_t G, int64_t M_total, int64_t N, int64_t K, int32_t fmt_a, int32_t fmt_b,
                    void* stream, void* workspace, size_t workspace_bytes) {
  const int dt = f8_dt(fmt_a, fmt_b);
  if (dt < 0) return GEMM_ERR_OPTS;
  return grouped_impl(dt, A, lda_m, lda_k, B, ldb_g, ldb_k, ldb_n, C, ldc, offsets, G, M_total, N, K,
                      stream, workspace, workspace_bytes);
}

size_t gemm_f16_grouped_workspace_bytes(int32_t G) {
  return (G < 1 || G > kMaxGroups) ? 0 : grouped_ws_bytes(G);
}


int gemm_f16_plan(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
                  int64_t ldb_n, const void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                  const gemm_f16_opts* opts, gemm_f16_plan_info* info) {
  return plan_impl(DT_F16, A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, opts, info);
}

int gemm_f16_plan_cus(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
                      int64_t ldb_n, const void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                      int32_t cus, const gemm_f16_opts* opts, gemm_f16_plan_info* info) {
  if (cus < 1 || cus > 65536) return GEMM_ERR_OPTS;
  return plan_impl(DT_F16, A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, opts, info, cus);
}

int gemm_f16_ex(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
                int64_t ldb_n, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream,
                void* workspace, size_t workspace_bytes, const gemm_f16_opts* opts) {
  return ex_impl(DT_F16, A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, stream, workspace,
                 workspace_bytes, opts);
}

int gemm_f16(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
             int64_t ldb_n, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
  return ex_impl(DT_F16, A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, stream, nullptr, 0,
                 nullptr);
}

size_t gemm_f16_workspace_bytes(int64_t M, int64_t N, int64_t K, const gemm_f16_opts* opts) {
  return ws_impl(DT_F16, M, N, K, opts);
}

int gemm_f16_noalloc(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
                     int64_t ldb_n, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                     void* stream) {
  return noalloc_impl(A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, stream);
}

int gemm_bf16_plan(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
                   int64_t ldb_n, const void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                   const gemm_f16_opts* opts, gemm_f16_plan_info* info) {
  return plan_impl(DT_BF16, A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, opts, info);
}

int gemm_bf16_ex(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
                 int64_t ldb_n, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream,
                 void* workspace, size_t workspace_bytes, const gemm_f16_opts* opts) {
  return ex_impl(DT_BF16, A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, stream, workspace,
                 workspace_bytes, opts);
}

int gemm_bf16(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
              int64_t ldb_n, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
  return ex_impl(DT_BF16, A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, stream, nullptr, 0,
                 nullptr);
}

size_t gemm_bf16_workspace_bytes(int64_t M, int64_t N, int64_t K, const gemm_f16_opts* opts) {
  return ws_impl(DT_BF16, M, N, K, opts);
}

// ---- pre-packed B
size_t gemm_f16_packed_b_bytes(int64_t K, int64_t N) { return packed_b_bytes(K, N); }

int gemm_f16_pack_b(const void* B, int64_t ldb_k, int64_t ldb_n, int64_t K, int64_t N, void* Bp,
                    void* stream) {
  if (!B || !Bp) return GEMM_ERR_NULL;
  if (K <= 0 || N <= 0) return GEMM_ERR_SHAPE;
  if (ldb_k <= 0 || ldb_n <= 0) return GEMM_ERR_STRIDE;
  int64_t spanB;
  if (!view_span(K, N, ldb_k, ldb_n, &spanB)) return GEMM_ERR_SHAPE;
  const size_t bytes = packed_b_bytes(K, N);
  if (bytes == 0 || K > tile_info(TILE_DMA256A128).max_k) return GEMM_ERR_SHAPE;
  if (((uintptr_t)Bp & 255u) != 0) return GEMM_ERR_WORKSPACE;
  const uintptr_t b0 = (uintptr_t)B, b1 = b0 + 2 * (uintptr_t)(spanB + 1);
  if (ranges_overlap(b0, b1, (uintptr_t)Bp, (uintptr_t)Bp + bytes)) return GEMM_ERR_ALIAS;
  return launch_pack_b((const uint16_t*)B, ldb_k, ldb_n, K, N, (uint16_t*)Bp, (hipStream_t)stream);
}

int gemm_f16_packed(const void* A, int64_t lda_m, int64_t lda_k, const void* Bp, void* C, int64_t ldc,
                    int64_t M, int64_t N, int64_t K, void* stream) {
  if (!A || !Bp || !C) return GEMM_ERR_NULL;
  if (M <= 0 || N <= 0 || K <= 0) return GEMM_ERR_SHAPE;
  if (lda_m <= 0 || lda_k <= 0) return GEMM_ERR_STRIDE;
  if (ldc < N) return GEMM_ERR_LDC;
  int64_t spanA, spanC;
  if (!view_span(M, K, lda_m, lda_k, &spanA) || !view_span(M, N, ldc, 1, &spanC)) return GEMM_ERR_SHAPE;
  const size_t bytes = packed_b_bytes(K, N);
  if (bytes == 0 || K > tile_info(TILE_DMA256A128).max_k) return GEMM_ERR_SHAPE;
  // The full-line-A tile's A path: K-contiguous, 16-byte aligned rows.
  if (classify(A, lda_m, lda_k) != PATH_KVEC || ((uintptr_t)Bp & 255u) != 0 ||
      lda_m > tile_info(TILE_DMA256A128).max_ld)
    return GEMM_ERR_LAYOUT;
  const uintptr_t a0 = (uintptr_t)A, a1 = a0 + 2 * (uintptr_t)(spanA + 1);
  const uintptr_t c0 = (uintptr_t)C, c1 = c0 + 2 * (uintptr_t)(spanC + 1);
  const uintptr_t p0 = (uintptr_t)Bp, p1 = p0 + bytes;
  if (ranges_overlap(c0, c1, a0, a1) || ranges_overlap(c0, c1, p0, p1)) return GEMM_ERR_ALIAS;
  return launch_packed_product(DT_F16, A, lda_m, lda_k, Bp, C, ldc, M, N, K, 4, (hipStream_t)stream);
}

static int f8_dt(int32_t fmt_a, int32_t fmt_b) {
  if ((fmt_a != 0 && fmt_a != 1) || (fmt_b != 0 && fmt_b != 1)) return -1;
  return DT_F8 + 2 * fmt_a + fmt_b;
}

int gemm_f8_plan(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
                 int64_t ldb_n, const void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                 int32_t fmt_a, int32_t fmt_b, const gemm_f16_opts* opts, gemm_f16_plan_info* info) {
  const int dt = f8_dt(fmt_a, fmt_b);
  if (dt < 0) return GEMM_ERR_OPTS;
  return plan_impl(dt, A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, opts, info);
}

int gemm_f8_plan_cus(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
                     int64_t ldb_n, const void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                     int32_t fmt_a, int32_t fmt_b, int32_t cus, const gemm_f16_opts* opts,
                     gemm_f16_plan_info* info) {
  const int dt = f8_dt(fmt_a, fmt_b);
  if (dt < 0 || cus < 1 || cus > 65536) return GEMM_ERR_OPTS;
  return plan_impl(dt, A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, opts, info, cus);
}

int gemm_f8_ex(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
               int64_t ldb_n, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, int32_t fmt_a,
               int32_t fmt_b, void* stream, void* workspace, size_t workspace_bytes,
               const gemm_f16_opts* opts) {
  const int dt = f8_dt(fmt_a, fmt_b);
  if (dt < 0) return GEMM_ERR_OPTS;
  return ex_impl(dt, A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, stream, workspace,
                 workspace_bytes, opts);
}

int gemm_f8(const void* A, int64_t lda_m, int64_t lda_k, const void* B, int64_t ldb_k,
            int64_t ldb_n, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, int32_t fmt_a,
            int32_t fmt_b, void* stream) {
  return gemm_f8_ex(A, lda_m, lda_k, B, ldb_k, ldb_n, C, ldc, M, N, K, fmt_a, fmt_b, stream,
                    nullptr, 0, nullptr);
}

size_t gemm_f8_workspace_bytes(int64_t M, int64_t N, int64_t K, const gemm_f16_opts* opts) {
  return ws_impl(DT_F8, M, N, K, opts);   // the same for every format pair
}

const char* gemm_f16_status_string(int status) {
  switch (status) {
    case GEMM_OK: return "success";
    case GEMM_ERR_NULL: return "A, B or C is NULL";
    case GEMM_ERR_SHAPE: return "M, N or K <= 0, an address span overflows int64, or the grid is too large";
    case GEMM_ERR_STRIDE: return "a stride of A or B is <= 0";
    case GEMM_ERR_LDC: return "ldc < N";
    case GEMM_ERR_ALIAS: return "C (or the workspace) overlaps an input";
    case GEMM_ERR_WORKSPACE: return "workspace too small or not 256-byte aligned";
    case GEMM_ERR_OPTS: return "invalid options (variant, split, panel or tile)";
    case GEMM_ERR_HIP: return "HIP runtime error";
    case GEMM_ERR_LAYOUT: return "operand layout not taken for this format (FP8: K-contiguous A and B, 16-byte aligned rows)";
    case GEMM_ERR_SCRATCH: return "the plan's workspace exceeds the fixed no-allocation scratch (GEMM_F16_SCRATCH_BYTES, 32 MiB)";
    default: return "unknown status";
  }
}

int gemm_f16_version(void) { return kVersion; }

}  // extern "C"
