/*
 * gemm_f16.h -- dense fp16 matrix multiply for AMD Instinct MI355X (gfx950).
 *
 *     C[M,N] = A[M,K] . B[K,N]
 *
 * fp16 (IEEE binary16) inputs, fp32 accumulation, fp16 output rounded to
 * nearest-even.  The operation is the one the pages define: every output is
 * the K-term dot product of a row of A and a column of B (TileLang tutorial
 * ch. 14, section 1.1; "Matrix multiplication and memory-access
 * optimisation", section 01; "Triton GEMM: from one output tile to addresses,
 * bounds and data reuse", introduction: no bias, activation, batch or
 * quantisation; fp16 in, fp32 accumulator, fp16 out).
 *
 * Addressing (Triton article, section "shape gives meaning, stride gives
 * addresses"): all strides are in ELEMENTS, not bytes, and all arithmetic on
 * them is 64-bit (same article, section "addresses and bounds in one short
 * kernel"):
 *     A[i,k] at A + i*lda_m + k*lda_k
 *     B[k,j] at B + k*ldb_k + j*ldb_n
 *     C[i,j] at C + i*ldc + j          (C is row-major with unit column stride)
 * Transposed views and positive-stride slices of larger buffers are legal.
 * Elements outside the M x K and K x N views are never read, and outputs
 * outside M x N (including the ldc - N padding of each C row) are never
 * written (same article, section "three dimensions that do not divide").
 *
 * Ownership: the caller owns A, B, C and any workspace; the library keeps no
 * pointer after a call returns.  Pointers are DEVICE pointers on the current
 * HIP device.  Every entry point that launches work is asynchronous on the
 * given hipStream_t (passed as void*, NULL = the default stream) and never
 * synchronises; a fault inside a kernel surfaces at the caller's next
 * synchronisation.
 *
 * Errors: arguments are validated on the host before anything is enqueued;
 * on any error nothing is launched and C is untouched.  Results are
 * deterministic: the same inputs and options give bit-identical C (no
 * atomics in any reduction).
 */
#ifndef GEMM_F16_H
#define GEMM_F16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes.  The argument contract follows the Triton article's wrapper
 * (section "addresses and bounds in one short kernel"): empty shapes, zero or
 * negative strides and outputs that share storage with inputs are outside
 * it. */
enum gemm_status {
  GEMM_OK = 0,
  GEMM_ERR_NULL = -1,      /* A, B or C is NULL                                  */
  GEMM_ERR_SHAPE = -2,     /* M, N or K <= 0, an address span overflows int64,   */
                           /* or the grid exceeds the launch limit               */
  GEMM_ERR_STRIDE = -3,    /* lda_m, lda_k, ldb_k or ldb_n <= 0                   */
  GEMM_ERR_LDC = -4,       /* ldc < N: two outputs would share an address        */
  GEMM_ERR_ALIAS = -5,     /* C's byte range overlaps A's or B's                 */
  GEMM_ERR_WORKSPACE = -6, /* the workspace given is smaller than required       */
  GEMM_ERR_OPTS = -7,      /* invalid forced variant, split, panel or tile       */
  GEMM_ERR_HIP = -8,       /* a HIP runtime call failed (no device, launch, ...) */
  GEMM_ERR_LAYOUT = -9,    /* operand layout not taken for the format (FP8 below) */
  GEMM_ERR_SCRATCH = -10   /* gemm_f16_noalloc: the plan needs more than the     */
                           /* library's fixed scratch (GEMM_F16_SCRATCH_BYTES)   */
};

/* Kernel families (gemm_f16_opts.variant / gemm_f16_plan_info.variant).
 *
 * STREAMK is the tail-wave scheduling of the TileLang tutorial, ch. 14,
 * section 4.2 (stream-K: spread the K iterations evenly over the compute
 * units instead of whole tiles), in a deterministic form: the tiles that
 * fill whole waves of the 256x256 tile run as in MAIN; the last sk_tiles
 * tiles, which would leave most compute units idle in a final partial wave,
 * are split into split_k K ranges each, written as fp32 partials to the
 * workspace, and a fix-up launch sums each output's ranges in ascending
 * order (no atomics, bit-reproducible for a given plan).  It needs the
 * 256x256 LDS-DMA tile (K-contiguous A; N-contiguous B with N % 8 == 0, or
 * K-contiguous B; every stride at most 2^23 elements); forcing it for other
 * layouts returns GEMM_ERR_OPTS.
 * AUTO picks SKINNY for M <= 64; SPLITK when the 128x128 tiles would fill
 * at most half the compute units and K >= 2048 (fp16 operands the 128x128
 * LDS-DMA tile reads as they lie), or K >= 2 max(M, N) and K >= 1024 (any
 * other operands); otherwise MAIN, which becomes STREAMK when the partial
 * wave is at most half full and K >= 2048, and, with every tile in the
 * tail, when all the 256x256 tiles together fill less than half a wave with
 * M, N >= 256 and K long enough: K >= 4096 under 3/16 of a wave, K >= 8192
 * from 3/16 to 5/16, K >= 3072 from 5/16 on or where the 128x128 LDS-DMA
 * tile does not take the call (fp16 and bfloat16 alike). */
enum gemm_variant {
  GEMM_VARIANT_AUTO = 0,    /* choose from the shape (the default)                */
  GEMM_VARIANT_MAIN = 1,    /* one workgroup per output tile, whole K            */
  GEMM_VARIANT_SKINNY = 2,  /* M <= 64: B streamed once, K split, fixed-order sum */
  GEMM_VARIANT_SPLITK = 3,  /* tiles x K ranges into fp32 partials, then a       */
                            /* second pass sums the ranges in fixed order        */
  GEMM_VARIANT_TILE64X32 = 4, /* main structure with the pages' 64x32x32 tile   */
  GEMM_VARIANT_STREAMK = 5   /* main tiles in whole waves, then the last        */
                             /* sk_tiles tiles split over K across the idle     */
                             /* compute units, summed by a fixed-order fix-up   */
};

typedef struct gemm_f16_opts {
  int32_t variant; /* enum gemm_variant                                          */
  int32_t split_k; /* K ranges for SPLITK/SKINNY/STREAMK; 0 = choose; 1..256      */
  int32_t panel;   /* raster group height in tiles; 0 = choose; -1 = plain       */
                   /* row-major tile order without XCD remapping; 1..4096        */
  int32_t tile;    /* main-kernel tile id (0 = choose; see gemm_f16_plan_info)   */
} gemm_f16_opts;

/* Tile ids (gemm_f16_opts.tile, gemm_f16_plan_info.tile_id):
 *   1  128x128x64 register path (every layout; fp16 and bfloat16)
 *   2  64x32x32, the pages' Triton geometry (forced only; fp16)
 *   3, 4, 5  skinny 16, 32 and 64-row tiles (SKINNY; 3 is also reported
 *      for the decode kernel)
 *   6  256x256 register path (fp16; where tile 13 cannot read the layout)
 *   7  128x128 LDS-DMA, 4-stage ring (fp16, bfloat16; K-contiguous A, B
 *      either way with N % 8 == 0 when B is N-contiguous; FP8 with
 *      K-contiguous B and K even)
 *   8  64x128 LDS-DMA, the same ring with two waves (as tile 7)
 *   13 256x256 LDS-DMA, 4-stage ring (fp16; the same layouts, any stride)
 *   14 256x256 LDS-DMA with 128-byte A rows (fp16, bfloat16; the same
 *      layouts, strides up to 2^23 elements)
 *   15 256x256 FP8 (the FP8 entry points only)
 * A tile that does not take the operand layout hands over to the next one
 * that does: fp16 along 7 -> 1, 8 -> 1 and 14 -> 13 -> 6, bfloat16 straight
 * to 1, FP8 to 15.
 * Forcing an id without kernels for the call's format returns
 * GEMM_ERR_OPTS. */

typedef struct gemm_f16_plan_info {
  int32_t variant;          /* the family that runs (never AUTO)                 */
  int32_t tile_m, tile_n, tile_k; /* workgroup tile                              */
  int32_t split_k;          /* K ranges (1 = none)                               */
  int32_t panel;            /* raster group height in tiles (-1 = plain order)   */
  int32_t a_path, b_path;   /* operand load path: 0 gather, 1 vector along K,    */
                            /* 2 vector along M (A) or N (B) with a transpose;   */
                            /* 3: packed (B) or realigned (A) into the workspace */
  int32_t tile_id;          /* the tile configuration chosen                     */
  int64_t grid;             /* workgroups in the first launch                    */
  int64_t grid2;            /* workgroups in the reduction launch (0 = none)     */
  uint64_t workspace_bytes; /* device workspace the call needs (0 = none)        */
  int64_t sk_tiles;         /* STREAMK: tiles split over K (0 otherwise)         */
} gemm_f16_plan_info;

/*
 * C := A.B  with automatic kernel choice.  Equivalent to gemm_f16_ex with no
 * workspace and default options.  If the chosen kernel needs a workspace
 * (split-K partials), it is allocated stream-ordered on `stream`
 * (hipMallocAsync) and released stream-ordered after the last launch.
 */
int gemm_f16(const void* A, int64_t lda_m, int64_t lda_k,
             const void* B, int64_t ldb_k, int64_t ldb_n,
             void* C, int64_t ldc,
             int64_t M, int64_t N, int64_t K, void* stream);

/*
 * As gemm_f16, with an optional caller-owned device workspace and options.
 * workspace may be NULL (the library allocates stream-ordered when needed);
 * otherwise it must hold at least gemm_f16_workspace_bytes(...) bytes, be
 * 256-byte aligned, and not overlap A, B or C.  The workspace needs no
 * initialisation and its contents are garbage afterwards.  opts may be NULL.
 *
 * Packing plan (AUTO only): with K-contiguous B (ldb_k == 1), M >= 16384 and
 * the MAIN (unsplit) or STREAMK family on the 256x256 LDS-DMA tile, the call
 * first packs B into the front of the workspace in the layout of
 * gemm_f16_pack_b (one pass over B) and then runs the packed-B kernels: the
 * direct K-major B stages take half a cache line per B row per DMA.  The
 * plan reports b_path 3 and workspace_bytes = gemm_f16_packed_b_bytes(K, N)
 * plus the stream-K partials.  It runs when workspace is NULL or holds that
 * many bytes; a smaller caller workspace gets the direct plan instead.
 * The same holds from M >= 1024 for a 16-bit B that the LDS-DMA tile cannot
 * read directly (rows not 16-byte aligned, or neither dimension contiguous),
 * which would otherwise take the element-wise path of the 128x128 tile: the
 * packing pass reads B through its strides.  SPLITK plans pack such a B
 * from M, N >= 256, their partials after it.
 * Realigning plan (AUTO only, MAIN/SPLITK/STREAMK, N >= 256): a 16-bit A
 * that the LDS-DMA tile cannot read (rows not 16-byte aligned or not
 * K-contiguous; an M-contiguous A only from M*N*K >= 2^33) is first copied
 * through its strides into the front of the workspace as M rows of
 * ceil(K/64)*64 elements (zero past K), 256-byte rounded, and the product
 * runs on that copy.  The plan reports a_path 3; a packed B and any
 * partials follow the copy.  Neither pass runs below M*N*K = 2^27.
 * Both give the same bits.  The *_workspace_bytes functions report split
 * workspaces only.  gemm_bf16_ex does the same; gemm_f8_ex too, for an FP8
 * B with K-contiguous rows, packed into 16 KiB blocks of 64 k (workspace
 * gemm_f16_packed_b_bytes((K + 1) / 2, N)); an N-contiguous FP8 B is never
 * packed.
 */
int gemm_f16_ex(const void* A, int64_t lda_m, int64_t lda_k,
                const void* B, int64_t ldb_k, int64_t ldb_n,
                void* C, int64_t ldc,
                int64_t M, int64_t N, int64_t K, void* stream,
                void* workspace, size_t workspace_bytes, const gemm_f16_opts* opts);

/*
 * The plan gemm_f16_ex would execute for these arguments, without launching
 * anything.  Performs the same validation (return codes as above) and fills
 * *info.  Needs the current HIP device only when opts ask for automatic
 * choices (the compute-unit count feeds them); GEMM_ERR_HIP otherwise.
 */
int gemm_f16_plan(const void* A, int64_t lda_m, int64_t lda_k,
                  const void* B, int64_t ldb_k, int64_t ldb_n,
                  const void* C, int64_t ldc,
                  int64_t M, int64_t N, int64_t K,
                  const gemm_f16_opts* opts, gemm_f16_plan_info* info);

/*
 * As gemm_f16_plan, for a device with `cus` compute units (1..65536, else
 * GEMM_ERR_OPTS), without querying any device: the dispatch rules of
 * TileLang tutorial ch. 14, sections 4.1-4.2 (split-K, stream-K) and the
 * tile choice, as a host computation.  For planning ahead and for tests of
 * the rules on hosts without a GPU.  The pointers are read for their
 * alignment only.
 */
int gemm_f16_plan_cus(const void* A, int64_t lda_m, int64_t lda_k,
                      const void* B, int64_t ldb_k, int64_t ldb_n,
                      const void* C, int64_t ldc,
                      int64_t M, int64_t N, int64_t K, int32_t cus,
                      const gemm_f16_opts* opts, gemm_f16_plan_info* info);

/* Workspace bytes gemm_f16_ex needs for this shape and these options
 * (0 when the plan has no K split).  Returns 0 for invalid arguments too. */
size_t gemm_f16_workspace_bytes(int64_t M, int64_t N, int64_t K, const gemm_f16_opts* opts);

/*
 * The same product with bfloat16 inputs and output: A, B and C hold
 * bfloat16 (the upper 16 bits of an IEEE binary32) instead of binary16;
 * accumulation is fp32 and C is rounded to nearest-even bfloat16.  The same
 * arguments, validation, options (every variant but TILE64X32; tiles 2, 6
 * and 13 hold fp16 kernels only, and forcing them, or the 64x32x32
 * variant, returns GEMM_ERR_OPTS), workspace contract and return codes as
 * the fp16 functions above.  The pages fix fp16; bfloat16 is
 * the same computation in the other 16-bit format the matrix cores take
 * (TileLang tutorial, ch. 14, section 5: lower-precision variants keep the
 * GEMM skeleton and change the matrix instruction).
 */
int gemm_bf16(const void* A, int64_t lda_m, int64_t lda_k,
              const void* B, int64_t ldb_k, int64_t ldb_n,
              void* C, int64_t ldc,
              int64_t M, int64_t N, int64_t K, void* stream);
int gemm_bf16_ex(const void* A, int64_t lda_m, int64_t lda_k,
                 const void* B, int64_t ldb_k, int64_t ldb_n,
                 void* C, int64_t ldc,
                 int64_t M, int64_t N, int64_t K, void* stream,
                 void* workspace, size_t workspace_bytes, const gemm_f16_opts* opts);
int gemm_bf16_plan(const void* A, int64_t lda_m, int64_t lda_k,
                   const void* B, int64_t ldb_k, int64_t ldb_n,
                   const void* C, int64_t ldc,
                   int64_t M, int64_t N, int64_t K,
                   const gemm_f16_opts* opts, gemm_f16_plan_info* info);
size_t gemm_bf16_workspace_bytes(int64_t M, int64_t N, int64_t K, const gemm_f16_opts* opts);

/*
 * C := A.B with OCP FP8 operands, fp32 accumulation and binary16 output
 * (round to nearest even): the FP8 variant of the TileLang tutorial, ch. 14,
 * section 5 (E4M3 and E5M2 operands with wider accumulation, the GEMM
 * skeleton kept, a K step of 64).  fmt_a and fmt_b give each operand's
 * format: 0 = E4M3 (the "FN" variant: no infinities, 448 the largest
 * finite value), 1 = E5M2; anything else is GEMM_ERR_OPTS.  A and B are one
 * byte per element; strides are in elements as for the 16-bit calls; C is
 * binary16 with row stride ldc.
 *
 * Layout: A must be K-contiguous (lda_k == 1).  B is either K-contiguous
 * (ldb_k == 1: the [N, K] weight layout, seen as a transposed view) or
 * N-contiguous (ldb_n == 1: B [K, N] row-major, with N a multiple of 16).
 * Row strides (lda_m, and ldb_n or ldb_k) are multiples of 16 and at most
 * 2^24, and A and B are 16-byte aligned; any other
 * layout returns GEMM_ERR_LAYOUT before anything is enqueued.  M, N and K are
 * masked as in the 16-bit calls (zero fill on K).  Variants: AUTO, MAIN,
 * SPLITK and STREAMK on the 256 x 256 x 64 FP8 tile (MAIN and SPLITK also
 * on the 128 x 128 and 64 x 128 LDS-DMA tiles, tile ids 7 and 8, for
 * K-contiguous B and K even: AUTO takes them below 80 tiles of 256 x 256 on
 * 256 compute units, and splits K there from K >= 4096),
 * and SKINNY (M <= 64
 * with N-contiguous B, M <= 16 with K-contiguous B): the decode kernel,
 * which widens the bytes to binary16 (exact for both formats) and runs the
 * 16-bit decode path; AUTO takes it up to 32 and 16 rows.  SKINNY outside
 * those bounds or with a forced tile, and TILE64X32, return GEMM_ERR_OPTS.
 * Workspace contract and other return codes as above.
 */
int gemm_f8(const void* A, int64_t lda_m, int64_t lda_k,
            const void* B, int64_t ldb_k, int64_t ldb_n,
            void* C, int64_t ldc,
            int64_t M, int64_t N, int64_t K, int32_t fmt_a, int32_t fmt_b, void* stream);
int gemm_f8_ex(const void* A, int64_t lda_m, int64_t lda_k,
               const void* B, int64_t ldb_k, int64_t ldb_n,
               void* C, int64_t ldc,
               int64_t M, int64_t N, int64_t K, int32_t fmt_a, int32_t fmt_b, void* stream,
               void* workspace, size_t workspace_bytes, const gemm_f16_opts* opts);
int gemm_f8_plan(const void* A, int64_t lda_m, int64_t lda_k,
                 const void* B, int64_t ldb_k, int64_t ldb_n,
                 const void* C, int64_t ldc,
                 int64_t M, int64_t N, int64_t K, int32_t fmt_a, int32_t fmt_b,
                 const gemm_f16_opts* opts, gemm_f16_plan_info* info);
/* gemm_f8_plan for a device with `cus` compute units, without any device
 * query (as gemm_f16_plan_cus; cus outside [1, 65536] is GEMM_ERR_OPTS). */
int gemm_f8_plan_cus(const void* A, int64_t lda_m, int64_t lda_k,
                     const void* B, int64_t ldb_k, int64_t ldb_n,
                     const void* C, int64_t ldc,
                     int64_t M, int64_t N, int64_t K, int32_t fmt_a, int32_t fmt_b, int32_t cus,
                     const gemm_f16_opts* opts, gemm_f16_plan_info* info);
size_t gemm_f8_workspace_bytes(int64_t M, int64_t N, int64_t K, const gemm_f16_opts* opts);

/*
 * Pre-packed static B: the C500 log's weight packing (B re-laid once,
 * outside the timed region, into the order the matrix instructions read
 * it), reported beside the general-stride path and never instead of it.
 * gemm_f16_pack_b reads B [K, N] through its element strides (any positive
 * strides) and writes Bp, an opaque device buffer of
 * gemm_f16_packed_b_bytes(K, N) bytes (256-byte aligned, not overlapping B):
 * 256-column panels of ceil(K/32) blocks of 16 KiB, each block the LDS image
 * of one K-major B stage of the 256 x 256 LDS-DMA tile, zero past N and K.
 * gemm_f16_packed computes C := A.B from A (K-contiguous, 16-byte aligned
 * rows at most 2^23 elements apart: GEMM_ERR_LAYOUT otherwise) and Bp
 * packed for the same K and N, on the main variant of that tile (no split,
 * no workspace; K above 2^36 is GEMM_ERR_SHAPE, as that tile counts its
 * 64-k steps in 32 bits).  Both are
 * asynchronous on `stream`; other return codes as gemm_f16.  The packed
 * buffer's layout is private to this library version.
 */
size_t gemm_f16_packed_b_bytes(int64_t K, int64_t N);
int gemm_f16_pack_b(const void* B, int64_t ldb_k, int64_t ldb_n, int64_t K, int64_t N, void* Bp,
                    void* stream);
int gemm_f16_packed(const void* A, int64_t lda_m, int64_t lda_k, const void* Bp,
                    void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Grouped product, one launch over G products that share N and K (the
 * TileLang tutorial, ch. 14, section 4.3: grouped GEMM with per-group row
 * counts, as for the experts of a mixture-of-experts layer):
 *
 *     for g in [0, G):  C[r, :] = A[r, :] . B_g   for r in [offsets[g], offsets[g+1])
 *
 *   A        [M_total, K], element strides (lda_m, lda_k): the rows of all
 *            groups, group by group (e.g. tokens sorted by expert).
 *   B        G matrices [K, N]; B_g[k,j] at B + g*ldb_g + k*ldb_k + j*ldb_n.
 *            ldb_g >= 0 (0: every group uses the same B).
 *   C        [M_total, N], row stride ldc >= N, column stride 1.
 *   offsets  DEVICE pointer to G + 1 int64 row offsets, non-decreasing,
 *            within [0, M_total].  They are read on the device (the host
 *            never needs the row counts).  Values outside [0, M_total] are
 *            clamped into it, so no access ever leaves the views above; with
 *            decreasing offsets, rows claimed by two groups get unspecified
 *            values.  Rows of C outside every group are not written.
 *   workspace  NULL (allocated stream-ordered) or at least
 *            gemm_f16_grouped_workspace_bytes(G) bytes, 256-byte aligned,
 *            not overlapping A, B or C; no initialisation needed.
 *
 * Same numerics, validation and return codes as gemm_f16; G must be in
 * [1, 2^20].  Asynchronous on `stream`; deterministic.
 */
int gemm_f16_grouped(const void* A, int64_t lda_m, int64_t lda_k,
                     const void* B, int64_t ldb_g, int64_t ldb_k, int64_t ldb_n,
                     void* C, int64_t ldc,
                     const int64_t* offsets, int32_t G,
                     int64_t M_total, int64_t N, int64_t K, void* stream,
                     void* workspace, size_t workspace_bytes);

/*
 * The grouped product with bfloat16 A, B and C (fp32 accumulation, output
 * rounded to nearest-even bfloat16): the same arguments, validation, return
 * codes and workspace as gemm_f16_grouped.
 */
int gemm_bf16_grouped(const void* A, int64_t lda_m, int64_t lda_k,
                      const void* B, int64_t ldb_g, int64_t ldb_k, int64_t ldb_n,
                      void* C, int64_t ldc,
                      const int64_t* offsets, int32_t G,
                      int64_t M_total, int64_t N, int64_t K, void* stream,
                      void* workspace, size_t workspace_bytes);

/*
 * The grouped product with FP8 A and B (formats fmt_a, fmt_b: 0 E4M3, 1 E5M2,
 * as for gemm_f8_ex), fp32 accumulation and binary16 C.  Strides of A and B
 * (and ldb_g) count bytes.  The layouts of gemm_f8_ex: A K-contiguous; every
 * B_g K-contiguous ([N, K] rows) or N-contiguous ([K, N] rows, N a multiple
 * of 16); 16-byte aligned bases and rows at most 2^24 bytes apart; ldb_g a
 * multiple of 16 (GEMM_ERR_LAYOUT otherwise).  Other arguments, return
 * codes and the workspace as for gemm_f16_grouped.
 */
int gemm_f8_grouped(const void* A, int64_t lda_m, int64_t lda_k,
                    const void* B, int64_t ldb_g, int64_t ldb_k, int64_t ldb_n,
                    void* C, int64_t ldc,
                    const int64_t* offsets, int32_t G,
                    int64_t M_total, int64_t N, int64_t K, int32_t fmt_a, int32_t fmt_b,
                    void* stream, void* workspace, size_t workspace_bytes);

/* Workspace bytes gemm_f16_grouped, gemm_bf16_grouped and gemm_f8_grouped
 * need for G groups (0 if G is invalid). */
size_t gemm_f16_grouped_workspace_bytes(int32_t G);

/*
 * For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation): C := A.B as
 * gemm_f16, with the same arguments, validation and return codes, but the
 * library allocates nothing.  The call never runs a packing plan, and a
 * plan's workspace (split-K, stream-K or decode partials) lives in a fixed
 * device array of GEMM_F16_SCRATCH_BYTES inside the library, one per GPU,
 * held until the process ends.  A plan that needs more returns
 * GEMM_ERR_SCRATCH before anything is enqueued (gemm_f16_plan with opts
 * NULL reports the workspace a shape needs, packing aside).  Every call on
 * one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (on different streams, or from several threads without ordering) race and
 * may give wrong results; calls ordered on one stream do not.  No kernel
 * reads scratch it has not written in the same call, so it needs no clearing.
 */
#define GEMM_F16_SCRATCH_BYTES ((size_t)32 << 20)
int gemm_f16_noalloc(const void* A, int64_t lda_m, int64_t lda_k,
                     const void* B, int64_t ldb_k, int64_t ldb_n,
                     void* C, int64_t ldc,
                     int64_t M, int64_t N, int64_t K, void* stream);

/* Static, NUL-terminated description of a return code. */
const char* gemm_f16_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int gemm_f16_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F16_H */
