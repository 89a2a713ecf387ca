/*
 * sk_gemm.h -- Stream-K GEMM for AMD Instinct MI355X (gfx950), C ABI.
 *
 * Every entry point computes, for m < M and n < N,
 *
 *     C[m][n] = RNE_bf16( sigma * sum_{k<K} a(m,k) * b(n,k) + bias[n] )
 *
 * with one persistent launch of at most grid_cap workgroups, in which each
 * workgroup owns a contiguous range of K-loop MAC iterations that may span
 * several output tiles ("Stream-k mxfp4 kernel", tritonBLAS pull request 74:
 * description and pull request overview).  A tile whose iterations are split
 * between workgroups is finished by its owner after it has added the fp32
 * partial tiles of the other workgroups in a fixed order, so the bits of C do
 * not depend on timing.  The bias, when present, runs along N, is broadcast
 * over the M rows and is added exactly once, after that aggregation ("Fix
 * StreamK Kernel Bias #67", Motivation and Technical Details).  The grid cap
 * mirrors a persistent GEMM confined to a chosen number of compute units
 * ("SM-constraint-GEMM by triton persistent kernel", description and Nsys
 * Results: a cap above the device's unit count is clamped to it).
 *
 * Layouts (all row-major, the K index contiguous):
 *   MXFP4  A uint8[M][K/2], B uint8[N][K/2]: two OCP E2M1 codes per byte, the
 *          even K index in the low nibble.  A_scale uint8[M][K/32],
 *          B_scale uint8[N][K/32]: OCP E8M0 (value 2^(e-127)), one per 32
 *          consecutive K elements starting at k = 0.  E8M0 0xFF (NaN) is
 *          undefined input.  sigma = 1.
 *   bf16   A uint16[M][K], B uint16[N][K] (bf16 bit patterns).  sigma = 1.
 *   MXFP8  A uint8[M][K], B uint8[N][K], OCP E4M3FN elements; A_scale
 *          uint8[M][K/32], B_scale uint8[N][K/32] E8M0 block scales as for
 *          MXFP4.  sigma = 1.
 *   MXFP6  A uint8[M][3K/4], B uint8[N][3K/4]: OCP E2M3 (SK_MXFP6_E2M3) or
 *          E3M2 (SK_MXFP6_E3M2) 6-bit codes packed as one little-endian bit
 *          stream per row (code k is bits 6k .. 6k+5 of the row, bit b of the
 *          stream being bit b % 8 of byte b / 8), so each block of 32
 *          elements is 24 bytes.  Scales as for MXFP4.  sigma = 1.
 *   mixed  SK_MXFP4_MXFP8: A as for MXFP4, B as for MXFP8; SK_MXFP8_MXFP4:
 *          A as for MXFP8, B as for MXFP4.  Scales as for MXFP4.  sigma = 1.
 *   fp8    A uint8[M][K], B uint8[N][K], OCP E4M3FN.  A_scale / B_scale are
 *          device pointers to one fp32 each (per-tensor), NULL meaning 1.0;
 *          sigma = A_scale * B_scale, applied to the fp32 sum before the bias
 *          (the bias is converted to fp32 for the add).
 *   bias   bf16[N] bit patterns, or NULL.
 *   C      bf16[M][N] bit patterns, written in full (every element).
 * B is stored N x K (the transpose of the usual K x N), so A and B are read
 * the same way.  C must not overlap any input.
 *
 * Precision: fp32 accumulation.  The one rounding to bf16 is round-to-
 * nearest-even of the fp32 value sigma*acc (+) bias taken exactly (the sum is
 * first rounded to odd in fp32, which keeps enough bits that the rounding to
 * bf16 after it is the correct rounding of the exact sum: adding the bias
 * never double-rounds).
 *
 * Ownership and asynchrony: all tensor pointers are device pointers owned by
 * the caller and must stay valid until the stream has passed the launch.
 * Calls enqueue on `stream` (a hipStream_t passed as void*; NULL is the
 * default stream) and return without waiting.  The library owns its scratch
 * (fp32 partial tiles, lock flags, an error word, and for the MX types a
 * k-step-major copy of the two scale arrays that a small kernel writes before
 * the GEMM on the same stream), kept per (device, stream), grown on demand and
 * freed by sk_release_workspace().  Device-side failures (a workgroup that
 * waited past its spin limit) are reported by sk_check().
 *
 * HIP graphs: a stream that is being captured is refused (SK_ERR_UNSUPPORTED,
 * nothing enqueued).  The lock flags of the fixup are compared with a
 * per-launch epoch that is a kernel argument, so a captured launch would
 * replay with a fixed epoch and an owner could take the flags of the previous
 * replay for this one's; the scratch may also have to grow, which needs a
 * synchronisation that capture forbids.
 *
 * Errors: every call returns an sk_status and never aborts.  Arguments are
 * checked before anything is launched:
 *   SK_ERR_ARG          a required pointer is NULL, M, N or K < 1, a size is
 *                       beyond the supported range (M < 2^31, N <= 2^22,
 *                       K <= 2^21, tiles * MAC iterations per tile < 2^31;
 *                       MX types: M * K / 32 and N * K / 32 below 2^31),
 *                       C overlaps an input, bf16 given scales, an unknown
 *                       dtype / policy, or sk_addmm without a bias;
 *   SK_ERR_ALIGN        an MX type with K not a multiple of 32 (whole
 *                       scale blocks), fp8 K not a multiple of 16, bf16 K
 *                       not a multiple of 8 (a row of A or B must be a whole
 *                       number of 16-byte chunks), or A, B, C not 16-byte
 *                       aligned, or bias not 2-byte aligned;
 *   SK_ERR_UNSUPPORTED  the current device is not gfx950, a tile override
 *                       names no compiled kernel for that dtype, or the stream
 *                       is being captured into a HIP graph;
 *   SK_ERR_HIP          a HIP runtime call failed;
 *   SK_ERR_NOMEM        scratch could not be allocated;
 *   SK_ERR_TIMEOUT      (sk_check only) a workgroup gave up waiting for a
 *                       partial tile; the affected output tiles are unwritten;
 *   SK_ERR_SCRATCH      (sk_gemm_mxfp4_noalloc only) the call needs more
 *                       scratch than its fixed buffer holds.
 */
#ifndef SK_GEMM_H
#define SK_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sk_status {
  SK_OK = 0,
  SK_ERR_ARG = 1,
  SK_ERR_ALIGN = 2,
  SK_ERR_UNSUPPORTED = 3,
  SK_ERR_HIP = 4,
  SK_ERR_NOMEM = 5,
  SK_ERR_TIMEOUT = 6,
  SK_ERR_SCRATCH = 7
} sk_status;

typedef enum sk_dtype {
  SK_MXFP4 = 0, SK_BF16 = 1, SK_FP8_E4M3 = 2, SK_MXFP8 = 3, SK_MXFP6_E2M3 = 4, SK_MXFP6_E3M2 = 5,
  SK_MXFP4_MXFP8 = 6, SK_MXFP8_MXFP4 = 7
} sk_dtype;

/* How output tiles are divided between the persistent workgroups.
 * HYBRID: whole tiles are dealt out round-robin ("data-parallel tail"), and
 *   only the tiles that would leave the last round unbalanced -- the
 *   remainder plus one full round -- are shared out by MAC iteration
 *   (Stream-K head); no head when the tile count is a multiple of the grid.
 * PURE_SK: every tile is shared out by MAC iteration.
 * PURE_DP: whole tiles round-robin, no iteration splitting (the "Persistent"
 *   path that the Stream-K switch turns off in "Fix StreamK Kernel Bias #67",
 *   Improve StreamK Testing). */
/* AUTO: the kernel and policy measured fastest at the nearest swept shape
 *   (the best-config search of "SM-constraint-GEMM by triton persistent
 *   kernel", description, checklist; the table is compiled into the library), else
 *   HYBRID with the kernel chosen by problem shape.  A fixed tile or kernel
 *   keeps its choice and runs HYBRID.  The sk_gemm_* and sk_addmm entry
 *   points use AUTO. */
typedef enum sk_policy {
  SK_POLICY_HYBRID = 0,
  SK_POLICY_PURE_SK = 1,
  SK_POLICY_PURE_DP = 2,
  SK_POLICY_AUTO = 3
} sk_policy;

/* sk_gemm_args.debug_flags bits (tests only). */
#define SK_DEBUG_DELAY 1u       /* each workgroup sleeps a seeded pseudo-random time before publishing its partial */
#define SK_DEBUG_DROP_SIGNAL 2u /* workgroup drop_signal_wg never publishes its partial tile's flag */
#define SK_DEBUG_RELAYOUT 4u    /* MX: always copy the scales into the kernel's lane order first, even where a
                                   kernel of at most 128-row tiles could read the caller's [rows][K/32] scales
                                   directly (K a whole number of k-steps, scale arrays 4-byte aligned) */

/* MXFP4: A, B packed E2M1; A_scale, B_scale E8M0 (required).  bias may be NULL.
 * The FP4 GEMM with Stream-K load balancing over the K-loop ("Stream-k mxfp4
 * kernel", author's description and pull request overview: the FP4 Stream-K
 * kernel behind the matmul_fp4 dispatch, with per-workgroup partial tiles and
 * lock flags).  Policy AUTO; grid_cap as for every entry point (<= 0: all the
 * stream's compute units).  stream is a hipStream_t passed as void*. */
sk_status sk_gemm_mxfp4(const uint8_t* A, const uint8_t* B, const uint8_t* A_scale, const uint8_t* B_scale,
                        const void* bias, void* C, int64_t M, int64_t N, int64_t K, int grid_cap, void* stream);

/* sk_gemm_mxfp4 for callers that cannot allocate device memory (code in a serving
 * loop that must not call hipMalloc, harnesses that forbid allocation): the same
 * arguments, kernels and result, with every piece of scratch -- lock flags and the
 * error word, fp32 partial tiles, the re-laid MX scales -- taken from one fixed
 * device array of the library (a static __device__ buffer of 8 KiB of flags plus
 * 32 MiB, of which each device the library runs on keeps its own copy until the
 * process ends).  Nothing is allocated, freed or grown, by this library or by any
 * library it calls, after the first call on a device, which looks up the array's
 * address and clears its flag words.
 *   Limits: partial tiles plus re-laid scales must fit in 32 MiB.  When the tuned
 *   plan's partial tiles do not fit, the same kernel runs data-parallel over whole
 *   tiles instead (MXFP4 sums are exact in fp32 in any order, so C is bit-for-bit
 *   the same); when the re-laid scales alone do not fit ((M + N) * K / 32 bytes,
 *   rounded up to whole tiles, about 32 MiB) the call returns SK_ERR_SCRATCH and
 *   enqueues nothing.
 *   Sharing: every call on a device uses that device's one array, which keeps the
 *   last call's contents; calls whose execution overlaps on one device (two
 *   streams, or two host threads without ordering) race on it and may give wrong
 *   results -- order them on one stream.  A device-side timeout is reported by
 *   sk_check on any stream of the device.  Errors otherwise as for sk_gemm_mxfp4;
 *   a capturing stream is refused the same way. */
sk_status sk_gemm_mxfp4_noalloc(const uint8_t* A, const uint8_t* B, const uint8_t* A_scale, const uint8_t* B_scale,
                                const void* bias, void* C, int64_t M, int64_t N, int64_t K, int grid_cap,
                                void* stream);

/* bf16 x bf16 -> bf16.  bias may be NULL.  The Stream-K matmul that the bias
 * page's correctness tests run on both the Persistent and the Stream-K path and
 * compare with torch.mm / torch.addmm ("Fix StreamK Kernel Bias #67", pull
 * request overview and the review comments on the two tests).  Policy AUTO. */
sk_status sk_gemm_bf16(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N, int64_t K,
                       int grid_cap, void* stream);

/* fp8 (E4M3FN) with per-tensor fp32 scales (device pointers to one float each, NULL = 1.0).  bias may be NULL.
 * The quantized mode of the Stream-K kernel, in which the bias is converted to
 * fp32 before it is added to the scaled sum ("Fix StreamK Kernel Bias #67",
 * Technical Details); the persistent grid may be capped to a number of compute
 * units ("SM-constraint-GEMM by triton persistent kernel", description).
 * Policy AUTO. */
sk_status sk_gemm_fp8(const uint8_t* A, const uint8_t* B, const float* A_scale, const float* B_scale,
                      const void* bias, void* C, int64_t M, int64_t N, int64_t K, int grid_cap, void* stream);

/* MXFP8: A, B E4M3FN elements; A_scale, B_scale E8M0 per 32 K (required).  bias may be NULL.
 * The same block-scaled contraction as MXFP4 with 8-bit elements: the quantized
 * mode in which the bias is turned into fp32 before it is added ("Fix StreamK
 * Kernel Bias #67", Technical Details), with the OCP MX v1.0 block scales of the
 * MXFP4 path ("Stream-k mxfp4 kernel", description). */
sk_status sk_gemm_mxfp8(const uint8_t* A, const uint8_t* B, const uint8_t* A_scale, const uint8_t* B_scale,
                        const void* bias, void* C, int64_t M, int64_t N, int64_t K, int grid_cap, void* stream);

/* Block-scaled operands of any OCP MX element type: a_fmt and b_fmt are
 * SK_MXFP4, SK_MXFP6_E2M3, SK_MXFP6_E3M2 or SK_MXFP8 (A and B laid out as for
 * that type, scales E8M0 [rows][K/32], required; bias may be NULL).  MXFP6
 * and the mixed MXFP4 x MXFP8 products are the other MX formats of the
 * quantized mode ("Fix StreamK Kernel Bias #67", Technical Details; MX formats
 * of "Stream-k mxfp4 kernel", description).  Equal formats run that type's
 * kernels (as sk_gemm_mxfp4 / sk_gemm_mxfp8 do); an MXFP4 operand with an
 * MXFP8 one runs the SK_MXFP4_MXFP8 / SK_MXFP8_MXFP4 kernels, in which the
 * scaled MFMA takes each operand in its own format.  Policy AUTO.  Errors as
 * for sk_gemm_mxfp4; SK_ERR_ARG also for a format that is not MX, and
 * SK_ERR_UNSUPPORTED for an MXFP6 operand with an operand of another format
 * (not compiled). */
sk_status sk_gemm_mx(sk_dtype a_fmt, sk_dtype b_fmt, const uint8_t* A, const uint8_t* B, const uint8_t* A_scale,
                     const uint8_t* B_scale, const void* bias, void* C, int64_t M, int64_t N, int64_t K, int grid_cap,
                     void* stream);

/* addmm(bias, A, B) = the dtype's GEMM with a bias that is required (alpha = beta = 1).
 * A_scale / B_scale as for that dtype (NULL for bf16).  The bias runs along N, is
 * broadcast over the M rows and is added once, after the partial tiles of a split
 * tile have been aggregated ("Fix StreamK Kernel Bias #67", Motivation and
 * Technical Details; the tests compare with torch.addmm, hence alpha = beta = 1).
 * Policy AUTO; SK_ERR_ARG when bias is NULL. */
sk_status sk_addmm(sk_dtype dtype, const void* bias, const void* A, const void* B, const void* A_scale,
                   const void* B_scale, void* C, int64_t M, int64_t N, int64_t K, int grid_cap, void* stream);

/* bf16 backward of C = A * B^T + bias (A [M][K], B [N][K], bias [N], as
 * stored by sk_gemm_bf16 / sk_addmm), given dC = dL/dC (bf16 [M][N]):
 *     dA[m][k]  = RNE_bf16( sum_n dC[m][n] * B[n][k] )      bf16 [M][K]
 *     dB[n][k]  = RNE_bf16( sum_m dC[m][n] * A[m][k] )      bf16 [N][K]
 *     dbias[n]  = RNE_bf16( sum_m dC[m][n] )                bf16 [N]
 * the gradients that the Stream-K matmul and addmm tests take and compare
 * with torch's for a, b and the bias ("Fix StreamK Kernel Bias #67", review
 * comments on the two Stream-K tests).  dA and dB run through the same
 * Stream-K kernels (policy AUTO, grid as for sk_gemm_bf16): the operands are
 * first transposed into K-contiguous copies in the library's scratch of
 * (device, stream), B^T for dA and dC^T, A^T for dB.  dbias is summed in fp32
 * in a fixed order.  Any of dA, dB, dbias may be NULL (not computed; at least
 * one is required); A may be NULL when dB is, B when dA is.  M, N and K must
 * be multiples of 8 (SK_ERR_ALIGN), the sizes as for the GEMMs this makes
 * (N <= 2^21 for dA, M <= 2^21 for dB, K <= 2^22), outputs must not overlap
 * inputs or each other (SK_ERR_ARG).  Precision as for sk_gemm_bf16: fp32
 * accumulation, one rounding. */
sk_status sk_gemm_bf16_backward(const void* dC, const void* A, const void* B, void* dA, void* dB, void* dbias,
                                int64_t M, int64_t N, int64_t K, int grid_cap, void* stream);

/* Full-control entry point: the same kernels with a chosen policy and tile, plus test hooks.
 * Zero-initialise and fill the fields you need.  The policies are the Stream-K
 * partition of the MAC-iteration space ("Stream-k mxfp4 kernel", description)
 * and the Persistent path the bias page's tests switch between ("Fix StreamK
 * Kernel Bias #67", pull request overview); errors as for sk_gemm_mxfp4. */
typedef struct sk_gemm_args {
  int32_t dtype;            /* sk_dtype */
  int32_t policy;           /* sk_policy */
  const void* A;
  const void* B;
  const void* A_scale;      /* MXFP4, MXFP8: uint8 [M][K/32]; fp8: device float* or NULL; bf16: NULL */
  const void* B_scale;
  const void* bias;         /* bf16[N] or NULL */
  void* C;                  /* bf16[M][N] */
  int64_t M, N, K;
  int32_t grid_cap;         /* <= 0: every compute unit */
  int32_t tile_m, tile_n;   /* 0, 0: automatic choice; else one of the compiled tiles of that dtype */
  void* stream;             /* hipStream_t */
  uint32_t debug_flags;     /* SK_DEBUG_* (tests only) */
  uint32_t delay_seed;      /* with SK_DEBUG_DELAY */
  int32_t drop_signal_wg;   /* with SK_DEBUG_DROP_SIGNAL */
  int32_t variant;          /* 0: automatic; k > 0: compiled kernel k-1 (see sk_variant_info), which must
                               match dtype and, for a direct-only kernel, the call (sk_variant_k_split);
                               SK_ERR_UNSUPPORTED otherwise; overrides tile_m, tile_n */
  uint64_t spin_limit_ticks;/* owner wait limit in ticks of the 100 MHz device clock; 0 = 2e8 (2 s) */
  uint64_t* trace;          /* NULL, or a device buffer of 32 uint64 per workgroup of the launch (sk_plan's
                               grid): a phase trace.  Wave 0 of workgroup w writes 100 MHz timestamps
                               (s_memrealtime) to trace[32 w + i]: i = 0 entry; 29 after the first
                               argument reads; 28 first stages' loads issued; 27 stage 0 landed; for its
                               work items j < 6, i = 1 + 4 j first k-step, 2 + 4 j k-steps done, 3 + 4 j
                               partial published / owner's waits done, 4 + 4 j item finished; 30 the item
                               count; 31 exit.  Words of items not reached are left as they were.  The
                               timing of traced calls is the same code's (the stores are wave 0's only);
                               the stamps let the phases of a persistent launch -- ramp, streaming,
                               fixup waits, epilogues -- be read per workgroup ("SM-constraint-GEMM by
                               triton persistent kernel", SM usage by nsys profile). */
} sk_gemm_args;

sk_status sk_gemm_ex(const sk_gemm_args* args);

/* The partition a call would use (host-only; no device work).  num_cus = 0 asks the current device.
 * Grid G = min(cap, compute units, work), with a cap above the unit count clamped
 * to it ("SM-constraint-GEMM by triton persistent kernel", Nsys Results: 133
 * requested on a 132-unit device ran 132); the Stream-K ranges split the MAC
 * iterations ("Stream-k mxfp4 kernel", description).  SK_ERR_ARG on a bad query,
 * SK_ERR_UNSUPPORTED when no compiled kernel has the requested tile. */
typedef struct sk_plan_query {
  int32_t dtype, policy;
  int64_t M, N, K;
  int32_t grid_cap;
  int32_t tile_m, tile_n;
  int32_t num_cus;
  int32_t variant;          /* as in sk_gemm_args */
} sk_plan_query;

typedef struct sk_plan_info {
  int32_t tile_m, tile_n, tile_k;   /* output tile and K elements per MAC iteration */
  int32_t tiles_m, tiles_n;
  int64_t tiles;                    /* T */
  int32_t iters_per_tile;           /* I = ceil(K / tile_k) */
  int32_t grid;                     /* G, persistent workgroups launched */
  int32_t policy;
  int32_t variant;                  /* index of the compiled kernel */
  int64_t sk_tiles;                 /* tiles [0, sk_tiles) are shared by iteration */
  int64_t sk_iters;                 /* S = sk_tiles * I */
  int64_t iters_per_wg;             /* q = S / G */
  int64_t iters_extra;              /* r = S % G: workgroups w < r get q + 1 iterations */
  int64_t scratch_bytes;            /* fp32 partial-tile scratch this call needs */
  int32_t threads;                  /* threads per workgroup */
  int32_t lds_bytes;                /* LDS per workgroup */
} sk_plan_info;

sk_status sk_plan(const sk_plan_query* q, sk_plan_info* out);

/* Stream-K iteration range [begin, end) of workgroup wg under plan p (host-only): the
 * contiguous range of MAC iterations each persistent workgroup owns ("Stream-k mxfp4
 * kernel", description).  SK_ERR_ARG for a NULL pointer or wg outside [0, grid). */
sk_status sk_plan_wg_range(const sk_plan_info* p, int32_t wg, int64_t* begin, int64_t* end);

/* One unit of a workgroup's work: MAC iterations [k0, k1) of output tile `tile`.
 * mode 0: finish the tile (epilogue); 1: publish the fp32 partial for the tile's
 * finisher; 2: add the partials of workgroups first .. wg-1 (descending), then finish. */
typedef struct sk_work_item {
  int64_t tile;
  int32_t k0, k1;
  int32_t mode;
  int32_t first;
} sk_work_item;

/* The ordered work list the kernel runs for workgroup wg under plan p (host-only; the
 * kernel walks the same list).  Writes at most max_items items; *count gets the total.
 * Contributors publish a partial tile and its lock flag, the finishing workgroup
 * aggregates them and then adds the bias ("Stream-k mxfp4 kernel", the per-workgroup
 * locks and P buffers of the Copilot comment; "Fix StreamK Kernel Bias #67",
 * Motivation).  SK_ERR_ARG for a NULL pointer or wg outside [0, grid). */
sk_status sk_plan_wg_work(const sk_plan_info* p, int32_t wg, sk_work_item* items, int32_t max_items,
                          int32_t* count);

/* Waits for `stream` (a hipStream_t), then reports (and clears) a device-side timeout
 * recorded in this device/stream's scratch since the last check: SK_ERR_TIMEOUT when an
 * owner gave up waiting for a contributor's lock flag (the per-workgroup locks of
 * "Stream-k mxfp4 kernel", Copilot comment), SK_ERR_UNSUPPORTED on a capturing stream,
 * SK_ERR_HIP when the runtime fails. */
sk_status sk_check(void* stream);

/* Waits for every stream that has scratch, then frees all scratch of every device.
 * The scratch is kept per (device, stream) rather than as one global buffer on the
 * default device ("Stream-k mxfp4 kernel", Copilot comment on the global Stream-K
 * scratch buffers). */
void sk_release_workspace(void);

/* Test hook: fill the current device/stream's scratch (grown to at least scratch_bytes) with
 * NaN partials and stale lock values, so a following call must not depend on their contents. */
sk_status sk_debug_poison_workspace(void* stream, int64_t scratch_bytes);

/* CU-partitioned streams.  A persistent GEMM held to a chosen set of compute
 * units exists so that other work can run on the remaining units of the same
 * device at the same time (the intra-device parallelism named in
 * "SM-constraint-GEMM by triton persistent kernel", description).
 *
 * sk_stream_create_cu_masked creates a HIP stream (default priority) whose
 * kernels run only on the compute units set in cu_mask: bit (i % 32) of word
 * i / 32 is CU i; `words` is the number of 32-bit words (1..64), and bits at
 * or above the device's CU count are ignored.  The calls of this library on
 * such a stream size their persistent grid to those units: grid_cap <= 0
 * means all of them and a larger cap is clamped to their number.  Returns
 * SK_ERR_ARG for a NULL pointer, a bad word count or a mask with no CU of the
 * device, SK_ERR_HIP if the runtime refuses the stream.  The caller owns the
 * stream and releases it (and the library's scratch kept for it) with
 * sk_stream_destroy, which first waits for the stream.
 *
 * sk_stream_cu_count reports the compute units kernels on `stream` may use
 * (every CU for the null stream or an unmasked stream).  For streams not
 * made here the count is read from the runtime the first time the library
 * sees the stream and kept for it. */
sk_status sk_stream_create_cu_masked(const uint32_t* cu_mask, int32_t words, void** stream);
sk_status sk_stream_destroy(void* stream);
sk_status sk_stream_cu_count(void* stream, int32_t* count);

/* Number of compiled kernels, and the shape of kernel `index` (host-only). */
int32_t sk_num_variants(void);
sk_status sk_variant_info(int32_t index, int32_t* dtype, int32_t* tile_m, int32_t* tile_n, int32_t* tile_k,
                          int32_t* threads, int32_t* lds_bytes);
/* How kernel `index` covers K (host-only; either pointer may be NULL).  *k_slices
 * > 1: each MAC iteration of tile_k elements is split into that many k-slices,
 * each multiplied by its own group of waves into accumulators of their own,
 * which are added once per tile (skinny problems: a 16 x 32 tile still keeps
 * four waves' loads in flight).  *direct_only = 1: the kernel reads MX scales
 * only straight from the caller's arrays, so it runs only where K is a
 * multiple of tile_k, both scale arrays are 16-byte aligned and
 * SK_DEBUG_RELAYOUT is not set; elsewhere the automatic choice passes it
 * over, and choosing it by index (sk_gemm_args.variant) gives
 * SK_ERR_UNSUPPORTED.  SK_ERR_ARG for an index out of range. */
sk_status sk_variant_k_split(int32_t index, int32_t* k_slices, int32_t* direct_only);

const char* sk_status_string(sk_status s);

#ifdef __cplusplus
}
#endif

#endif /* SK_GEMM_H */
