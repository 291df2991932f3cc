/*
 * bsfp8 -- block-scaled fp8 weight GEMM for small row counts on AMD MI355X (gfx950).
 *
 * The operation (page "recipes/docker-images/mia-tp4/adapter/wo_a_w8.py", module docstring and
 * kernels _wo_a_partial_w8 / _wo_a_mid_kernel): a weight is stored as e4m3 ("float8_e4m3fn")
 * codes q[g][n][k] plus one exponent byte b per 32x32 block; the weight value is
 * bf16(e4m3(q) * 2^(b-127)), rebuilt exactly in registers. For bf16 activations X the library
 * computes, per group g,
 *
 *     Y[m][g][n] = sum_k X[m][g*K + k] * W[g][n][k]
 *
 * with fp32 accumulation and a fixed summation order, and stores Y as bf16 (RNE) or fp32.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless stated "host". bf16 values are passed as their 16-bit
 *     patterns (uint16_t). The caller owns every buffer; the library allocates nothing in the
 *     per-call functions and keeps no state between calls, apart from the static scratch array
 *     of bsfp8_gemm_no_alloc (and its address, looked up once per device).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Per-call functions
 *     only enqueue work: they never synchronise or allocate, so they can be captured in a HIP
 *     graph. The "prepare" functions are synchronous: they enqueue, wait for the stream and
 *     return a verdict.
 *   - Every shape, stride, alignment or scale-layout mismatch is reported as a negative status
 *     before anything is enqueued; nothing is silently degraded (page
 *     "recipes/docker-images/mia-tp4/adapter/shared_pad_k.py", module docstring, last paragraph).
 *   - Sizes are int64_t; an empty problem (M == 0) is a valid no-op.
 */
#ifndef BSFP8_H
#define BSFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSFP8_ABI_VERSION 1

/* Symbols of the shared library; everything else in it is hidden. */
#if defined(__GNUC__) || defined(__clang__)
#define BSFP8_API __attribute__((visibility("default")))
#else
#define BSFP8_API
#endif

typedef enum bsfp8_status {
  BSFP8_OK = 0,
  BSFP8_NOT_EXACT = 1,      /* make_twin verdict: the twin does not rebuild the weight (not an error) */
  BSFP8_EINVAL = -1,        /* null pointer where one is required, bad enum value, or an output
                               buffer overlapping an input, the workspace or another output */
  BSFP8_ESHAPE = -2,        /* sizes out of range or not multiples of the 32x32 block */
  BSFP8_ESCALE = -3,        /* a block scale is not a positive finite power of two */
  BSFP8_ESTRIDE = -4,       /* leading dimension too small or misaligned, pointer not 16-byte aligned */
  BSFP8_EWORKSPACE = -5,    /* workspace missing or smaller than bsfp8_workspace_bytes() */
  BSFP8_EHIP = -6           /* a HIP runtime call failed */
} bsfp8_status;

typedef enum bsfp8_out {
  BSFP8_OUT_BF16 = 0,       /* y is uint16_t bf16 patterns, round-half-to-even from fp32 */
  BSFP8_OUT_F32 = 1         /* y is float (the LM-head logits of page
                               "recipes/docker-images/mia-tp4/docs/tp4-adapters.md", row draft_head_fp8) */
} bsfp8_out;

/* Human-readable name of a status code (static string, never NULL). */
BSFP8_API const char* bsfp8_strerror(int status);

/* BSFP8_ABI_VERSION of the built library. */
BSFP8_API int bsfp8_abi_version(void);

/* ------------------------------------------------------------------------------------------
 * Prepare (load time; synchronous)
 * ------------------------------------------------------------------------------------------ */

/* fp32 block scales -> exponent bytes.
 * Page "shared_pad_k.py", function _pad_weight: a block-fp8 weight [N,K] carries fp32 scales
 * [N/32, K/32] that must be positive powers of two (zero fraction bits and > 0).
 *   scales   : float [rows][cols], row-major, contiguous (device).
 *   exp_out  : uint8_t [rows][cols] (device); byte = fp32 exponent field (2^(b-127) == scale).
 *   n_bad_out: host, nullable; receives the number of refused scales.
 * Refused: fraction bits set, zero, negative, subnormal, +inf, NaN. Returns BSFP8_ESCALE if any
 * scale is refused (exp_out then holds 0 at those positions), BSFP8_ESHAPE if rows or cols < 0. */
BSFP8_API int bsfp8_scales_from_f32(const float* scales, int64_t rows, int64_t cols, uint8_t* exp_out,
                          int64_t* n_bad_out, void* stream);

/* bf16 weight -> e4m3 twin, accepted only when it rebuilds the weight bit for bit.
 * Page "wo_a_w8.py", function make_twin. Per 32x32 block: amax = max|w|; the block exponent e is
 * the least integer with max(amax, 2^-126) <= 448 * 2^e, clamped to [-127, 127]; q = e4m3 RNE of
 * w * 2^-e; the block is exact when bf16(e4m3(q) * 2^e) equals w in every bit.
 *   w        : uint16_t bf16 [G][R][D] (device), R and D multiples of 32.
 *   q_out    : uint8_t [G][R][D] (device).
 *   e_out    : uint8_t [G][R/32][D/32] (device), byte = e + 127.
 *   block_ok : uint8_t [G][R/32][D/32] (device, nullable): 1 exact, 0 not.
 *   n_bad_out: host, nullable: number of blocks that are not exact.
 * A block holding inf or NaN is never exact; it gets exponent byte 255 and codes 0x7F (e4m3 NaN).
 * Returns BSFP8_OK when every block is exact, BSFP8_NOT_EXACT otherwise (the page then keeps the
 * bf16 weight); outputs are written in both cases. */
BSFP8_API int bsfp8_make_twin(const uint16_t* w, int64_t G, int64_t R, int64_t D, uint8_t* q_out,
                    uint8_t* e_out, uint8_t* block_ok, int64_t* n_bad_out, void* stream);

/* bsfp8_make_twin without the synchronisation, for loading many layers: the encoder is enqueued
 * on `stream` and the call returns at once; the verdict stays on the device. Same rule, outputs
 * and page as bsfp8_make_twin.
 *   n_bad_dev: device int64_t, 8-byte aligned: the number of blocks that are not exact is ADDED to
 *              it (the caller zeroes it first; one counter may gather several layers). The twin
 *              is exact iff the count it received is 0.
 * Allocates nothing and does not wait, so it may be captured in a graph (zero the counter with a
 * kernel, not a memset node, before each replay that should count from zero). Returns BSFP8_OK once
 * enqueued, BSFP8_ESHAPE / ESTRIDE / EINVAL as bsfp8_make_twin (EINVAL also for a missing or
 * misaligned n_bad_dev, or one that overlaps w or an output), BSFP8_EHIP on a launch failure. */
BSFP8_API int bsfp8_make_twin_async(const uint16_t* w, int64_t G, int64_t R, int64_t D, uint8_t* q_out,
                                    uint8_t* e_out, uint8_t* block_ok, int64_t* n_bad_dev, void* stream);

/* bf16 weight -> e4m3 twin with one exponent per row and 32 columns, accepted only when it rebuilds
 * the weight bit for bit. Page "recipes/docker-images/mia-tp4/docs/tp4-adapters.md", row
 * draft_main_proj: each rank keeps its output columns as e4m3 with per-(row, 32-column)
 * power-of-two scales, checked to reproduce the weight exactly. The per-block rule is the one of
 * bsfp8_make_twin, applied to 1x32 blocks.
 *   w        : uint16_t bf16 [G][N][K] (device, 16-byte aligned), K a multiple of 32.
 *   q_out    : uint8_t [G][N][K] (device, 16-byte aligned).
 *   e_out    : uint8_t [G][N][K/32] (device), byte = e + 127 (255 for a block holding inf or NaN).
 *   block_ok : uint8_t [G][N][K/32] (device, nullable): 1 exact, 0 not.
 *   n_bad_out: host, nullable: number of blocks that are not exact.
 * Returns BSFP8_OK when every block is exact, BSFP8_NOT_EXACT otherwise; outputs are written in
 * both cases. */
BSFP8_API int bsfp8_make_twin_row32(const uint16_t* w, int64_t G, int64_t N, int64_t K, uint8_t* q_out,
                                    uint8_t* e_out, uint8_t* block_ok, int64_t* n_bad_out, void* stream);

/* Pad the contraction dimension of a twin: codes [G][N][K] -> [G][N][K_pad] with zero codes,
 * exponents [G][N/32][K/32] -> [G][N/32][K_pad/32] with byte 127 (factor 1.0).
 * Page "shared_pad_k.py", module docstring (WHAT THE PATCH DOES, item 1) and _pad_weight: the
 * weight is padded with zeros and its scales with ones. K, K_pad multiples of 32, K_pad >= K.
 * Asynchronous (no verdict). */
BSFP8_API int bsfp8_pad_k_weight(const uint8_t* q, const uint8_t* e, int64_t G, int64_t N, int64_t K,
                       int64_t K_pad, uint8_t* q_pad, uint8_t* e_pad, void* stream);

/* Standalone dequantisation of a twin to bf16 (page "wo_a_w8.py", _dequant_kernel and
 * dequant_into_scratch): w_out[g][n][k] = bf16(e4m3(q) * 2^(b-127)), exact.
 *   q: [G][N][K], e: [G][N/32][K/32], w_out: uint16_t [G][N][K] (all device, caller-owned);
 *   N and K multiples of 32, K <= 2^24; q and w_out 16-byte aligned. Asynchronous.
 * Returns BSFP8_ESHAPE (N or K not a multiple of 32, negative sizes, K > 2^24), BSFP8_EINVAL
 * (a missing pointer, w_out overlapping q or e), BSFP8_ESTRIDE (misaligned q or w_out), BSFP8_EHIP
 * on a launch failure; nothing to do (a zero size) is BSFP8_OK. */
BSFP8_API int bsfp8_dequant(const uint8_t* q, const uint8_t* e, int64_t G, int64_t N, int64_t K,
                  uint16_t* w_out, void* stream);

/* ------------------------------------------------------------------------------------------
 * Per call (asynchronous, graph-capturable, no allocation, no synchronisation)
 * ------------------------------------------------------------------------------------------ */

/* Pad activations: x [M][ldx] with group g at columns [g*K, (g+1)*K) -> x_pad [M][G*K_pad]
 * (contiguous), group g at [g*K_pad, g*K_pad + K) and zeros in [g*K_pad + K, (g+1)*K_pad).
 * Page "shared_pad_k.py", _pad_input (its tail stays zero). ldx >= G*K. */
BSFP8_API int bsfp8_pad_k_input(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t K,
                      int64_t K_pad, uint16_t* x_pad, void* stream);

/* Workspace bytes the GEMM entry points need for this shape (0 when no split of K across
 * workgroups is used). split_k as in the GEMM calls (0 = built-in table). The workspace holds,
 * for the one-pass kernels, one 64-bit exchange slot per output (rows rounded up to 16) and node
 * of the pairwise-combine tree over the splits, and for the tile kernel the fp32 partials
 * [splits][M][G][N] its reduce kernel sums. It must be ZERO-FILLED once after allocation; every
 * call leaves the exchange slots at zero again (the second partner of each node clears its slot).
 * One workspace must not be used by two calls that can run at the same time (e.g. on two
 * streams). */
BSFP8_API size_t bsfp8_workspace_bytes(int64_t M, int64_t G, int64_t N, int64_t K, int split_k);

/* The GEMM. Page "wo_a_w8.py": _wo_a_partial_w8 (2..8 rows) and _wo_a_mid_kernel (9..192 rows).
 *   x       : uint16_t bf16 [M][ldx] (device, 16-byte aligned), group g at columns [g*K,(g+1)*K);
 *             ldx >= G*K and ldx % 8 == 0.
 *   q, e    : twin codes [G][N][K] and exponent bytes [G][N/32][K/32] (device; q 16-byte, e 4-byte aligned);
 *             N and K multiples of 32. Exponent byte 255 and e4m3 NaN codes give NaN outputs.
 *             The kernels read e in aligned 4-byte words: when its size is not a multiple of 4,
 *             up to 3 bytes past its end are read (within the same word, hence the same page);
 *             they never reach a result.
 *   split_k : number of workgroups that share one output tile's K range (fixed-order reduction);
 *             0 = the built-in table for this shape; otherwise 1..64.
 *   ws      : workspace of ws_bytes >= bsfp8_workspace_bytes(M,G,N,K,split_k) (may be NULL when
 *             that is 0).
 *   y       : [M][G][N] contiguous, bf16 (uint16_t) or float per out_dtype (device, 16-byte
 *             aligned); must not overlap x, q, e or ws (BSFP8_EINVAL).
 * Summation order: each output is an fp32 sum over 128-wide K chunks in a fixed order that
 * depends only on (M, G, N, split_k) and on K rounded up to a multiple of 128, so results are
 * bitwise reproducible run to run, and K zero-padded within the same multiple of 128 (e.g.
 * 576 -> 640) gives bitwise the same Y (page "shared_pad_k.py", LOSSLESS).
 * bsfp8_gemm_small takes 1 <= M <= 16, bsfp8_gemm_mid 1 <= M <= 256; bsfp8_gemm picks small for
 * M <= 8 and mid above (page "wo_a_w8.py", module docstring: 2..8 rows vs 9..192 rows). */
BSFP8_API int bsfp8_gemm_small(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
                     const uint8_t* q, const uint8_t* e, int split_k, void* ws, size_t ws_bytes,
                     void* y, int out_dtype, void* stream);
BSFP8_API int bsfp8_gemm_mid(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
                   const uint8_t* q, const uint8_t* e, int split_k, void* ws, size_t ws_bytes,
                   void* y, int out_dtype, void* stream);
BSFP8_API int bsfp8_gemm(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
               const uint8_t* q, const uint8_t* e, int split_k, void* ws, size_t ws_bytes,
               void* y, int out_dtype, void* stream);

/* bsfp8_gemm without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Arguments,
 * plans, kernels, summation order and results are those of bsfp8_gemm with the same split_k
 * (bitwise the same Y). A plan that needs a workspace uses a fixed array in the library's own
 * device memory instead: BSFP8_NO_ALLOC_SCRATCH_BYTES bytes, of which each GPU the library runs
 * on holds its own copy until the process ends. The call allocates nothing; it enqueues a small zero-fill
 * kernel before a plan whose exchange slots must start at zero. Errors as bsfp8_gemm, plus
 * BSFP8_EWORKSPACE (nothing enqueued) when the plan's workspace (bsfp8_workspace_bytes) exceeds
 * BSFP8_NO_ALLOC_SCRATCH_BYTES, and BSFP8_EHIP when the array's address cannot be looked up.
 * Every call on one GPU shares that GPU's array: calls that can overlap on one GPU (two streams,
 * two threads) race and must not be made; calls ordered on one stream are safe. */
#define BSFP8_NO_ALLOC_SCRATCH_BYTES (16u << 20)
BSFP8_API int bsfp8_gemm_no_alloc(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
                                  const uint8_t* q, const uint8_t* e, int split_k, void* y, int out_dtype,
                                  void* stream);

/* The GEMM on a twin with one exponent per row and 32 columns (bsfp8_make_twin_row32): the GEMV
 * of page "recipes/docker-images/mia-tp4/docs/tp4-adapters.md", row draft_main_proj, for up to
 * 16 rows. W[g][n][k] = bf16(e4m3(q[g][n][k]) * 2^(e[g][n][k/32] - 127)); otherwise arguments,
 * layouts, summation order and errors as bsfp8_gemm, with 1 <= M <= 16 (0 is a no-op) and
 * K % 128 == 0. The workspace (exchange slots when K is split over workgroups) is sized by
 * bsfp8_workspace_bytes_row32 and must be zero-filled once after allocation. */
BSFP8_API size_t bsfp8_workspace_bytes_row32(int64_t M, int64_t G, int64_t N, int64_t K, int split_k);
BSFP8_API int bsfp8_gemm_row32(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
                               const uint8_t* q, const uint8_t* e, int split_k, void* ws, size_t ws_bytes,
                               void* y, int out_dtype, void* stream);

/* ------------------------------------------------------------------------------------------
 * MXFP8 activations and the fp8 x fp8 GEMM (W8A8; per call, asynchronous, no allocation)
 *
 * Page "recipes/docker-images/mia-tp4/adapter/shared_pad_k.py" (module docstring, DIAGNOSIS and
 * LOSSLESS): the pages' MXFP8 linear quantizes its bf16 input itself into e4m3 values with one
 * power-of-two (E8M0) scale per 32 consecutive values of a row and multiplies that with the
 * block-fp8 weight. The pages do not print the quantizer; the rule here is OCP Microscaling (MX)
 * v1.0 for MXFP8: per 32-value block, s = floor(log2(max |v|)) - 8 clamped to [-127, 127]
 * (an all-zero block gets -127), each element e4m3(v * 2^-s) rounded to nearest even and
 * saturated at +-448; a block holding inf or NaN gets scale byte 255 and e4m3 NaN codes
 * (0x7F, or 0xFF for a negative sign). Unlike the bf16 path this is lossy: it is the pages'
 * comparison path, not the exact twin GEMM.
 * ------------------------------------------------------------------------------------------ */

/* bf16 activations -> MXFP8 codes and scale bytes.
 *   x  : uint16_t bf16 [M][ldx] (device, 16-byte aligned), ldx >= L, ldx % 8 == 0.
 *   xq : uint8_t e4m3 codes [M][L] (device, contiguous, 16-byte aligned).
 *   xs : uint8_t scale bytes [M][L/32] (device, contiguous), byte = s + 127 (2^(byte-127)).
 * L % 32 == 0. Deterministic and exact (every decision is an integer one). */
BSFP8_API int bsfp8_quantize_mx(const uint16_t* x, int64_t ldx, int64_t M, int64_t L, uint8_t* xq,
                                uint8_t* xs, void* stream);

/* Y[m][g][n] = sum_k Xmx[m][g*K + k] * W[g][n][k], with Xmx = e4m3(xq) * 2^(xs - 127) per
 * 32-value row block and W = e4m3(q) * 2^(e - 127) per 32x32 weight block (the weight's block
 * exponent serves as the MX scale of each row's 32-value piece).
 *   xq, xs : codes [M][ldq] (16-byte aligned) and scale bytes [M][ldq/32] (4-byte aligned), group g
 *            at columns [g*K, (g+1)*K) (e.g. the output of bsfp8_quantize_mx with L = G*K);
 *            ldq >= G*K and ldq % 128 == 0.
 *   q, e   : the weight twin as for bsfp8_gemm (q 16-byte aligned, e 4-byte aligned).
 *   y      : [M][G][N] bf16 (RNE) or fp32 per out_dtype (16-byte aligned).
 * 1 <= M <= 256 (M == 0 is a no-op), N % 32 == 0, K % 128 == 0 and K <= 8192. The products run
 * on the block-scaled fp8 MFMA with fp32 accumulation across 128-wide chunks; the hardware sums
 * each group of eight adjacent products inside the instruction with a precision of about 2^-14
 * of the group's largest product (measured), so results are not those of an exact sum rounded
 * once. The summation order is fixed by the built-in configuration: bitwise reproducible. */
BSFP8_API int bsfp8_gemm_mx(const uint8_t* xq, const uint8_t* xs, int64_t ldq, int64_t M, int64_t G,
                            int64_t N, int64_t K, const uint8_t* q, const uint8_t* e, void* y,
                            int out_dtype, void* stream);

/* ------------------------------------------------------------------------------------------
 * MXFP8 output epilogue (per call, asynchronous, no allocation)
 *
 * Page "recipes/docker-images/mia-tp4/adapter/wo_a_w8.py": its module docstring reports the
 * MXFP8-epilogue path (what production runs), and in `install` the dropped-weight path and
 * small_mx hand the fp32 split partials [S][M][G][N] of _partial_w8 to a kernel that sums them
 * and quantises the sum to MXFP8 in one pass, where the plain path sums them with _wo_a_reduce and
 * rounds to bf16. Neither the quantiser nor the order of that sum is printed. Here:
 *   - the partials are added in fp32 in a fixed order (bsfp8_sum_order);
 *   - the sum, viewed as [M][L] (L = G*N for the GEMM), is quantised per 32 consecutive values of
 *     a row with the rule of bsfp8_quantize_mx (OCP MX v1.0: s = floor(log2 amax) - 8 clamped to
 *     [-127, 127], e4m3 RNE with saturation at 448, scale byte s + 127; byte 255 and e4m3 NaN
 *     codes for a block holding inf or NaN);
 *   - codes are [M][L] and scale bytes [M][L/32], both row-major (the pages' consumer wants its
 *     scales in a swizzled layout of its own, which is not reproduced).
 * ------------------------------------------------------------------------------------------ */

typedef enum bsfp8_sum_order {
  BSFP8_SUM_ASCENDING = 0,  /* ((p0 + p1) + p2) + ... : the order of the page's _wo_a_reduce */
  BSFP8_SUM_PAIRWISE = 1    /* pairwise tree over the split index: p2i + p2i+1, an unpaired last
                               partial carried up unchanged, repeated until one value is left */
} bsfp8_sum_order;

/* Fixed-order sum of S fp32 partials and MXFP8 quantisation of the sum.
 *   part  : float [S][M][L] (device, contiguous, 16-byte aligned).
 *   S     : 1..64 partials (S = 1 quantises part itself).
 *   order : a bsfp8_sum_order.
 *   yq    : uint8_t e4m3 codes [M][L] (device, contiguous, 16-byte aligned).
 *   ys    : uint8_t scale bytes [M][L/32] (device, contiguous).
 * L % 32 == 0 and L >= 32; M == 0 is a no-op. Every addition is an IEEE fp32 addition and every
 * quantisation decision an integer one, so the result is bit-exact and deterministic. */
BSFP8_API int bsfp8_reduce_quantize_mx(const float* part, int64_t S, int64_t M, int64_t L, int order,
                                       uint8_t* yq, uint8_t* ys, void* stream);

/* Workspace bytes of bsfp8_gemm_mxfp8 for this shape and split_k (never 0 for a valid shape:
 * the fp32 results, one copy per split, may pass through it). Nothing in it needs clearing; one
 * workspace must not be used by two calls that can run at the same time. */
BSFP8_API size_t bsfp8_workspace_bytes_mxfp8(int64_t M, int64_t G, int64_t N, int64_t K, int split_k);

/* The GEMM of bsfp8_gemm with the MXFP8 epilogue: the fp32 results of the plan that
 * bsfp8_plan_info(..., path 3) reports for (M, G, N, K, split_k) - the sum itself with one split,
 * else each split's partial - go to ws, and the epilogue adds the partials in the order of that
 * plan's own combine (pairwise for the one-pass kernels, ascending for the tile kernel), so the
 * quantised values are exactly the fp32 outputs of bsfp8_gemm_config with that configuration and
 * chunks per split (out_dtype = BSFP8_OUT_F32). That is bsfp8_gemm's own plan, except on the
 * decode shapes where bsfp8_gemm takes the paired kernel: its 8-row tiles hold a quarter of an MX
 * block, so this call keeps the 16-row decode plan, whose fused form quantises whole blocks.
 *   x, ldx, M, G, N, K, q, e, split_k : as bsfp8_gemm (1 <= M <= 256).
 *   ws    : >= bsfp8_workspace_bytes_mxfp8(M, G, N, K, split_k) bytes (device, 16-byte aligned).
 *   yq    : uint8_t e4m3 codes [M][G*N] (device, contiguous, 16-byte aligned).
 *   ys    : uint8_t scale bytes [M][G*N/32] (device, contiguous).
 * For a decode plan with one split (up to 16 rows, K a multiple of 128, at most 32 chunks) one
 * fused kernel computes and quantises 32 output columns per workgroup; otherwise two kernels run
 * on `stream`, the GEMM (writing the fp32 results into ws) and the epilogue. Both forms give the
 * same bits. */
BSFP8_API int bsfp8_gemm_mxfp8(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
                               const uint8_t* q, const uint8_t* e, int split_k, void* ws, size_t ws_bytes,
                               uint8_t* yq, uint8_t* ys, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSFP8_H */
