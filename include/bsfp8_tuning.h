/*
 * bsfp8 tuning interface: run the GEMM with an explicit kernel configuration, and describe the
 * plan the built-in table picks. For sweeps and reports; applications use bsfp8.h.
 *
 * The GEMM computed is the one of bsfp8_gemm (page "recipes/docker-images/mia-tp4/adapter/
 * wo_a_w8.py", kernels _wo_a_partial_w8 and _wo_a_mid_kernel, whose launch parameters are
 * likewise a row-count table of tile sizes and splits).
 */
#ifndef BSFP8_TUNING_H
#define BSFP8_TUNING_H

#include "bsfp8.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Number of compiled kernel configurations (valid `cfg` values are 0 .. n-1). */
BSFP8_API int bsfp8_num_configs(void);

/* Tile of configuration `cfg`: out[0] = rows of X per workgroup (BM), out[1] = weight rows per
 * workgroup (NB), out[2] = threads per workgroup, out[3] = 128-wide K chunks per wave per pass,
 * out[4] = waves along the weight rows, out[5] = waves along K (each output's fp32 sum is the
 * ascending chain of the chunks one wave owns, so two plans with the same waves along K and the
 * same chunks per split give bitwise the same outputs), out[6] = kernel kind: 0 = staged
 * (multi-pass, X in LDS), 1 = one-pass with the X rows in LDS (at most 16 rows of X per
 * workgroup), 2 = one-pass with both operands in registers, 3 = tile kernel (X shared through
 * LDS; out[3] = chunks in flight; with more than one split each workgroup writes an fp32 partial
 * tile and a second kernel adds the partials in ascending split order), 4 = one-pass decode
 * kernel (X, exponents and weights streamed into LDS; out[0] rows of X per workgroup), 5 = slab
 * kernel (X shared through an LDS ring of 512-wide K slabs; out[3] = ring stages; splits begin
 * on slab boundaries). For kinds
 * 1, 2 and 4 the chunks per split must be at most out[3] * out[5]; for kind 3 at most 64. Kinds 3
 * and 5 take K in whole 128-wide chunks (K % 128 == 0), and so do the kind-4 configurations
 * except those built for a ragged last chunk (a call with K % 128 != 0 is refused with
 * BSFP8_EINVAL by the others).
 * out[7] bit 0 = 1 when the configuration reads one exponent per weight row and 32 columns (it
 * then runs only through bsfp8_gemm_row32_config); out[7] >> 8 = the XCDs per group of an
 * XCD-grouped tile map (0: none; such a configuration takes only G = 8 / that value and a number
 * of n-blocks it divides, else BSFP8_EINVAL). Returns BSFP8_EINVAL for an unknown cfg. `out` is
 * host memory of 8 ints. */
BSFP8_API int bsfp8_config_info(int cfg, int* out);

/* Plan the built-in table picks. path: 0 = small, 1 = mid, 2 = what bsfp8_gemm picks, 3 = what
 * bsfp8_gemm_mxfp8 picks.
 * out (host, 8 ints): cfg, BM, NB, kchunks, chunks per split, splits, m-blocks, workgroups.
 * Returns a status as the GEMM calls would for this shape. */
BSFP8_API int bsfp8_plan_info(int64_t M, int64_t G, int64_t N, int64_t K, int split_k, int path, int* out);

/* Workspace bytes for an explicit configuration and chunks per split (cps >= 1). */
BSFP8_API size_t bsfp8_workspace_bytes_config(int64_t M, int64_t G, int64_t N, int64_t K, int cfg, int cps);

/* The GEMM with an explicit configuration `cfg` and `cps` 128-wide K chunks per split (the
 * number of splits is ceil(ceil(K/128) / cps)). Arguments and errors otherwise as bsfp8_gemm;
 * 1 <= M <= 256. N must be a multiple of the configuration's NB (else BSFP8_ESHAPE).
 * Row-scale configurations (out[7] of bsfp8_config_info) give BSFP8_EINVAL. */
BSFP8_API int bsfp8_gemm_config(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
                      const uint8_t* q, const uint8_t* e, int cfg, int cps, void* ws,
                      size_t ws_bytes, void* y, int out_dtype, void* stream);

/* bsfp8_gemm_mxfp8 with an explicit configuration and chunks per split, and its workspace bytes
 * (splits * M * G * N * 4). Arguments and errors otherwise as bsfp8_gemm_mxfp8 and
 * bsfp8_gemm_config; the epilogue adds the partials in the order of the configuration's own
 * combine, so the codes quantise exactly the fp32 output of bsfp8_gemm_config(cfg, cps). */
BSFP8_API size_t bsfp8_workspace_bytes_mxfp8_config(int64_t M, int64_t G, int64_t N, int64_t K, int cfg, int cps);
BSFP8_API int bsfp8_gemm_mxfp8_config(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N,
                                      int64_t K, const uint8_t* q, const uint8_t* e, int cfg, int cps,
                                      void* ws, size_t ws_bytes, uint8_t* yq, uint8_t* ys, void* stream);

/* The same for a row-scale configuration, on a twin with one exponent per row and 32 columns
 * (e [G][N][K/32], as bsfp8_gemm_row32); other configurations give BSFP8_EINVAL. */
BSFP8_API int bsfp8_gemm_row32_config(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N,
                                      int64_t K, const uint8_t* q, const uint8_t* e, int cfg, int cps, void* ws,
                                      size_t ws_bytes, void* y, int out_dtype, void* stream);

/* fp8 x fp8 GEMM (bsfp8_gemm_mx) configurations. out (host, 6 ints) of bsfp8_mx_config_info:
 * rows of X per workgroup, weight rows per workgroup, threads, chunks per ring stage, ring stages,
 * waves along K. bsfp8_mx_plan returns the configuration bsfp8_gemm_mx picks (or a negative
 * status). bsfp8_gemm_mx_config runs an explicit configuration; arguments and errors otherwise as
 * bsfp8_gemm_mx (BSFP8_ESHAPE when N is not a multiple of the configuration's weight rows). */
BSFP8_API int bsfp8_mx_num_configs(void);
BSFP8_API int bsfp8_mx_config_info(int cfg, int* out);
BSFP8_API int bsfp8_mx_plan(int64_t M, int64_t G, int64_t N);
BSFP8_API int bsfp8_gemm_mx_config(const uint8_t* xq, const uint8_t* xs, int64_t ldq, int64_t M, int64_t G,
                                   int64_t N, int64_t K, const uint8_t* q, const uint8_t* e, int cfg,
                                   void* y, int out_dtype, void* stream);

/* Plain-read floor, a measurement aid: one kernel that reads `bytes` of device memory at p once,
 * with the GEMM's load shape (16 bytes per lane, one contiguous kilobyte per wave load,
 * non-temporal, every load of a workgroup's share issued before any is used), on nwg workgroups
 * of 512 threads that each read one contiguous share, and computes nothing else. Timed over the
 * same distinct weight copies and in the same graph replay as a GEMM (the measurement protocol of
 * page "recipes/docker-images/mia-tp4/adapter/shared_pad_k.py", MEASUREMENT: distinct weight
 * copies so that the cache is cold, captured graphs, interleaved rounds), it gives the floor a
 * GEMM that streams those bytes can reach on this machine; bytes = 0 times a bare launch.
 * With slab_bytes > 0 every workgroup also reads the whole slab of its group (workgroup b takes
 * group b * slab_groups / nwg; LDS-mode loads of one kilobyte per wave): the floor of a GEMM
 * whose workgroups also each read the activation rows of their group, as the GEMMs do. The slab
 * is read before the share, or, with flags = BSFP8_FLOOR_SLAB_INTERLEAVED, spread evenly over
 * the steps of the share (each step's slab loads issued just before its share loads, as a GEMM
 * issues each chunk's activations before its weights); flags = 0 otherwise.
 * With out_bytes > 0 each workgroup then also writes its contiguous share of `out` (16 bytes per
 * lane; non-temporal stores for shares of 16 KB and more): the floor of a kernel that reads those
 * bytes and stores that many output bytes.
 *   p    : device memory, 16-byte aligned, at least `bytes` long (may be NULL when bytes = 0);
 *          bytes < 2^31.
 *   slab : device memory, 16-byte aligned, slab_groups x slab_bytes long (NULL when slab_bytes
 *          = 0); slab_bytes a multiple of 16, 1 <= slab_groups <= nwg, the whole below 2^31.
 *   sink : device uint32_t [nwg]; written only when a workgroup's fold of the data equals a fixed
 *          constant (it keeps the loads alive), so its contents are meaningless.
 *   out  : device memory, 16-byte aligned, out_bytes long (NULL when out_bytes = 0); out_bytes a
 *          multiple of 16 below 2^31; receives the workgroups' folds (meaningless contents).
 * Returns BSFP8_EINVAL (nwg outside 1..65536, no sink, out or slab missing, slab_groups out of
 * range, an unknown flag, out or sink overlapping p, the slab or each other), BSFP8_ESTRIDE (misaligned p, slab or
 * out, slab_bytes or out_bytes not a multiple of 16), BSFP8_ESHAPE (bytes, the slab or out_bytes
 * too large), BSFP8_EHIP on a launch failure. */
#define BSFP8_FLOOR_SLAB_INTERLEAVED 1
BSFP8_API int bsfp8_read_floor(const void* p, size_t bytes, int nwg, const void* slab, size_t slab_bytes,
                               int slab_groups, int flags, uint32_t* sink, void* out, size_t out_bytes,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSFP8_TUNING_H */
