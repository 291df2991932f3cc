// Internal declarations shared by the bsfp8 HIP sources (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bsfp8.h"

namespace bsfp8 {

// One output tile of a workgroup is BM x NB (rows of X x rows of W); K is walked in 128-wide
// chunks. See gemm.hip for the meaning of each field.
struct GemmShape {
  int64_t ldx;
  int M, G, N, K;
};

struct GemmPlan {
  int cfg;          // index into the kernel configuration table
  int BM, NB;       // workgroup tile
  int kchunks;      // ceil(K / 128)
  int cps;          // chunks per split
  int splits;       // workgroups sharing one tile's K range
  int mblocks;      // ceil(M / BM)
  int nblocks;      // N / NB (per group)
  size_t ws_bytes;  // workspace needed (0 when splits == 1)
};

enum Path { PATH_SMALL = 0, PATH_MID = 1 };

// Picks the kernel configuration and split for a shape; returns a bsfp8_status. allow_pair = false
// leaves out the paired decode kernel (the MXFP8-epilogue GEMM quantises whole 32-row blocks).
int plan_gemm(const GemmShape& s, int path, int split_k, GemmPlan* plan, bool allow_pair = true);
// Plan for an explicit configuration index and chunks per split.
int plan_with(const GemmShape& s, int cfg, int cps, GemmPlan* plan);
// Plan of the MXFP8-epilogue GEMM (bsfp8_gemm_mxfp8).
int plan_gemm_mxfp8(const GemmShape& s, int split_k, GemmPlan* plan);
// Plan for weights with one exponent per row and 32 columns (M <= 16, K % 128 == 0).
int plan_gemm_row32(const GemmShape& s, int split_k, GemmPlan* plan);
// 1 when configuration `cfg` reads exponents per row and 32 columns.
int gemm_config_row_scales(int cfg);
int num_gemm_configs();
// BM, NB, threads, chunks per wave per pass of a configuration.
int gemm_config_info(int cfg, int* out);
// partials != 0: leave fp32 results in ws for a later kernel instead of writing y: the result
// itself when the plan has one split, else the partial of every split ([splits][M][G][N]), in
// the order gemm_partials_order names.
// yq, ys non-null: the kernel quantises its fp32 results to MXFP8 itself (codes [M][G*N], scale
// bytes [M][G*N/32]) instead of writing y; only for one split and a configuration whose tile
// holds whole 32-column blocks (else BSFP8_EINVAL, before anything is launched).
int launch_gemm(const GemmShape& s, const GemmPlan& p, const uint16_t* x, const uint8_t* q,
                const uint8_t* e, void* ws, void* y, int out_f32, hipStream_t stream, int partials = 0,
                uint8_t* yq = nullptr, uint8_t* ys = nullptr);
// Order in which a plan's own combine adds its split partials: BSFP8_SUM_ASCENDING (tile kernel
// and its reduce kernel) or BSFP8_SUM_PAIRWISE (the one-pass kernels' exchange tree).
int gemm_partials_order(const GemmPlan& p);
// 1 when the plan's workspace must hold zeros before the launch (the one-pass kernels' exchange
// slots; the tile kernel's partials are written whole).
int gemm_ws_needs_zero(const GemmPlan& p);
// Workspace of launch_gemm with partials: splits * M * G * N fp32 values.
size_t gemm_partials_bytes(const GemmShape& s, const GemmPlan& p);

// The MXFP8 epilogue (epilogue.hip): fixed-order sum of S fp32 partials [S][M][L], then MXFP8
// quantisation along L (codes [M][L], scale bytes [M][L/32]).
int launch_reduce_quantize_mx(const float* part, int S, int64_t M, int64_t L, int order, uint8_t* yq,
                              uint8_t* ys, hipStream_t stream);
// The fused form (decode plans with one split): GEMM and epilogue in one kernel. Returns
// BSFP8_EINVAL when the plan is not a 16-row decode plan with one split.
int launch_decode_mxfp8(const GemmShape& s, const GemmPlan& p, const uint16_t* x, const uint8_t* q,
                        const uint8_t* e, uint8_t* yq, uint8_t* ys, hipStream_t stream);

int launch_scales_from_f32(const float* s, int64_t n, uint8_t* out, unsigned long long* bad,
                           hipStream_t stream);
int launch_make_twin(const uint16_t* w, int64_t G, int64_t R, int64_t D, uint8_t* q, uint8_t* e,
                     uint8_t* ok, unsigned long long* bad, hipStream_t stream);
int launch_make_twin_row32(const uint16_t* w, int64_t G, int64_t N, int64_t K, uint8_t* q, uint8_t* e,
                           uint8_t* ok, unsigned long long* bad, hipStream_t stream);
int launch_pad_k_weight(const uint8_t* q, const uint8_t* e, int64_t G, int64_t N, int64_t K,
                        int64_t K_pad, uint8_t* q_pad, uint8_t* e_pad, hipStream_t stream);
int launch_pad_k_input(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t K,
                       int64_t K_pad, uint16_t* x_pad, hipStream_t stream);
int launch_dequant(const uint8_t* q, const uint8_t* e, int64_t G, int64_t N, int64_t K,
                   uint16_t* w, hipStream_t stream);

// MXFP8 activations and the fp8 x fp8 GEMM (mx.hip)
int launch_quantize_mx(const uint16_t* x, int64_t ldx, int64_t M, int64_t L, uint8_t* xq, uint8_t* xs,
                       hipStream_t stream);
int launch_gemm_mx(const uint8_t* xq, const uint8_t* xs, int64_t ldq, int M, int G, int N, int K,
                   const uint8_t* q, const uint8_t* e, void* y, int out_f32, int cfg, hipStream_t stream);
int num_mx_configs();
int mx_config_info(int cfg, int* out);
int mx_pick(int M, int G, int N);

// Plain-read floor of a weight stream (measure.hip): reads `bytes` once with the GEMM's load shape,
// then, with out_bytes > 0, writes that many bytes to out.
int launch_read_floor(const void* p, size_t bytes, int nwg, const void* slab, size_t slab_bytes, int slab_groups,
                      int interleave, uint32_t* sink, void* out, size_t out_bytes, hipStream_t stream);

// Static scratch of bsfp8_gemm_no_alloc (scratch.hip): the array's address on the device of
// `stream` (the current device for a null stream), looked up once per device.
int scratch_for_stream(hipStream_t stream, void** out);
// Zero-fills `bytes` (a multiple of 16) at p with a kernel on `stream`.
int launch_clear(void* p, size_t bytes, hipStream_t stream);

inline int hip_status(hipError_t err) { return err == hipSuccess ? BSFP8_OK : BSFP8_EHIP; }

}  // namespace bsfp8
