// C ABI of the bsfp8 library: argument checks, dispatch and the synchronous prepare calls.
// Everything that computes runs in the HIP kernels of gemm.hip and prep.hip.

#include <stdint.h>

#include <initializer_list>

#include "bsfp8_tuning.h"
#include "internal.h"

using namespace bsfp8;

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// A buffer's byte range, for the check that outputs overlap no input, workspace or other output
// (the kernels read the inputs while other workgroups write the outputs).
struct Range {
  const void* p;
  size_t n;
};
inline bool overlap(Range a, Range b) {
  if (!a.p || !b.p || !a.n || !b.n) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}
inline bool outputs_alias(std::initializer_list<Range> outs, std::initializer_list<Range> others) {
  for (const Range* o = outs.begin(); o != outs.end(); ++o) {
    for (const Range* r = others.begin(); r != others.end(); ++r)
      if (overlap(*o, *r)) return true;
    for (const Range* o2 = o + 1; o2 != outs.end(); ++o2)
      if (overlap(*o, *o2)) return true;
  }
  return false;
}
// Bytes of x [M][ldx] (bf16) that a GEMM reads, of the codes and of the exponent bytes.
inline size_t x_span(const GemmShape& s) { return ((size_t)(s.M - 1) * s.ldx + (size_t)s.G * s.K) * 2; }
inline size_t q_span(const GemmShape& s) { return (size_t)s.G * s.N * s.K; }
inline size_t e_span(const GemmShape& s, bool row_exps) {
  return (size_t)s.G * (row_exps ? s.N : s.N / 32) * (s.K / 32);
}
inline size_t y_span(const GemmShape& s, int out_dtype) {
  return (size_t)s.M * s.G * s.N * (out_dtype == BSFP8_OUT_F32 ? 4 : 2);
}
// y against x, q, e and the workspace (BSFP8_EINVAL on overlap)
inline int check_gemm_alias(const GemmShape& s, const void* x, const void* q, const void* e, bool row_exps,
                            const void* ws, size_t ws_bytes, const void* y, int out_dtype) {
  return outputs_alias({{y, y_span(s, out_dtype)}},
                       {{x, x_span(s)}, {q, q_span(s)}, {e, e_span(s, row_exps)}, {ws, ws_bytes}})
             ? BSFP8_EINVAL
             : BSFP8_OK;
}
// MXFP8 outputs (codes [M][G*N], scale bytes [M][G*N/32]) against the inputs, the workspace and
// each other
inline bool mxfp8_alias(const GemmShape& s, const void* x, const void* q, const void* e, const void* ws,
                        size_t ws_bytes, const void* yq, const void* ys) {
  const size_t L = (size_t)s.G * s.N;
  return outputs_alias({{yq, (size_t)s.M * L}, {ys, (size_t)s.M * L / 32}},
                       {{x, x_span(s)}, {q, q_span(s)}, {e, e_span(s, false)}, {ws, ws_bytes}});
}

// Size checks shared by the GEMM entry points and the plan report; fills `shape`.
int check_dims(int64_t M, int64_t G, int64_t N, int64_t K, int split_k, int64_t max_m,
               GemmShape* shape) {
  if (M < 0 || M > max_m || G < 1 || N < 32 || K < 32) return BSFP8_ESHAPE;
  if (N % 32 || K % 32) return BSFP8_ESHAPE;
  if (G > 4096 || N > (1 << 24) || K > (1 << 24) || G * N > (1 << 26)) return BSFP8_ESHAPE;
  if (split_k < 0 || split_k > 64) return BSFP8_EINVAL;
  shape->ldx = G * K;
  shape->M = (int)M;
  shape->G = (int)G;
  shape->N = (int)N;
  shape->K = (int)K;
  return BSFP8_OK;
}

// Checks shared by the GEMM entry points; fills `shape`.
int check_gemm(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
               const uint8_t* q, const uint8_t* e, void* y, int out_dtype, int split_k,
               int64_t max_m, GemmShape* shape) {
  if (out_dtype != BSFP8_OUT_BF16 && out_dtype != BSFP8_OUT_F32) return BSFP8_EINVAL;
  int st = check_dims(M, G, N, K, split_k, max_m, shape);
  if (st != BSFP8_OK) return st;
  if (M > 0 && (!x || !q || !e || !y)) return BSFP8_EINVAL;
  if (ldx < G * K || ldx % 8) return BSFP8_ESTRIDE;
  // every operand is addressed with 32-bit byte offsets
  if (M > 0 && ((M - 1) * ldx + G * K) * 2 >= ((int64_t)1 << 31)) return BSFP8_ESHAPE;
  if (G * N * K >= ((int64_t)1 << 31)) return BSFP8_ESHAPE;
  // the kernels read exponent bytes as 4-byte words (one word = the four blocks of a chunk)
  if (M > 0 && (!aligned16(x) || !aligned16(q) || !aligned16(y) || (reinterpret_cast<uintptr_t>(e) & 3)))
    return BSFP8_ESTRIDE;
  shape->ldx = ldx;
  return BSFP8_OK;
}

int run_gemm(int path, int64_t max_m, const uint16_t* x, int64_t ldx, int64_t M, int64_t G,
             int64_t N, int64_t K, const uint8_t* q, const uint8_t* e, int split_k, void* ws,
             size_t ws_bytes, void* y, int out_dtype, void* stream) {
  GemmShape s;
  int st = check_gemm(x, ldx, M, G, N, K, q, e, y, out_dtype, split_k, max_m, &s);
  if (st != BSFP8_OK || M == 0) return st;
  GemmPlan p;
  st = plan_gemm(s, path, split_k, &p);
  if (st != BSFP8_OK) return st;
  if (p.ws_bytes > 0 && (!ws || ws_bytes < p.ws_bytes || !aligned16(ws))) return BSFP8_EWORKSPACE;
  st = check_gemm_alias(s, x, q, e, false, ws, ws_bytes, y, out_dtype);
  if (st != BSFP8_OK) return st;
  return launch_gemm(s, p, x, q, e, ws, y, out_dtype == BSFP8_OUT_F32, as_stream(stream));
}

// Device counter for the synchronous prepare calls: allocate, run, read back, free.
struct Counter {
  unsigned long long* dev = nullptr;
  ~Counter() {
    if (dev) (void)hipFree(dev);
  }
  int init(hipStream_t s) {
    if (hipMalloc(reinterpret_cast<void**>(&dev), sizeof(unsigned long long)) != hipSuccess) return BSFP8_EHIP;
    return hip_status(hipMemsetAsync(dev, 0, sizeof(unsigned long long), s));
  }
  int read(hipStream_t s, unsigned long long* out) {
    if (hipMemcpyAsync(out, dev, sizeof(*out), hipMemcpyDeviceToHost, s) != hipSuccess) return BSFP8_EHIP;
    return hip_status(hipStreamSynchronize(s));
  }
};

// Size, alignment and stride checks of the fp8 x fp8 GEMM.
int check_gemm_mx(const uint8_t* xq, const uint8_t* xs, int64_t ldq, int64_t M, int64_t G, int64_t N,
                  int64_t K, const uint8_t* q, const uint8_t* e, void* y, int out_dtype) {
  if (out_dtype != BSFP8_OUT_BF16 && out_dtype != BSFP8_OUT_F32) return BSFP8_EINVAL;
  if (M < 0 || M > 256 || G < 1 || N < 32 || K < 128 || N % 32 || K % 128) return BSFP8_ESHAPE;
  if (K > 8192 || G > 4096 || N > (1 << 24) || G * N > (1 << 26)) return BSFP8_ESHAPE;
  if (M > 0 && (!xq || !xs || !q || !e || !y)) return BSFP8_EINVAL;
  if (ldq < G * K || ldq % 128) return BSFP8_ESTRIDE;
  if (!aligned16(xq) || !aligned16(q) || !aligned16(y) || (reinterpret_cast<uintptr_t>(xs) & 3) ||
      (reinterpret_cast<uintptr_t>(e) & 3))
    return BSFP8_ESTRIDE;
  if (M > 0) {
    const size_t xqb = (size_t)(M - 1) * ldq + (size_t)G * K;
    const size_t xsb = (size_t)(M - 1) * (ldq / 32) + (size_t)G * K / 32;
    const size_t yb = (size_t)M * G * N * (out_dtype == BSFP8_OUT_F32 ? 4 : 2);
    if (outputs_alias({{y, yb}}, {{xq, xqb}, {xs, xsb}, {q, (size_t)G * N * K}, {e, (size_t)G * (N / 32) * (K / 32)}}))
      return BSFP8_EINVAL;
  }
  return BSFP8_OK;
}

// The GEMM with the MXFP8 epilogue, when `fuse`: the fused decode kernel for a decode plan with one
// split, or the plan's own kernel quantising its output where its tile holds whole 32-column
// blocks; otherwise the GEMM into the workspace (fp32 results or split partials) and the
// epilogue kernel.
int run_gemm_mxfp8(const GemmShape& s, const GemmPlan& p, const uint16_t* x, const uint8_t* q,
                   const uint8_t* e, void* ws, size_t ws_bytes, uint8_t* yq, uint8_t* ys, bool fuse,
                   hipStream_t stream) {
  if (!ws || ws_bytes < gemm_partials_bytes(s, p) || !aligned16(ws)) return BSFP8_EWORKSPACE;
  if (mxfp8_alias(s, x, q, e, ws, ws_bytes, yq, ys)) return BSFP8_EINVAL;
  if (fuse) {
    int fst = launch_decode_mxfp8(s, p, x, q, e, yq, ys, stream);
    if (fst != BSFP8_EINVAL) return fst;
    fst = launch_gemm(s, p, x, q, e, nullptr, nullptr, 1, stream, 0, yq, ys);   // in-kernel epilogue
    if (fst != BSFP8_EINVAL) return fst;
  }
  int st = launch_gemm(s, p, x, q, e, ws, nullptr, 1, stream, /*partials=*/1);
  if (st != BSFP8_OK) return st;
  return launch_reduce_quantize_mx(reinterpret_cast<const float*>(ws), p.splits, s.M, (int64_t)s.G * s.N,
                                   gemm_partials_order(p), yq, ys, stream);
}

}  // namespace

extern "C" {

const char* bsfp8_strerror(int status) {
  switch (status) {
    case BSFP8_OK: return "ok";
    case BSFP8_NOT_EXACT: return "twin does not rebuild the weight exactly";
    case BSFP8_EINVAL: return "invalid argument";
    case BSFP8_ESHAPE: return "unsupported shape";
    case BSFP8_ESCALE: return "block scale is not a positive finite power of two";
    case BSFP8_ESTRIDE: return "bad leading dimension or alignment";
    case BSFP8_EWORKSPACE: return "workspace missing or too small";
    case BSFP8_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int bsfp8_abi_version(void) { return BSFP8_ABI_VERSION; }

int bsfp8_scales_from_f32(const float* scales, int64_t rows, int64_t cols, uint8_t* exp_out,
                          int64_t* n_bad_out, void* stream) {
  if (rows < 0 || cols < 0) return BSFP8_ESHAPE;
  const int64_t n = rows * cols;
  if (n_bad_out) *n_bad_out = 0;
  if (n == 0) return BSFP8_OK;
  if (!scales || !exp_out) return BSFP8_EINVAL;
  if (outputs_alias({{exp_out, (size_t)n}}, {{scales, (size_t)n * 4}})) return BSFP8_EINVAL;
  hipStream_t s = as_stream(stream);
  Counter c;
  int st = c.init(s);
  if (st != BSFP8_OK) return st;
  st = launch_scales_from_f32(scales, n, exp_out, c.dev, s);
  if (st != BSFP8_OK) return st;
  unsigned long long bad = 0;
  st = c.read(s, &bad);
  if (st != BSFP8_OK) return st;
  if (n_bad_out) *n_bad_out = (int64_t)bad;
  return bad ? BSFP8_ESCALE : BSFP8_OK;
}

int bsfp8_make_twin(const uint16_t* w, int64_t G, int64_t R, int64_t D, uint8_t* q_out,
                    uint8_t* e_out, uint8_t* block_ok, int64_t* n_bad_out, void* stream) {
  if (G < 0 || R < 0 || D < 0 || R % 32 || D % 32) return BSFP8_ESHAPE;
  if (n_bad_out) *n_bad_out = 0;
  if (G * R * D == 0) return BSFP8_OK;
  if (!w || !q_out || !e_out) return BSFP8_EINVAL;
  if (!aligned16(w) || !aligned16(q_out)) return BSFP8_ESTRIDE;
  {
    const size_t n = (size_t)G * R * D, nb = n / 1024;
    if (outputs_alias({{q_out, n}, {e_out, nb}, {block_ok, nb}}, {{w, n * 2}})) return BSFP8_EINVAL;
  }
  hipStream_t s = as_stream(stream);
  Counter c;
  int st = c.init(s);
  if (st != BSFP8_OK) return st;
  st = launch_make_twin(w, G, R, D, q_out, e_out, block_ok, c.dev, s);
  if (st != BSFP8_OK) return st;
  unsigned long long bad = 0;
  st = c.read(s, &bad);
  if (st != BSFP8_OK) return st;
  if (n_bad_out) *n_bad_out = (int64_t)bad;
  return bad ? BSFP8_NOT_EXACT : BSFP8_OK;
}

int bsfp8_make_twin_async(const uint16_t* w, int64_t G, int64_t R, int64_t D, uint8_t* q_out,
                          uint8_t* e_out, uint8_t* block_ok, int64_t* n_bad_dev, void* stream) {
  if (G < 0 || R < 0 || D < 0 || R % 32 || D % 32) return BSFP8_ESHAPE;
  if (!n_bad_dev || reinterpret_cast<uintptr_t>(n_bad_dev) % 8) return BSFP8_EINVAL;
  if (G * R * D == 0) return BSFP8_OK;
  if (!w || !q_out || !e_out) return BSFP8_EINVAL;
  if (!aligned16(w) || !aligned16(q_out)) return BSFP8_ESTRIDE;
  {
    const size_t n = (size_t)G * R * D, nb = n / 1024;
    if (outputs_alias({{q_out, n}, {e_out, nb}, {block_ok, nb}, {n_bad_dev, 8}}, {{w, n * 2}})) return BSFP8_EINVAL;
  }
  return launch_make_twin(w, G, R, D, q_out, e_out, block_ok, reinterpret_cast<unsigned long long*>(n_bad_dev),
                          as_stream(stream));
}

int bsfp8_make_twin_row32(const uint16_t* w, int64_t G, int64_t N, int64_t K, uint8_t* q_out, uint8_t* e_out,
                          uint8_t* block_ok, int64_t* n_bad_out, void* stream) {
  if (G < 0 || N < 0 || K < 0 || K % 32) return BSFP8_ESHAPE;
  if (n_bad_out) *n_bad_out = 0;
  if (G * N * K == 0) return BSFP8_OK;
  if (!w || !q_out || !e_out) return BSFP8_EINVAL;
  if (!aligned16(w) || !aligned16(q_out)) return BSFP8_ESTRIDE;
  {
    const size_t n = (size_t)G * N * K, nb = n / 32;
    if (outputs_alias({{q_out, n}, {e_out, nb}, {block_ok, nb}}, {{w, n * 2}})) return BSFP8_EINVAL;
  }
  hipStream_t s = as_stream(stream);
  Counter c;
  int st = c.init(s);
  if (st != BSFP8_OK) return st;
  st = launch_make_twin_row32(w, G, N, K, q_out, e_out, block_ok, c.dev, s);
  if (st != BSFP8_OK) return st;
  unsigned long long bad = 0;
  st = c.read(s, &bad);
  if (st != BSFP8_OK) return st;
  if (n_bad_out) *n_bad_out = (int64_t)bad;
  return bad ? BSFP8_NOT_EXACT : BSFP8_OK;
}

int bsfp8_pad_k_weight(const uint8_t* q, const uint8_t* e, int64_t G, int64_t N, int64_t K,
                       int64_t K_pad, uint8_t* q_pad, uint8_t* e_pad, void* stream) {
  if (G < 0 || N < 0 || K < 0 || N % 32 || K % 32 || K_pad % 32 || K_pad < K) return BSFP8_ESHAPE;
  if (G * N * K_pad == 0) return BSFP8_OK;
  if (!q_pad || !e_pad || (K > 0 && (!q || !e))) return BSFP8_EINVAL;
  if ((K > 0 && !aligned16(q)) || !aligned16(q_pad)) return BSFP8_ESTRIDE;
  if (outputs_alias({{q_pad, (size_t)G * N * K_pad}, {e_pad, (size_t)G * (N / 32) * (K_pad / 32)}},
                    {{q, (size_t)G * N * K}, {e, (size_t)G * (N / 32) * (K / 32)}}))
    return BSFP8_EINVAL;
  return launch_pad_k_weight(q, e, G, N, K, K_pad, q_pad, e_pad, as_stream(stream));
}

int bsfp8_pad_k_input(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t K,
                      int64_t K_pad, uint16_t* x_pad, void* stream) {
  if (M < 0 || G < 1 || K < 0 || K % 32 || K_pad % 32 || K_pad < K) return BSFP8_ESHAPE;
  if (ldx < G * K) return BSFP8_ESTRIDE;
  if (M == 0 || K_pad == 0) return BSFP8_OK;
  if (!x_pad || (K > 0 && !x)) return BSFP8_EINVAL;
  if (outputs_alias({{x_pad, (size_t)M * G * K_pad * 2}}, {{x, ((size_t)(M - 1) * ldx + (size_t)G * K) * 2}}))
    return BSFP8_EINVAL;
  return launch_pad_k_input(x, ldx, M, G, K, K_pad, x_pad, as_stream(stream));
}

int bsfp8_dequant(const uint8_t* q, const uint8_t* e, int64_t G, int64_t N, int64_t K,
                  uint16_t* w_out, void* stream) {
  if (G < 0 || N < 0 || K < 0 || N % 32 || K % 32 || K > (1 << 24)) return BSFP8_ESHAPE;
  if (G * N * K == 0) return BSFP8_OK;
  if (!q || !e || !w_out) return BSFP8_EINVAL;
  if (!aligned16(q) || !aligned16(w_out)) return BSFP8_ESTRIDE;
  if (outputs_alias({{w_out, (size_t)G * N * K * 2}}, {{q, (size_t)G * N * K}, {e, (size_t)G * (N / 32) * (K / 32)}}))
    return BSFP8_EINVAL;
  return launch_dequant(q, e, G, N, K, w_out, as_stream(stream));
}

size_t bsfp8_workspace_bytes(int64_t M, int64_t G, int64_t N, int64_t K, int split_k) {
  if (M <= 0 || G < 1 || N < 32 || K < 32 || N % 32 || K % 32 || split_k < 0 || split_k > 64) return 0;
  if (M > 256 || G > 4096 || N > (1 << 24) || K > (1 << 24)) return 0;
  GemmShape s{G * K, (int)M, (int)G, (int)N, (int)K};
  size_t need = 0;
  for (int path = PATH_SMALL; path <= PATH_MID; ++path) {
    if (path == PATH_SMALL && M > 16) continue;
    GemmPlan p;
    if (plan_gemm(s, path, split_k, &p) == BSFP8_OK && p.ws_bytes > need) need = p.ws_bytes;
  }
  return need;
}

int bsfp8_gemm_small(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
                     const uint8_t* q, const uint8_t* e, int split_k, void* ws, size_t ws_bytes,
                     void* y, int out_dtype, void* stream) {
  return run_gemm(PATH_SMALL, 16, x, ldx, M, G, N, K, q, e, split_k, ws, ws_bytes, y, out_dtype, stream);
}

int bsfp8_gemm_mid(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
                   const uint8_t* q, const uint8_t* e, int split_k, void* ws, size_t ws_bytes,
                   void* y, int out_dtype, void* stream) {
  return run_gemm(PATH_MID, 256, x, ldx, M, G, N, K, q, e, split_k, ws, ws_bytes, y, out_dtype, stream);
}

int bsfp8_gemm(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
               const uint8_t* q, const uint8_t* e, int split_k, void* ws, size_t ws_bytes, void* y,
               int out_dtype, void* stream) {
  const int path = M <= 8 ? PATH_SMALL : PATH_MID;
  return run_gemm(path, 256, x, ldx, M, G, N, K, q, e, split_k, ws, ws_bytes, y, out_dtype, stream);
}

int bsfp8_gemm_no_alloc(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
                        const uint8_t* q, const uint8_t* e, int split_k, void* y, int out_dtype, void* stream) {
  GemmShape s;
  int st = check_gemm(x, ldx, M, G, N, K, q, e, y, out_dtype, split_k, 256, &s);
  if (st != BSFP8_OK || M == 0) return st;
  GemmPlan p;
  st = plan_gemm(s, M <= 8 ? PATH_SMALL : PATH_MID, split_k, &p);
  if (st != BSFP8_OK) return st;
  hipStream_t hs = as_stream(stream);
  void* ws = nullptr;
  if (p.ws_bytes > 0) {
    if (p.ws_bytes > BSFP8_NO_ALLOC_SCRATCH_BYTES) return BSFP8_EWORKSPACE;
    st = scratch_for_stream(hs, &ws);
    if (st != BSFP8_OK) return st;
  }
  st = check_gemm_alias(s, x, q, e, false, ws, p.ws_bytes, y, out_dtype);
  if (st != BSFP8_OK) return st;
  if (gemm_ws_needs_zero(p)) {
    st = launch_clear(ws, p.ws_bytes, hs);
    if (st != BSFP8_OK) return st;
  }
  return launch_gemm(s, p, x, q, e, ws, y, out_dtype == BSFP8_OUT_F32, hs);
}

size_t bsfp8_workspace_bytes_row32(int64_t M, int64_t G, int64_t N, int64_t K, int split_k) {
  if (M <= 0 || M > 16 || G < 1 || N < 32 || K < 128 || N % 32 || K % 128 || split_k < 0 || split_k > 64) return 0;
  if (G > 4096 || N > (1 << 24) || K > (1 << 24)) return 0;
  GemmShape s{G * K, (int)M, (int)G, (int)N, (int)K};
  GemmPlan p;
  return plan_gemm_row32(s, split_k, &p) == BSFP8_OK ? p.ws_bytes : 0;
}

int bsfp8_gemm_row32(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
                     const uint8_t* q, const uint8_t* e, int split_k, void* ws, size_t ws_bytes, void* y,
                     int out_dtype, void* stream) {
  GemmShape s;
  int st = check_gemm(x, ldx, M, G, N, K, q, e, y, out_dtype, split_k, 16, &s);
  if (st != BSFP8_OK || M == 0) return st;
  GemmPlan p;
  st = plan_gemm_row32(s, split_k, &p);
  if (st != BSFP8_OK) return st;
  if (p.ws_bytes > 0 && (!ws || ws_bytes < p.ws_bytes || !aligned16(ws))) return BSFP8_EWORKSPACE;
  st = check_gemm_alias(s, x, q, e, true, ws, ws_bytes, y, out_dtype);
  if (st != BSFP8_OK) return st;
  return launch_gemm(s, p, x, q, e, ws, y, out_dtype == BSFP8_OUT_F32, as_stream(stream));
}

int bsfp8_gemm_row32_config(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
                            const uint8_t* q, const uint8_t* e, int cfg, int cps, void* ws, size_t ws_bytes,
                            void* y, int out_dtype, void* stream) {
  if (!gemm_config_row_scales(cfg)) return BSFP8_EINVAL;
  GemmShape s;
  int st = check_gemm(x, ldx, M, G, N, K, q, e, y, out_dtype, 0, 256, &s);
  if (st != BSFP8_OK || M == 0) return st;
  GemmPlan p;
  st = plan_with(s, cfg, cps, &p);
  if (st != BSFP8_OK) return st;
  if (p.ws_bytes > 0 && (!ws || ws_bytes < p.ws_bytes || !aligned16(ws))) return BSFP8_EWORKSPACE;
  st = check_gemm_alias(s, x, q, e, true, ws, ws_bytes, y, out_dtype);
  if (st != BSFP8_OK) return st;
  return launch_gemm(s, p, x, q, e, ws, y, out_dtype == BSFP8_OUT_F32, as_stream(stream));
}

int bsfp8_read_floor(const void* p, size_t bytes, int nwg, const void* slab, size_t slab_bytes, int slab_groups,
                     int flags, uint32_t* sink, void* out, size_t out_bytes, void* stream) {
  if (nwg < 1 || nwg > 65536 || !sink || (out_bytes && !out)) return BSFP8_EINVAL;
  if (flags & ~BSFP8_FLOOR_SLAB_INTERLEAVED) return BSFP8_EINVAL;
  if (slab_bytes && (!slab || slab_groups < 1 || slab_groups > nwg)) return BSFP8_EINVAL;
  if (bytes && (!p || !aligned16(p))) return BSFP8_ESTRIDE;
  if (out_bytes && (!aligned16(out) || out_bytes % 16)) return BSFP8_ESTRIDE;
  if (slab_bytes && (!aligned16(slab) || slab_bytes % 16)) return BSFP8_ESTRIDE;
  if (bytes >= ((size_t)1 << 31) || out_bytes >= ((size_t)1 << 31)) return BSFP8_ESHAPE;
  if (slab_bytes && slab_bytes * (size_t)slab_groups >= ((size_t)1 << 31)) return BSFP8_ESHAPE;
  const size_t slab_span = slab_bytes ? slab_bytes * (size_t)slab_groups : 0;
  if (outputs_alias({{out, out_bytes}, {sink, (size_t)nwg * 4}}, {{p, bytes}, {slab, slab_span}}))
    return BSFP8_EINVAL;
  return launch_read_floor(p, bytes, nwg, slab, slab_bytes, slab_bytes ? slab_groups : 1,
                           (flags & BSFP8_FLOOR_SLAB_INTERLEAVED) != 0, sink, out, out_bytes, as_stream(stream));
}

int bsfp8_num_configs(void) { return num_gemm_configs(); }

int bsfp8_config_info(int cfg, int* out) {
  if (!out) return BSFP8_EINVAL;
  return gemm_config_info(cfg, out);
}

int bsfp8_plan_info(int64_t M, int64_t G, int64_t N, int64_t K, int split_k, int path, int* out) {
  if (!out) return BSFP8_EINVAL;
  if (path < 0 || path > 3) return BSFP8_EINVAL;
  const int p_eff = path >= 2 ? (M <= 8 ? PATH_SMALL : PATH_MID) : path;
  const int64_t max_m = p_eff == PATH_SMALL && path != 2 ? 16 : 256;
  GemmShape s;
  int st = check_dims(M, G, N, K, split_k, max_m, &s);
  if (st != BSFP8_OK) return st;
  if (M == 0) return BSFP8_ESHAPE;
  GemmPlan p;
  st = path == 3 ? plan_gemm_mxfp8(s, split_k, &p) : plan_gemm(s, p_eff, split_k, &p);
  if (st != BSFP8_OK) return st;
  out[0] = p.cfg;
  out[1] = p.BM;
  out[2] = p.NB;
  out[3] = p.kchunks;
  out[4] = p.cps;
  out[5] = p.splits;
  out[6] = p.mblocks;
  out[7] = (int)((int64_t)p.splits * s.G * p.nblocks * p.mblocks);
  return BSFP8_OK;
}

size_t bsfp8_workspace_bytes_config(int64_t M, int64_t G, int64_t N, int64_t K, int cfg, int cps) {
  if (M <= 0 || M > 256 || G < 1 || N < 32 || K < 32 || N % 32 || K % 32 || cps < 1) return 0;
  GemmShape s{G * K, (int)M, (int)G, (int)N, (int)K};
  GemmPlan p;
  if (plan_with(s, cfg, cps, &p) != BSFP8_OK) return 0;
  return p.ws_bytes;
}

int bsfp8_gemm_config(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
                      const uint8_t* q, const uint8_t* e, int cfg, int cps, void* ws,
                      size_t ws_bytes, void* y, int out_dtype, void* stream) {
  if (gemm_config_row_scales(cfg)) return BSFP8_EINVAL;       // those read [G][N][K/32] exponents
  GemmShape s;
  int st = check_gemm(x, ldx, M, G, N, K, q, e, y, out_dtype, 0, 256, &s);
  if (st != BSFP8_OK || M == 0) return st;
  GemmPlan p;
  st = plan_with(s, cfg, cps, &p);
  if (st != BSFP8_OK) return st;
  if (p.ws_bytes > 0 && (!ws || ws_bytes < p.ws_bytes || !aligned16(ws))) return BSFP8_EWORKSPACE;
  st = check_gemm_alias(s, x, q, e, false, ws, ws_bytes, y, out_dtype);
  if (st != BSFP8_OK) return st;
  return launch_gemm(s, p, x, q, e, ws, y, out_dtype == BSFP8_OUT_F32, as_stream(stream));
}

int bsfp8_quantize_mx(const uint16_t* x, int64_t ldx, int64_t M, int64_t L, uint8_t* xq, uint8_t* xs,
                      void* stream) {
  if (M < 0 || L < 32 || L % 32 || M > (1 << 24) || L > (1 << 26)) return BSFP8_ESHAPE;
  if (M == 0) return BSFP8_OK;
  if (!x || !xq || !xs) return BSFP8_EINVAL;
  if (ldx < L || ldx % 8 || !aligned16(x) || !aligned16(xq)) return BSFP8_ESTRIDE;
  if (outputs_alias({{xq, (size_t)M * L}, {xs, (size_t)M * L / 32}}, {{x, ((size_t)(M - 1) * ldx + L) * 2}}))
    return BSFP8_EINVAL;
  return launch_quantize_mx(x, ldx, M, L, xq, xs, as_stream(stream));
}

int bsfp8_gemm_mx(const uint8_t* xq, const uint8_t* xs, int64_t ldq, int64_t M, int64_t G, int64_t N,
                  int64_t K, const uint8_t* q, const uint8_t* e, void* y, int out_dtype, void* stream) {
  const int st = check_gemm_mx(xq, xs, ldq, M, G, N, K, q, e, y, out_dtype);
  if (st != BSFP8_OK || M == 0) return st;
  return launch_gemm_mx(xq, xs, ldq, (int)M, (int)G, (int)N, (int)K, q, e, y, out_dtype == BSFP8_OUT_F32,
                        mx_pick((int)M, (int)G, (int)N), as_stream(stream));
}

int bsfp8_mx_num_configs(void) { return num_mx_configs(); }

int bsfp8_mx_config_info(int cfg, int* out) {
  if (!out) return BSFP8_EINVAL;
  return mx_config_info(cfg, out);
}

int bsfp8_mx_plan(int64_t M, int64_t G, int64_t N) {
  if (M < 1 || M > 256 || G < 1 || N < 32 || N % 32) return BSFP8_ESHAPE;
  return mx_pick((int)M, (int)G, (int)N);
}

int bsfp8_gemm_mx_config(const uint8_t* xq, const uint8_t* xs, int64_t ldq, int64_t M, int64_t G,
                         int64_t N, int64_t K, const uint8_t* q, const uint8_t* e, int cfg, void* y,
                         int out_dtype, void* stream) {
  const int st = check_gemm_mx(xq, xs, ldq, M, G, N, K, q, e, y, out_dtype);
  if (st != BSFP8_OK || M == 0) return st;
  return launch_gemm_mx(xq, xs, ldq, (int)M, (int)G, (int)N, (int)K, q, e, y, out_dtype == BSFP8_OUT_F32, cfg,
                        as_stream(stream));
}

int bsfp8_reduce_quantize_mx(const float* part, int64_t S, int64_t M, int64_t L, int order, uint8_t* yq,
                             uint8_t* ys, void* stream) {
  if (order != BSFP8_SUM_ASCENDING && order != BSFP8_SUM_PAIRWISE) return BSFP8_EINVAL;
  if (S < 1 || S > 64) return BSFP8_EINVAL;
  if (M < 0 || L < 32 || L % 32 || M > (1 << 24) || L > (1 << 26)) return BSFP8_ESHAPE;
  if (M == 0) return BSFP8_OK;
  if (S * M * L > ((int64_t)1 << 40)) return BSFP8_ESHAPE;
  if (!part || !yq || !ys) return BSFP8_EINVAL;
  if (!aligned16(part) || !aligned16(yq)) return BSFP8_ESTRIDE;
  if (outputs_alias({{yq, (size_t)M * L}, {ys, (size_t)M * L / 32}}, {{part, (size_t)S * M * L * 4}}))
    return BSFP8_EINVAL;
  return launch_reduce_quantize_mx(part, (int)S, M, L, order, yq, ys, as_stream(stream));
}

size_t bsfp8_workspace_bytes_mxfp8(int64_t M, int64_t G, int64_t N, int64_t K, int split_k) {
  GemmShape s;
  if (M <= 0 || check_dims(M, G, N, K, split_k, 256, &s) != BSFP8_OK) return 0;
  GemmPlan p;
  return plan_gemm_mxfp8(s, split_k, &p) == BSFP8_OK ? gemm_partials_bytes(s, p) : 0;
}

int bsfp8_gemm_mxfp8(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
                     const uint8_t* q, const uint8_t* e, int split_k, void* ws, size_t ws_bytes, uint8_t* yq,
                     uint8_t* ys, void* stream) {
  GemmShape s;
  int st = check_gemm(x, ldx, M, G, N, K, q, e, yq, BSFP8_OUT_F32, split_k, 256, &s);
  if (st != BSFP8_OK || M == 0) return st;
  if (!ys) return BSFP8_EINVAL;
  GemmPlan p;
  st = plan_gemm_mxfp8(s, split_k, &p);
  if (st != BSFP8_OK) return st;
  return run_gemm_mxfp8(s, p, x, q, e, ws, ws_bytes, yq, ys, /*fuse=*/true, as_stream(stream));
}

size_t bsfp8_workspace_bytes_mxfp8_config(int64_t M, int64_t G, int64_t N, int64_t K, int cfg, int cps) {
  GemmShape s;
  if (M <= 0 || check_dims(M, G, N, K, 0, 256, &s) != BSFP8_OK || gemm_config_row_scales(cfg)) return 0;
  GemmPlan p;
  return plan_with(s, cfg, cps, &p) == BSFP8_OK ? gemm_partials_bytes(s, p) : 0;
}

int bsfp8_gemm_mxfp8_config(const uint16_t* x, int64_t ldx, int64_t M, int64_t G, int64_t N, int64_t K,
                            const uint8_t* q, const uint8_t* e, int cfg, int cps, void* ws, size_t ws_bytes,
                            uint8_t* yq, uint8_t* ys, void* stream) {
  if (gemm_config_row_scales(cfg)) return BSFP8_EINVAL;
  GemmShape s;
  int st = check_gemm(x, ldx, M, G, N, K, q, e, yq, BSFP8_OUT_F32, 0, 256, &s);
  if (st != BSFP8_OK || M == 0) return st;
  if (!ys) return BSFP8_EINVAL;
  GemmPlan p;
  st = plan_with(s, cfg, cps, &p);
  if (st != BSFP8_OK) return st;
  return run_gemm_mxfp8(s, p, x, q, e, ws, ws_bytes, yq, ys, /*fuse=*/false, as_stream(stream));
}

}  // extern "C"
