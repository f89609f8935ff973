// C ABI of libmxq: host-side validation and kernel dispatch. Every check runs
// before any launch, so an argument error writes nothing; the calls never
// allocate, free or synchronize.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/mxq.h"

namespace mxq {
hipError_t launch_quant_mxfp8(const void*, int64_t, int64_t, int64_t, void*, void*, void*, void*, hipStream_t);
hipError_t launch_quant_mxfp8_multi(int, const void* const*, const int64_t*, const int64_t*, const int64_t*,
                                    void* const*, void* const*, void* const*, void* const*, hipStream_t);
hipError_t launch_quant_mxfp4(const void*, int64_t, int64_t, int64_t, void*, void*, void*, void*, hipStream_t);
hipError_t launch_quant_mxfp4_multi(int, const void* const*, const int64_t*, const int64_t*, const int64_t*,
                                    void* const*, void* const*, void* const*, void* const*, hipStream_t);
hipError_t launch_quant_fp8_block(int, const void*, int64_t, int64_t, int64_t, void*, float*, void*, float*,
                                  hipStream_t);
hipError_t launch_quant_nvfp4_token(const void*, int64_t, int64_t, int64_t, void*, void*, float*, hipStream_t);
hipError_t launch_quant_nvfp4(const void*, int64_t, int64_t, int64_t, int, int64_t, int, int, uint32_t, void*, void*,
                              float*, uint32_t*, int64_t, int, uint64_t, hipStream_t);
hipError_t launch_quant_nvfp4_2d(const void*, int64_t, int64_t, int64_t, int64_t, void*, void*, void*, void*, float*,
                                 uint32_t*, int64_t, hipStream_t);
hipError_t launch_dequant(int, const void*, const void*, const float*, int, int64_t, int64_t, int64_t, void*, int,
                          hipStream_t);
hipError_t launch_dequant_t(int, const void*, const void*, const float*, int, int64_t, int64_t, int64_t,
                            const int32_t*, int64_t, void*, int64_t, hipStream_t);
hipError_t launch_swiglu_nvfp4(const float*, int64_t, int64_t, void*, void*, void*, float*, hipStream_t);
hipError_t launch_combine(const float*, int64_t, int64_t, int64_t, int64_t, const int64_t*, const float*, float*,
                          hipStream_t);
hipError_t launch_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void* A, const void* sA, const float* tA,
                       int tA_mode, const void* B, const void* sB, const float* tB, int tB_mode, float* C,
                       int64_t ldc, hipStream_t st);
hipError_t launch_grouped_gemm(int fmt, int64_t groups, const int64_t* offsets, int vary_k, int64_t total, int64_t M,
                               int64_t N, int64_t K, const int32_t* a_row_index, int64_t a_rows, const void* A,
                               const void* sA, const float* tA, int tA_mode, const void* B, const void* sB,
                               const float* tB, int tB_mode, float* C, void* ws, hipStream_t st);
size_t grouped_gemm_ws_bytes(int64_t groups);
hipError_t launch_gemm_batch(int fmt, int n, const int64_t* M, const int64_t* N, const int64_t* K,
                             const void* const* A, const void* const* sA, const float* const* tA, const int* tA_mode,
                             const void* const* B, const void* const* sB, const float* const* tB, const int* tB_mode,
                             float* const* C, const int64_t* ldc, hipStream_t st);
}  // namespace mxq

namespace {

constexpr int64_t kMaxRowCols = 16384;       // register-resident NVFP4 row quantizer
constexpr int64_t kMaxGridBlocks = 0x7FFFFFFF;
// GEMM operand reads use 32-bit buffer offsets: a 256-row tile of K-contiguous rows,
// or (gather) the whole gathered operand, must span less than 2^31 bytes.
constexpr int64_t kMaxGemmK = int64_t(1) << 22;
inline int64_t gemm_row_bytes(mxq_format fmt, int64_t k) {
  return fmt == MXQ_BF16 ? 2 * k : fmt == MXQ_MXFP8 ? k : k / 2;   // NVFP4, MXFP4: two per byte
}

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool al4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
inline hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }
inline mxq_status hip_status(hipError_t e) { return e == hipSuccess ? MXQ_OK : MXQ_ERR_HIP; }

}  // namespace

extern "C" {

int mxq_abi_version(void) { return MXQ_ABI_VERSION; }

const char* mxq_status_string(mxq_status s) {
  switch (s) {
    case MXQ_OK: return "ok";
    case MXQ_ERR_NULL: return "required pointer is NULL";
    case MXQ_ERR_SHAPE: return "invalid shape (negative, not a multiple of the block, or beyond a limit)";
    case MXQ_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case MXQ_ERR_FORMAT: return "unsupported format, scope or option combination";
    case MXQ_ERR_WORKSPACE: return "workspace missing or too small";
    case MXQ_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

size_t mxq_scale_bytes(mxq_format fmt, int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  if ((fmt == MXQ_MXFP8 || fmt == MXQ_MXFP4) && cols % 32 == 0) return (size_t)(rows * (cols / 32));
  if (fmt == MXQ_NVFP4 && cols % 16 == 0) return (size_t)(rows * (cols / 16));
  return 0;
}

size_t mxq_workspace_bytes(int op, int64_t a, int64_t b, int64_t c) {
  (void)b;
  if (op == MXQ_OP_QUANTIZE_NVFP4) return c > 0 ? (size_t)(((c * 4) + 255) / 256 * 256) : 0;
  if (op == MXQ_OP_GROUPED_GEMM) return a > 0 ? mxq::grouped_gemm_ws_bytes(a) : 0;
  return 0;
}

mxq_status quantize_mxfp8(const void* x, int64_t rows, int64_t cols, int64_t ld_x, void* q_row, void* s_row,
                          void* q_colT, void* s_colT, void* stream) {
  if (rows < 0 || cols < 0) return MXQ_ERR_SHAPE;
  const bool do_row = q_row || s_row, do_col = q_colT || s_colT;
  if (!x || (!do_row && !do_col)) return MXQ_ERR_NULL;
  if ((do_row && (!q_row || !s_row)) || (do_col && (!q_colT || !s_colT))) return MXQ_ERR_NULL;
  if (cols % 32) return MXQ_ERR_SHAPE;
  if (do_col && rows % 32) return MXQ_ERR_SHAPE;
  if (ld_x < cols) return MXQ_ERR_SHAPE;
  if (ld_x % 8 || !al16(x) || (do_row && !al16(q_row)) || (do_col && !al16(q_colT))) return MXQ_ERR_ALIGN;
  if (rows == 0 || cols == 0) return MXQ_OK;
  if (((rows + 127) / 128) * ((cols + 127) / 128) > kMaxGridBlocks) return MXQ_ERR_SHAPE;
  return hip_status(mxq::launch_quant_mxfp8(x, rows, cols, ld_x, do_row ? q_row : nullptr, s_row,
                                            do_col ? q_colT : nullptr, s_colT, S(stream)));
}

mxq_status quantize_mxfp4(const void* x, int64_t rows, int64_t cols, int64_t ld_x, void* q_row, void* s_row,
                          void* q_colT, void* s_colT, void* stream) {
  if (rows < 0 || cols < 0) return MXQ_ERR_SHAPE;
  const bool do_row = q_row || s_row, do_col = q_colT || s_colT;
  if (!x || (!do_row && !do_col)) return MXQ_ERR_NULL;
  if ((do_row && (!q_row || !s_row)) || (do_col && (!q_colT || !s_colT))) return MXQ_ERR_NULL;
  if (cols % 32) return MXQ_ERR_SHAPE;
  if (do_col && rows % 32) return MXQ_ERR_SHAPE;
  if (ld_x < cols) return MXQ_ERR_SHAPE;
  if (ld_x % 8 || !al16(x) || (do_row && !al16(q_row)) || (do_col && !al16(q_colT))) return MXQ_ERR_ALIGN;
  if (rows == 0 || cols == 0) return MXQ_OK;
  if (((rows + 127) / 128) * ((cols + 127) / 128) > kMaxGridBlocks) return MXQ_ERR_SHAPE;
  return hip_status(mxq::launch_quant_mxfp4(x, rows, cols, ld_x, do_row ? q_row : nullptr, s_row,
                                            do_col ? q_colT : nullptr, s_colT, S(stream)));
}

}  // extern "C"

namespace {
mxq_status quantize_mx_multi(const mxq_mxfp8_tensor* tensors, int count, bool fp4, void* stream) {
  if (count < 1 || count > MXQ_MXFP8_MULTI_MAX) return MXQ_ERR_SHAPE;
  if (!tensors) return MXQ_ERR_NULL;
  const void* x[MXQ_MXFP8_MULTI_MAX];
  int64_t rows[MXQ_MXFP8_MULTI_MAX], cols[MXQ_MXFP8_MULTI_MAX], ld[MXQ_MXFP8_MULTI_MAX];
  void *qr[MXQ_MXFP8_MULTI_MAX], *sr[MXQ_MXFP8_MULTI_MAX], *qc[MXQ_MXFP8_MULTI_MAX], *sc[MXQ_MXFP8_MULTI_MAX];
  int n = 0;
  int64_t blocks = 0;
  bool mode_set = false, mode_row = false, mode_col = false;
  for (int i = 0; i < count; ++i) {
    const mxq_mxfp8_tensor& t = tensors[i];
    if (t.rows < 0 || t.cols < 0) return MXQ_ERR_SHAPE;
    if (t.rows == 0 || t.cols == 0) continue;                 // empty tensors are skipped
    const bool do_row = t.q_row || t.s_row, do_col = t.q_colT || t.s_colT;
    if (!t.x || (!do_row && !do_col)) return MXQ_ERR_NULL;
    if ((do_row && (!t.q_row || !t.s_row)) || (do_col && (!t.q_colT || !t.s_colT))) return MXQ_ERR_NULL;
    if (mode_set && (do_row != mode_row || do_col != mode_col)) return MXQ_ERR_FORMAT;
    mode_set = true; mode_row = do_row; mode_col = do_col;
    if (t.cols % 32) return MXQ_ERR_SHAPE;
    if (do_col && t.rows % 32) return MXQ_ERR_SHAPE;
    if (t.ld_x < t.cols) return MXQ_ERR_SHAPE;
    if (t.ld_x % 8 || !al16(t.x) || (do_row && !al16(t.q_row)) || (do_col && !al16(t.q_colT))) return MXQ_ERR_ALIGN;
    blocks += ((t.rows + 127) / 128) * ((t.cols + 127) / 128);
    x[n] = t.x; rows[n] = t.rows; cols[n] = t.cols; ld[n] = t.ld_x;
    qr[n] = do_row ? t.q_row : nullptr; sr[n] = t.s_row; qc[n] = do_col ? t.q_colT : nullptr; sc[n] = t.s_colT;
    ++n;
  }
  if (blocks > kMaxGridBlocks) return MXQ_ERR_SHAPE;
  if (n == 0) return MXQ_OK;
  return hip_status(fp4 ? mxq::launch_quant_mxfp4_multi(n, x, rows, cols, ld, qr, sr, qc, sc, S(stream))
                        : mxq::launch_quant_mxfp8_multi(n, x, rows, cols, ld, qr, sr, qc, sc, S(stream)));
}
}  // namespace

extern "C" {

mxq_status quantize_mxfp8_multi(const mxq_mxfp8_tensor* tensors, int count, void* stream) {
  return quantize_mx_multi(tensors, count, false, stream);
}

mxq_status quantize_mxfp4_multi(const mxq_mxfp8_tensor* tensors, int count, void* stream) {
  return quantize_mx_multi(tensors, count, true, stream);
}

mxq_status quantize_fp8_block_act(const void* x, int64_t rows, int64_t cols, int64_t ld_x, void* q_row, float* s_row,
                                  void* q_colT, float* s_colT, void* stream) {
  if (rows < 0 || cols < 0) return MXQ_ERR_SHAPE;
  const bool do_row = q_row || s_row, do_col = q_colT || s_colT;
  if (!x || (!do_row && !do_col)) return MXQ_ERR_NULL;
  if ((do_row && (!q_row || !s_row)) || (do_col && (!q_colT || !s_colT))) return MXQ_ERR_NULL;
  if (ld_x < cols || cols % 8) return MXQ_ERR_SHAPE;
  if (do_row && cols % 128) return MXQ_ERR_SHAPE;
  if (do_col && rows % 128) return MXQ_ERR_SHAPE;
  if (ld_x % 8 || !al16(x) || (do_row && (!al16(q_row) || !al4(s_row))) || (do_col && (!al16(q_colT) || !al4(s_colT))))
    return MXQ_ERR_ALIGN;
  if (rows == 0 || cols == 0) return MXQ_OK;
  if (((rows + 127) / 128) * ((cols + 127) / 128) > kMaxGridBlocks) return MXQ_ERR_SHAPE;
  return hip_status(mxq::launch_quant_fp8_block(0, x, rows, cols, ld_x, do_row ? q_row : nullptr, s_row,
                                                do_col ? q_colT : nullptr, s_colT, S(stream)));
}

mxq_status quantize_fp8_block_weight(const void* x, int64_t rows, int64_t cols, int64_t ld_x, void* q_row, float* s_row,
                                     void* q_colT, float* s_colT, void* stream) {
  if (rows < 0 || cols < 0) return MXQ_ERR_SHAPE;
  const bool do_row = q_row || s_row, do_col = q_colT || s_colT;
  if (!x || (!do_row && !do_col)) return MXQ_ERR_NULL;
  if ((do_row && (!q_row || !s_row)) || (do_col && (!q_colT || !s_colT))) return MXQ_ERR_NULL;
  if (rows % 128 || cols % 128 || ld_x < cols) return MXQ_ERR_SHAPE;
  if (ld_x % 8 || !al16(x) || (do_row && (!al16(q_row) || !al4(s_row))) || (do_col && (!al16(q_colT) || !al4(s_colT))))
    return MXQ_ERR_ALIGN;
  if (rows == 0 || cols == 0) return MXQ_OK;
  if ((rows / 128) * (cols / 128) > kMaxGridBlocks) return MXQ_ERR_SHAPE;
  return hip_status(mxq::launch_quant_fp8_block(1, x, rows, cols, ld_x, do_row ? q_row : nullptr, s_row,
                                                do_col ? q_colT : nullptr, s_colT, S(stream)));
}

mxq_status quantize_nvfp4_per_token(const void* x, int64_t tokens, int64_t hidden, int64_t ld_x, void* q_packed,
                                    void* s_block, float* s_token, void* stream) {
  if (tokens < 0 || hidden < 0) return MXQ_ERR_SHAPE;
  if (!x || !q_packed || !s_block || !s_token) return MXQ_ERR_NULL;
  if (hidden % 16 || hidden > kMaxRowCols || ld_x < hidden) return MXQ_ERR_SHAPE;
  if (ld_x % 8 || !al16(x) || !al4(q_packed) || !al4(s_token)) return MXQ_ERR_ALIGN;
  if (tokens == 0 || hidden == 0) return MXQ_OK;
  return hip_status(mxq::launch_quant_nvfp4_token(x, tokens, hidden, ld_x, q_packed, s_block, s_token, S(stream)));
}

namespace {
mxq_status quantize_nvfp4_any(const void* x, int64_t rows, int64_t cols, int64_t ld_x, mxq_scope scope,
                              int64_t group_rows, int transpose, const int8_t* rht_signs16, void* q, void* s, float* t,
                              void* workspace, size_t workspace_bytes, int sr, uint64_t seed, void* stream) {
  if (rows < 0 || cols < 0) return MXQ_ERR_SHAPE;
  if (!x || !q || !s || !t) return MXQ_ERR_NULL;
  if (scope != MXQ_SCOPE_ROW && scope != MXQ_SCOPE_TENSOR && scope != MXQ_SCOPE_GROUP) return MXQ_ERR_FORMAT;
  if (transpose != 0 && transpose != 1) return MXQ_ERR_FORMAT;
  if (transpose && scope == MXQ_SCOPE_ROW) return MXQ_ERR_FORMAT;
  uint32_t neg_mask = 0;
  if (rht_signs16) {
    for (int i = 0; i < 16; ++i) {
      if (rht_signs16[i] == -1) neg_mask |= 1u << i;
      else if (rht_signs16[i] != 1) return MXQ_ERR_FORMAT;
    }
  }
  if (ld_x < cols) return MXQ_ERR_SHAPE;
  const int64_t out_rows = transpose ? cols : rows;
  if (transpose) {
    if (rows % 16 || cols % 8) return MXQ_ERR_SHAPE;
  } else {
    if (cols % 16 || cols > kMaxRowCols) return MXQ_ERR_SHAPE;
  }
  int64_t n_scopes = 1;
  if (scope == MXQ_SCOPE_ROW) n_scopes = out_rows;
  if (scope == MXQ_SCOPE_GROUP) {
    if (group_rows <= 0 || out_rows % group_rows) return MXQ_ERR_SHAPE;
    if (transpose && group_rows % 8) return MXQ_ERR_SHAPE;
    n_scopes = out_rows / group_rows;
  }
  if (ld_x % 8 || !al16(x) || !al4(q) || !al4(t)) return MXQ_ERR_ALIGN;
  if (transpose && !al16(q)) return MXQ_ERR_ALIGN;
  if (scope != MXQ_SCOPE_ROW) {
    if (!workspace || workspace_bytes < (size_t)(n_scopes * 4)) return MXQ_ERR_WORKSPACE;
    if (!al4(workspace)) return MXQ_ERR_ALIGN;
  }
  if (rows == 0 || cols == 0) return MXQ_OK;
  return hip_status(mxq::launch_quant_nvfp4(x, rows, cols, ld_x, (int)scope, group_rows, transpose,
                                            rht_signs16 != nullptr, neg_mask, q, s, t, (uint32_t*)workspace,
                                            n_scopes, sr, seed, S(stream)));
}
}  // namespace

mxq_status quantize_nvfp4(const void* x, int64_t rows, int64_t cols, int64_t ld_x, mxq_scope scope,
                          int64_t group_rows, int transpose, const int8_t* rht_signs16, void* q, void* s, float* t,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return quantize_nvfp4_any(x, rows, cols, ld_x, scope, group_rows, transpose, rht_signs16, q, s, t, workspace,
                            workspace_bytes, 0, 0, stream);
}

mxq_status quantize_nvfp4_stochastic(const void* x, int64_t rows, int64_t cols, int64_t ld_x, mxq_scope scope,
                                     int64_t group_rows, int transpose, const int8_t* rht_signs16, uint64_t seed,
                                     void* q, void* s, float* t, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  return quantize_nvfp4_any(x, rows, cols, ld_x, scope, group_rows, transpose, rht_signs16, q, s, t, workspace,
                            workspace_bytes, 1, seed, stream);
}

mxq_status quantize_nvfp4_2d(const void* x, int64_t rows, int64_t cols, int64_t ld_x, mxq_scope scope,
                             int64_t group_rows, void* q_row, void* s_row, void* q_colT, void* s_colT, float* t,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 0 || cols < 0) return MXQ_ERR_SHAPE;
  const bool do_row = q_row || s_row, do_col = q_colT || s_colT;
  if (!x || !t || (!do_row && !do_col)) return MXQ_ERR_NULL;
  if ((do_row && (!q_row || !s_row)) || (do_col && (!q_colT || !s_colT))) return MXQ_ERR_NULL;
  if (scope != MXQ_SCOPE_TENSOR && scope != MXQ_SCOPE_GROUP) return MXQ_ERR_FORMAT;
  if (rows % 16 || cols % 16 || cols > kMaxRowCols || ld_x < cols) return MXQ_ERR_SHAPE;
  const int64_t gr = scope == MXQ_SCOPE_TENSOR ? rows : group_rows;
  if (scope == MXQ_SCOPE_GROUP && (group_rows <= 0 || group_rows % 16 || rows % group_rows)) return MXQ_ERR_SHAPE;
  if (ld_x % 8 || !al16(x) || !al4(t) || (do_row && !al4(q_row)) || (do_col && !al16(q_colT))) return MXQ_ERR_ALIGN;
  if (rows == 0 || cols == 0) return MXQ_OK;
  const int64_t n_scopes = rows / gr;
  if (!workspace || workspace_bytes < (size_t)(n_scopes * 4)) return MXQ_ERR_WORKSPACE;
  if (!al4(workspace)) return MXQ_ERR_ALIGN;
  if ((rows + 255) / 256 * ((cols + 127) / 128) > kMaxGridBlocks) return MXQ_ERR_SHAPE;
  return hip_status(mxq::launch_quant_nvfp4_2d(x, rows, cols, ld_x, gr, do_row ? q_row : nullptr, s_row,
                                               do_col ? q_colT : nullptr, s_colT, t, (uint32_t*)workspace, n_scopes,
                                               S(stream)));
}

mxq_status dequantize(mxq_format fmt, const void* q, const void* s, const float* t, mxq_scope t_scope,
                      int64_t group_rows, int64_t rows, int64_t cols, void* out, mxq_out_dtype out_dtype,
                      void* stream) {
  if (rows < 0 || cols < 0) return MXQ_ERR_SHAPE;
  if (fmt != MXQ_MXFP8 && fmt != MXQ_NVFP4 && fmt != MXQ_MXFP4) return MXQ_ERR_FORMAT;
  if (out_dtype != MXQ_OUT_BF16 && out_dtype != MXQ_OUT_F32) return MXQ_ERR_FORMAT;
  if (!q || !s || !out || (fmt == MXQ_NVFP4 && !t)) return MXQ_ERR_NULL;
  if ((fmt == MXQ_MXFP8 || fmt == MXQ_MXFP4) && cols % 32) return MXQ_ERR_SHAPE;
  if (fmt == MXQ_NVFP4 && cols % 16) return MXQ_ERR_SHAPE;
  int tm = 0;
  if (fmt == MXQ_NVFP4) {
    if (t_scope == MXQ_SCOPE_ROW) tm = 0;
    else if (t_scope == MXQ_SCOPE_TENSOR) tm = 1;
    else if (t_scope == MXQ_SCOPE_GROUP) {
      tm = 2;
      if (group_rows <= 0 || rows % group_rows) return MXQ_ERR_SHAPE;
    } else return MXQ_ERR_FORMAT;
  }
  if (!al16(q) || !al16(out)) return MXQ_ERR_ALIGN;
  if (rows == 0 || cols == 0) return MXQ_OK;
  return hip_status(mxq::launch_dequant((int)fmt, q, s, t, tm, group_rows, rows, cols, out,
                                        out_dtype == MXQ_OUT_F32, S(stream)));
}

mxq_status dequantize_transposed(mxq_format fmt, const void* q, const void* s, const float* t, mxq_scope t_scope,
                                 int64_t groups, int64_t group_rows, int64_t cols, const int32_t* src_row,
                                 int64_t out_cols, void* out_bf16, int64_t ld_out, void* stream) {
  if (groups < 0 || group_rows < 0 || cols < 0 || out_cols < 0) return MXQ_ERR_SHAPE;
  if (fmt != MXQ_MXFP8 && fmt != MXQ_NVFP4 && fmt != MXQ_BF16) return MXQ_ERR_FORMAT;
  if (!q || !out_bf16 || (fmt != MXQ_BF16 && !s) || (fmt == MXQ_NVFP4 && !t)) return MXQ_ERR_NULL;
  int tm = 0;
  if (fmt == MXQ_NVFP4) {
    if (t_scope == MXQ_SCOPE_ROW) tm = 0;
    else if (t_scope == MXQ_SCOPE_TENSOR) tm = 1;
    else if (t_scope == MXQ_SCOPE_GROUP) tm = 2;
    else return MXQ_ERR_FORMAT;
  }
  if (cols % (fmt == MXQ_MXFP8 ? 32 : 16)) return MXQ_ERR_SHAPE;
  if (!src_row && out_cols > group_rows) return MXQ_ERR_SHAPE;
  if (out_cols % 8 || ld_out < out_cols || ld_out % 8) return MXQ_ERR_SHAPE;
  if (groups > 65535 || (cols + 63) / 64 > 65535 || (out_cols + 63) / 64 > kMaxGridBlocks) return MXQ_ERR_SHAPE;
  if (!al16(q) || !al16(out_bf16)) return MXQ_ERR_ALIGN;
  if (groups == 0 || group_rows == 0 || cols == 0 || out_cols == 0) return MXQ_OK;
  return hip_status(mxq::launch_dequant_t((int)fmt, q, s, t, tm, groups, group_rows, cols, src_row, out_cols,
                                          out_bf16, ld_out, S(stream)));
}

static int scope_mode(mxq_scope sc) {
  return sc == MXQ_SCOPE_ROW ? 0 : sc == MXQ_SCOPE_TENSOR ? 1 : sc == MXQ_SCOPE_GROUP ? 2 : -1;
}

mxq_status gemm_block_scaled(mxq_format fmt, int64_t M, int64_t N, int64_t K, const void* A, const void* sA,
                             const float* tA, mxq_scope tA_scope, const void* B, const void* sB, const float* tB,
                             mxq_scope tB_scope, float* C, int64_t ldc, void* stream) {
  if (M < 0 || N < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (fmt != MXQ_MXFP8 && fmt != MXQ_NVFP4 && fmt != MXQ_BF16 && fmt != MXQ_MXFP4) return MXQ_ERR_FORMAT;
  if (!A || !B || !C) return MXQ_ERR_NULL;
  if (fmt != MXQ_BF16 && (!sA || !sB)) return MXQ_ERR_NULL;
  int ta = -1, tb = -1;
  if (fmt == MXQ_NVFP4) {
    if (!tA || !tB) return MXQ_ERR_NULL;
    ta = scope_mode(tA_scope);
    tb = scope_mode(tB_scope);
    if (ta != 0 && ta != 1) return MXQ_ERR_FORMAT;
    if (tb != 0 && tb != 1) return MXQ_ERR_FORMAT;
  }
  if (fmt != MXQ_BF16 && K % 32) return MXQ_ERR_SHAPE;
  if (fmt == MXQ_BF16 && K % 8) return MXQ_ERR_SHAPE;
  if (K > kMaxGemmK || ldc < N) return MXQ_ERR_SHAPE;
  if (!al16(A) || !al16(B) || !al4(C)) return MXQ_ERR_ALIGN;
  if (M == 0 || N == 0) return MXQ_OK;
  return hip_status(mxq::launch_gemm((int)fmt, M, N, K, A, sA, tA, ta, B, sB, tB, tb, C, ldc, S(stream)));
}

mxq_status gemm_block_scaled_batch(mxq_format fmt, const mxq_gemm_problem* problems, int count, void* stream) {
  if (count < 1 || count > MXQ_GEMM_BATCH_MAX) return MXQ_ERR_SHAPE;
  if (!problems) return MXQ_ERR_NULL;
  if (fmt != MXQ_MXFP8 && fmt != MXQ_NVFP4 && fmt != MXQ_BF16 && fmt != MXQ_MXFP4) return MXQ_ERR_FORMAT;
  int64_t M[MXQ_GEMM_BATCH_MAX], N[MXQ_GEMM_BATCH_MAX], K[MXQ_GEMM_BATCH_MAX], ldc[MXQ_GEMM_BATCH_MAX];
  const void *A[MXQ_GEMM_BATCH_MAX], *sA[MXQ_GEMM_BATCH_MAX], *B[MXQ_GEMM_BATCH_MAX], *sB[MXQ_GEMM_BATCH_MAX];
  const float *tA[MXQ_GEMM_BATCH_MAX], *tB[MXQ_GEMM_BATCH_MAX];
  int ta[MXQ_GEMM_BATCH_MAX], tb[MXQ_GEMM_BATCH_MAX];
  float* C[MXQ_GEMM_BATCH_MAX];
  int n = 0;
  for (int i = 0; i < count; ++i) {
    const mxq_gemm_problem& q = problems[i];
    if (q.M < 0 || q.N < 0 || q.K < 0) return MXQ_ERR_SHAPE;
    if (q.M == 0 || q.N == 0) continue;                       // empty problems are skipped
    if (!q.A || !q.B || !q.C) return MXQ_ERR_NULL;
    if (fmt != MXQ_BF16 && (!q.sA || !q.sB)) return MXQ_ERR_NULL;
    int a_mode = 0, b_mode = 0;
    if (fmt == MXQ_NVFP4) {
      if (!q.tA || !q.tB) return MXQ_ERR_NULL;
      a_mode = scope_mode(q.tA_scope);
      b_mode = scope_mode(q.tB_scope);
      if ((a_mode != 0 && a_mode != 1) || (b_mode != 0 && b_mode != 1)) return MXQ_ERR_FORMAT;
    }
    if (fmt != MXQ_BF16 && q.K % 32) return MXQ_ERR_SHAPE;
    if (fmt == MXQ_BF16 && q.K % 8) return MXQ_ERR_SHAPE;
    if (q.K > kMaxGemmK || q.ldc < q.N) return MXQ_ERR_SHAPE;
    if (!al16(q.A) || !al16(q.B) || !al4(q.C)) return MXQ_ERR_ALIGN;
    M[n] = q.M; N[n] = q.N; K[n] = q.K; ldc[n] = q.ldc;
    A[n] = q.A; sA[n] = q.sA; tA[n] = q.tA; ta[n] = a_mode;
    B[n] = q.B; sB[n] = q.sB; tB[n] = q.tB; tb[n] = b_mode;
    C[n] = q.C;
    ++n;
  }
  if (n == 0) return MXQ_OK;
  int64_t blocks = 0;
  for (int i = 0; i < n; ++i) blocks += ((M[i] + 127) / 128) * ((N[i] + 127) / 128) + 8;
  if (blocks > kMaxGridBlocks) return MXQ_ERR_SHAPE;
  return hip_status(mxq::launch_gemm_batch((int)fmt, n, M, N, K, A, sA, tA, ta, B, sB, tB, tb, C, ldc, S(stream)));
}

mxq_status gemm_fp8_blockwise(int64_t M, int64_t N, int64_t K, const void* A, const float* sA, const void* B,
                              const float* sB, int b_blocks, float* C, int64_t ldc, void* stream) {
  if (M < 0 || N < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (!A || !sA || !B || !sB || !C) return MXQ_ERR_NULL;
  if (b_blocks != 0 && b_blocks != 1) return MXQ_ERR_FORMAT;
  if (K % 128 || K > kMaxGemmK || ldc < N) return MXQ_ERR_SHAPE;
  if (!al16(A) || !al16(B) || !al4(sA) || !al4(sB) || !al4(C)) return MXQ_ERR_ALIGN;
  if (M == 0 || N == 0) return MXQ_OK;
  return hip_status(mxq::launch_gemm(5, M, N, K, A, sA, nullptr, 0, B, sB, nullptr, b_blocks, C, ldc, S(stream)));
}

mxq_status gemm_fp8_blockwise_batch(const mxq_fp8_block_problem* problems, int count, void* stream) {
  if (count < 1 || count > MXQ_GEMM_BATCH_MAX) return MXQ_ERR_SHAPE;
  if (!problems) return MXQ_ERR_NULL;
  int64_t M[MXQ_GEMM_BATCH_MAX], N[MXQ_GEMM_BATCH_MAX], K[MXQ_GEMM_BATCH_MAX], ldc[MXQ_GEMM_BATCH_MAX];
  const void *A[MXQ_GEMM_BATCH_MAX], *sA[MXQ_GEMM_BATCH_MAX], *B[MXQ_GEMM_BATCH_MAX], *sB[MXQ_GEMM_BATCH_MAX];
  const float* none[MXQ_GEMM_BATCH_MAX] = {};
  int ta[MXQ_GEMM_BATCH_MAX] = {}, tb[MXQ_GEMM_BATCH_MAX];
  float* C[MXQ_GEMM_BATCH_MAX];
  int n = 0;
  int64_t blocks = 0;
  for (int i = 0; i < count; ++i) {
    const mxq_fp8_block_problem& q = problems[i];
    if (q.M < 0 || q.N < 0 || q.K < 0) return MXQ_ERR_SHAPE;
    if (q.M == 0 || q.N == 0) continue;                       // empty problems are skipped
    if (!q.A || !q.sA || !q.B || !q.sB || !q.C) return MXQ_ERR_NULL;
    if (q.b_blocks != 0 && q.b_blocks != 1) return MXQ_ERR_FORMAT;
    if (q.K % 128 || q.K > kMaxGemmK || q.ldc < q.N) return MXQ_ERR_SHAPE;
    if (!al16(q.A) || !al16(q.B) || !al4(q.sA) || !al4(q.sB) || !al4(q.C)) return MXQ_ERR_ALIGN;
    blocks += ((q.M + 127) / 128 * ((q.N + 127) / 128) + 7) / 8 * 8;
    if (blocks > kMaxGridBlocks) return MXQ_ERR_SHAPE;
    M[n] = q.M; N[n] = q.N; K[n] = q.K; ldc[n] = q.ldc;
    A[n] = q.A; sA[n] = q.sA; B[n] = q.B; sB[n] = q.sB; tb[n] = q.b_blocks; C[n] = q.C;
    ++n;
  }
  if (n == 0) return MXQ_OK;
  return hip_status(mxq::launch_gemm_batch(5, n, M, N, K, A, sA, none, ta, B, sB, none, tb, C, ldc, S(stream)));
}

mxq_status gemm_mxfp8_matrix_core(int64_t M, int64_t N, int64_t K, const void* A, const void* sA, const void* B,
                                  const void* sB, float* C, int64_t ldc, void* stream) {
  if (M < 0 || N < 0 || K < 0) return MXQ_ERR_SHAPE;
  if (!A || !sA || !B || !sB || !C) return MXQ_ERR_NULL;
  if (K % 32 || K > kMaxGemmK || ldc < N) return MXQ_ERR_SHAPE;
  if (!al16(A) || !al16(B) || !al4(C)) return MXQ_ERR_ALIGN;
  if (M == 0 || N == 0) return MXQ_OK;
  return hip_status(mxq::launch_gemm(6, M, N, K, A, sA, nullptr, 0, B, sB, nullptr, 0, C, ldc, S(stream)));
}

}  // extern "C"

namespace {

// Host checks shared by both grouped entry points; on MXQ_OK, *empty says the call has
// no work and *ta / *tb hold the decode-scale modes.
mxq_status grouped_check(mxq_format fmt, int64_t groups, const int64_t* offsets, int vary_k, int64_t total,
                         int64_t M, int64_t N, int64_t K, const int32_t* a_row_index, int64_t a_rows, const void* A,
                         const void* sA, const float* tA, mxq_scope tA_scope, const void* B, const void* sB,
                         const float* tB, mxq_scope tB_scope, const float* C, bool* empty, int* ta, int* tb) {
  if (groups < 0 || total < 0 || M < 0 || N < 0 || K < 0 || a_rows < 0) return MXQ_ERR_SHAPE;
  if (fmt != MXQ_MXFP8 && fmt != MXQ_NVFP4 && fmt != MXQ_BF16 && fmt != MXQ_MXFP4 && fmt != MXQ_BF16_NVFP4T)
    return MXQ_ERR_FORMAT;
  if (vary_k != 0 && vary_k != 1 && vary_k != 2) return MXQ_ERR_FORMAT;
  if (vary_k == 2 && fmt != MXQ_BF16) return MXQ_ERR_FORMAT;   // K-major A: BF16 only
  if (fmt == MXQ_BF16_NVFP4T) {
    // BF16 A x the stacked NVFP4 weights (groups, K, N), read transposed, one scale per group
    if (vary_k || a_row_index) return MXQ_ERR_FORMAT;
    if (!offsets || !A || !B || !C) return MXQ_ERR_NULL;
    if (!sB || !tB) return MXQ_ERR_NULL;
    if (scope_mode(tB_scope) != 2) return MXQ_ERR_FORMAT;
    if (K % 8 || N % 16 || K > kMaxGemmK) return MXQ_ERR_SHAPE;
    if (K * (N / 2) > 0x7FFFFFFF) return MXQ_ERR_SHAPE;  // one weight's bytes: 32-bit buffer offsets
    if (!al16(A) || !al16(B) || !al4(C)) return MXQ_ERR_ALIGN;
    *ta = -1;
    *tb = 2;
    *empty = groups == 0 || N == 0 || total == 0;
    return MXQ_OK;
  }
  if (vary_k && fmt == MXQ_NVFP4) return MXQ_ERR_FORMAT;
  if (vary_k && a_row_index) return MXQ_ERR_FORMAT;
  if (!offsets || !A || !B || !C) return MXQ_ERR_NULL;
  if (fmt != MXQ_BF16 && (!sA || !sB)) return MXQ_ERR_NULL;
  *ta = -1;
  *tb = -1;
  if (fmt == MXQ_NVFP4) {
    if (!tA || !tB) return MXQ_ERR_NULL;
    *ta = scope_mode(tA_scope);
    *tb = scope_mode(tB_scope);
    if (*ta != 0 && *ta != 1) return MXQ_ERR_FORMAT;
    if (*tb != 0 && *tb != 2) return MXQ_ERR_FORMAT;    // per B row, or per group (expert)
  }
  if (!vary_k) {
    if (fmt != MXQ_BF16 && K % 32) return MXQ_ERR_SHAPE;
    if (fmt == MXQ_BF16 && K % 8) return MXQ_ERR_SHAPE;
    if (K > kMaxGemmK) return MXQ_ERR_SHAPE;
    if (a_row_index && a_rows * gemm_row_bytes(fmt, K) > 0x7FFFFFFF) return MXQ_ERR_SHAPE;
  } else {
    if (total % ((fmt == MXQ_MXFP8 || fmt == MXQ_MXFP4) ? 32 : 8)) return MXQ_ERR_SHAPE;
    if (total > kMaxGemmK) return MXQ_ERR_SHAPE;
    if (vary_k == 2 && M % 8) return MXQ_ERR_SHAPE;            // 16-byte rows of the K-major A
  }
  if (!al16(A) || !al16(B) || !al4(C)) return MXQ_ERR_ALIGN;
  *empty = groups == 0 || N == 0 || (vary_k ? M == 0 : total == 0);
  return MXQ_OK;
}

// Scratch of grouped_gemm_block_scaled_noalloc: the device-side tile prefix ((groups + 1)
// int64, fully rewritten by every call before any tile reads it) lives in this
// file-scope device array instead of a caller workspace. Each GPU the library runs on
// holds its own copy until the process ends. In host code `scratch` names a host-side
// stand-in, never the device memory: its device address is looked up once per device
// (hipGetSymbolAddress with that device current) and only that address is passed on.
constexpr int64_t kNoAllocMaxGroups = MXQ_NOALLOC_MAX_GROUPS;
__device__ __align__(256) int64_t scratch[kNoAllocMaxGroups + 1];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on the first call on that device).
mxq_status current_device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MXQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MXQ_ERR_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MXQ_OK;
}

}  // namespace

extern "C" {

mxq_status grouped_gemm_block_scaled(mxq_format fmt, int64_t groups, const int64_t* offsets, int vary_k,
                                     int64_t total, int64_t M, int64_t N, int64_t K, const int32_t* a_row_index,
                                     int64_t a_rows, const void* A, const void* sA, const float* tA, mxq_scope tA_scope,
                                     const void* B, const void* sB, const float* tB, mxq_scope tB_scope, float* C,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  int ta = -1, tb = -1;
  const mxq_status st = grouped_check(fmt, groups, offsets, vary_k, total, M, N, K, a_row_index, a_rows, A, sA, tA,
                                      tA_scope, B, sB, tB, tB_scope, C, &empty, &ta, &tb);
  if (st != MXQ_OK || empty) return st;
  if (!workspace || workspace_bytes < mxq::grouped_gemm_ws_bytes(groups)) return MXQ_ERR_WORKSPACE;
  if (!al16(workspace)) return MXQ_ERR_ALIGN;
  return hip_status(mxq::launch_grouped_gemm(fmt == MXQ_BF16_NVFP4T ? 7 : (int)fmt, groups, offsets, vary_k, total,
                                             M, N, K, a_row_index, a_row_index ? a_rows : total, A, sA,
                                             tA, ta, B, sB, tB, tb, C, workspace, S(stream)));
}

mxq_status grouped_gemm_block_scaled_noalloc(mxq_format fmt, int64_t groups, const int64_t* offsets, int vary_k,
                                             int64_t total, int64_t M, int64_t N, int64_t K,
                                             const int32_t* a_row_index, int64_t a_rows, const void* A,
                                             const void* sA, const float* tA, mxq_scope tA_scope, const void* B,
                                             const void* sB, const float* tB, mxq_scope tB_scope, float* C,
                                             void* stream) {
  bool empty = false;
  int ta = -1, tb = -1;
  const mxq_status st = grouped_check(fmt, groups, offsets, vary_k, total, M, N, K, a_row_index, a_rows, A, sA, tA,
                                      tA_scope, B, sB, tB, tB_scope, C, &empty, &ta, &tb);
  if (st != MXQ_OK) return st;
  if (groups > kNoAllocMaxGroups) return MXQ_ERR_WORKSPACE;      // beyond the static scratch
  if (empty) return MXQ_OK;
  void* ws = nullptr;
  const mxq_status ss = current_device_scratch(&ws);
  if (ss != MXQ_OK) return ss;
  return hip_status(mxq::launch_grouped_gemm(fmt == MXQ_BF16_NVFP4T ? 7 : (int)fmt, groups, offsets, vary_k, total,
                                             M, N, K, a_row_index, a_row_index ? a_rows : total, A, sA,
                                             tA, ta, B, sB, tB, tb, C, ws, S(stream)));
}

mxq_status moe_swiglu_quantize_nvfp4(const float* gate_up, int64_t rows, int64_t inter, void* h_bf16, void* q,
                                     void* s, float* t, void* stream) {
  if (rows < 0 || inter < 0) return MXQ_ERR_SHAPE;
  if (!gate_up || !q || !s || !t) return MXQ_ERR_NULL;
  if (inter % 16 || inter > kMaxRowCols) return MXQ_ERR_SHAPE;
  if (!al16(gate_up) || !al4(q) || (h_bf16 && !al16(h_bf16)) || !al4(t)) return MXQ_ERR_ALIGN;
  if (rows == 0 || inter == 0) return MXQ_OK;
  return hip_status(mxq::launch_swiglu_nvfp4(gate_up, rows, inter, h_bf16, q, s, t, S(stream)));
}

mxq_status moe_combine(const float* o_slots, int64_t total_slots, int64_t tokens, int64_t topk, int64_t hidden,
                       const int64_t* slot_of, const float* weights, float* y, void* stream) {
  if (tokens < 0 || topk < 0 || hidden < 0 || total_slots < 0) return MXQ_ERR_SHAPE;
  if (!o_slots || !slot_of || !weights || !y) return MXQ_ERR_NULL;
  if (hidden % 4) return MXQ_ERR_SHAPE;
  if (!al16(o_slots) || !al16(y)) return MXQ_ERR_ALIGN;
  if (tokens == 0 || hidden == 0) return MXQ_OK;
  if (tokens > kMaxGridBlocks) return MXQ_ERR_SHAPE;
  return hip_status(mxq::launch_combine(o_slots, total_slots, tokens, topk, hidden, slot_of, weights, y, S(stream)));
}

}  // extern "C"
