// C ABI of the QoQ W4A8 library: argument validation, then launches on the
// caller's stream.  Declarations and the contract of every entry point are in
// include/qoq.h.
#include "../../include/qoq.h"

#include <hip/hip_runtime_api.h>

#include "qoq_internal.h"

namespace {

constexpr int64_t kMaxK = 139648;   // largest multiple of 128 with 127*121*K < 2^31
constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

// shape rules shared by the weight and GEMM calls; group 0 = per-channel weights
// (accepted by the calls that document it)
int check_nk(int64_t N, int64_t K, int32_t group, bool allow_pc = false) {
  if (group != 128 && !(allow_pc && group == 0)) return QOQ_ERR_UNSUPPORTED;
  if (N <= 0 || K <= 0 || N % 16 != 0 || K % 128 != 0) return QOQ_ERR_INVALID;
  if (K > kMaxK) return QOQ_ERR_UNSUPPORTED;
  if (N > kMaxDim || N * K / 2 > kMaxDim * 8) return QOQ_ERR_UNSUPPORTED;
  return QOQ_OK;
}

int check_gemm(int64_t M, int64_t N, int64_t K, int32_t group, bool allow_pc = false) {
  int st = check_nk(N, K, group, allow_pc);
  if (st != QOQ_OK) return st;
  if (M < 0) return QOQ_ERR_INVALID;
  if (M > kMaxDim) return QOQ_ERR_UNSUPPORTED;
  // row / column indices are 32-bit inside the kernels; element offsets are 64-bit
  if ((M + 63) / 64 > 65535) return QOQ_ERR_UNSUPPORTED;
  return QOQ_OK;
}

}  // namespace

extern "C" {

int qoq_version(void) { return 2; }

const char *qoq_status_string(int status) {
  switch (status) {
    case QOQ_OK: return "ok";
    case QOQ_ERR_INVALID: return "invalid argument (null pointer or shape not allowed)";
    case QOQ_ERR_UNSUPPORTED: return "unsupported configuration (group not allowed here or size beyond limits)";
    case QOQ_ERR_ALIGNMENT: return "pointer alignment requirement not met";
    case QOQ_ERR_WORKSPACE: return "workspace smaller than required";
    case QOQ_ERR_HIP: return "HIP runtime error at launch";
    case QOQ_ERR_SCRATCH: return "shape needs more scratch than the static array holds (QOQ_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int qoq_weight_buffer_sizes(int64_t N, int64_t K, int32_t group, size_t *packed_w_bytes,
                            size_t *group_meta_bytes, size_t *s_w_bytes) {
  int st = check_nk(N, K, group, true);
  if (st != QOQ_OK) return st;
  if (packed_w_bytes) *packed_w_bytes = static_cast<size_t>(N) * static_cast<size_t>(K) / 2;
  if (group_meta_bytes)
    *group_meta_bytes = group == 0 ? static_cast<size_t>(N) : static_cast<size_t>(N) * static_cast<size_t>(K / 128) * 2;
  if (s_w_bytes) *s_w_bytes = static_cast<size_t>(N) * 2;
  return QOQ_OK;
}

int qoq_quantize_pack_weights(const void *w_fp16, int64_t N, int64_t K, int32_t group, void *packed_w,
                              void *group_meta, void *s_w_fp16, void *stream) {
  int st = check_nk(N, K, group, true);
  if (st != QOQ_OK) return st;
  if (!w_fp16 || !packed_w || !group_meta || !s_w_fp16) return QOQ_ERR_INVALID;
  if (!aligned(w_fp16, 16) || !aligned(packed_w, 16) || !aligned(group_meta, group == 0 ? 1 : 2) ||
      !aligned(s_w_fp16, 2))
    return QOQ_ERR_ALIGNMENT;
  if (group == 0)
    qoq::launch_quantize_pack_weights_pc(w_fp16, N, K, packed_w, group_meta, s_w_fp16, as_stream(stream));
  else
    qoq::launch_quantize_pack_weights(w_fp16, N, K, packed_w, group_meta, s_w_fp16, as_stream(stream));
  return launch_status();
}

int qoq_quantize_activations(const void *x_fp16, int64_t M, int64_t K, void *qx_i8, void *s_x_fp16,
                             void *stream) {
  if (M < 0 || K <= 0 || K % 8 != 0) return QOQ_ERR_INVALID;
  if (M > kMaxDim || K > kMaxDim / 2) return QOQ_ERR_UNSUPPORTED;
  if (M == 0) return QOQ_OK;
  if (!x_fp16 || !qx_i8 || !s_x_fp16) return QOQ_ERR_INVALID;
  if (!aligned(x_fp16, 16) || !aligned(qx_i8, 16) || !aligned(s_x_fp16, 2)) return QOQ_ERR_ALIGNMENT;
  qoq::launch_quantize_activations(x_fp16, M, K, qx_i8, s_x_fp16, as_stream(stream));
  return launch_status();
}

int qoq_quantize_activations_rowsum(const void *x_fp16, int64_t M, int64_t K, void *qx_i8, void *s_x_fp16,
                                    int32_t *t_x, void *stream) {
  if (M < 0 || K <= 0 || K % 8 != 0) return QOQ_ERR_INVALID;
  if (M > kMaxDim || K > kMaxDim / 2) return QOQ_ERR_UNSUPPORTED;
  if (M == 0) return QOQ_OK;
  if (!x_fp16 || !qx_i8 || !s_x_fp16 || !t_x) return QOQ_ERR_INVALID;
  if (!aligned(x_fp16, 16) || !aligned(qx_i8, 16) || !aligned(s_x_fp16, 2) || !aligned(t_x, 4))
    return QOQ_ERR_ALIGNMENT;
  qoq::launch_quantize_activations_rowsum(x_fp16, M, K, qx_i8, s_x_fp16, t_x, as_stream(stream));
  return launch_status();
}

int qoq_quantize_activations_tiled(const void *x_fp16, int64_t M, int64_t K, void *qx_tiled, void *s_x_fp16,
                                   void *stream) {
  if (M < 0 || K <= 0 || K % 64 != 0) return QOQ_ERR_INVALID;
  if (M > qoq::kTiledMaxM || K > kMaxDim / 2) return QOQ_ERR_UNSUPPORTED;
  if (M == 0) return QOQ_OK;
  if (!x_fp16 || !qx_tiled || !s_x_fp16) return QOQ_ERR_INVALID;
  if (!aligned(x_fp16, 16) || !aligned(qx_tiled, 16) || !aligned(s_x_fp16, 2)) return QOQ_ERR_ALIGNMENT;
  qoq::launch_quantize_activations_tiled(x_fp16, M, K, qx_tiled, s_x_fp16, as_stream(stream));
  return launch_status();
}

int qoq_quantize_activations_rowsum_tiled(const void *x_fp16, int64_t M, int64_t K, void *qx_tiled,
                                          void *s_x_fp16, int32_t *t_x, void *stream) {
  if (M < 0 || K <= 0 || K % 64 != 0) return QOQ_ERR_INVALID;
  if (M > qoq::kTiledMaxM || K > kMaxDim / 2) return QOQ_ERR_UNSUPPORTED;
  if (M == 0) return QOQ_OK;
  if (!x_fp16 || !qx_tiled || !s_x_fp16 || !t_x) return QOQ_ERR_INVALID;
  if (!aligned(x_fp16, 16) || !aligned(qx_tiled, 16) || !aligned(s_x_fp16, 2) || !aligned(t_x, 4))
    return QOQ_ERR_ALIGNMENT;
  qoq::launch_quantize_activations_rowsum_tiled(x_fp16, M, K, qx_tiled, s_x_fp16, t_x, as_stream(stream));
  return launch_status();
}

static int fused_common_checks(int64_t M, int64_t K, int32_t layout, const void *qx, const void *s_x,
                               const int32_t *t_x) {
  if (M < 0 || K <= 0 || K % 8 != 0 || (layout != 0 && layout != 1)) return QOQ_ERR_INVALID;
  if (layout == 1 && K % 64 != 0) return QOQ_ERR_INVALID;
  if (K > qoq::kFusedMaxK || M > kMaxDim || (layout == 1 && M > qoq::kTiledMaxM)) return QOQ_ERR_UNSUPPORTED;
  if (M == 0) return QOQ_OK;
  if (!qx || !s_x) return QOQ_ERR_INVALID;
  if (!aligned(qx, 16) || !aligned(s_x, 2) || (t_x && !aligned(t_x, 4))) return QOQ_ERR_ALIGNMENT;
  return 1;   // proceed
}

int qoq_rmsnorm_quantize(const void *x_fp16, const void *gamma_fp16, float eps, int64_t M, int64_t K,
                         int32_t layout, void *qx, void *s_x_fp16, int32_t *t_x, void *stream) {
  if (!(eps > 0.0f) || eps > 1.0e30f) return QOQ_ERR_INVALID;
  const int st = fused_common_checks(M, K, layout, qx, s_x_fp16, t_x);
  if (st != 1) return st;
  if (!x_fp16 || !gamma_fp16) return QOQ_ERR_INVALID;
  if (!aligned(x_fp16, 16) || !aligned(gamma_fp16, 16)) return QOQ_ERR_ALIGNMENT;
  qoq::launch_rmsnorm_quantize(x_fp16, gamma_fp16, eps, M, K, layout, qx, s_x_fp16, t_x, as_stream(stream));
  return launch_status();
}

int qoq_silu_mul_quantize(const void *gate_fp16, const void *up_fp16, int64_t ld, int64_t M, int64_t K,
                          int32_t layout, void *qx, void *s_x_fp16, int32_t *t_x, void *stream) {
  if (ld < K || ld % 8 != 0) return QOQ_ERR_INVALID;
  const int st = fused_common_checks(M, K, layout, qx, s_x_fp16, t_x);
  if (st != 1) return st;
  if (!gate_fp16 || !up_fp16) return QOQ_ERR_INVALID;
  if (ld > kMaxDim) return QOQ_ERR_UNSUPPORTED;
  if (!aligned(gate_fp16, 16) || !aligned(up_fp16, 16)) return QOQ_ERR_ALIGNMENT;
  qoq::launch_silu_mul_quantize(gate_fp16, up_fp16, ld, M, K, layout, qx, s_x_fp16, t_x, as_stream(stream));
  return launch_status();
}

int qoq_rmsnorm(const void *x_fp16, const void *gamma_fp16, float eps, int64_t M, int64_t K, void *y_fp16,
                void *stream) {
  if (!(eps > 0.0f) || eps > 1.0e30f || M < 0 || K <= 0 || K % 8 != 0) return QOQ_ERR_INVALID;
  if (K > qoq::kFusedMaxK || M > kMaxDim) return QOQ_ERR_UNSUPPORTED;
  if (M == 0) return QOQ_OK;
  if (!x_fp16 || !gamma_fp16 || !y_fp16) return QOQ_ERR_INVALID;
  if (!aligned(x_fp16, 16) || !aligned(gamma_fp16, 16) || !aligned(y_fp16, 16)) return QOQ_ERR_ALIGNMENT;
  qoq::launch_rmsnorm_quantize(x_fp16, gamma_fp16, eps, M, K, -1, y_fp16, nullptr, nullptr, as_stream(stream));
  return launch_status();
}

int qoq_silu_mul_quantize_workspace_bytes(int64_t M, int64_t K, size_t *bytes) {
  if (M < 0 || K <= 0 || K % 8 != 0 || !bytes) return QOQ_ERR_INVALID;
  if (K > qoq::kFusedMaxK || M > kMaxDim) return QOQ_ERR_UNSUPPORTED;
  *bytes = qoq::silu_split_workspace(M, K);
  return QOQ_OK;
}

int qoq_silu_mul_quantize_ws(const void *gate_fp16, const void *up_fp16, int64_t ld, int64_t M, int64_t K,
                             int32_t layout, void *qx, void *s_x_fp16, void *workspace, size_t workspace_bytes,
                             void *stream) {
  if (ld < K || ld % 8 != 0) return QOQ_ERR_INVALID;
  const int st = fused_common_checks(M, K, layout, qx, s_x_fp16, nullptr);
  if (st != 1) return st;
  if (!gate_fp16 || !up_fp16) return QOQ_ERR_INVALID;
  if (ld > kMaxDim) return QOQ_ERR_UNSUPPORTED;
  if (!aligned(gate_fp16, 16) || !aligned(up_fp16, 16)) return QOQ_ERR_ALIGNMENT;
  const size_t need = qoq::silu_split_workspace(M, K);
  if (need == 0) {                                  // one pass, as qoq_silu_mul_quantize
    qoq::launch_silu_mul_quantize(gate_fp16, up_fp16, ld, M, K, layout, qx, s_x_fp16, nullptr, as_stream(stream));
    return launch_status();
  }
  if (!workspace || workspace_bytes < need) return QOQ_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return QOQ_ERR_ALIGNMENT;
  qoq::launch_silu_mul_quantize_split(gate_fp16, up_fp16, ld, M, K, layout == 1, qx, s_x_fp16, workspace,
                                      as_stream(stream));
  return launch_status();
}

int qoq_silu_mul(const void *gate_fp16, const void *up_fp16, int64_t ld, int64_t M, int64_t K, void *h_fp16,
                 void *stream) {
  if (M < 0 || K <= 0 || K % 8 != 0 || ld < K || ld % 8 != 0) return QOQ_ERR_INVALID;
  if (K > qoq::kFusedMaxK || M > kMaxDim || ld > kMaxDim) return QOQ_ERR_UNSUPPORTED;
  if (M == 0) return QOQ_OK;
  if (!gate_fp16 || !up_fp16 || !h_fp16) return QOQ_ERR_INVALID;
  if (!aligned(gate_fp16, 16) || !aligned(up_fp16, 16) || !aligned(h_fp16, 16)) return QOQ_ERR_ALIGNMENT;
  qoq::launch_silu_mul_quantize(gate_fp16, up_fp16, ld, M, K, -1, h_fp16, nullptr, nullptr, as_stream(stream));
  return launch_status();
}

int qoq_kv4_page_bytes(int64_t h_kv, int64_t head_dim, size_t *bytes) {
  if (h_kv <= 0 || !bytes) return QOQ_ERR_INVALID;
  if (head_dim != 128 || h_kv > 1024) return QOQ_ERR_UNSUPPORTED;
  *bytes = static_cast<size_t>(h_kv) * qoq::kKv4PageBytes;
  return QOQ_OK;
}

int qoq_kv4_write(const void *k_new, const void *v_new, int64_t B, int64_t n_new, int64_t h_kv, int64_t head_dim,
                  const int32_t *positions, const int32_t *page_table, int64_t max_pages, void *kv_pool,
                  int64_t num_pages, void *stream) {
  if (B < 0 || n_new < 0 || h_kv <= 0 || max_pages <= 0 || num_pages <= 0) return QOQ_ERR_INVALID;
  if (num_pages > INT32_MAX || max_pages > (int64_t{1} << 24)) return QOQ_ERR_UNSUPPORTED;
  if (head_dim != 128 || h_kv > 1024 || B > 65535 || n_new > (int64_t{1} << 19)) return QOQ_ERR_UNSUPPORTED;
  if (B == 0 || n_new == 0) return QOQ_OK;
  if (!k_new || !v_new || !positions || !page_table || !kv_pool) return QOQ_ERR_INVALID;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(positions, 4) || !aligned(page_table, 4) ||
      !aligned(kv_pool, 16))
    return QOQ_ERR_ALIGNMENT;
  qoq::launch_kv4_write(k_new, v_new, B, n_new, h_kv, positions, page_table, max_pages, num_pages, kv_pool,
                        as_stream(stream));
  return launch_status();
}

int qoq_smooth_attention_lambda(const void *k_samples, int64_t n, int64_t h_kv, int64_t head_dim, float alpha,
                                void *lambda_f32, void *stream) {
  if (n < 1 || h_kv < 1 || !(alpha >= 0.0f && alpha <= 1.0f)) return QOQ_ERR_INVALID;
  if (head_dim != 128 || h_kv > 65535 || n > (int64_t{1} << 30) / h_kv) return QOQ_ERR_UNSUPPORTED;
  if (!k_samples || !lambda_f32) return QOQ_ERR_INVALID;
  if (!aligned(k_samples, 2) || !aligned(lambda_f32, 4)) return QOQ_ERR_ALIGNMENT;
  qoq::launch_smooth_lambda(k_samples, n, h_kv, alpha, lambda_f32, as_stream(stream));
  return launch_status();
}

int qoq_smooth_attention_fold(const void *w_q, const void *w_k, const void *lambda_f32, int64_t h, int64_t h_kv,
                              int64_t head_dim, int64_t d_model, void *w_q_out, void *w_k_out, void *stream) {
  if (h < 1 || h_kv < 1 || d_model < 1 || h % h_kv != 0) return QOQ_ERR_INVALID;
  if (head_dim != 128 || h > 4096 || d_model > (int64_t{1} << 20)) return QOQ_ERR_UNSUPPORTED;
  if (!w_q || !w_k || !lambda_f32 || !w_q_out || !w_k_out) return QOQ_ERR_INVALID;
  if (!aligned(w_q, 2) || !aligned(w_k, 2) || !aligned(lambda_f32, 4) || !aligned(w_q_out, 2) ||
      !aligned(w_k_out, 2))
    return QOQ_ERR_ALIGNMENT;
  qoq::launch_smooth_fold(w_q, w_k, lambda_f32, h, h_kv, d_model, w_q_out, w_k_out, as_stream(stream));
  return launch_status();
}

static int kv4_attn_checks(int64_t B, int64_t h, int64_t h_kv, int64_t head_dim, int64_t max_len, int64_t max_pages) {
  if (B < 0 || h <= 0 || h_kv <= 0 || max_len <= 0 || max_pages <= 0 || h % h_kv != 0) return QOQ_ERR_INVALID;
  if (head_dim != 128 || h / h_kv > 16 || B > 65535 || h_kv > 1024) return QOQ_ERR_UNSUPPORTED;
  if (max_pages > (int64_t{1} << 24)) return QOQ_ERR_UNSUPPORTED;
  if (max_len > max_pages * qoq::kKv4PageTokens) return QOQ_ERR_INVALID;
  return QOQ_OK;
}

int qoq_kv4_attention_workspace_bytes(int64_t B, int64_t h, int64_t h_kv, int64_t head_dim, int64_t max_len,
                                      size_t *bytes) {
  const int st = kv4_attn_checks(B, h, h_kv, head_dim, max_len, (max_len + qoq::kKv4PageTokens - 1) /
                                                                   qoq::kKv4PageTokens);
  if (st != QOQ_OK) return st;
  if (!bytes) return QOQ_ERR_INVALID;
  *bytes = B == 0 ? 0 : qoq::kv4_workspace_need(B, h, h_kv, max_len);
  return QOQ_OK;
}

int qoq_kv4_decode_attention(const void *q, const void *kv_pool, int64_t num_pages, const int32_t *page_table,
                             int64_t max_pages, const int32_t *seq_lens, int64_t B, int64_t h, int64_t h_kv,
                             int64_t head_dim, int64_t max_len, void *out, void *workspace, size_t workspace_bytes,
                             void *stream) {
  const int st = kv4_attn_checks(B, h, h_kv, head_dim, max_len, max_pages);
  if (st != QOQ_OK) return st;
  if (num_pages <= 0) return QOQ_ERR_INVALID;
  if (num_pages > INT32_MAX) return QOQ_ERR_UNSUPPORTED;
  if (B == 0) return QOQ_OK;
  if (!q || !kv_pool || !page_table || !seq_lens || !out) return QOQ_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(kv_pool, 16) || !aligned(page_table, 4) || !aligned(seq_lens, 4) ||
      !aligned(out, 16))
    return QOQ_ERR_ALIGNMENT;
  const size_t need = qoq::kv4_workspace_need(B, h, h_kv, max_len);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return QOQ_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return QOQ_ERR_ALIGNMENT;
  }
  qoq::launch_kv4_attention(q, kv_pool, num_pages, page_table, max_pages, seq_lens, B, h, h_kv, max_len, out,
                            workspace, as_stream(stream));
  return launch_status();
}

static int gemm_tiled_common(const void *qx_tiled, const void *s_x_fp16, const void *packed_w,
                             const void *group_meta, const void *s_w_fp16, void *out, int out_kind, int64_t M,
                             int64_t N, int64_t K, void *stream) {
  int st = check_gemm(M, N, K, 128);
  if (st != QOQ_OK) return st;
  if (M > qoq::kTiledMaxM) return QOQ_ERR_UNSUPPORTED;
  if (M == 0) return QOQ_OK;
  if (!qx_tiled || !packed_w || !group_meta || !out) return QOQ_ERR_INVALID;
  if (out_kind == 0 && (!s_x_fp16 || !s_w_fp16)) return QOQ_ERR_INVALID;
  if (!aligned(qx_tiled, 16) || !aligned(packed_w, 16) || !aligned(group_meta, 16) || !aligned(out, 16))
    return QOQ_ERR_ALIGNMENT;
  if (out_kind == 0 && (!aligned(s_x_fp16, 2) || !aligned(s_w_fp16, 2))) return QOQ_ERR_ALIGNMENT;
  qoq::launch_w4a8_gemm_tiled(qx_tiled, s_x_fp16, packed_w, group_meta, s_w_fp16, out, out_kind, M, N, K,
                              as_stream(stream));
  return launch_status();
}

int qoq_w4a8_gemm_tiled(const void *qx_tiled, const void *s_x_fp16, const void *packed_w, const void *group_meta,
                        const void *s_w_fp16, void *out_fp16, int64_t M, int64_t N, int64_t K, void *stream) {
  return gemm_tiled_common(qx_tiled, s_x_fp16, packed_w, group_meta, s_w_fp16, out_fp16, 0, M, N, K, stream);
}

int qoq_w4a8_gemm_tiled_i32(const void *qx_tiled, const void *packed_w, const void *group_meta, int32_t *acc_i32,
                            int64_t M, int64_t N, int64_t K, void *stream) {
  return gemm_tiled_common(qx_tiled, nullptr, packed_w, group_meta, nullptr, acc_i32, 1, M, N, K, stream);
}

const char *qoq_gemm_tiled_plan(int64_t M, int64_t N, int64_t K) {
  if (check_gemm(M, N, K, 128) != QOQ_OK || M == 0 || M > qoq::kTiledMaxM) return "invalid";
  return qoq::gemm_tiled_plan_name(M, N, K);
}

static int gemm_pc_tiled_common(const void *qx_tiled, const void *s_x_fp16, const int32_t *t_x,
                                const void *packed_w, const void *zeros, const void *s_w_fp16, void *out,
                                int out_kind, int64_t M, int64_t N, int64_t K, void *stream) {
  int st = check_gemm(M, N, K, 128);
  if (st != QOQ_OK) return st;
  if (M > qoq::kTiledMaxM) return QOQ_ERR_UNSUPPORTED;
  if (M == 0) return QOQ_OK;
  if (!qx_tiled || !t_x || !packed_w || !zeros || !out) return QOQ_ERR_INVALID;
  if (out_kind == 0 && (!s_x_fp16 || !s_w_fp16)) return QOQ_ERR_INVALID;
  if (!aligned(qx_tiled, 16) || !aligned(packed_w, 16) || !aligned(out, 16) || !aligned(t_x, 4))
    return QOQ_ERR_ALIGNMENT;
  if (out_kind == 0 && (!aligned(s_x_fp16, 2) || !aligned(s_w_fp16, 2))) return QOQ_ERR_ALIGNMENT;
  qoq::launch_w4a8_gemm_pc_tiled(qx_tiled, s_x_fp16, t_x, packed_w, zeros, s_w_fp16, out, out_kind, M, N, K,
                                 as_stream(stream));
  return launch_status();
}

int qoq_w4a8_gemm_pc_tiled(const void *qx_tiled, const void *s_x_fp16, const int32_t *t_x, const void *packed_w,
                           const void *zeros, const void *s_w_fp16, void *out_fp16, int64_t M, int64_t N, int64_t K,
                           void *stream) {
  return gemm_pc_tiled_common(qx_tiled, s_x_fp16, t_x, packed_w, zeros, s_w_fp16, out_fp16, 0, M, N, K, stream);
}

int qoq_w4a8_gemm_pc_tiled_i32(const void *qx_tiled, const int32_t *t_x, const void *packed_w, const void *zeros,
                               int32_t *acc_i32, int64_t M, int64_t N, int64_t K, void *stream) {
  return gemm_pc_tiled_common(qx_tiled, nullptr, t_x, packed_w, zeros, nullptr, acc_i32, 1, M, N, K, stream);
}

static int gemm_pc_common(const void *qx_i8, const void *s_x_fp16, const int32_t *t_x, const void *packed_w,
                          const void *zeros, const void *s_w_fp16, void *out, int out_kind, int64_t M, int64_t N,
                          int64_t K, void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_gemm(M, N, K, 128);
  if (st != QOQ_OK) return st;
  if (M == 0) return QOQ_OK;
  if (!qx_i8 || !t_x || !packed_w || !zeros || !out) return QOQ_ERR_INVALID;
  if (out_kind == 0 && (!s_x_fp16 || !s_w_fp16)) return QOQ_ERR_INVALID;
  if (!aligned(qx_i8, 16) || !aligned(packed_w, 16) || !aligned(out, 16) || !aligned(t_x, 4))
    return QOQ_ERR_ALIGNMENT;
  if (out_kind == 0 && (!aligned(s_x_fp16, 2) || !aligned(s_w_fp16, 2))) return QOQ_ERR_ALIGNMENT;
  const size_t need = qoq::gemm_workspace_need(M, N, K);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return QOQ_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return QOQ_ERR_ALIGNMENT;
  }
  qoq::launch_w4a8_gemm_pc(qx_i8, s_x_fp16, t_x, packed_w, zeros, s_w_fp16, out, out_kind, M, N, K, workspace,
                           as_stream(stream));
  return launch_status();
}

int qoq_w4a8_gemm_pc(const void *qx_i8, const void *s_x_fp16, const int32_t *t_x, const void *packed_w,
                     const void *zeros, const void *s_w_fp16, void *out_fp16, int64_t M, int64_t N, int64_t K,
                     void *workspace, size_t workspace_bytes, void *stream) {
  return gemm_pc_common(qx_i8, s_x_fp16, t_x, packed_w, zeros, s_w_fp16, out_fp16, 0, M, N, K, workspace,
                        workspace_bytes, stream);
}

int qoq_w4a8_gemm_pc_i32(const void *qx_i8, const int32_t *t_x, const void *packed_w, const void *zeros,
                         int32_t *acc_i32, int64_t M, int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                         void *stream) {
  return gemm_pc_common(qx_i8, nullptr, t_x, packed_w, zeros, nullptr, acc_i32, 1, M, N, K, workspace,
                        workspace_bytes, stream);
}

int qoq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group, size_t *bytes) {
  int st = check_gemm(M, N, K, group, true);
  if (st != QOQ_OK) return st;
  if (!bytes) return QOQ_ERR_INVALID;
  *bytes = M == 0 ? 0 : qoq::gemm_workspace_need(M, N, K);
  return QOQ_OK;
}

static int gemm_common(const void *qx_i8, const void *s_x_fp16, const void *packed_w, const void *group_meta,
                       const void *s_w_fp16, void *out, int out_kind, int64_t M, int64_t N, int64_t K,
                       int32_t group, void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_gemm(M, N, K, group);
  if (st != QOQ_OK) return st;
  if (M == 0) return QOQ_OK;
  if (!qx_i8 || !packed_w || !group_meta || !out) return QOQ_ERR_INVALID;
  if (out_kind == 0 && (!s_x_fp16 || !s_w_fp16)) return QOQ_ERR_INVALID;
  if (!aligned(qx_i8, 16) || !aligned(packed_w, 16) || !aligned(group_meta, 16) || !aligned(out, 16))
    return QOQ_ERR_ALIGNMENT;
  if (out_kind == 0 && (!aligned(s_x_fp16, 2) || !aligned(s_w_fp16, 2))) return QOQ_ERR_ALIGNMENT;
  const size_t need = qoq::gemm_workspace_need(M, N, K);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return QOQ_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return QOQ_ERR_ALIGNMENT;
  }
  qoq::launch_w4a8_gemm(qx_i8, s_x_fp16, packed_w, group_meta, s_w_fp16, out, out_kind, M, N, K, workspace,
                        as_stream(stream));
  return launch_status();
}

int qoq_w4a8_gemm(const void *qx_i8, const void *s_x_fp16, const void *packed_w, const void *group_meta,
                  const void *s_w_fp16, void *out_fp16, int64_t M, int64_t N, int64_t K, int32_t group,
                  void *workspace, size_t workspace_bytes, void *stream) {
  return gemm_common(qx_i8, s_x_fp16, packed_w, group_meta, s_w_fp16, out_fp16, 0, M, N, K, group, workspace,
                     workspace_bytes, stream);
}

int qoq_w4a8_gemm_i32(const void *qx_i8, const void *packed_w, const void *group_meta, int32_t *acc_i32,
                      int64_t M, int64_t N, int64_t K, int32_t group, void *workspace, size_t workspace_bytes,
                      void *stream) {
  return gemm_common(qx_i8, nullptr, packed_w, group_meta, nullptr, acc_i32, 1, M, N, K, group, workspace,
                     workspace_bytes, stream);
}

const char *qoq_gemm_plan(int64_t M, int64_t N, int64_t K) {
  if (check_gemm(M, N, K, 128) != QOQ_OK || M == 0) return "invalid";
  return qoq::gemm_plan_name(M, N, K);
}

int qoq_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group, size_t *bytes) {
  int st = check_gemm(M, N, K, group);
  if (st != QOQ_OK) return st;
  if (!bytes) return QOQ_ERR_INVALID;
  if (M > kMaxDim || K > kMaxDim / 2) return QOQ_ERR_UNSUPPORTED;
  *bytes = M == 0 ? 0 : qoq::linear_workspace_need(M, N, K);
  return QOQ_OK;
}

int qoq_w4a8_linear(const void *x_fp16, const void *packed_w, const void *group_meta, const void *s_w_fp16,
                    void *out_fp16, void *s_x_fp16, int64_t M, int64_t N, int64_t K, int32_t group,
                    void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_gemm(M, N, K, group);
  if (st != QOQ_OK) return st;
  if (M > kMaxDim || K > kMaxDim / 2) return QOQ_ERR_UNSUPPORTED;
  if (M == 0) return QOQ_OK;
  if (!x_fp16 || !packed_w || !group_meta || !s_w_fp16 || !out_fp16) return QOQ_ERR_INVALID;
  if (!aligned(x_fp16, 16) || !aligned(packed_w, 16) || !aligned(group_meta, 16) || !aligned(out_fp16, 16) ||
      !aligned(s_w_fp16, 2) || !aligned(s_x_fp16, 2))
    return QOQ_ERR_ALIGNMENT;
  const size_t need = qoq::linear_workspace_need(M, N, K);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return QOQ_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return QOQ_ERR_ALIGNMENT;
  }
  qoq::launch_w4a8_linear(x_fp16, packed_w, group_meta, s_w_fp16, out_fp16, s_x_fp16, M, N, K, workspace,
                          as_stream(stream));
  return launch_status();
}

int qoq_w4a8_linear_noalloc(const void *x_fp16, const void *packed_w, const void *group_meta,
                            const void *s_w_fp16, void *out_fp16, void *s_x_fp16, int64_t M, int64_t N,
                            int64_t K, int32_t group, void *stream) {
  static_assert(qoq::kScratchBytes == QOQ_SCRATCH_BYTES, "scratch size in the header");
  int st = check_gemm(M, N, K, group);
  if (st != QOQ_OK) return st;
  if (M > kMaxDim || K > kMaxDim / 2) return QOQ_ERR_UNSUPPORTED;
  if (M == 0) return QOQ_OK;
  if (!x_fp16 || !packed_w || !group_meta || !s_w_fp16 || !out_fp16) return QOQ_ERR_INVALID;
  if (!aligned(x_fp16, 16) || !aligned(packed_w, 16) || !aligned(group_meta, 16) || !aligned(out_fp16, 16) ||
      !aligned(s_w_fp16, 2) || !aligned(s_x_fp16, 2))
    return QOQ_ERR_ALIGNMENT;
  const size_t need = qoq::linear_workspace_need(M, N, K);
  if (need > qoq::kScratchBytes) return QOQ_ERR_SCRATCH;
  void *ws = nullptr;
  if (need > 0 && qoq::linear_scratch(&ws) != hipSuccess) return QOQ_ERR_HIP;
  qoq::launch_w4a8_linear(x_fp16, packed_w, group_meta, s_w_fp16, out_fp16, s_x_fp16, M, N, K, ws,
                          as_stream(stream));
  return launch_status();
}

const char *qoq_linear_plan(int64_t M, int64_t N, int64_t K) {
  if (check_gemm(M, N, K, 128) != QOQ_OK || M == 0) return "invalid";
  return qoq::linear_plan_name(M, N, K);
}

const char *qoq_linear_config_name(int index) { return qoq::linear_config_name(index); }

int qoq_gemm_plan_splits(int64_t M, int64_t N, int64_t K) {
  const int st = check_gemm(M, N, K, 128);
  if (st != QOQ_OK) return st;
  if (M == 0) return QOQ_ERR_INVALID;
  return qoq::gemm_plan_splits(M, N, K);
}

const char *qoq_gemm_config_name(int index) { return qoq::gemm_config_name(index); }

int qoq_set_plan_override(const char *gemm_config, int32_t splits, const char *regime,
                          const char *linear_config) {
  return qoq::set_plan_override(gemm_config, splits, regime, linear_config) == 0 ? QOQ_OK : QOQ_ERR_INVALID;
}

int qoq_dequantize_packed(const void *packed_w, const void *group_meta, int64_t N, int64_t K, int32_t group,
                          void *w_i8, void *stream) {
  int st = check_nk(N, K, group);
  if (st != QOQ_OK) return st;
  if (!packed_w || !group_meta || !w_i8) return QOQ_ERR_INVALID;
  if (!aligned(packed_w, 16) || !aligned(group_meta, 2) || !aligned(w_i8, 16)) return QOQ_ERR_ALIGNMENT;
  qoq::launch_dequantize_packed(packed_w, group_meta, N, K, w_i8, as_stream(stream));
  return launch_status();
}

int qoq_stream_copy(const void *src, void *dst, size_t bytes, void *stream) {
  if (!src || !dst || bytes % 16 != 0) return QOQ_ERR_INVALID;
  if (!aligned(src, 16) || !aligned(dst, 16)) return QOQ_ERR_ALIGNMENT;
  if (bytes == 0) return QOQ_OK;
  qoq::launch_stream_copy(src, dst, bytes, as_stream(stream));
  return launch_status();
}

int qoq_stream_read(const void *src, size_t bytes, void *sink, int unroll, int blocks, void *stream) {
  if (!src || !sink || bytes % 16 != 0 || blocks <= 0 || unroll <= 0) return QOQ_ERR_INVALID;
  if (!aligned(src, 16) || !aligned(sink, 4)) return QOQ_ERR_ALIGNMENT;
  if (bytes == 0) return QOQ_OK;
  qoq::launch_stream_read(src, bytes, sink, unroll, blocks, as_stream(stream));
  return launch_status();
}

int qoq_mfma_peak_operands(const void *a, size_t a_bytes, const void *b, size_t b_bytes, int iters, int blocks,
                           void *sink, void *stream) {
  if (!a || !b || !sink || iters <= 0 || blocks <= 0 || a_bytes < 16 || b_bytes < 16) return QOQ_ERR_INVALID;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sink, 4)) return QOQ_ERR_ALIGNMENT;
  qoq::launch_mfma_peak_operands(a, a_bytes, b, b_bytes, iters, blocks, sink, as_stream(stream));
  return launch_status();
}

int qoq_mfma_peak(int iters, int blocks, void *sink, void *stream) {
  if (iters <= 0 || blocks <= 0 || !sink) return QOQ_ERR_INVALID;
  if (!aligned(sink, 4)) return QOQ_ERR_ALIGNMENT;
  qoq::launch_mfma_peak(iters, blocks, sink, as_stream(stream));
  return launch_status();
}

int qoq_mfma_probe32(const void *a_frag, const void *b_frag, void *d_frag, void *stream) {
  if (!a_frag || !b_frag || !d_frag) return QOQ_ERR_INVALID;
  if (!aligned(a_frag, 16) || !aligned(b_frag, 16) || !aligned(d_frag, 16)) return QOQ_ERR_ALIGNMENT;
  qoq::launch_mfma_probe32(a_frag, b_frag, d_frag, as_stream(stream));
  return launch_status();
}

int qoq_mfma_probe(const void *a_frag, const void *b_frag, void *d_frag, void *stream) {
  if (!a_frag || !b_frag || !d_frag) return QOQ_ERR_INVALID;
  if (!aligned(a_frag, 16) || !aligned(b_frag, 16) || !aligned(d_frag, 16)) return QOQ_ERR_ALIGNMENT;
  qoq::launch_mfma_probe(a_frag, b_frag, d_frag, as_stream(stream));
  return launch_status();
}

}  // extern "C"
