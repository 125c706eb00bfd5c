// Host-side launchers shared between the C-ABI layer and the kernel files.
// Arguments are validated by the C-ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace qoq {

void launch_quantize_activations(const void *x, int64_t M, int64_t K, void *qx, void *sx,
                                 hipStream_t stream);
void launch_quantize_pack_weights(const void *w, int64_t N, int64_t K, void *packed, void *meta,
                                  void *sw, hipStream_t stream);
void launch_quantize_pack_weights_pc(const void *w, int64_t N, int64_t K, void *packed, void *zeros, void *sw,
                                     hipStream_t stream);
// codes in the tiled layout of the few-token GEMM (tiled_offset in qoq_device.h);
// qx holds round_up(M, 16) * K bytes, rows past M are not written
void launch_quantize_activations_tiled(const void *x, int64_t M, int64_t K, void *qx, void *sx,
                                       hipStream_t stream);
void launch_quantize_activations_rowsum(const void *x, int64_t M, int64_t K, void *qx, void *sx, void *tx,
                                        hipStream_t stream);
void launch_quantize_activations_rowsum_tiled(const void *x, int64_t M, int64_t K, void *qx, void *sx, void *tx,
                                              hipStream_t stream);

// producers with the quantization fused in (tiled 1: codes in the tiled layout,
// M <= kTiledMaxM; 0: row-major; -1: no quantization, the fp16 value itself into
// qx as [M, K] fp16); tx may be null (no code sums); K % 8 == 0, K <= kFusedMaxK;
// gate / up rows have stride ld elements
constexpr int64_t kFusedMaxK = 32768;
void launch_rmsnorm_quantize(const void *x, const void *gamma, float eps, int64_t M, int64_t K, int tiled,
                             void *qx, void *sx, void *tx, hipStream_t stream);
// SwiGLU + quantization of a few long rows in two passes over 2048-value slices,
// with a workspace of one 32-bit maximum per (row, slice); 0 slices: not split
#ifndef QOQ_SILU_SPLIT_MAX_M
#define QOQ_SILU_SPLIT_MAX_M 64
#endif
constexpr int64_t kSiluSplitMaxM = QOQ_SILU_SPLIT_MAX_M;
int silu_split_slices(int64_t M, int64_t K);
size_t silu_split_workspace(int64_t M, int64_t K);
void launch_silu_mul_quantize_split(const void *gate, const void *up, int64_t ld, int64_t M, int64_t K, bool tiled,
                                    void *qx, void *sx, void *ws, hipStream_t stream);
void launch_silu_mul_quantize(const void *gate, const void *up, int64_t ld, int64_t M, int64_t K, int tiled,
                              void *qx, void *sx, void *tx, hipStream_t stream);

// KV4 cache (head dim 128, 64-token pages, the layout described in qoq_kv4.hip)
constexpr int kKv4PageTokens = 64;
constexpr int kKv4PageBytes = 8704;              // per (page, KV head): K, V codes + fp16 stats
#ifndef QOQ_KV4_TARGET_WG
#define QOQ_KV4_TARGET_WG 512
#endif
constexpr int64_t kKv4TargetWorkgroups = QOQ_KV4_TARGET_WG;
#ifndef QOQ_KV4_MAX_SPLITS
#define QOQ_KV4_MAX_SPLITS 64
#endif
constexpr int64_t kKv4MaxSplits = QOQ_KV4_MAX_SPLITS;
int kv4_splits(int64_t B, int64_t h_kv, int64_t max_len);
size_t kv4_workspace_need(int64_t B, int64_t h, int64_t h_kv, int64_t max_len);
void launch_kv4_write(const void *k_new, const void *v_new, int64_t B, int64_t n_new, int64_t h_kv,
                      const int *positions, const int *page_table, int64_t max_pages, int64_t num_pages, void *pool,
                      hipStream_t stream);
void launch_smooth_lambda(const void *k, int64_t n, int64_t h_kv, float alpha, void *lam, hipStream_t stream);
void launch_smooth_fold(const void *wq, const void *wk, const void *lam, int64_t h, int64_t h_kv, int64_t dm,
                        void *wq_out, void *wk_out, hipStream_t stream);
void launch_kv4_attention(const void *q, const void *pool, int64_t num_pages, const int *page_table,
                          int64_t max_pages, const int *seq_lens, int64_t B, int64_t h, int64_t h_kv,
                          int64_t max_len, void *out, void *ws, hipStream_t stream);

// GEMM: out_kind 0 = fp16 epilogue, 1 = INT32 accumulators; ws holds at least
// gemm_workspace_need(M, N, K) bytes (may be null when that is 0)
void launch_w4a8_gemm(const void *qx, const void *sx, const void *packed, const void *meta,
                      const void *sw, void *out, int out_kind, int64_t M, int64_t N, int64_t K, void *ws,
                      hipStream_t stream);
// per-channel weights: B = raw codes, epilogue acc - zeros[n] * tx[m] (same plans
// and workspace as the per-group GEMM)
void launch_w4a8_gemm_pc(const void *qx, const void *sx, const void *tx, const void *packed, const void *zeros,
                         const void *sw, void *out, int out_kind, int64_t M, int64_t N, int64_t K, void *ws,
                         hipStream_t stream);
// tiled activation codes (M <= kTiledMaxM): few-token kernels only, no workspace
constexpr int64_t kTiledMaxM = 64;
void launch_w4a8_gemm_tiled(const void *qx, const void *sx, const void *packed, const void *meta, const void *sw,
                            void *out, int out_kind, int64_t M, int64_t N, int64_t K, hipStream_t stream);
void launch_w4a8_gemm_pc_tiled(const void *qx, const void *sx, const void *tx, const void *packed, const void *zeros,
                               const void *sw, void *out, int out_kind, int64_t M, int64_t N, int64_t K,
                               hipStream_t stream);
const char *gemm_tiled_plan_name(int64_t M, int64_t N, int64_t K);
size_t gemm_workspace_need(int64_t M, int64_t N, int64_t K);
int gemm_plan_splits(int64_t M, int64_t N, int64_t K);
const char *gemm_plan_name(int64_t M, int64_t N, int64_t K);

// linear = quantize + GEMM (fused kernel for a few tokens, tiled codes up to
// kTiledMaxM tokens); ws holds at least linear_workspace_need(M, N, K) bytes,
// 256-byte aligned
void launch_w4a8_linear(const void *x, const void *packed, const void *meta, const void *sw, void *out,
                        void *sx_out, int64_t M, int64_t N, int64_t K, void *ws, hipStream_t stream);
size_t linear_workspace_need(int64_t M, int64_t N, int64_t K);
// device address of the static scratch array on the current device (looked up once
// per device); hipSuccess or the lookup's error
hipError_t linear_scratch(void **ptr);
constexpr size_t kScratchBytes = size_t{64} << 20;
const char *linear_plan_name(int64_t M, int64_t N, int64_t K);
const char *linear_config_name(int index);
const char *gemm_config_name(int index);
// planner overrides for measurement and verification (qoq_set_plan_override):
// 0, or -1 for an unknown name or a negative split factor
int set_plan_override(const char *gemm_config, int splits, const char *regime, const char *linear_config);

void launch_dequantize_packed(const void *packed, const void *meta, int64_t N, int64_t K, void *w_i8,
                              hipStream_t stream);
void launch_stream_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);
void launch_stream_read(const void *src, size_t bytes, void *sink, int unroll, int blocks, hipStream_t stream);
void launch_mfma_peak(int iters, int blocks, void *sink, hipStream_t stream);
void launch_mfma_peak_operands(const void *a, size_t a_bytes, const void *b, size_t b_bytes, int iters, int blocks,
                               void *sink, hipStream_t stream);
void launch_mfma_probe32(const void *a, const void *b, void *d, hipStream_t stream);
void launch_mfma_probe(const void *a, const void *b, void *d, hipStream_t stream);

}  // namespace qoq
