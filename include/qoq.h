/*
 * qoq.h — C ABI of the QoQ W4A8 per-group GEMM library for MI355X (gfx950).
 *
 * The method (QServe / QoQ, "QServe: W4A8KV4 Quantization and System Co-design for
 * Efficient LLM Serving", sections "渐进式组量化" progressive group quantization,
 * "保护性量化范围" protective quantization range and "逐组W4A8 GEMM中的快速反量化"
 * per-group fast dequantization):
 *   weights    W [N,K] fp16  -> level 0: per-output-channel symmetric INT8 codes in
 *                               the protective range [-119, 119], fp16 scale s_W[n]
 *                            -> level 1: per group of 128 consecutive k, asymmetric
 *                               UINT4 codes with a UINT4 zero z and a UINT8 scale s_u8
 *   activations X [M,K] fp16 -> per-token symmetric INT8 codes qx, fp16 scale s_X[m]
 *   GEMM       acc[m,n] = sum_k qx[m,k] * (q_u4[n,k] - z[n,k/128]) * s_u8[n,k/128]
 *              (exact INT32; the dequantized weight always fits INT8)
 *              out[m,n] = fp16( float(acc) * (float(s_X[m]) * float(s_W[n])) )
 *
 * Conventions shared by every call
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or retains them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *     compute call validates its arguments on the host, then enqueues its kernels on
 *     `stream` and returns without synchronising.
 *   - Return value: QOQ_OK (0) or a negative qoq_status.  On any error nothing is
 *     launched and no output is touched.  No C++ exception crosses this interface.
 *   - The library holds no mutable global state; calls are thread-safe.  Calls on
 *     different streams that write the same output race, as any GPU work does.
 *   - group == 128 (per-group weights); group == 0 selects per-channel weights where
 *     a call documents it.  Anything else: QOQ_ERR_UNSUPPORTED.
 *   - Shapes: N % 16 == 0, K % 128 == 0, 0 < K <= 139648 (keeps every INT32
 *     accumulator exact: 127 * 121 * K < 2^31), M >= 0 (M == 0 is a no-op).
 *   - Inputs must be finite; behaviour for inf/NaN inputs is unspecified.
 *
 * Storage layout of the packed weights (this library's own order; the pages fix only
 * that weights, zeros and scales are stored offline in the order the kernel consumes
 * them so that each lane issues one 128-bit load — "QServe：把 W4A8KV4 ..." review,
 * §3.2 compute-aware weight reordering):
 *   strip b = n / 16, c = n % 16, group j = k / 128, G = K / 128,
 *   k = 128 j + 64 half + 16 h + i   (half in {0,1}, h in 0..3, i in 0..15)
 *   packed_w[((b*G + j)*64 + 16*h + c)*16 + i]
 *       = q_u4[n, 128j + 16h + i] | q_u4[n, 128j + 64 + 16h + i] << 4      (uint8)
 *   group_meta[(b*G + j)*16 + c] = s_u8[n, j] | z[n, j] << 8               (uint16)
 *   s_w: fp16 [N], natural order.
 */
#ifndef QOQ_H
#define QOQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QOQ_OK = 0,
  QOQ_ERR_INVALID = -1,      /* null pointer, negative or non-multiple shape */
  QOQ_ERR_UNSUPPORTED = -2,  /* group != 128, K beyond the exact-INT32 limit */
  QOQ_ERR_ALIGNMENT = -3,    /* pointer not aligned as the call requires */
  QOQ_ERR_WORKSPACE = -4,    /* workspace smaller than qoq_gemm_workspace_bytes */
  QOQ_ERR_HIP = -5,          /* the HIP runtime reported an error at launch */
  QOQ_ERR_SCRATCH = -6       /* the shape needs more than QOQ_SCRATCH_BYTES of scratch */
} qoq_status;

/* Library ABI version (increments when a signature, an entry point or the storage
 * layout changes; 2 adds the per-channel variant and the linear entry point). */
int qoq_version(void);

/* Human-readable text of a qoq_status value; never NULL, static storage. */
const char *qoq_status_string(int status);

/* Sizes in bytes of the three buffers qoq_quantize_pack_weights writes for W [N,K]:
 * group 128: packed_w = N*K/2, group_meta = 2*N*K/128, s_w = 2*N;
 * group 0 (per-channel weights): packed_w = N*K/2, group_meta = N (the zeros, one
 * byte per output channel), s_w = 2*N.  Any output pointer may be NULL.
 * Errors: INVALID for bad N/K, UNSUPPORTED for any other group. */
int qoq_weight_buffer_sizes(int64_t N, int64_t K, int32_t group, size_t *packed_w_bytes,
                            size_t *group_meta_bytes, size_t *s_w_bytes);

/* Offline weight quantization and packing ("QServe ..." summary, progressive group
 * quantization and protective quantization range; review §3.1):
 *   s_W[n] = fp16(max_k |W[n,k]| / 119)            (fp32 IEEE divide, then RNE to fp16)
 *   q_s8   = clamp(rint(W / s_W), -119, 119)         (0 for a row whose s_W is 0)
 *   per group: lo = min(0, min q_s8), hi = max(0, max q_s8),
 *   s_u8 = max(1, ceil((hi - lo) / 15)), z = clamp(rne(-lo / s_u8), 0, 15),
 *   q_u4 = clamp(z + rne(q_s8 / s_u8), 0, 15)        (rne = round half to even)
 * w_fp16: [N,K] row-major fp16, 16-byte aligned.  packed_w: N*K/2 bytes, 16-byte
 * aligned.  group_meta: N*K/128 uint16, 2-byte aligned.  s_w_fp16: N fp16.
 * Errors: INVALID, UNSUPPORTED, ALIGNMENT, HIP. */
int qoq_quantize_pack_weights(const void *w_fp16, int64_t N, int64_t K, int32_t group,
                              void *packed_w, void *group_meta, void *s_w_fp16, void *stream);

/* group == 0 selects the per-channel format (the W4A8 variant without groups, whose
 * zero point leaves the main loop: "QServe ..." summary, per-channel fast
 * dequantization; integer quantization with a zero point, one per channel):
 *   lo = min(0, min_k W[n,k]), hi = max(0, max_k W[n,k])   (fp32)
 *   s_W[n] = fp16((hi - lo) / 15)                          (fp32 subtract and divide)
 *   z[n]   = clamp(rint(-lo / s_W), 0, 15),  q = clamp(z + rint(W / s_W), 0, 15)
 *   (a row whose s_W is 0: q = 0, z = 0)
 * packed_w: the codes in the same storage layout as above; group_meta receives the
 * zeros (uint8 [N], no alignment requirement); s_w_fp16 [N]. */

/* Per-token symmetric INT8 activation quantization (the activation side of the
 * epilogue scale s_W x s_X, "QServe ..." summary; symmetric quantizer of
 * "01 inference papers and experiments" §4.1):
 *   s_X[m] = fp16(max_k |X[m,k]| / 127), qx = clamp(rint(X / s_X), -127, 127)
 *   (all-zero token: s_X = 0, qx = 0).
 * x_fp16: [M,K] row-major fp16; qx_i8: [M,K] row-major int8; s_x_fp16: [M] fp16.
 * K % 8 == 0 here (the GEMM itself needs K % 128 == 0); x and qx 16-byte aligned.
 * Errors: INVALID, ALIGNMENT, HIP. */
int qoq_quantize_activations(const void *x_fp16, int64_t M, int64_t K, void *qx_i8,
                             void *s_x_fp16, void *stream);

/* qoq_quantize_activations plus the per-token code sums of the per-channel epilogue:
 * t_x[m] = sum_k qx[m, k] (INT32 [M], 4-byte aligned; the "t_X" of the per-channel
 * epilogue term t_X x (z_W ⊙ s_W), taken over the quantized activations so the
 * epilogue is exact).  Errors: INVALID, ALIGNMENT, HIP. */
int qoq_quantize_activations_rowsum(const void *x_fp16, int64_t M, int64_t K, void *qx_i8,
                                    void *s_x_fp16, int32_t *t_x, void *stream);

/* qoq_quantize_activations with the codes in the tiled layout that the few-token
 * GEMM reads (qoq_w4a8_gemm_tiled): the codes of rows 16*rb .. +15 and k = 64*kb ..
 * +63 form a 1 KB block at byte (rb * K/64 + kb) * 1024, in which the 16 bytes
 * k = 64*kb + 16*q .. +15 of row 16*rb + r sit at offset (16*q + r) * 16 — the order
 * in which the 16x16x64 INT8 matrix instruction takes its A operand, one 16-byte
 * load per lane.  This is the compute-order layout idea the pages apply to the
 * weights ("QServe：把 W4A8KV4 ..." review §3.2), applied here to the activations by
 * the kernel that produces them.  qx_tiled: round_up(M, 16) * K bytes, 16-byte
 * aligned; the rows past M of the last block are not written (the GEMM does not
 * read them).  s_x_fp16 as for qoq_quantize_activations.  M <= 64, K % 64 == 0.
 * Errors: INVALID, UNSUPPORTED (M > 64), ALIGNMENT, HIP. */
int qoq_quantize_activations_tiled(const void *x_fp16, int64_t M, int64_t K, void *qx_tiled,
                                   void *s_x_fp16, void *stream);

/* qoq_quantize_activations_tiled plus the per-token code sums t_x of
 * qoq_quantize_activations_rowsum (INT32 [M], 4-byte aligned): the inputs of the
 * per-channel GEMM on tiled codes (qoq_w4a8_gemm_pc_tiled).  M <= 64, K % 64 == 0.
 * Errors: INVALID, UNSUPPORTED (M > 64), ALIGNMENT, HIP. */
int qoq_quantize_activations_rowsum_tiled(const void *x_fp16, int64_t M, int64_t K, void *qx_tiled,
                                          void *s_x_fp16, int32_t *t_x, void *stream);

/* The producers of the GEMM's INT8 activations with the quantization fused in
 * ("QServe：把 W4A8KV4 ..." review, runtime precision mapping §3.2 and data path
 * step 2: fused into the preceding normalization kernel for the QKV projection and
 * the first FFN layer, into the preceding activation kernel for the second FFN
 * layer).  Each forms the fp16 value the unfused pipeline would write, in
 * registers, and quantizes it per token exactly as qoq_quantize_activations (same
 * codes and s_X); t_x (NULL or INT32 [M], 4-byte aligned) also receives the code
 * sums of qoq_quantize_activations_rowsum.
 *   layout 0: qx row-major [M,K]; layout 1: the tiled layout of
 *   qoq_quantize_activations_tiled (M <= 64, K % 64 == 0, round_up(M,16)*K bytes).
 * K % 8 == 0 and K <= 32768 (one row in registers); qx 16-byte aligned, s_x_fp16 [M].
 * Errors: INVALID, UNSUPPORTED (K > 32768; layout 1 with M > 64), ALIGNMENT, HIP. */

/* RMSNorm (the normalization of the Llama / Qwen workloads) + quantization:
 *   y = fp16(fp32(fp32(x * inv) * gamma)), inv = fp32(1 / fp32(sqrt(fp32(mean +
 *   eps)))), mean = fp32(sum_k x^2 / K) with the sum in fp64 (IEEE operations).
 * x_fp16 [M,K] row-major and gamma_fp16 [K], both 16-byte aligned; eps > 0. */
int qoq_rmsnorm_quantize(const void *x_fp16, const void *gamma_fp16, float eps, int64_t M,
                         int64_t K, int32_t layout, void *qx, void *s_x_fp16, int32_t *t_x,
                         void *stream);

/* SwiGLU activation + quantization: h = fp16(gate * up / (1 + exp(-gate))), the
 * expression evaluated in fp64 and rounded once.  gate_fp16 and up_fp16: [M,K]
 * with row stride ld elements (ld >= K, ld % 8 == 0; e.g. the two halves of a fused
 * gate+up projection output [M, 2K]: gate = out, up = out + K, ld = 2K), 16-byte
 * aligned. */
int qoq_silu_mul_quantize(const void *gate_fp16, const void *up_fp16, int64_t ld, int64_t M,
                          int64_t K, int32_t layout, void *qx, void *s_x_fp16, int32_t *t_x,
                          void *stream);

/* The same result without the code sums, for a few long rows split over workgroups
 * without repetition: pass 1 forms each 2048-value slice of a row and writes its
 * maximum magnitude to the workspace, pass 2 quantizes every slice with the row
 * maximum (the same codes and scales as qoq_silu_mul_quantize, bit for bit).
 * workspace: caller-owned device memory of qoq_silu_mul_quantize_workspace_bytes
 * (one 32-bit value per row and slice; 0 bytes, and one pass, above 64 rows or
 * below 2049 values per row), 4-byte aligned, no initialization, nothing kept
 * between calls; overlapping calls need separate workspaces.
 * Errors: as qoq_silu_mul_quantize, WORKSPACE when the workspace is NULL or smaller
 * than reported. */
int qoq_silu_mul_quantize_workspace_bytes(int64_t M, int64_t K, size_t *bytes);
int qoq_silu_mul_quantize_ws(const void *gate_fp16, const void *up_fp16, int64_t ld, int64_t M,
                             int64_t K, int32_t layout, void *qx, void *s_x_fp16, void *workspace,
                             size_t workspace_bytes, void *stream);

/* The same kernels without the quantization (the unfused pipeline's normalization and
 * activation kernels): the fp16 values the fused entry points quantize, [M,K]
 * row-major fp16, 16-byte aligned.  Same arguments and errors otherwise. */
int qoq_rmsnorm(const void *x_fp16, const void *gamma_fp16, float eps, int64_t M, int64_t K,
                void *y_fp16, void *stream);
int qoq_silu_mul(const void *gate_fp16, const void *up_fp16, int64_t ld, int64_t M, int64_t K,
                 void *h_fp16, void *stream);

/* ------------------------------------------------------------------------------
 * KV4: paged, per-head dynamic INT4 KV cache and decode attention ("QServe: W4A8KV4
 * ..." summary: attention o_h = softmax(q_h K_{h_KV}^T / sqrt(D)) V_{h_KV}, h_KV =
 * h / r; asymmetric integer quantization; a paged KV cache keeping each head's FP16
 * scale and zero inside the page right after its quantized features; KV4 attention
 * in FP16.  "QServe：把 W4A8KV4 ..." review §3.2 and §4 steps 4-5.)
 * Head dim 128, 64 tokens per page.  The pool is caller-owned device memory of
 * num_pages x qoq_kv4_page_bytes bytes (16-byte aligned); a page holds, for each KV
 * head, the K and V codes of its 64 token slots (in the operand order of the
 * attention kernel's matrix instructions) followed by each slot's fp16 K scale and
 * zero (one 32-bit word per token) and each four slots' fp16 V scales then V zeros
 * (16 bytes per four tokens); the byte-level layout is described with the kernels
 * (qoq_kv4.hip).  page_table: int32 [B, max_pages], the pool page
 * of each 64-token span of each sequence (pages of different sequences distinct).
 * num_pages: pages in the pool.  Positions, page ids and seq_lens are device data the
 * host cannot check; the kernels guard them: the write skips a token whose position
 * falls outside the table or whose page id lies outside [0, num_pages), the attention
 * clamps page ids to that range and seq_lens to [1, max_len] (a bad table gives wrong
 * values, never an access outside the buffers).  The write skips a whole 16-token
 * block when its position or page is out of range.
 * ------------------------------------------------------------------------------ */

/* Bytes of one page (all h_kv heads).  Errors: INVALID, UNSUPPORTED (head_dim != 128). */
int qoq_kv4_page_bytes(int64_t h_kv, int64_t head_dim, size_t *bytes);

/* KV write: quantize n_new new tokens per sequence into the cache.  k_new, v_new: fp16
 * [B, n_new, h_kv, 128] (16-byte aligned); token i of sequence b goes to position
 * positions[b] + i.  Per token and KV head, over the range [lo, hi] = [min x, max x]
 * of its 128 values ("QServe ..." summary, integer quantization; review §3.2, FP16
 * scale and zero per head): s = fp16(fp32(hi - lo) / 15), z = rne(-lo / s), codes
 * clamp(z + rne(x / s), 0, 15) (fp32 IEEE quotients).  Where s = 0 (a constant
 * vector) or |z| > 1024 (q - z would leave FP16's exact integers), the same over
 * [min(lo, 0), max(hi, 0)] (z in [0, 15] then); s = 0 for an all-zero vector,
 * codes and z 0; s and z stored as fp16.  One wave per (KV head, sequence, 16-token block of positions): a V word
 * holds four tokens, so each block's words are assembled once, merged with the
 * tokens already there; calls for the same pages must not overlap.  n_new <= 2^19,
 * B <= 65535, the sequence's positions below 2^30.
 * Errors: INVALID, UNSUPPORTED, ALIGNMENT, HIP. */
int qoq_kv4_write(const void *k_new, const void *v_new, int64_t B, int64_t n_new, int64_t h_kv,
                  int64_t head_dim, const int32_t *positions, const int32_t *page_table,
                  int64_t max_pages, void *kv_pool, int64_t num_pages, void *stream);

/* SmoothAttention, offline ("QServe: W4A8KV4 ..." summary, SmoothAttention: the keys'
 * outlier channels are scaled down by lambda and the queries up by the same factor,
 * Z = (Q Lambda)(K Lambda^-1)^T; review §4.2: folded into W_Q and W_K, no runtime
 * cost).  Scales from key samples: k_samples fp16 [n, h_kv, 128] (2-byte aligned),
 * lambda_f32 out [h_kv, 128] (4-byte aligned): for channel i of KV head g,
 * a_i = max_n |k[n, g, i]|, and the RoPE pair (i, i + 64) shares
 * lambda = max(a_i, a_{i+64})^alpha (alpha = 0.5: the IEEE fp32 square root; other
 * alpha in [0, 1]: the double-precision power rounded to fp32); a pair that is 0 on
 * every sample keeps lambda = 1.  One workgroup per KV head (offline use).
 * Errors: INVALID (n, h_kv < 1, alpha outside [0, 1]), UNSUPPORTED (head_dim != 128,
 * h_kv > 65535, n * h_kv > 2^30), ALIGNMENT, HIP. */
int qoq_smooth_attention_lambda(const void *k_samples, int64_t n, int64_t h_kv, int64_t head_dim,
                                float alpha, void *lambda_f32, void *stream);

/* Folds lambda into the projections: w_q fp16 [h * 128, d_model] row-major (the query
 * heads' output channels), w_k fp16 [h_kv * 128, d_model]; row (head, i) of w_q becomes
 * fp16(fp32(w) * lambda[head / (h / h_kv), i]) and row (g, i) of w_k becomes
 * fp16(w / lambda[g, i]) (IEEE fp32 quotient).  Outputs may be the inputs (in place).
 * Errors: INVALID (h % h_kv, sizes < 1, null pointers), UNSUPPORTED (head_dim != 128,
 * h > 4096, d_model > 2^20), ALIGNMENT (2-byte weights, 4-byte lambda), HIP. */
int qoq_smooth_attention_fold(const void *w_q, const void *w_k, const void *lambda_f32, int64_t h,
                              int64_t h_kv, int64_t head_dim, int64_t d_model, void *w_q_out,
                              void *w_k_out, void *stream);

/* Workspace for qoq_kv4_decode_attention (0 when one workgroup per (sequence, KV
 * head) covers the sequence): split partials, no initialization needed.
 * Errors: INVALID, UNSUPPORTED. */
int qoq_kv4_attention_workspace_bytes(int64_t B, int64_t h, int64_t h_kv, int64_t head_dim,
                                      int64_t max_len, size_t *bytes);

/* Decode attention of one new token per sequence over its cached tokens:
 *   o[b, head] = softmax(q[b, head] . K_hat / sqrt(128)) V_hat over the seq_lens[b]
 *   cached tokens of KV head head / (h / h_kv), K_hat = fp16((code - z) * s).
 * q: fp16 [B, h, 128]; out: fp16 [B, h, 128] (16-byte aligned); seq_lens: int32 [B],
 * 1 <= seq_lens[b] <= max_len <= 64 * max_pages; h % h_kv == 0, h / h_kv <= 16.
 * Products on the matrix cores with FP16 inputs and FP32 accumulation; the
 * softmax in FP32 with the probabilities rounded to FP16 for the second product.
 * workspace: qoq_kv4_attention_workspace_bytes (WORKSPACE when smaller).
 * Errors: INVALID, UNSUPPORTED, ALIGNMENT, WORKSPACE, HIP. */
int qoq_kv4_decode_attention(const void *q, const void *kv_pool, int64_t num_pages,
                             const int32_t *page_table, int64_t max_pages, const int32_t *seq_lens,
                             int64_t B, int64_t h, int64_t h_kv, int64_t head_dim, int64_t max_len,
                             void *out, void *workspace, size_t workspace_bytes, void *stream);

/* Workspace in bytes the GEMM entry points need for this problem (0 for M == 0).
 * It is non-zero when the plan splits the K groups of each output tile over several
 * workgroups ("QServe：把 W4A8KV4 ..." review §3.2: split-k when the batch is small;
 * here for any shape whose output tiles alone would leave compute units idle):
 * splits x M x N INT32 partial sums, written by the GEMM kernel and summed by a second
 * kernel that applies the epilogue (both enqueued on `stream`).  The workspace is
 * caller-owned device memory, 16-byte aligned, needs no initialization and holds
 * nothing between calls; calls that may run concurrently need separate workspaces.
 * Errors: INVALID, UNSUPPORTED. */
int qoq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group, size_t *bytes);

/* W4A8 per-group GEMM with the fp16 epilogue ("QServe ..." summary, per-group
 * W4A8 GEMM fast dequantization and the epilogue O = (Q_X Q_W) ⊙ (s_W x s_X);
 * review §4 step 3: INT4 -> INT8 by multiply-then-subtract in registers, INT8
 * matrix-core products, INT32 accumulation, fp16 output):
 *   out[m,n] = fp16( float(acc[m,n]) * (float(s_X[m]) * float(s_W[n])) )
 * qx_i8 [M,K] int8 (16-byte aligned), s_x_fp16 [M], packed_w / group_meta / s_w_fp16
 * as written by qoq_quantize_pack_weights for the same N, K (packed_w and group_meta
 * 16-byte aligned); out_fp16 [M,N] row-major fp16 (16-byte aligned).  workspace: see
 * qoq_gemm_workspace_bytes (may be NULL when that reports 0; WORKSPACE when it is
 * NULL or smaller than reported, ALIGNMENT when not 16-byte aligned).
 * Errors: INVALID, UNSUPPORTED, ALIGNMENT, WORKSPACE, HIP. */
int qoq_w4a8_gemm(const void *qx_i8, const void *s_x_fp16, const void *packed_w,
                  const void *group_meta, const void *s_w_fp16, void *out_fp16, int64_t M,
                  int64_t N, int64_t K, int32_t group, void *workspace,
                  size_t workspace_bytes, void *stream);

/* Same main loop as qoq_w4a8_gemm with an INT32 epilogue: acc_i32 [M,N] row-major
 * (16-byte aligned) receives the exact integer accumulators (for bit-exact
 * verification).
 * Errors: as qoq_w4a8_gemm. */
int qoq_w4a8_gemm_i32(const void *qx_i8, const void *packed_w, const void *group_meta,
                      int32_t *acc_i32, int64_t M, int64_t N, int64_t K, int32_t group,
                      void *workspace, size_t workspace_bytes, void *stream);

/* qoq_w4a8_gemm for M <= 64 with the activation codes in the tiled layout of
 * qoq_quantize_activations_tiled: same arithmetic and results; the few-token
 * kernels only (no split-K workspace).  Errors: as qoq_w4a8_gemm, UNSUPPORTED for
 * M > 64. */
int qoq_w4a8_gemm_tiled(const void *qx_tiled, const void *s_x_fp16, const void *packed_w,
                        const void *group_meta, const void *s_w_fp16, void *out_fp16, int64_t M,
                        int64_t N, int64_t K, void *stream);

/* The same with the INT32 epilogue (exact accumulators, as qoq_w4a8_gemm_i32). */
int qoq_w4a8_gemm_tiled_i32(const void *qx_tiled, const void *packed_w, const void *group_meta,
                            int32_t *acc_i32, int64_t M, int64_t N, int64_t K, void *stream);

/* Name of the configuration qoq_w4a8_gemm_tiled launches ("invalid" for a shape it
 * rejects). */
const char *qoq_gemm_tiled_plan(int64_t M, int64_t N, int64_t K);

/* W4A8 GEMM on per-channel weights ("QServe ..." summary, per-channel fast
 * dequantization: O = (Q_X Q_W) ⊙ (s_W x s_X) - t_X x (z_W ⊙ s_W); the main loop
 * multiplies the raw UINT4 codes, the zero point is applied in the epilogue):
 *   acc[m,n] = sum_k qx[m,k] * q[n,k] - z[n] * t_x[m]   (= sum_k qx (q - z), exact)
 *   out[m,n] = fp16( float(acc) * (float(s_X[m]) * float(s_W[n])) )
 * packed_w / zeros / s_w_fp16 as written by qoq_quantize_pack_weights with group 0;
 * t_x from qoq_quantize_activations_rowsum; other buffers, the workspace (the size
 * qoq_gemm_workspace_bytes reports for the shape) and errors as for qoq_w4a8_gemm. */
int qoq_w4a8_gemm_pc(const void *qx_i8, const void *s_x_fp16, const int32_t *t_x,
                     const void *packed_w, const void *zeros, const void *s_w_fp16,
                     void *out_fp16, int64_t M, int64_t N, int64_t K, void *workspace,
                     size_t workspace_bytes, void *stream);

/* The same with the INT32 epilogue: acc_i32 [M,N] receives acc exactly. */
int qoq_w4a8_gemm_pc_i32(const void *qx_i8, const int32_t *t_x, const void *packed_w,
                         const void *zeros, int32_t *acc_i32, int64_t M, int64_t N, int64_t K,
                         void *workspace, size_t workspace_bytes, void *stream);

/* qoq_w4a8_gemm_pc for M <= 64 with the activation codes in the tiled layout of
 * qoq_quantize_activations_rowsum_tiled (t_x as written by it): same arithmetic and
 * results; the few-token kernels of qoq_w4a8_gemm_tiled (same plan, no workspace).
 * Errors: as qoq_w4a8_gemm_pc, UNSUPPORTED for M > 64. */
int qoq_w4a8_gemm_pc_tiled(const void *qx_tiled, const void *s_x_fp16, const int32_t *t_x,
                           const void *packed_w, const void *zeros, const void *s_w_fp16,
                           void *out_fp16, int64_t M, int64_t N, int64_t K, void *stream);

/* The same with the INT32 epilogue (acc exactly, as qoq_w4a8_gemm_pc_i32). */
int qoq_w4a8_gemm_pc_tiled_i32(const void *qx_tiled, const int32_t *t_x, const void *packed_w,
                               const void *zeros, int32_t *acc_i32, int64_t M, int64_t N, int64_t K,
                               void *stream);

/* Workspace in bytes qoq_w4a8_linear needs for this problem: 0 when the fused
 * kernel serves it (qoq_linear_plan names a fused configuration), otherwise room for
 * the codes (M <= 64: round_up(M, 16)*K bytes, tiled; else M*K, row-major) and s_X
 * (2*M bytes), each rounded up to 256 bytes, plus, for M > 64,
 * qoq_gemm_workspace_bytes.  Errors: INVALID, UNSUPPORTED. */
int qoq_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group, size_t *bytes);

/* The runtime step in one call: per-token activation quantization followed by the
 * W4A8 GEMM with its fp16 epilogue — the same arithmetic, codes, scales and fp16
 * results as qoq_quantize_activations + qoq_w4a8_gemm ("QServe ..." summary: the
 * activation quantization is fused into the kernel that feeds the GEMM, so it costs
 * no pass of its own).  For a few tokens, where the library's measured table (or, for
 * shapes it does not cover, M <= 2 and K <= 8192) says it is faster (see
 * qoq_linear_plan), one kernel does both: each workgroup quantizes the token rows
 * into LDS and runs the GEMM on them; otherwise up to 64 tokens the codes go through
 * the tiled layout
 * (qoq_quantize_activations_tiled + qoq_w4a8_gemm_tiled); beyond, row-major.
 * x_fp16 [M,K] row-major fp16 (16-byte aligned); packed_w / group_meta / s_w_fp16 as
 * for qoq_w4a8_gemm; out_fp16 [M,N] (16-byte aligned); s_x_fp16: NULL, or [M] fp16
 * that receives the token scales.  workspace: caller-owned device memory of
 * qoq_linear_workspace_bytes (may be NULL when that is 0), 256-byte aligned, no
 * initialization needed; calls that may run concurrently need separate workspaces.
 * Errors: INVALID, UNSUPPORTED, ALIGNMENT, WORKSPACE, HIP. */
int qoq_w4a8_linear(const void *x_fp16, const void *packed_w, const void *group_meta,
                    const void *s_w_fp16, void *out_fp16, void *s_x_fp16, int64_t M, int64_t N,
                    int64_t K, int32_t group, void *workspace, size_t workspace_bytes,
                    void *stream);

/* Size of the library's static scratch array (one per GPU, held until the process
 * ends) that qoq_w4a8_linear_noalloc uses in place of a workspace. */
#define QOQ_SCRATCH_BYTES (64u << 20)

/* qoq_w4a8_linear for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same
 * kernels, arguments, results and errors, minus the workspace.  The codes, token
 * scales and split-K partial sums go to a static device array of QOQ_SCRATCH_BYTES
 * (its address looked up once per device, on the first call with that device
 * current); no call allocates or frees anything.  A shape whose
 * qoq_linear_workspace_bytes exceeds QOQ_SCRATCH_BYTES returns QOQ_ERR_SCRATCH
 * before anything is launched.  Every byte the kernels read from the array is
 * written earlier in the same call, so it needs no clearing.  All calls on one GPU
 * share its array: calls that may overlap in time on one GPU (other streams, other
 * threads) race and must be serialized by the caller.
 * Errors: INVALID, UNSUPPORTED, ALIGNMENT, SCRATCH, HIP. */
int qoq_w4a8_linear_noalloc(const void *x_fp16, const void *packed_w, const void *group_meta,
                            const void *s_w_fp16, void *out_fp16, void *s_x_fp16, int64_t M,
                            int64_t N, int64_t K, int32_t group, void *stream);

/* Name of the kernel configuration qoq_w4a8_linear uses for this shape: a fused
 * configuration, or the qoq_gemm_tiled_plan (M <= 64) / qoq_gemm_plan name when it
 * quantizes and multiplies in two kernels ("invalid" for a shape it rejects).  A linear
 * override (qoq_set_plan_override) forces the choice where the shape allows it. */
const char *qoq_linear_plan(int64_t M, int64_t N, int64_t K);

/* Name of the index-th fused linear configuration, NULL past the last. */
const char *qoq_linear_config_name(int index);

/* Name of the kernel configuration qoq_w4a8_gemm launches for this shape (static
 * string, "invalid" for a shape the GEMM rejects).  Used to match profiler output. */
const char *qoq_gemm_plan(int64_t M, int64_t N, int64_t K);

/* Split-K factor of that plan (1 = no split; > 1 = workgroups per output tile, which
 * then needs the workspace), or a negative qoq_status for a shape the GEMM rejects
 * (INVALID also for M == 0).  A split override (qoq_set_plan_override) forces n
 * (clamped to [1, min(16, K/128)]) for the kernels that support split-K. */
int qoq_gemm_plan_splits(int64_t M, int64_t N, int64_t K);

/* Name of the index-th kernel configuration the library contains (0-based), NULL past
 * the last.  Forcing one of these names (qoq_set_plan_override) makes the GEMM entry
 * points use that configuration for every shape. */
const char *qoq_gemm_config_name(int index);

/* Planner overrides, for measurement and verification only: results are identical
 * under every override, only the speed changes.
 *   gemm_config    a name from qoq_gemm_config_name, used for every GEMM shape
 *                  (tiled-code entry points take it only if it is a few-token
 *                  configuration); NULL or "" = none
 *   splits         split-K factor for the kernels that support it (clamped to
 *                  [1, min(16, K/128)]); 0 = none
 *   regime         "skinny" (few-token kernels) or "tiled" (tile kernels); NULL or
 *                  "" = none
 *   linear_config  a name from qoq_linear_config_name or "unfused"; NULL or "" = none
 * The call replaces all four values at once (all NULL / 0 clears them).  Their
 * initial values come from the environment, read once per process:
 * QOQ_GEMM_CONFIG, QOQ_GEMM_SPLITS, QOQ_GEMM_REGIME, QOQ_LINEAR_CONFIG.  The values
 * are process-wide: set them only while no other thread plans or launches a GEMM.
 * Errors: INVALID for an unknown name or a negative split factor (nothing changes). */
int qoq_set_plan_override(const char *gemm_config, int32_t splits, const char *regime,
                          const char *linear_config);

/* ---- diagnostics (verification and measurement; not on the GEMM path) ---- */

/* Dequantize packed weights with the GEMM's own in-register routine:
 * w_i8 [N,K] row-major int8 = (q_u4 - z) * s_u8.  Same buffer rules as the GEMM.
 * Errors: INVALID, UNSUPPORTED, ALIGNMENT, HIP. */
int qoq_dequantize_packed(const void *packed_w, const void *group_meta, int64_t N,
                          int64_t K, int32_t group, void *w_i8, void *stream);

/* Plain device-to-device copy kernel of `bytes` bytes (bytes % 16 == 0, both
 * pointers 16-byte aligned): the streaming ceiling and the reference for hardware
 * byte counters.  Errors: INVALID, ALIGNMENT, HIP. */
int qoq_stream_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Read-only streaming kernel over `bytes` bytes (bytes % 16 == 0, src 16-byte
 * aligned): `blocks` workgroups of 256 threads, each thread keeping `unroll` (1, 4
 * or 8) 16-byte loads in flight; `sink` (4 bytes, device) is written only in a case
 * the data never produces.  Measures the practical HBM read ceiling for a given
 * size.  Errors: INVALID, ALIGNMENT, HIP. */
int qoq_stream_read(const void *src, size_t bytes, void *sink, int unroll, int blocks, void *stream);

/* MFMA-only throughput kernel: `blocks` workgroups of 4 waves, each wave running
 * `iters` rounds of 4 independent v_mfma_i32_32x32x32_i8 on register operands
 * (65536 INT8 ops each; 262144 ops per wave per round).  Measures the practical INT8 matrix-core ceiling; `sink`
 * (4 bytes, device) is written only in a case that does not occur.
 * Errors: INVALID, ALIGNMENT, HIP. */
int qoq_mfma_peak(int iters, int blocks, void *sink, void *stream);

/* qoq_mfma_peak on operands read from memory: each lane loads eight A fragments
 * from `a` and eight B fragments from `b` (16 bytes each, at positions spread over
 * the buffers; a_bytes, b_bytes >= 16) and the loop cycles through them.  Fed with
 * a GEMM's own activation codes and dequantized weights it gives the matrix-core
 * ceiling for that data: the chip's clock under MFMA load depends on how much the
 * operands toggle.  Errors: INVALID, ALIGNMENT, HIP. */
int qoq_mfma_peak_operands(const void *a, size_t a_bytes, const void *b, size_t b_bytes, int iters,
                           int blocks, void *sink, void *stream);

/* One v_mfma_i32_16x16x64_i8 on a single wave: lane l supplies 16 A bytes at
 * a_frag + 16*l and 16 B bytes at b_frag + 16*l and receives its 4 INT32 results at
 * d_frag + 16*l.  Used to pin the operand and result lane layout.
 * Errors: INVALID, ALIGNMENT, HIP. */
int qoq_mfma_probe(const void *a_frag, const void *b_frag, void *d_frag, void *stream);

/* One v_mfma_i32_32x32x32_i8 on a single wave: lane l supplies 16 A bytes at
 * a_frag + 16*l and 16 B bytes at b_frag + 16*l and receives its 16 INT32 results at
 * d_frag + 64*l.  Errors: INVALID, ALIGNMENT, HIP. */
int qoq_mfma_probe32(const void *a_frag, const void *b_frag, void *d_frag, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QOQ_H */
