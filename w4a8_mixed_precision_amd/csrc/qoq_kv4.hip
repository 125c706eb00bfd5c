// KV4: per-head dynamic INT4 KV cache write and decode attention (gfx950).
//
// "QServe: W4A8KV4 Quantization and System Co-design ..." summary: the attention
// o_h = softmax(q_h K_{h_KV}^T / sqrt(D)) V_{h_KV}, h_KV = floor(h / r); the integer
// quantizer round(X / s + z), s = (max - min) / 15, dequantized (Q - z) s; a paged
// KV cache with each head's FP16 scale and zero stored in the page right after its
// quantized features; KV4 attention in FP16.  "QServe：把 W4A8KV4 ..." review §3.2
// (per-head dynamic KV quantization, online update) and §4 steps 4-5 (decode reads
// INT4 K / V from pages with two operations per element to dequantize, FP16 QK and
// SV products; the write path quantizes each new token's k / v per head).
//
// MI355X mapping (this library's own): both contractions run on the matrix cores
// (v_mfma_f32_16x16x16_f16: FP16 inputs, FP32 accumulation); dequantization on the
// vector ALU with packed FP16 (bias 1024 + code, exact subtraction of 1024 + z, one
// rounded multiply by s: two packed operations per pair of values).  A wave works
// on blocks of 16 tokens and keeps everything in registers:
//   S^T = K_hat q^T      A = K_hat (16 tokens x 16 dims per k step), B = q^T
//                        -> lane l holds head l % 16, tokens 4 (l / 16) + i
//   online softmax per head (the lane's own head)
//   O^T += V_hat^T P^T   A = V_hat^T (16 dims x 16 tokens), B = P^T straight from
//                        the softmax registers -> lane l holds head l % 16
// so the cache is stored in the matrix instructions' operand order (below), one
// 16-byte load per lane per 16-token block for K and one for V.
//
// Page layout (kPageTokens tokens, head dim 128): for page p and KV head g, kPageBytes
// at (p * H_KV + g) * kPageBytes:
//   [0, 4096)     K codes, 16-token block b at b * 1024; lane slot L = 16 qd + t
//                 (token t of the block, dim quarter qd) at L * 16: byte 2j + e
//                 holds dims 16 j + 4 qd + 2 e (low nibble) and + 1 (high nibble),
//                 j = 0..7, e = 0, 1
//   [4096, 8192)  V codes, block b at 4096 + b * 1024; lane slot L = 16 qt + dd
//                 (token quarter qt, dim dd of a 16-dim block) at L * 16: byte
//                 2 cb + e holds tokens 4 qt + 2 e (low) and + 1 (high) of dim
//                 16 cb + dd, cb = 0..7
//   [8192, 8704)  fp16 K scales [64], K zeros [64], V scales [64], V zeros [64]
#include "qoq_device.h"
#include "qoq_internal.h"

#include <math.h>

#include <algorithm>

namespace qoq {

namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kP = kKv4PageTokens;           // tokens per page (64)
constexpr int kKCodes = 0;
constexpr int kVCodes = kP * kD / 2;          // 4096
constexpr int kKScale = 2 * kVCodes;          // 8192
constexpr int kKZero = kKScale + 2 * kP;
constexpr int kVScale = kKZero + 2 * kP;
constexpr int kVZero = kVScale + 2 * kP;
static_assert(kVZero + 2 * kP == kKv4PageBytes, "page layout");

__device__ __forceinline__ f4 mfma_f16(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h2 bits_h2(unsigned u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ unsigned h2_bits(h2 v) { return __builtin_bit_cast(unsigned, v); }

// two 4-bit codes (low, high nibble of byte b) -> fp16 pair (1024 + c0, 1024 + c1)
__device__ __forceinline__ h2 biased_pair(unsigned b) {
  return bits_h2((b & 0xfu) | ((b & 0xf0u) << 12) | 0x64006400u);
}

// ---------------------------------------------------------------------------
// KV write: one wave per (sequence, KV head); the new tokens of the sequence one
// after another (the V bytes it touches hold two tokens, so one writer per page).
// Lane l holds dims 2l, 2l + 1.  Quantization (per token and head): range widened
// to contain 0, s = fp16(fp32(hi - lo) / 15), z = rne(-lo / s), q = clamp(z +
// rne(x / s), 0, 15), fp32 IEEE quotients; s and z stored as fp16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_min_f32(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off, 64));
  return v;
}

// codes of the lane's two values and the vector's (s, z)
__device__ __forceinline__ void kv_quant2(float x0, float x1, unsigned &c0, unsigned &c1, __half &sh, __half &zh) {
  const float lo = fminf(wave_min_f32(fminf(x0, x1)), 0.0f);
  const float hi = fmaxf(wave_max_f32(fmaxf(x0, x1)), 0.0f);
  float range = hi - lo;
  __asm__ volatile("" : "+v"(range));                 // fp32 difference, then the divide
  sh = __float2half_rn(__fdiv_rn(range, 15.0f));
  const float s = __half2float(sh);
  if (s == 0.0f) {
    c0 = c1 = 0u;
    zh = __float2half_rn(0.0f);
    return;
  }
  const float z = rintf(__fdiv_rn(-lo, s));
  zh = __float2half_rn(z);
  c0 = static_cast<unsigned>(fminf(fmaxf(z + rintf(__fdiv_rn(x0, s)), 0.0f), 15.0f));
  c1 = static_cast<unsigned>(fminf(fmaxf(z + rintf(__fdiv_rn(x1, s)), 0.0f), 15.0f));
}

// Positions and page ids are data the host cannot check: a token whose position
// falls outside the page table, or whose page id lies outside the pool, is skipped
// (a bad table gives wrong contents, never an access outside the buffers).
__global__ __launch_bounds__(64) void kv4_write_kernel(const __half *__restrict__ k_new,
                                                       const __half *__restrict__ v_new, int n_new, int h_kv,
                                                       const int *__restrict__ positions,
                                                       const int *__restrict__ page_table, int max_pages,
                                                       int num_pages, uint8_t *__restrict__ pool) {
  const int b = blockIdx.y, g = blockIdx.x, lane = threadIdx.x;
  const int d0 = 2 * lane;
  for (int i = 0; i < n_new; ++i) {
    const int pos = positions[b] + i;                  // the same in every lane
    if (pos < 0 || pos / kP >= max_pages) continue;
    const int page = page_table[static_cast<size_t>(b) * max_pages + pos / kP];
    if (page < 0 || page >= num_pages) continue;
    const int slot = pos % kP;
    uint8_t *pg = pool + (static_cast<size_t>(page) * h_kv + g) * kKv4PageBytes;
    const size_t src = ((static_cast<size_t>(b) * n_new + i) * h_kv + g) * kD + d0;
    const unsigned kw = *reinterpret_cast<const unsigned *>(k_new + src);
    const unsigned vw = *reinterpret_cast<const unsigned *>(v_new + src);
    unsigned c0, c1;
    __half sh, zh;
    // K: dims d0, d0 + 1 share one byte
    kv_quant2(half_bits_to_float(kw & 0xffffu), half_bits_to_float(kw >> 16), c0, c1, sh, zh);
    {
      const int blk = slot >> 4, t = slot & 15;
      const int j = d0 >> 4, qd = (d0 & 15) >> 2, e = (d0 & 3) >> 1;
      pg[kKCodes + blk * 1024 + (16 * qd + t) * 16 + 2 * j + e] = static_cast<uint8_t>(c0 | (c1 << 4));
      if (lane == 0) {
        reinterpret_cast<__half *>(pg + kKScale)[slot] = sh;
        reinterpret_cast<__half *>(pg + kKZero)[slot] = zh;
      }
    }
    // V: one nibble of each of two bytes (the other nibble is a neighbouring token)
    kv_quant2(half_bits_to_float(vw & 0xffffu), half_bits_to_float(vw >> 16), c0, c1, sh, zh);
    {
      const int blk = slot >> 4, t = slot & 15;
      const int qt = t >> 2, ti = t & 3, e = ti >> 1, hi = ti & 1;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int d = d0 + u;
        const int cb = d >> 4, dd = d & 15;
        uint8_t *p = pg + kVCodes + blk * 1024 + (16 * qt + dd) * 16 + 2 * cb + e;
        const unsigned c = u ? c1 : c0;
        const unsigned old = *p;
        *p = static_cast<uint8_t>(hi ? ((old & 0x0fu) | (c << 4)) : ((old & 0xf0u) | c));
      }
      if (lane == 0) {
        reinterpret_cast<__half *>(pg + kVScale)[slot] = sh;
        reinterpret_cast<__half *>(pg + kVZero)[slot] = zh;
      }
    }
    __syncthreads();                                   // the next token may share V bytes
  }
}

// ---------------------------------------------------------------------------
// Decode attention.  Workgroup (split s, KV head g, sequence b), 4 waves; the split
// covers 16-token blocks [s * bps, min(nblk, (s + 1) * bps)), wave w every 4th of
// them.  Per wave: m, l (fp32, for the lane's head) and O^T (32 fp32 per lane).  The
// waves merge through LDS; one split writes o directly, several write unnormalized
// partials (O, m, l) that kv4_combine_kernel merges.
// ---------------------------------------------------------------------------
constexpr int kAttnWaves = 4;

struct AttnPartial {
  float o[8][4];
  float m, l;
};

__global__ __launch_bounds__(64 * kAttnWaves) void kv4_attention_kernel(
    const __half *__restrict__ q, const uint8_t *__restrict__ pool, const int *__restrict__ page_table,
    int max_pages, int num_pages, const int *__restrict__ seq_lens, int max_len, int h, int h_kv, int bps,
    float scale, __half *__restrict__ out, float *__restrict__ ws_o, float *__restrict__ ws_ml) {
  __shared__ float red[kAttnWaves][34][64];
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int splits = gridDim.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = h / h_kv;
  const int hl = lane & 15, quad = lane >> 4;
  const int len = min(max(seq_lens[b], 1), max_len);   // data: clamped to what the table covers
  const int nblk = (len + 15) >> 4;
  const int blk0 = s * bps, blk1 = min(nblk, blk0 + bps);

  // q^T as the B operand of S^T = K_hat q^T: lane holds head hl, dims 16 j + 4 quad + 0..3
  h4 qf[8];
  {
    const int head = g * r + hl;
    const __half *qr = q + (static_cast<size_t>(b) * h + (hl < r ? head : 0)) * kD;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint2 w = hl < r ? *reinterpret_cast<const uint2 *>(qr + 16 * j + 4 * quad) : make_uint2(0u, 0u);
      qf[j] = __builtin_bit_cast(h4, w);
    }
  }
  float m = -INFINITY, l = 0.0f;
  f4 o[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) o[cb] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int blk = blk0 + wave; blk < blk1; blk += kAttnWaves) {
    const int tok0 = blk * 16;
    const int page = min(max(page_table[static_cast<size_t>(b) * max_pages + tok0 / kP], 0), num_pages - 1);
    const uint8_t *pg = pool + (static_cast<size_t>(page) * h_kv + g) * kKv4PageBytes;
    const int pb = (tok0 % kP) >> 4;                  // block within the page
    // loads: K fragment (token hl), V fragment (tokens 4 quad + 0..3), their stats
    const uint4 kc = *reinterpret_cast<const uint4 *>(pg + kKCodes + pb * 1024 + lane * 16);
    const uint4 vc = *reinterpret_cast<const uint4 *>(pg + kVCodes + pb * 1024 + lane * 16);
    const int tk = pb * 16 + hl;                       // the lane's K token in the page
    const int tv = pb * 16 + 4 * quad;                 // first of the lane's V tokens
    unsigned ks = reinterpret_cast<const unsigned short *>(pg + kKScale)[tk];
    unsigned kz = reinterpret_cast<const unsigned short *>(pg + kKZero)[tk];
    uint2 vs = *reinterpret_cast<const uint2 *>(pg + kVScale + 2 * tv);
    uint2 vz = *reinterpret_cast<const uint2 *>(pg + kVZero + 2 * tv);
    // tokens past the sequence: scale and zero 0 -> dequantized 0, whatever the codes
    if (tok0 + hl >= len) ks = kz = 0u;
    {
      const int valid = len - (tok0 + 4 * quad);        // how many of the 4 V tokens exist
      if (valid < 4) {
        const unsigned keep0 = valid > 0 ? 0xffffu : 0u, keep1 = valid > 1 ? 0xffff0000u : 0u;
        const unsigned keep2 = valid > 2 ? 0xffffu : 0u;
        vs.x &= keep0 | keep1;
        vz.x &= keep0 | keep1;
        vs.y &= keep2;
        vz.y &= keep2;
      }
    }
    // K_hat fragment: (1024 + c) - (1024 + z), times s (two packed ops per pair)
    const h2 kbias = bits_h2((kz | (kz << 16)) ^ 0x80008000u) - bits_h2(0x64006400u);   // -z - 1024
    const h2 ks2 = bits_h2(ks | (ks << 16));
    const unsigned kw[4] = {kc.x, kc.y, kc.z, kc.w};
    f4 st = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const unsigned w = kw[j >> 1] >> (16 * (j & 1));
      const h2 p0 = (biased_pair(w & 0xffu) + kbias) * ks2;
      const h2 p1 = (biased_pair((w >> 8) & 0xffu) + kbias) * ks2;
      const h4 a = {p0[0], p0[1], p1[0], p1[1]};
      st = mfma_f16(a, qf[j], st);
    }
    // scores of the lane's head for tokens tok0 + 4 quad + i; softmax update
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = (tok0 + 4 * quad + i < len) ? st[i] * scale : -INFINITY;
    float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const float mn = fmaxf(m, bm);                     // finite: every block has a valid token
    const float alpha = expf(m - mn);                  // m = -inf at first: 0
    float p[4], ps = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = expf(sc[i] - mn);
      ps += p[i];
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l = l * alpha + ps;
    m = mn;
    const h4 pf = {static_cast<_Float16>(p[0]), static_cast<_Float16>(p[1]), static_cast<_Float16>(p[2]),
                   static_cast<_Float16>(p[3])};
    // V_hat^T fragments and O^T += V_hat^T P^T
    const h2 vs01 = bits_h2(vs.x), vs23 = bits_h2(vs.y);
    const h2 vb01 = bits_h2(vz.x ^ 0x80008000u) - bits_h2(0x64006400u);
    const h2 vb23 = bits_h2(vz.y ^ 0x80008000u) - bits_h2(0x64006400u);
    const unsigned vw[4] = {vc.x, vc.y, vc.z, vc.w};
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const unsigned w = vw[cb >> 1] >> (16 * (cb & 1));
      const h2 p0 = (biased_pair(w & 0xffu) + vb01) * vs01;
      const h2 p1 = (biased_pair((w >> 8) & 0xffu) + vb23) * vs23;
      const h4 a = {p0[0], p0[1], p1[0], p1[1]};
      o[cb] = mfma_f16(a, pf, o[cb] * alpha);
    }
  }

  // merge the waves: partials through LDS, wave 0 combines
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][cb * 4 + i][lane] = o[cb][i];
  red[wave][32][lane] = m;
  red[wave][33][lane] = l;
  __syncthreads();
  if (wave != 0) return;
  float mm = -INFINITY;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) mm = fmaxf(mm, red[w][32][lane]);
  float ll = 0.0f, f[kAttnWaves];
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) {
    const float mw = red[w][32][lane];
    f[w] = mw == -INFINITY ? 0.0f : expf(mw - mm);    // a wave with no block adds nothing
    ll += red[w][33][lane] * f[w];
  }
  const int head = g * r + hl;
  if (hl >= r) return;
  if (splits == 1) {
    const float inv = 1.0f / ll;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      __half v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float acc = 0.0f;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) acc += red[w][cb * 4 + i][lane] * f[w];
        v4[i] = __float2half_rn(acc * inv);
      }
      // O^T row (dim) 16 cb + 4 quad + i, column (head) hl
      *reinterpret_cast<uint2 *>(out + (static_cast<size_t>(b) * h + head) * kD + 16 * cb + 4 * quad) =
          *reinterpret_cast<const uint2 *>(v4);
    }
    return;
  }
  const size_t pidx = (static_cast<size_t>(s) * gridDim.z + b) * h + head;
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) {
    f4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) acc += red[w][cb * 4 + i][lane] * f[w];
      v[i] = acc;
    }
    *reinterpret_cast<f4 *>(ws_o + pidx * kD + 16 * cb + 4 * quad) = v;
  }
  if (quad == 0) {
    ws_ml[2 * pidx] = mm;
    ws_ml[2 * pidx + 1] = ll;
  }
}

// o[b, head] = sum_s O_s exp(m_s - m) / sum_s l_s exp(m_s - m); a split with no
// tokens has m = -inf and adds nothing
__global__ __launch_bounds__(kD) void kv4_combine_kernel(const float *__restrict__ ws_o,
                                                         const float *__restrict__ ws_ml, int splits, int bh,
                                                         __half *__restrict__ out) {
  const int row = blockIdx.x, d = threadIdx.x;
  float mm = -INFINITY;
  for (int s = 0; s < splits; ++s) mm = fmaxf(mm, ws_ml[2 * (static_cast<size_t>(s) * bh + row)]);
  float acc = 0.0f, ll = 0.0f;
  for (int s = 0; s < splits; ++s) {
    const size_t p = static_cast<size_t>(s) * bh + row;
    const float ms = ws_ml[2 * p];
    if (ms == -INFINITY) continue;
    const float f = expf(ms - mm);
    ll += ws_ml[2 * p + 1] * f;
    acc += ws_o[p * kD + d] * f;
  }
  out[static_cast<size_t>(row) * kD + d] = __float2half_rn(acc / ll);
}

}  // namespace

int kv4_splits(int64_t B, int64_t h_kv, int64_t max_len) {
  const int64_t nblk = (max_len + 15) / 16;
  const int64_t want = (kKv4TargetWorkgroups + B * h_kv - 1) / (B * h_kv);
  // at least 4 blocks (one per wave) per split, at most kKv4MaxSplits splits
  const int64_t s = std::min<int64_t>({want, (nblk + 3) / 4, kKv4MaxSplits});
  return static_cast<int>(std::max<int64_t>(1, s));
}

size_t kv4_workspace_need(int64_t B, int64_t h, int64_t h_kv, int64_t max_len) {
  const int s = kv4_splits(B, h_kv, max_len);
  if (s == 1) return 0;
  return static_cast<size_t>(s) * B * h * (kD + 2) * sizeof(float);
}

void launch_kv4_write(const void *k_new, const void *v_new, int64_t B, int64_t n_new, int64_t h_kv,
                      const int *positions, const int *page_table, int64_t max_pages, int64_t num_pages, void *pool,
                      hipStream_t st) {
  hipLaunchKernelGGL(kv4_write_kernel, dim3(static_cast<unsigned>(h_kv), static_cast<unsigned>(B)), dim3(64), 0, st,
                     static_cast<const __half *>(k_new), static_cast<const __half *>(v_new), static_cast<int>(n_new),
                     static_cast<int>(h_kv), positions, page_table, static_cast<int>(max_pages),
                     static_cast<int>(num_pages), static_cast<uint8_t *>(pool));
}

void launch_kv4_attention(const void *q, const void *pool, int64_t num_pages, const int *page_table,
                          int64_t max_pages, const int *seq_lens, int64_t B, int64_t h, int64_t h_kv,
                          int64_t max_len, void *out, void *ws, hipStream_t st) {
  const int splits = kv4_splits(B, h_kv, max_len);
  const int64_t nblk = (max_len + 15) / 16;
  const int bps = static_cast<int>((nblk + splits - 1) / splits);
  float *wo = static_cast<float *>(ws);
  float *wml = splits > 1 ? wo + static_cast<size_t>(splits) * B * h * kD : nullptr;
  const float scale = 1.0f / sqrtf(static_cast<float>(kD));
  hipLaunchKernelGGL(kv4_attention_kernel,
                     dim3(static_cast<unsigned>(splits), static_cast<unsigned>(h_kv), static_cast<unsigned>(B)),
                     dim3(64 * kAttnWaves), 0, st, static_cast<const __half *>(q),
                     static_cast<const uint8_t *>(pool), page_table, static_cast<int>(max_pages),
                     static_cast<int>(num_pages), seq_lens, static_cast<int>(max_len), static_cast<int>(h),
                     static_cast<int>(h_kv), bps, scale, static_cast<__half *>(out), wo, wml);
  if (splits > 1)
    hipLaunchKernelGGL(kv4_combine_kernel, dim3(static_cast<unsigned>(B * h)), dim3(kD), 0, st, wo, wml, splits,
                       static_cast<int>(B * h), static_cast<__half *>(out));
}

}  // namespace qoq
