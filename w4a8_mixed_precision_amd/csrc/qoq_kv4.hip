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
// vector ALU with packed FP16.  A wave works on blocks of 16 tokens and keeps
// everything in registers:
//   S^T = K_hat q^T      A = K_hat (16 tokens x 16 dims per k step), B = q^T
//                        -> lane l holds head l % 16, tokens 4 (l / 16) + i
//   online softmax per head (the lane's own head), base 2
//   O^T += V_hat^T P^T   A = V_hat^T (16 dims x 16 tokens), B = P^T straight from
//                        the softmax registers -> lane l holds head l % 16
// so the cache is stored in the matrix instructions' operand order (below), one
// 16-byte load per lane per 16-token block for K and one for V.
//
// Dequantization of a pair of codes: the codes sit in nibbles k and k + 4 of a
// 32-bit word, so one and-or with 0x000f000f (nibbles 0 and 4) or 0x00f000f0 (1 and
// 5) against the fp16 bit pattern of 1024 or 64 (whose mantissa steps are 1 and 1/16)
// gives the fp16 pair (base + c0, base + c1) exactly; nibbles 2, 6 and 3, 7 the same
// after one shift by 8.  Then (base + c) - (base + z) = c - z exactly, and one
// rounded multiply by s: K_hat = fp16((c - z) s).  Two packed FP16 operations per
// pair of values after the extraction.
//
// Page layout (kPageTokens = 64 tokens, head dim 128): for page p and KV head g,
// kPageBytes at (p * H_KV + g) * kPageBytes:
//   [0, 4096)     K codes, 16-token block b at b * 1024; lane slot L = 16 qd + t
//                 (token t of the block, dim quarter qd) at L * 16; 32-bit word u
//                 (u = 0..3) of the slot, nibble k (bits 4k..4k+3) holds dim
//                 16 (2u + (k >> 1 & 1)) + 4 qd + 2 (k & 1) + (k >> 2)
//   [4096, 8192)  V codes, block b at 4096 + b * 1024; lane slot L = 16 qt + dd
//                 (token quarter qt, dim dd of a 16-dim block) at L * 16; word u,
//                 nibble k holds token 4 qt + 2 (k & 1) + (k >> 2) of dim
//                 16 (2u + (k >> 1 & 1)) + dd
//   [8192, 8448)  K statistics: token t at 8192 + 4t, fp16 scale (low half) and
//                 fp16 zero (high half)
//   [8448, 8704)  V statistics: tokens 4 qg .. 4 qg + 3 at 8448 + 16 qg, their four
//                 fp16 scales then their four fp16 zeros
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
constexpr int kKStats = 2 * kVCodes;          // 8192: (scale, zero) per token
constexpr int kVStats = kKStats + 4 * kP;     // 8448: 4 scales, 4 zeros per 4 tokens
static_assert(kVStats + 4 * kP == kKv4PageBytes, "page layout");

__device__ __forceinline__ f4 mfma_f16(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h2 bits_h2(unsigned u) { return __builtin_bit_cast(h2, u); }

constexpr unsigned kBase1024 = 0x64006400u, kBase64 = 0x54005400u;

// The extraction masks live in registers so that (w & mask) | base is one
// v_and_or_b32 (the base from a scalar register; one scalar operand per
// instruction); as literals the compiler splits it into an and and an or.
struct NibbleMasks {
  unsigned lo, hi;
};
__device__ __forceinline__ NibbleMasks nibble_masks() {
  NibbleMasks m;
  __asm__ volatile("v_mov_b32 %0, 0x000f000f" : "=v"(m.lo));
  __asm__ volatile("v_mov_b32 %0, 0x00f000f0" : "=v"(m.hi));
  return m;
}
__device__ __forceinline__ unsigned and_or(unsigned w, unsigned mask, unsigned base) {
  unsigned r;
  __asm__("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "v"(mask), "s"(base));
  return r;
}
// nibbles 0 and 4 of w -> (1024 + c0, 1024 + c4); nibbles 1 and 5 -> (64 + c1, 64 + c5)
__device__ __forceinline__ h2 pair_lo(unsigned w, const NibbleMasks &nm) { return bits_h2(and_or(w, nm.lo, kBase1024)); }
__device__ __forceinline__ h2 pair_hi(unsigned w, const NibbleMasks &nm) { return bits_h2(and_or(w, nm.hi, kBase64)); }

// -(base + z) for a pair of fp16 zeros (exact: z is an integer in [-1024, 1024], so
// base + z lies within FP16's exact integers for base 64 and 1024, and so does
// (base + c) - (base + z) = c - z)
__device__ __forceinline__ h2 neg_biased(unsigned zz, unsigned base) {
  const h2 v = bits_h2(zz) + bits_h2(base);
  return bits_h2(__builtin_bit_cast(unsigned, v) ^ 0x80008000u);
}

// ---------------------------------------------------------------------------
// KV write: one wave per (KV head, sequence, 16-token block of positions), four
// consecutive blocks per workgroup (single-wave workgroups leave most of the chip
// idle: the dispatcher, not the work, sets the pace).  The block is the one 16-token
// block of the page that the new tokens' positions fall in (counted from the one
// holding the sequence's first new position), so no two waves of a launch touch the
// same page words.  Lane
// l = 4 t + u holds dims 32 u .. 32 u + 31 of token t of the block (K and V, all
// loads issued at once); per token and head: the vector's own range (widened to
// contain 0 only where kv_scale_zero says so), s = fp16(fp32(hi - lo) / 15),
// z = rne(-lo / s), q = clamp(z + rne(x / s), 0, 15),
// fp32 IEEE quotients, s and z stored as fp16; min and max over the token's four
// lanes by two xor steps.  Word u of every K slot of token t takes its nibbles from
// dims 32 u .. 32 u + 31 only, so lane (t, u) builds those four words in registers;
// the wave's K stores cover 256 contiguous bytes each.  A V word holds four tokens,
// so the V codes go through LDS and each V word is assembled once for the block,
// merged with the nibbles of tokens outside the new range.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float quad_max_f32(float v) {
  v = fmaxf(v, __shfl_xor(v, 1, 64));
  return fmaxf(v, __shfl_xor(v, 2, 64));
}
__device__ __forceinline__ float quad_min_f32(float v) {
  v = fminf(v, __shfl_xor(v, 1, 64));
  return fminf(v, __shfl_xor(v, 2, 64));
}

// Scale and zero of one vector from its minimum and maximum: the quantizer over
// the vector's own range, s = fp16(fp32(hi - lo) / 15), z = rne(fp32(-lo / s));
// where that has no usable result (s = 0: a constant vector; |z| > kZLimit: a
// narrow range far from 0, where q - z would leave FP16's exact integers) the same
// over the range widened to contain 0, which puts z in [0, 15].  s == 0 on return
// only for an all-zero vector (z = 0 then).
constexpr float kZLimit = 1024.0f;

__device__ __forceinline__ void kv_scale_zero_once(float lo, float hi, __half &sh, float &s, float &z) {
  float range = hi - lo;
  __asm__ volatile("" : "+v"(range));                 // fp32 difference, then the divide
  sh = __float2half_rn(__fdiv_rn(range, 15.0f));
  s = __half2float(sh);
  z = s == 0.0f ? 0.0f : rintf(__fdiv_rn(-lo, s));
}

__device__ __forceinline__ void kv_scale_zero(float lo, float hi, __half &sh, float &s, float &z) {
  kv_scale_zero_once(lo, hi, sh, s, z);
  if (s == 0.0f || fabsf(z) > kZLimit) kv_scale_zero_once(fminf(lo, 0.0f), fmaxf(hi, 0.0f), sh, s, z);
}

// codes of the lane's 32 values and the token's (s, z); the token's 128 values sit
// in four consecutive lanes
__device__ __forceinline__ void kv_quant32(const float (&x)[32], unsigned (&c)[32], __half &sh, __half &zh) {
  float lo = x[0], hi = x[0];
#pragma unroll
  for (int j = 1; j < 32; ++j) {
    lo = fminf(lo, x[j]);
    hi = fmaxf(hi, x[j]);
  }
  float s, z;
  kv_scale_zero(quad_min_f32(lo), quad_max_f32(hi), sh, s, z);
  if (s == 0.0f) {
#pragma unroll
    for (int j = 0; j < 32; ++j) c[j] = 0u;
    zh = __float2half_rn(0.0f);
    return;
  }
  zh = __float2half_rn(z);
  // x / s as x * fp32(1 / s): |x / s| <= |z| + 15.5 <= 1040 here (x lies in the
  // range, whose low end is -z s to half a step), so the product (two roundings)
  // and the correctly rounded quotient differ by at most 1040 (2^-23 + 2^-24) <
  // 2^-12, and rint decides the same way unless the product lies within 2^-12 of a
  // half-integer; those rare values take the IEEE divide (a branch the wave takes
  // only when one of its lanes needs it)
  const float y = __fdiv_rn(1.0f, s);
  float q[32];
  float gap = 1.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    q[j] = x[j] * y;
    gap = fminf(gap, half_gap(q[j]));
  }
  if (__ballot(gap < 0x1p-12f) != 0) {
#pragma unroll
    for (int j = 0; j < 32; ++j)
      if (half_gap(q[j]) < 0x1p-12f) q[j] = __fdiv_rn(x[j], s);
  }
#pragma unroll
  for (int j = 0; j < 32; ++j) c[j] = static_cast<unsigned>(fminf(fmaxf(z + rintf(q[j]), 0.0f), 15.0f));
}

__device__ __forceinline__ unsigned half_bits(__half h) { return __builtin_bit_cast(unsigned short, h); }

__device__ __forceinline__ void halves_to_f32(const uint4 (&w)[4], float (&x)[32]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned d[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * i + 2 * e] = half_bits_to_float(d[e] & 0xffffu);
      x[8 * i + 2 * e + 1] = half_bits_to_float(d[e] >> 16);
    }
  }
}

constexpr int kWriteWaves = 4;                     // 16-token blocks (one per wave) per workgroup

// Positions and page ids are data the host cannot check: a block whose position
// falls outside the page table, or whose page id lies outside the pool, is skipped
// (a bad table gives wrong contents, never an access outside the buffers).
__global__ __launch_bounds__(64 * kWriteWaves) __attribute__((amdgpu_waves_per_eu(4))) void kv4_write_block_kernel(
    const __half *__restrict__ k_new, const __half *__restrict__ v_new, int n_new, int h_kv,
    const int *__restrict__ positions, const int *__restrict__ page_table, int max_pages, int num_pages,
    uint8_t *__restrict__ pool) {
  __shared__ __attribute__((aligned(16))) uint8_t vcode_all[kWriteWaves][16][kD];
  const int g = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint8_t(&vcode)[16][kD] = vcode_all[wave];
  const int pos0 = positions[b];                     // the same in the whole workgroup
  if (pos0 < 0 || pos0 >= (1 << 30)) return;         // past any page table (max_pages <= 2^24)
  const int blk = pos0 / 16 + kWriteWaves * static_cast<int>(blockIdx.z) + wave;   // absolute 16-token block
  const int p_lo = max(pos0, 16 * blk), p_hi = min(pos0 + n_new, 16 * blk + 16);
  int page = -1;
  if (p_lo < p_hi && blk / 4 < max_pages) page = page_table[static_cast<size_t>(b) * max_pages + blk / 4];
  // the same in the whole wave; an inactive wave skips its work but meets the barrier
  const bool active = page >= 0 && page < num_pages;
  uint8_t *pg = pool + (static_cast<size_t>(active ? page : 0) * h_kv + g) * kKv4PageBytes;
  const int pb = blk & 3;                            // block within the page
  if (active) {
    const int t = lane >> 2, u = lane & 3;
    const int p = 16 * blk + t;
    const bool fresh = p >= p_lo && p < p_hi;        // the same in the token's four lanes

    float kx[32], vx[32];
    {
      uint4 kw[4], vw[4];
      const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
      const size_t src = ((static_cast<size_t>(b) * n_new + (fresh ? p - pos0 : 0)) * h_kv + g) * kD + 32 * u;
      const uint4 *kp = reinterpret_cast<const uint4 *>(k_new + src);
      const uint4 *vp = reinterpret_cast<const uint4 *>(v_new + src);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kw[i] = fresh ? kp[i] : zero;
        vw[i] = fresh ? vp[i] : zero;
      }
      halves_to_f32(kw, kx);
      halves_to_f32(vw, vx);
    }
    unsigned kc[32], vc[32];
    __half ksh, kzh, vsh, vzh;
    kv_quant32(kx, kc, ksh, kzh);
    kv_quant32(vx, vc, vsh, vzh);

    if (fresh) {
      // K: word u of slot (qd, t); nibble k holds dim 32 u + 16 (k >> 1 & 1) + 4 qd + 2 (k & 1) + (k >> 2)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        unsigned w = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) w |= kc[16 * ((k >> 1) & 1) + 4 * qd + 2 * (k & 1) + (k >> 2)] << (4 * k);
        *reinterpret_cast<unsigned *>(pg + kKCodes + pb * 1024 + (16 * qd + t) * 16 + 4 * u) = w;
      }
      if (u == 0) {
        const int slot = p & 63;
        *reinterpret_cast<unsigned *>(pg + kKStats + 4 * slot) = half_bits(ksh) | (half_bits(kzh) << 16);
        __half *vst = reinterpret_cast<__half *>(pg + kVStats + 16 * (slot >> 2));
        vst[slot & 3] = vsh;
        vst[4 + (slot & 3)] = vzh;
      }
    }
    unsigned d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = vc[4 * i] | (vc[4 * i + 1] << 8) | (vc[4 * i + 2] << 16) | (vc[4 * i + 3] << 24);
    uint4 *dst = reinterpret_cast<uint4 *>(&vcode[t][32 * u]);
    dst[0] = make_uint4(d[0], d[1], d[2], d[3]);
    dst[1] = make_uint4(d[4], d[5], d[6], d[7]);
  }
  __syncthreads();
  if (!active) return;
  // V: lane slot L = lane (token quarter qt, dim dd), its four words; nibble k of
  // word w holds token 4 qt + 2 (k & 1) + (k >> 2) of dim 16 (2w + (k >> 1 & 1)) + dd
  const int qt = lane >> 4, dd = lane & 15;
  const int t_lo = p_lo - 16 * blk, t_hi = p_hi - 16 * blk;
  if (4 * qt + 4 <= t_lo || 4 * qt >= t_hi) return;  // none of this slot's tokens is new
  const bool whole = 4 * qt >= t_lo && 4 * qt + 4 <= t_hi;
  unsigned *wp = reinterpret_cast<unsigned *>(pg + kVCodes + pb * 1024 + lane * 16);
#pragma unroll
  for (int wu = 0; wu < 4; ++wu) {
    unsigned w = whole ? 0u : wp[wu];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int tk = 4 * qt + 2 * (k & 1) + (k >> 2);
      if (tk >= t_lo && tk < t_hi) {
        const int dk = 16 * (2 * wu + ((k >> 1) & 1)) + dd;
        w = (w & ~(0xfu << (4 * k))) | (static_cast<unsigned>(vcode[tk][dk]) << (4 * k));
      }
    }
    wp[wu] = w;
  }
}

__device__ __forceinline__ float wave_min_f32(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off, 64));
  return v;
}

// codes of the lane's two values and the vector's (s, z)
__device__ __forceinline__ void kv_quant2(float x0, float x1, unsigned &c0, unsigned &c1, __half &sh, __half &zh) {
  float s, z;
  kv_scale_zero(wave_min_f32(fminf(x0, x1)), wave_max_f32(fmaxf(x0, x1)), sh, s, z);
  if (s == 0.0f) {
    c0 = c1 = 0u;
    zh = __float2half_rn(0.0f);
    return;
  }
  zh = __float2half_rn(z);
  c0 = static_cast<unsigned>(fminf(fmaxf(z + rintf(__fdiv_rn(x0, s)), 0.0f), 15.0f));
  c1 = static_cast<unsigned>(fminf(fmaxf(z + rintf(__fdiv_rn(x1, s)), 0.0f), 15.0f));
}

// Few new tokens per sequence (decode): lane l quantizes dims 2l, 2l + 1 of each new
// token of the block in turn (same arithmetic as above, min and max over the whole
// wave), stages the codes in LDS and writes each token's K words as it goes; V words
// as above.  Per token: two quotients per lane instead of the block kernel's 32 for
// each of the 16 tokens it covers whether new or not.
__global__ __launch_bounds__(64) void kv4_write_tokens_kernel(const __half *__restrict__ k_new,
                                                              const __half *__restrict__ v_new, int n_new, int h_kv,
                                                              const int *__restrict__ positions,
                                                              const int *__restrict__ page_table, int max_pages,
                                                              int num_pages, uint8_t *__restrict__ pool) {
  __shared__ uint8_t kcode[16][kD], vcode[16][kD];
  const int g = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int pos0 = positions[b];                     // the same in every lane
  if (pos0 < 0 || pos0 >= (1 << 30)) return;         // past any page table (max_pages <= 2^24)
  const int blk = pos0 / 16 + static_cast<int>(blockIdx.z);     // absolute 16-token block
  const int p_lo = max(pos0, 16 * blk), p_hi = min(pos0 + n_new, 16 * blk + 16);
  if (p_lo >= p_hi || blk / 4 >= max_pages) return;
  const int page = page_table[static_cast<size_t>(b) * max_pages + blk / 4];
  if (page < 0 || page >= num_pages) return;
  uint8_t *pg = pool + (static_cast<size_t>(page) * h_kv + g) * kKv4PageBytes;
  const int pb = blk & 3;                            // block within the page
  const int d0 = 2 * lane;
  for (int p = p_lo; p < p_hi; ++p) {
    const int t = p & 15, slot = p & 63;
    const size_t src = ((static_cast<size_t>(b) * n_new + (p - pos0)) * h_kv + g) * kD + d0;
    const unsigned kw = *reinterpret_cast<const unsigned *>(k_new + src);
    const unsigned vw = *reinterpret_cast<const unsigned *>(v_new + src);
    unsigned c0, c1;
    __half ksh, kzh, vsh, vzh;
    kv_quant2(half_bits_to_float(kw & 0xffffu), half_bits_to_float(kw >> 16), c0, c1, ksh, kzh);
    kcode[t][d0] = static_cast<uint8_t>(c0);
    kcode[t][d0 + 1] = static_cast<uint8_t>(c1);
    kv_quant2(half_bits_to_float(vw & 0xffffu), half_bits_to_float(vw >> 16), c0, c1, vsh, vzh);
    vcode[t][d0] = static_cast<uint8_t>(c0);
    vcode[t][d0 + 1] = static_cast<uint8_t>(c1);
    if (lane == 0) {
      *reinterpret_cast<unsigned *>(pg + kKStats + 4 * slot) = half_bits(ksh) | (half_bits(kzh) << 16);
      __half *vst = reinterpret_cast<__half *>(pg + kVStats + 16 * (slot >> 2));
      vst[slot & 3] = vsh;
      vst[4 + (slot & 3)] = vzh;
    }
    __syncthreads();
    if (lane < 16) {                                 // K: word u of slot (qd, t), this token only
      const int qd = lane >> 2, u = lane & 3;
      unsigned w = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int d = 16 * (2 * u + ((k >> 1) & 1)) + 4 * qd + 2 * (k & 1) + (k >> 2);
        w |= static_cast<unsigned>(kcode[t][d]) << (4 * k);
      }
      *reinterpret_cast<unsigned *>(pg + kKCodes + pb * 1024 + (16 * qd + t) * 16 + 4 * u) = w;
    }
  }
  // V: lane slot L = lane (token quarter qt, dim dd), its four words; nibble k of
  // word u holds token 4 qt + 2 (k & 1) + (k >> 2) of dim 16 (2u + (k >> 1 & 1)) + dd
  const int qt = lane >> 4, dd = lane & 15;
  const int t_lo = p_lo - 16 * blk, t_hi = p_hi - 16 * blk;
  if (4 * qt + 4 <= t_lo || 4 * qt >= t_hi) return;  // none of this slot's tokens is new
  const bool whole = 4 * qt >= t_lo && 4 * qt + 4 <= t_hi;
  unsigned *wp = reinterpret_cast<unsigned *>(pg + kVCodes + pb * 1024 + lane * 16);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    unsigned w = whole ? 0u : wp[u];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int t = 4 * qt + 2 * (k & 1) + (k >> 2);
      if (t >= t_lo && t < t_hi) {
        const int d = 16 * (2 * u + ((k >> 1) & 1)) + dd;
        w = (w & ~(0xfu << (4 * k))) | (static_cast<unsigned>(vcode[t][d]) << (4 * k));
      }
    }
    wp[u] = w;
  }
}

// ---------------------------------------------------------------------------
// Decode attention.  Workgroup (split s, KV head g, sequence b), kAttnWaves waves;
// the split covers 16-token blocks [s * bps, min(nblk, (s + 1) * bps)) (bps a
// multiple of 4, so splits start on page boundaries), wave w every kAttnWaves-th
// of them.  The page ids of a 64-page window sit one per lane and are read with
// readlane; each wave keeps the next block's codes and statistics in flight while
// it computes the current one (a two-slot ring).  Per wave: m, l (fp32, for the
// lane's head, scores in base-2 units; l summed over the lane's own tokens until
// the end) and O^T (32 fp32 per lane).  The running
// maximum is raised only when a score exceeds it by more than 2^kLazy: in between
// the weights exp2(score - m) stay below 2^kLazy, and the final division by l
// (accumulated against the same m) is unchanged.  The waves merge through LDS; one
// split writes o directly, several write unnormalized partials (O, m, l) that
// kv4_combine_kernel merges.
// ---------------------------------------------------------------------------
#ifndef QOQ_KV4_WAVES
#define QOQ_KV4_WAVES 4
#endif
constexpr int kAttnWaves = QOQ_KV4_WAVES;
constexpr int kWindowBlocks = 4 * 64;              // blocks of the 64 pages one wave's lanes name
constexpr float kLazy = 8.0f;

struct KvBlock {                                   // raw data of one 16-token block, one lane's share
  uint4 kc, vc;                                    // K codes (token hl), V codes (tokens 4 quad + 0..3)
  unsigned ks;                                     // fp16 scale | fp16 zero << 16 of K token hl
  uint4 vs;                                        // fp16 scales (x, y), zeros (z, w) of V tokens 4 quad + 0..3
};

// Buffer loads: the (page, head) section is a buffer resource (its base in scalar
// registers, its size as the range: a load past it returns zeros), the block
// offset a scalar, the lane offsets constant vector registers; no per-block vector
// address arithmetic.  A decode step reads each cached token once, so every load
// carries the streaming (non-temporal) cache hint (kStream, the `nt` bit of the
// cache-policy operand): 3-5 % faster on the decode shapes measured.
typedef unsigned u4v __attribute__((ext_vector_type(4)));
constexpr int kBufferWord3 = 0x00020000;           // raw 32-bit data format
constexpr int kStream = 2;                         // cache policy: non-temporal

__device__ __forceinline__ uint4 as_uint4(u4v v) { return make_uint4(v.x, v.y, v.z, v.w); }

__device__ __forceinline__ void load_block(KvBlock &r, const uint8_t *__restrict__ pool, int page, int h_kv, int g,
                                           int blk, unsigned lane_off, unsigned ks_off, unsigned vs_off) {
  const int pb = blk & 3;                          // block within the page
  const uint8_t *sec = pool + (static_cast<size_t>(page) * h_kv + g) * kKv4PageBytes;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(sec), 0, kKv4PageBytes, kBufferWord3);
  r.kc = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs, lane_off, kKCodes + pb * 1024, kStream));
  r.vc = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs, lane_off, kVCodes + pb * 1024, kStream));
  r.ks = __builtin_amdgcn_raw_buffer_load_b32(rs, ks_off, kKStats + pb * 64, kStream);
  r.vs = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(rs, vs_off, kVStats + pb * 64, kStream));
}

// one block: scores S^T = K_hat q^T, online softmax update, O^T += V_hat^T P^T.
// TAIL: the block ends past the sequence (the masked last block of a sequence).
template <bool TAIL>
__device__ __forceinline__ void attend_block(const KvBlock &rb, int blk, int len, int hl, int quad, float c2,
                                             const NibbleMasks &nm, const h4 (&qf)[8], float &m, float &l,
                                             f4 (&o)[8]) {
  const int tok0 = blk * 16;
  unsigned kst = rb.ks;
  uint4 vst = rb.vs;
  // tokens past the sequence: scale and zero 0 -> dequantized 0, whatever the codes
  if (TAIL) {
    if (tok0 + hl >= len) kst = 0u;
    const int valid = len - (tok0 + 4 * quad);        // how many of the lane's 4 V tokens exist
    if (valid < 4) {
      const unsigned keep01 = (valid > 0 ? 0xffffu : 0u) | (valid > 1 ? 0xffff0000u : 0u);
      const unsigned keep23 = valid > 2 ? 0xffffu : 0u;
      vst.x &= keep01;
      vst.z &= keep01;
      vst.y &= keep23;
      vst.w &= keep23;
    }
  }
  // K_hat fragments (token hl, one scale and zero for the lane)
  const unsigned kz = (kst >> 16) * 0x10001u, ks = (kst & 0xffffu) * 0x10001u;
  const h2 kb1024 = neg_biased(kz, kBase1024), kb64 = neg_biased(kz, kBase64), ks2 = bits_h2(ks);
  const unsigned kw[4] = {rb.kc.x, rb.kc.y, rb.kc.z, rb.kc.w};
  f4 st0 = f4{0.0f, 0.0f, 0.0f, 0.0f}, st1 = st0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const unsigned w = kw[u], w8 = w >> 8;
    const h2 a0 = (pair_lo(w, nm) + kb1024) * ks2, a1 = (pair_hi(w, nm) + kb64) * ks2;    // dims 16 (2u) + 4 quad + 0..3
    const h2 b0 = (pair_lo(w8, nm) + kb1024) * ks2, b1 = (pair_hi(w8, nm) + kb64) * ks2;  // dims 16 (2u + 1) + ...
    st0 = mfma_f16(h4{a0[0], a0[1], a1[0], a1[1]}, qf[2 * u], st0);
    st1 = mfma_f16(h4{b0[0], b0[1], b1[0], b1[1]}, qf[2 * u + 1], st1);
  }
  // base-2 scores of the lane's head for tokens tok0 + 4 quad + i
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] = (st0[i] + st1[i]) * c2;
  if (TAIL) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = (tok0 + 4 * quad + i < len) ? sc[i] : -INFINITY;
  }
  const float lm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  // m is the same in the 4 lanes of a head; it is raised (for every head of the wave
  // at once) only when some score exceeds it by more than kLazy, m = -inf at first
  if (__builtin_amdgcn_ballot_w64(lm > m + kLazy)) {
    float bm = fmaxf(lm, __shfl_xor(lm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));             // finite: every block has a valid token
    const float mn = fmaxf(m, bm);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    l *= alpha;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) o[cb] *= alpha;
    m = mn;
  }
  // the lane's share of the denominator (its 4 tokens); summed over the 4 lanes at the end
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = __builtin_amdgcn_exp2f(sc[i] - m);
    l += p[i];
  }
  const h4 pf = {static_cast<_Float16>(p[0]), static_cast<_Float16>(p[1]), static_cast<_Float16>(p[2]),
                 static_cast<_Float16>(p[3])};
  // V_hat^T fragments (tokens 4 quad + 0, 1 and + 2, 3) and O^T += V_hat^T P^T
  const h2 vs01 = bits_h2(vst.x), vs23 = bits_h2(vst.y);
  const h2 vb01 = neg_biased(vst.z, kBase1024), vb23 = neg_biased(vst.w, kBase64);
  const unsigned vw[4] = {rb.vc.x, rb.vc.y, rb.vc.z, rb.vc.w};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const unsigned w = vw[u], w8 = w >> 8;
    const h2 a0 = (pair_lo(w, nm) + vb01) * vs01, a1 = (pair_hi(w, nm) + vb23) * vs23;    // dim 16 (2u) + l % 16
    const h2 b0 = (pair_lo(w8, nm) + vb01) * vs01, b1 = (pair_hi(w8, nm) + vb23) * vs23;  // dim 16 (2u + 1) + l % 16
    o[2 * u] = mfma_f16(h4{a0[0], a0[1], a1[0], a1[1]}, pf, o[2 * u]);
    o[2 * u + 1] = mfma_f16(h4{b0[0], b0[1], b1[0], b1[1]}, pf, o[2 * u + 1]);
  }
}

// at most 128 registers per lane: four waves per SIMD, no accumulation registers
__global__ __launch_bounds__(64 * kAttnWaves) __attribute__((amdgpu_waves_per_eu(4))) void kv4_attention_kernel(
    const __half *__restrict__ q, const uint8_t *__restrict__ pool, const int *__restrict__ page_table,
    int max_pages, int num_pages, const int *__restrict__ seq_lens, int max_len, int h, int h_kv, int bps,
    float c2, __half *__restrict__ out, float *__restrict__ ws_o, float *__restrict__ ws_ml) {
  __shared__ float red[kAttnWaves][34][64];
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int splits = gridDim.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = h / h_kv;
  const int hl = lane & 15, quad = lane >> 4;
  const int blk0 = s * bps;
  // the first window's page ids (one per lane), requested before the length is known
  const int *ptab = page_table + static_cast<size_t>(b) * max_pages;
  const int first_pi = (blk0 >> 2) + lane;
  const int first_page = first_pi < max_pages ? ptab[first_pi] : 0;
  const int len = min(max(seq_lens[b], 1), max_len);   // data: clamped to what the table covers
  const int nblk = (len + 15) >> 4;
  const int blk1 = min(nblk, blk0 + bps);

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
  const NibbleMasks nm = nibble_masks();
  float m = -INFINITY, l = 0.0f;
  f4 o[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) o[cb] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  const unsigned lane_off = 16u * lane, ks_off = 4u * hl, vs_off = 16u * quad;
  for (int w0 = blk0; w0 < blk1; w0 += kWindowBlocks) {
    const int wend = min(blk1, w0 + kWindowBlocks);
    const int pg0 = w0 >> 2;                           // w0 is a page boundary
    const int pi = pg0 + lane;
    const int id = w0 == blk0 ? first_page : (pi < max_pages ? ptab[pi] : 0);
    const int mypage = min(max(id, 0), num_pages - 1);
    // Full blocks: three per trip, two blocks in flight ahead of the one computed.
    // Inside the loop every load and every block is unconditional (a load past the
    // range reloads its last block, which is not used), so the wait before each
    // block counts only the loads issued before it, never the prefetches behind it.
    const int wfull = min(wend, len >> 4);
    if (w0 < wfull) {
      const int last = wfull - 1;
      KvBlock ring0, ring1, ring2;
      auto fetch = [&](KvBlock &r, int bk) {
        const int ld = min(bk, last);
        load_block(r, pool, __builtin_amdgcn_readlane(mypage, (ld >> 2) - pg0), h_kv, g, ld, lane_off, ks_off,
                   vs_off);
      };
      int blk = w0 + wave;
      const int mine = blk < wfull ? (wfull - blk + kAttnWaves - 1) / kAttnWaves : 0;   // this wave's blocks
      fetch(ring0, blk);
      fetch(ring1, blk + kAttnWaves);
      int i = 0;
      for (; i + 3 <= mine; i += 3, blk += 3 * kAttnWaves) {
        fetch(ring2, blk + 2 * kAttnWaves);
        attend_block<false>(ring0, blk, len, hl, quad, c2, nm, qf, m, l, o);
        fetch(ring0, blk + 3 * kAttnWaves);
        attend_block<false>(ring1, blk + kAttnWaves, len, hl, quad, c2, nm, qf, m, l, o);
        fetch(ring1, blk + 4 * kAttnWaves);
        attend_block<false>(ring2, blk + 2 * kAttnWaves, len, hl, quad, c2, nm, qf, m, l, o);
      }
      // the last one or two (already in ring0, ring1)
      if (i < mine) attend_block<false>(ring0, blk, len, hl, quad, c2, nm, qf, m, l, o);
      if (i + 1 < mine) attend_block<false>(ring1, blk + kAttnWaves, len, hl, quad, c2, nm, qf, m, l, o);
    }
    // the sequence's partial last block, by the wave the interleaving gives it
    const int tb = nblk - 1;
    if ((len & 15) && tb >= w0 && tb < wend && (tb - w0) % kAttnWaves == wave) {
      KvBlock rt;
      load_block(rt, pool, __builtin_amdgcn_readlane(mypage, (tb >> 2) - pg0), h_kv, g, tb, lane_off, ks_off, vs_off);
      attend_block<true>(rt, tb, len, hl, quad, c2, nm, qf, m, l, o);
    }
  }

  // the head's denominator: the 4 lanes' shares
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
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
    f[w] = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - mm);   // a wave with no block adds nothing
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

// o[b, head] = sum_s O_s 2^(m_s - m) / sum_s l_s 2^(m_s - m) (base-2 maxima); a split
// with no tokens has m = -inf, O = 0, l = 0 and adds nothing.  One workgroup of
// kCombineWaves waves per (b, head): the maxima a thread per split, then wave w
// takes splits w, w + kCombineWaves, ... with no branch in the loop, two dims per
// lane, and the waves' sums meet in LDS.
constexpr int kCombineWaves = 4;

__global__ __launch_bounds__(64 * kCombineWaves) void kv4_combine_kernel(const float *__restrict__ ws_o,
                                                                        const float *__restrict__ ws_ml,
                                                                        int splits, int bh,
                                                                        __half *__restrict__ out) {
  __shared__ float red_m[kCombineWaves];
  __shared__ float red_o[kCombineWaves][2 * 64 + 1];
  const int row = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float mm = -INFINITY;
  for (int s = threadIdx.x; s < splits; s += 64 * kCombineWaves)
    mm = fmaxf(mm, ws_ml[2 * (static_cast<size_t>(s) * bh + row)]);
  mm = wave_max_f32(mm);
  if (lane == 0) red_m[wave] = mm;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kCombineWaves; ++w) mm = fmaxf(mm, red_m[w]);   // finite: split 0 holds the first token
  float a0 = 0.0f, a1 = 0.0f, ll = 0.0f;
#pragma unroll 4
  for (int s = wave; s < splits; s += kCombineWaves) {
    const size_t p = static_cast<size_t>(s) * bh + row;
    const float ms = ws_ml[2 * p];
    const float f = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - mm);
    ll += ws_ml[2 * p + 1] * f;
    const float2 v = *reinterpret_cast<const float2 *>(ws_o + p * kD + 2 * lane);
    a0 += v.x * f;
    a1 += v.y * f;
  }
  red_o[wave][2 * lane] = a0;
  red_o[wave][2 * lane + 1] = a1;
  if (lane == 0) red_o[wave][128] = ll;
  __syncthreads();
  if (wave != 0) return;
  float s0 = 0.0f, s1 = 0.0f, sl = 0.0f;
#pragma unroll
  for (int w = 0; w < kCombineWaves; ++w) {
    s0 += red_o[w][2 * lane];
    s1 += red_o[w][2 * lane + 1];
    sl += red_o[w][128];
  }
  const float inv = 1.0f / sl;
  __half2 r;
  r.x = __float2half_rn(s0 * inv);
  r.y = __float2half_rn(s1 * inv);
  *reinterpret_cast<__half2 *>(out + static_cast<size_t>(row) * kD + 2 * lane) = r;
}

// ---------------------------------------------------------------------------
// SmoothAttention ("QServe: W4A8KV4 ..." summary, SmoothAttention: Z = (Q Lambda)
// (K Lambda^-1)^T, lambda_i = max|K_i|^alpha with the RoPE pair constraint
// lambda_i = lambda_{i+D/2} = max(max|K_i|, max|K_{i+D/2}|)^alpha; review §4.2:
// folded offline into the query and key projections).  Offline kernels: the
// scales from key samples, and the folding into W_Q, W_K.
// ---------------------------------------------------------------------------
constexpr int kSmoothRowGroups = 8;                // sample rows split over the waves of a workgroup

// one workgroup per KV head: 8 x 128 threads (row group, dim) take the channel
// maxima over the samples, then the pair maximum and its power; a pair that never
// leaves 0 keeps lambda = 1
__global__ __launch_bounds__(kSmoothRowGroups * kD) void smooth_lambda_kernel(const __half *__restrict__ k, int n,
                                                                             int h_kv, float alpha,
                                                                             float *__restrict__ lam) {
  __shared__ float part[kSmoothRowGroups][kD];
  const int g = blockIdx.x, d = threadIdx.x % kD, rg = threadIdx.x / kD;
  float m = 0.0f;
#pragma unroll 4
  for (int i = rg; i < n; i += kSmoothRowGroups)
    m = fmaxf(m, fabsf(__half2float(k[(static_cast<size_t>(i) * h_kv + g) * kD + d])));
  part[rg][d] = m;
  __syncthreads();
  if (threadIdx.x < kD / 2) {
    float p = 0.0f;
#pragma unroll
    for (int r = 0; r < kSmoothRowGroups; ++r) p = fmaxf(p, fmaxf(part[r][d], part[r][d + kD / 2]));
    float l;
    if (p == 0.0f)
      l = 1.0f;
    else if (alpha == 0.5f)
      l = __builtin_sqrtf(p);                        // IEEE square root
    else
      l = static_cast<float>(pow(static_cast<double>(p), static_cast<double>(alpha)));
    lam[g * kD + d] = l;
    lam[g * kD + d + kD / 2] = l;
  }
}

// W_Q rows of query head hq, channel i: fp16(fp32(w) * lambda[hq / r, i]); W_K rows
// of KV head g, channel i: fp16(w / lambda[g, i]) (IEEE quotient).  In place allowed.
__global__ __launch_bounds__(256) void smooth_fold_kernel(const __half *__restrict__ wq, const __half *__restrict__ wk,
                                                         const float *__restrict__ lam, int h, int h_kv, int dm,
                                                         __half *__restrict__ wq_out, __half *__restrict__ wk_out) {
  const size_t nq = static_cast<size_t>(h) * kD * dm, nk = static_cast<size_t>(h_kv) * kD * dm;
  const int r = h / h_kv;
  for (size_t e = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < nq + nk;
       e += static_cast<size_t>(gridDim.x) * blockDim.x) {
    if (e < nq) {
      const size_t row = e / dm;
      const int hq = static_cast<int>(row / kD), i = static_cast<int>(row % kD);
      wq_out[e] = mul_round_half(__half2float(wq[e]), lam[(hq / r) * kD + i]);
    } else {
      const size_t f = e - nq, row = f / dm;
      const int g = static_cast<int>(row / kD), i = static_cast<int>(row % kD);
      wk_out[f] = __float2half_rn(__fdiv_rn(__half2float(wk[f]), lam[g * kD + i]));
    }
  }
}

}  // namespace

// up to this many new tokens per sequence the per-token write kernel (measured on
// MI355X: decode writes of one token per sequence take about half the time of the
// block kernel, which quantizes all 16 token slots of a block)
constexpr int64_t kWriteFewTokens = 4;

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
  // 16-token blocks spanned by n_new consecutive positions from any start
  const unsigned nz = static_cast<unsigned>((n_new + 14) / 16 + 1);
  const bool few = n_new <= kWriteFewTokens;
  const unsigned gz = few ? nz : (nz + kWriteWaves - 1) / kWriteWaves;
  hipLaunchKernelGGL(few ? kv4_write_tokens_kernel : kv4_write_block_kernel,
                     dim3(static_cast<unsigned>(h_kv), static_cast<unsigned>(B), gz), dim3(few ? 64 : 64 * kWriteWaves),
                     0, st,
                     static_cast<const __half *>(k_new), static_cast<const __half *>(v_new), static_cast<int>(n_new),
                     static_cast<int>(h_kv), positions, page_table, static_cast<int>(max_pages),
                     static_cast<int>(num_pages), static_cast<uint8_t *>(pool));
}

void launch_kv4_attention(const void *q, const void *pool, int64_t num_pages, const int *page_table,
                          int64_t max_pages, const int *seq_lens, int64_t B, int64_t h, int64_t h_kv,
                          int64_t max_len, void *out, void *ws, hipStream_t st) {
  const int splits = kv4_splits(B, h_kv, max_len);
  const int64_t nblk = (max_len + 15) / 16;
  const int bps = static_cast<int>(((nblk + splits - 1) / splits + 3) / 4 * 4);   // whole pages per split
  float *wo = static_cast<float *>(ws);
  float *wml = splits > 1 ? wo + static_cast<size_t>(splits) * B * h * kD : nullptr;
  // scores in base 2: q . k / sqrt(128) * log2(e)
  const float c2 = static_cast<float>(1.4426950408889634 / 11.313708498984761);
  hipLaunchKernelGGL(kv4_attention_kernel,
                     dim3(static_cast<unsigned>(splits), static_cast<unsigned>(h_kv), static_cast<unsigned>(B)),
                     dim3(64 * kAttnWaves), 0, st, static_cast<const __half *>(q),
                     static_cast<const uint8_t *>(pool), page_table, static_cast<int>(max_pages),
                     static_cast<int>(num_pages), seq_lens, static_cast<int>(max_len), static_cast<int>(h),
                     static_cast<int>(h_kv), bps, c2, static_cast<__half *>(out), wo, wml);
  if (splits > 1)
    hipLaunchKernelGGL(kv4_combine_kernel, dim3(static_cast<unsigned>(B * h)), dim3(64 * kCombineWaves), 0, st, wo,
                       wml, splits,
                       static_cast<int>(B * h), static_cast<__half *>(out));
}

}  // namespace qoq

namespace qoq {

void launch_smooth_lambda(const void *k, int64_t n, int64_t h_kv, float alpha, void *lam, hipStream_t st) {
  hipLaunchKernelGGL(smooth_lambda_kernel, dim3(static_cast<unsigned>(h_kv)), dim3(kSmoothRowGroups * kD), 0, st,
                     static_cast<const __half *>(k), static_cast<int>(n), static_cast<int>(h_kv), alpha,
                     static_cast<float *>(lam));
}

void launch_smooth_fold(const void *wq, const void *wk, const void *lam, int64_t h, int64_t h_kv, int64_t dm,
                        void *wq_out, void *wk_out, hipStream_t st) {
  const size_t total = static_cast<size_t>(h + h_kv) * kD * dm;
  const unsigned blocks = static_cast<unsigned>(std::min<size_t>((total + 255) / 256, 8192));
  hipLaunchKernelGGL(smooth_fold_kernel, dim3(blocks), dim3(256), 0, st, static_cast<const __half *>(wq),
                     static_cast<const __half *>(wk), static_cast<const float *>(lam), static_cast<int>(h),
                     static_cast<int>(h_kv), static_cast<int>(dm), static_cast<__half *>(wq_out),
                     static_cast<__half *>(wk_out));
}

}  // namespace qoq
