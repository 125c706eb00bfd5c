// Device helpers shared by the library's HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qoq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 128;       // weights per (output channel, group)
constexpr int kWQmax = 119;       // protective range of the level-0 weight codes
constexpr int kXQmax = 127;       // symmetric INT8 activation range

// ---------------------------------------------------------------------------
// fp16 helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float half_bits_to_float(unsigned bits) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(bits)));
}

// max over the 8 halves of a 16-byte chunk of |x|, as an fp16 bit pattern with the
// sign cleared (for non-NaN values the integer order of these patterns is the order
// of the magnitudes, subnormals and infinities included)
__device__ __forceinline__ unsigned absmax_bits8(uint4 v, unsigned acc) {
  unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    unsigned lo = w[i] & 0x7fffu;
    unsigned hi = (w[i] >> 16) & 0x7fffu;
    acc = max(acc, max(lo, hi));
  }
  return acc;
}

// fp16(fp32(a * b)): the product is rounded to fp32 first, then to fp16.  The empty
// asm pins the fp32 product in a register, so the compiler cannot fold multiply and
// narrowing into one mixed-precision FMA (a single rounding of the exact product,
// which differs from the two-step rounding whenever the fp32 product lands on an
// fp16 tie).
__device__ __forceinline__ __half mul_round_half(float a, float b) {
  float p = a * b;
  __asm__ volatile("" : "+v"(p));
  return __float2half_rn(p);
}

// symmetric scale: fp16( fp32(absmax) / qmax ) with an IEEE-correct fp32 divide
__device__ __forceinline__ __half sym_scale(unsigned absmax_bits, float qmax) {
  float q = __fdiv_rn(half_bits_to_float(absmax_bits), qmax);
  __asm__ volatile("" : "+v"(q));     // the fp32 quotient is rounded before narrowing
  return __float2half_rn(q);
}

// code = clamp(rint(x / s), -qmax, qmax); s == 0 gives 0
__device__ __forceinline__ int sym_code(float x, float s, float qmax) {
  if (s == 0.0f) return 0;
  float r = rintf(__fdiv_rn(x, s));
  r = fminf(fmaxf(r, -qmax), qmax);
  return static_cast<int>(r);
}

// Activation codes for a row-constant scale s, with rcp = fp32(1 / s) (IEEE divide):
// the same values as sym_code(x, s, 127), i.e. rint of the correctly rounded fp32
// quotient, clamped.  q = fp32(x * rcp) is within |x/s| * 2^-22 of that quotient
// (two roundings against one), far below 2^-12 for every |x/s| this scale allows
// (under 2^8: s is at least about absmax / 190 even after fp16 subnormal rounding),
// so rint(q) decides the same way unless q lies within 2^-12 of a half-integer;
// those rare elements take the IEEE divide, in a branch the whole wave takes only
// when one of its lanes needs it (a per-lane branch is turned into a divide for
// every element plus a select).  Saves the divide sequence per element, which made
// the quantizer vector-ALU bound.

// fp32(1 / s) for quant_chunk8 (0 for s == 0, never used then)
__device__ __forceinline__ float act_rcp(float s) { return s == 0.0f ? 0.0f : __fdiv_rn(1.0f, s); }

// rint(q) clamped to [-127, 127], as an integer
__device__ __forceinline__ int act_int(float q) {
  return static_cast<int>(fminf(fmaxf(rintf(q), -static_cast<float>(kXQmax)), static_cast<float>(kXQmax)));
}

// distance of q from the nearest half-integer (v_fract: q - floor(q))
__device__ __forceinline__ float half_gap(float q) { return fabsf(__builtin_amdgcn_fractf(q) - 0.5f); }

// 8 fp16 activations (one 16-byte chunk) -> 8 INT8 codes with scale s (rcp = act_rcp(s))
__device__ __forceinline__ uint2 quant_chunk8(uint4 v, float s, float rcp) {
  const unsigned w[4] = {v.x, v.y, v.z, v.w};
  float x[8], q[8];
  float gap = 1.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = half_bits_to_float((w[i >> 1] >> (16 * (i & 1))) & 0xffffu);
    q[i] = x[i] * rcp;
    gap = fminf(gap, half_gap(q[i]));
  }
  if (__ballot(gap < 0x1p-12f) != 0) {          // uniform: rare
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (half_gap(q[i]) < 0x1p-12f) q[i] = __fdiv_rn(x[i], s);
  }
  if (s == 0.0f) return make_uint2(0u, 0u);
  int c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = act_int(q[i]);
  // bytes 0 of c[0..3] and c[4..7] (v_perm_b32 selector: byte 4 of the first
  // operand, byte 0 of the second, ...)
  const unsigned lo01 = __builtin_amdgcn_perm(static_cast<unsigned>(c[1]), static_cast<unsigned>(c[0]), 0x0c0c0400u);
  const unsigned lo23 = __builtin_amdgcn_perm(static_cast<unsigned>(c[3]), static_cast<unsigned>(c[2]), 0x04000c0cu);
  const unsigned hi01 = __builtin_amdgcn_perm(static_cast<unsigned>(c[5]), static_cast<unsigned>(c[4]), 0x0c0c0400u);
  const unsigned hi23 = __builtin_amdgcn_perm(static_cast<unsigned>(c[7]), static_cast<unsigned>(c[6]), 0x04000c0cu);
  return make_uint2(lo01 | lo23, hi01 | hi23);
}

// ---------------------------------------------------------------------------
// wave-wide reductions (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, static_cast<unsigned>(__shfl_xor(static_cast<int>(v), off, 64)));
  return v;
}
__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
  return v;
}

// ---------------------------------------------------------------------------
// exact integer a / b rounded half to even (b > 0)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int rne_div(int a, int b) {
  int fl = (a >= 0) ? a / b : -((-a + b - 1) / b);   // floor(a / b)
  int r = a - fl * b;                                 // 0 <= r < b
  int up = (2 * r > b) || (2 * r == b && (fl & 1));
  return fl + up;
}

// ---------------------------------------------------------------------------
// INT4 -> INT8 dequantization by multiply-then-subtract, four weights per 32-bit
// register ("QServe ..." summary, per-group fast dequantization; review §3.2:
// the 8-bit scale is applied to four byte lanes at once and the zero point is
// subtracted afterwards; the protective range keeps every byte product in range).
//
// Each byte lane holds an unsigned code q in [0,15].  For one group the constants
// are s2 = s | s << 16 and, per 16-bit half, c16 = ((128 - z*s) * 257) mod 2^16.
// v_pk_mad_u16 computes q_lo*s + 256*q_hi*s + c16 modulo 2^16, which is congruent
// to (q_lo*s - z*s + 128) + 256*(q_hi*s - z*s + 128).  Every q*s and z*s is at most
// 255 and every q*s - z*s + 128 lies in [7, 249], so that integer is in [0, 2^16)
// and its two bytes are exactly the biased values.  XOR 0x80 per byte then turns
// each biased byte into the two's-complement INT8 (q - z)*s.
// ---------------------------------------------------------------------------
struct GroupConsts {
  unsigned s2;
  unsigned c;
};

__device__ __forceinline__ GroupConsts group_consts(unsigned meta16) {
  unsigned s = meta16 & 0xffu;
  unsigned z = (meta16 >> 8) & 0xffu;
  int bias = 128 - static_cast<int>(z * s);                 // in [-127, 128]
  unsigned c16 = static_cast<unsigned>(bias * 257) & 0xffffu;
  GroupConsts g;
  g.s2 = s | (s << 16);
  g.c = c16 | (c16 << 16);
  return g;
}

__device__ __forceinline__ unsigned dequant4(unsigned codes4, GroupConsts g) {
  u16x2 q = __builtin_bit_cast(u16x2, codes4);
  u16x2 s = __builtin_bit_cast(u16x2, g.s2);
  u16x2 c = __builtin_bit_cast(u16x2, g.c);
  u16x2 r = q * s + c;
  return __builtin_bit_cast(unsigned, r) ^ 0x80808080u;
}

// One lane's 16 packed bytes (32 codes of one column and one group) -> the two
// 16-byte B operands of a pair of 16x16x64 MFMAs: lo nibbles give the first
// 64-wide k block, hi nibbles the second.
__device__ __forceinline__ void dequant_lane(uint4 p, GroupConsts g, v4i &b_lo, v4i &b_hi) {
  unsigned w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    unsigned lo = w[r] & 0x0f0f0f0fu;
    unsigned hi = (w[r] >> 4) & 0x0f0f0f0fu;
    b_lo[r] = static_cast<int>(dequant4(lo, g));
    b_hi[r] = static_cast<int>(dequant4(hi, g));
  }
}

// Per-channel variant: the UINT4 codes themselves are the B operand (0..15 fit an
// INT8 lane); the zero point is applied in the epilogue as z * t.  Unpacking only:
// AND / SHIFT / AND per 8 codes ("QServe ..." summary, per-channel fast
// dequantization: three logic operations per register).
__device__ __forceinline__ void unpack_lane(uint4 p, v4i &b_lo, v4i &b_hi) {
  unsigned w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    b_lo[r] = static_cast<int>(w[r] & 0x0f0f0f0fu);
    b_hi[r] = static_cast<int>((w[r] >> 4) & 0x0f0f0f0fu);
  }
}

// B operand of one lane: dequantized INT8 weights (per-group, PC = false) or the
// raw codes (per-channel, PC = true)
template <bool PC>
__device__ __forceinline__ void weights_lane(uint4 p, unsigned meta16, v4i &b_lo, v4i &b_hi) {
  if constexpr (PC)
    unpack_lane(p, b_lo, b_hi);
  else
    dequant_lane(p, group_consts(meta16), b_lo, b_hi);
}

// Tiled activation codes (the few-token GEMM's A operand): the codes of a 16-row
// block and a 64-wide k block are 1 KB, stored in the order the 16x16x64 INT8 MFMA
// takes its A operand (lane l = 16*kq + r: row r, k = 16*kq .. +15), so that a
// 16-byte load per lane reads a block as 1 KB of consecutive bytes.  Blocks are
// row-block major: block (rb, kb) starts at (rb * K/64 + kb) * 1024.
__host__ __device__ __forceinline__ size_t tiled_offset(int row, int k, int K) {
  return ((static_cast<size_t>(row >> 4) * (K >> 6) + (k >> 6)) * 64 + ((k >> 4) & 3) * 16 + (row & 15)) * 16 +
         (k & 15);
}

__device__ __forceinline__ v4i mfma16x16x64(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v16i mfma32x32x32(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

}  // namespace qoq
