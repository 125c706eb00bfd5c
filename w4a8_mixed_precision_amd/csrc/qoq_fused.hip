// Producers of the GEMM's INT8 activations with the quantization fused in (gfx950).
//
// "QServe：把 W4A8KV4 ..." review, runtime precision mapping (§3.2) and data path
// step 2: the activation quantization of the QKV projection and of the first FFN
// layer is fused into the preceding normalization kernel, that of the second FFN
// layer into the preceding activation kernel; blocks are FP16 in and out.  The
// fp16 value the unfused pipeline would write (RMSNorm output, SiLU(gate) * up) is
// formed in registers and quantized per token exactly as the standalone quantizer
// does, so the codes equal quantize(fp16 value).  Optional t[m] = sum_k codes (the
// per-channel epilogue term, "QServe ..." summary, per-channel fast dequantization:
// precomputed by the memory-bound kernel before the GEMM).
//
// Precision (the pages fix only FP16 in / out):
//   RMSNorm: sum of squares in fp64 (each fp16 square is exact there), mean =
//     fp32(sum / K), inv = fp32(1 / fp32(sqrt(fp32(mean + eps)))) with IEEE
//     operations, y = fp16(fp32(fp32(x * inv) * gamma)).
//   SiLU(gate) * up = gate * up / (1 + exp(-gate)) in fp64, rounded once to fp16.
#include "qoq_device.h"
#include "qoq_internal.h"

#include <algorithm>

namespace qoq {

namespace {

constexpr int kFThreads = 256;
constexpr int kFChunks = 16;            // 16 chunks x 8 values x 256 threads: K <= 32768

__device__ __forceinline__ double block_sum_f64(double v, double *red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();                       // red may still be read from a previous use
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < kFThreads / 64; ++w) s += red[w];   // same order in every thread
  return s;
}

__device__ __forceinline__ unsigned block_max_u32(unsigned v, unsigned *red) {
  v = wave_max_u32(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  unsigned m = 0;
#pragma unroll
  for (int w = 0; w < kFThreads / 64; ++w) m = max(m, red[w]);
  return m;
}

__device__ __forceinline__ int block_sum_i32(int v, int *red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < kFThreads / 64; ++w) s += red[w];
  return s;
}

// fp16 bits of the 8 values of a chunk -> codes, stored row-major or tiled
template <bool TILED>
__device__ __forceinline__ void store_codes(int8_t *__restrict__ qx, int row, int K, int idx, uint2 q) {
  if (TILED)
    *reinterpret_cast<uint2 *>(qx + tiled_offset(row, 8 * idx, K)) = q;
  else
    reinterpret_cast<uint2 *>(qx + static_cast<size_t>(row) * K)[idx] = q;
}

// Quantize the fp16 values y (register chunks, fp16 bits) of one row, given their
// maximum magnitude (fp16 bits): s_X, the codes of this part's slots, the code sum.
template <bool TILED, bool ROWSUM>
__device__ __forceinline__ void quantize_row(const uint4 (&y)[kFChunks], unsigned amax, int row, int K,
                                             int8_t *__restrict__ qx, __half *__restrict__ sx,
                                             int *__restrict__ tx, int *ired) {
  const int nchunk = K >> 3;
  const int part = blockIdx.y, parts = gridDim.y;
  const __half sh = sym_scale(amax, static_cast<float>(kXQmax));
  const float s = __half2float(sh);
  const float rcp = act_rcp(s);
  if (threadIdx.x == 0 && part == 0) sx[row] = sh;
  int tsum = 0;
#pragma unroll
  for (int c = 0; c < kFChunks; ++c) {
    const int idx = threadIdx.x + c * kFThreads;
    if (idx < nchunk && c % parts == part) {
      const uint2 q = quant_chunk8(y[c], s, rcp);
      store_codes<TILED>(qx, row, K, idx, q);
      if (ROWSUM)
        tsum += __builtin_amdgcn_sdot4(static_cast<int>(q.x), 0x01010101, 0, false) +
                __builtin_amdgcn_sdot4(static_cast<int>(q.y), 0x01010101, 0, false);
    }
  }
  if (ROWSUM) {
    const int t = block_sum_i32(tsum, ired);
    if (threadIdx.x == 0) tx[row] = t;
  }
}

__device__ __forceinline__ unsigned pack_half2(__half lo, __half hi) {
  return static_cast<unsigned>(__half_as_ushort(lo)) | (static_cast<unsigned>(__half_as_ushort(hi)) << 16);
}

// ---------------------------------------------------------------------------
// RMSNorm + quantization.  One row per blockIdx.x; gridDim.y workgroups share a
// row (each recomputes the row's statistics and quantizes its share of the slots).
// ---------------------------------------------------------------------------
template <bool TILED, bool ROWSUM>
__global__ __launch_bounds__(kFThreads) void rmsnorm_quant_kernel(const __half *__restrict__ x,
                                                                  const __half *__restrict__ gamma, float eps,
                                                                  int K, int8_t *__restrict__ qx,
                                                                  __half *__restrict__ sx, int *__restrict__ tx) {
  __shared__ double dred[kFThreads / 64];
  __shared__ unsigned ured[kFThreads / 64];
  __shared__ int ired[kFThreads / 64];
  const int row = blockIdx.x;
  const int nchunk = K >> 3;
  const uint4 *xr = reinterpret_cast<const uint4 *>(x + static_cast<size_t>(row) * K);
  const uint4 *gr = reinterpret_cast<const uint4 *>(gamma);
  uint4 v[kFChunks], g[kFChunks];
#pragma unroll
  for (int c = 0; c < kFChunks; ++c) {          // every load first: all in flight together
    const int idx = threadIdx.x + c * kFThreads;
    v[c] = idx < nchunk ? xr[idx] : make_uint4(0u, 0u, 0u, 0u);
    g[c] = idx < nchunk ? gr[idx] : make_uint4(0u, 0u, 0u, 0u);
  }
  double ss = 0.0;
#pragma unroll
  for (int c = 0; c < kFChunks; ++c) {
    if (threadIdx.x + c * kFThreads >= nchunk) continue;   // past the row (whole slots skipped)
    const unsigned w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double xv = static_cast<double>(half_bits_to_float((w[i >> 1] >> (16 * (i & 1))) & 0xffffu));
      ss += xv * xv;                             // each square is exact in fp64
    }
  }
  const double sum = block_sum_f64(ss, dred);
  const float mean = static_cast<float>(sum / static_cast<double>(K));
  const float inv = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(mean, eps)));

  unsigned amax = 0;
#pragma unroll
  for (int c = 0; c < kFChunks; ++c) {
    if (threadIdx.x + c * kFThreads >= nchunk) continue;
    const unsigned w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
    const unsigned gw[4] = {g[c].x, g[c].y, g[c].z, g[c].w};
    unsigned o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = half_bits_to_float(w[i] & 0xffffu), x1 = half_bits_to_float(w[i] >> 16);
      const float g0 = half_bits_to_float(gw[i] & 0xffffu), g1 = half_bits_to_float(gw[i] >> 16);
      float t0 = x0 * inv, t1 = x1 * inv;
      __asm__ volatile("" : "+v"(t0), "+v"(t1));   // fp32(x * inv) is rounded before the gamma product
      o[i] = pack_half2(mul_round_half(t0, g0), mul_round_half(t1, g1));
    }
    v[c] = make_uint4(o[0], o[1], o[2], o[3]);
    amax = absmax_bits8(v[c], amax);
  }
  amax = block_max_u32(amax, ured);
  quantize_row<TILED, ROWSUM>(v, amax, row, K, qx, sx, tx, ired);
}

// ---------------------------------------------------------------------------
// SiLU(gate) * up + quantization.  gate and up rows have stride ld (elements).
// One workgroup per row (gridDim.y == 1): every value exactly (fp64) in
// registers, then the quantization.  Several per row (gridDim.y > 1, few tokens):
// the row maximum needs every value, the codes only this part's, so all values are
// first formed in fp32 (within 2^-20 relative of the exact ones), the exact fp64
// values are taken for the candidates of the maximum (fp32 magnitude within 2^-12
// of the fp32 maximum) and for this part's slots.
// ---------------------------------------------------------------------------
__device__ __forceinline__ __half silu_mul_exact(float gf, float uf) {
  const double gd = static_cast<double>(gf), ud = static_cast<double>(uf);
  const _Float16 h = static_cast<_Float16>(gd * ud / (1.0 + exp(-gd)));   // one rounding, fp64 -> fp16
  return __ushort_as_half(__builtin_bit_cast(unsigned short, h));
}

// fp32 with the accurate expf (about 1 ulp) and an IEEE divide; gate * up is exact
// in fp32 (two 11-bit significands): relative error well under 2^-20
__device__ __forceinline__ float silu_mul_fast(float gf, float uf) {
  return gf * uf / (1.0f + expf(-gf));
}

template <bool TILED, bool ROWSUM>
__global__ __launch_bounds__(kFThreads) void silu_mul_quant_kernel(const __half *__restrict__ gate,
                                                                   const __half *__restrict__ up, int ld, int K,
                                                                   int8_t *__restrict__ qx,
                                                                   __half *__restrict__ sx,
                                                                   int *__restrict__ tx) {
  __shared__ unsigned ured[kFThreads / 64];
  __shared__ int ired[kFThreads / 64];
  const int row = blockIdx.x;
  const int part = blockIdx.y, parts = gridDim.y;
  const int nchunk = K >> 3;
  const uint4 *gr = reinterpret_cast<const uint4 *>(gate + static_cast<size_t>(row) * ld);
  const uint4 *ur = reinterpret_cast<const uint4 *>(up + static_cast<size_t>(row) * ld);
  uint4 a[kFChunks], b[kFChunks];
#pragma unroll
  for (int c = 0; c < kFChunks; ++c) {
    const int idx = threadIdx.x + c * kFThreads;
    a[c] = idx < nchunk ? gr[idx] : make_uint4(0u, 0u, 0u, 0u);
    b[c] = idx < nchunk ? ur[idx] : make_uint4(0u, 0u, 0u, 0u);
  }
  unsigned amax = 0;
  if (parts == 1) {
#pragma unroll
    for (int c = 0; c < kFChunks; ++c) {
      if (threadIdx.x + c * kFThreads >= nchunk) continue;   // past the row (whole slots skipped)
      const unsigned gw[4] = {a[c].x, a[c].y, a[c].z, a[c].w};
      const unsigned uw[4] = {b[c].x, b[c].y, b[c].z, b[c].w};
      unsigned o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = pack_half2(silu_mul_exact(half_bits_to_float(gw[i] & 0xffffu), half_bits_to_float(uw[i] & 0xffffu)),
                          silu_mul_exact(half_bits_to_float(gw[i] >> 16), half_bits_to_float(uw[i] >> 16)));
      a[c] = make_uint4(o[0], o[1], o[2], o[3]);
      amax = absmax_bits8(a[c], amax);
    }
    amax = block_max_u32(amax, ured);
  } else {
    float fmax = 0.0f;
#pragma unroll
    for (int c = 0; c < kFChunks; ++c) {
      if (threadIdx.x + c * kFThreads >= nchunk) continue;
      const unsigned gw[4] = {a[c].x, a[c].y, a[c].z, a[c].w};
      const unsigned uw[4] = {b[c].x, b[c].y, b[c].z, b[c].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned sh = 16 * (i & 1);
        fmax = fmaxf(fmax, fabsf(silu_mul_fast(half_bits_to_float((gw[i >> 1] >> sh) & 0xffffu),
                                               half_bits_to_float((uw[i >> 1] >> sh) & 0xffffu))));
      }
    }
    fmax = __uint_as_float(block_max_u32(__float_as_uint(fmax), ured));   // non-negative: bit order = value order
    const float cut = fmax * (1.0f - 0x1p-12f);
#pragma unroll
    for (int c = 0; c < kFChunks; ++c) {
      if (threadIdx.x + c * kFThreads >= nchunk) continue;
      const unsigned gw[4] = {a[c].x, a[c].y, a[c].z, a[c].w};
      const unsigned uw[4] = {b[c].x, b[c].y, b[c].z, b[c].w};
      const bool mine = c % parts == part;
      unsigned o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned sh = 16 * (i & 1);
        const float gf = half_bits_to_float((gw[i >> 1] >> sh) & 0xffffu);
        const float uf = half_bits_to_float((uw[i >> 1] >> sh) & 0xffffu);
        const bool cand = fabsf(silu_mul_fast(gf, uf)) >= cut;
        if (mine || cand) {
          const unsigned hb = __half_as_ushort(silu_mul_exact(gf, uf));
          if (cand) amax = max(amax, hb & 0x7fffu);
          o[i >> 1] |= hb << sh;
        }
      }
      if (mine) a[c] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    amax = block_max_u32(amax, ured);
  }
  quantize_row<TILED, ROWSUM>(a, amax, row, K, qx, sx, tx, ired);
}

}  // namespace

// workgroups per row: as for the standalone quantizer (a few tokens spread a row
// over up to one workgroup per register slot); one when the code sum is wanted
unsigned fused_row_parts(int64_t M, int64_t K, bool rowsum) {
  if (rowsum) return 1;
  const int64_t slots = (K / 8 + kFThreads - 1) / kFThreads;
  return static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>(slots, 256 / M)));
}

void launch_rmsnorm_quantize(const void *x, const void *gamma, float eps, int64_t M, int64_t K, int tiled,
                             void *qx, void *sx, void *tx, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(M), fused_row_parts(M, K, tx != nullptr));
  const __half *xp = static_cast<const __half *>(x);
  const __half *gp = static_cast<const __half *>(gamma);
  int8_t *q = static_cast<int8_t *>(qx);
  __half *s = static_cast<__half *>(sx);
  int *t = static_cast<int *>(tx);
  const int k = static_cast<int>(K);
  if (tiled) {
    if (t) hipLaunchKernelGGL((rmsnorm_quant_kernel<true, true>), grid, dim3(kFThreads), 0, st, xp, gp, eps, k, q, s, t);
    else hipLaunchKernelGGL((rmsnorm_quant_kernel<true, false>), grid, dim3(kFThreads), 0, st, xp, gp, eps, k, q, s, t);
  } else {
    if (t) hipLaunchKernelGGL((rmsnorm_quant_kernel<false, true>), grid, dim3(kFThreads), 0, st, xp, gp, eps, k, q, s, t);
    else hipLaunchKernelGGL((rmsnorm_quant_kernel<false, false>), grid, dim3(kFThreads), 0, st, xp, gp, eps, k, q, s, t);
  }
}

void launch_silu_mul_quantize(const void *gate, const void *up, int64_t ld, int64_t M, int64_t K, int tiled,
                              void *qx, void *sx, void *tx, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(M), fused_row_parts(M, K, tx != nullptr));
  const __half *gp = static_cast<const __half *>(gate);
  const __half *up_ = static_cast<const __half *>(up);
  int8_t *q = static_cast<int8_t *>(qx);
  __half *s = static_cast<__half *>(sx);
  int *t = static_cast<int *>(tx);
  const int k = static_cast<int>(K), l = static_cast<int>(ld);
  if (tiled) {
    if (t) hipLaunchKernelGGL((silu_mul_quant_kernel<true, true>), grid, dim3(kFThreads), 0, st, gp, up_, l, k, q, s, t);
    else hipLaunchKernelGGL((silu_mul_quant_kernel<true, false>), grid, dim3(kFThreads), 0, st, gp, up_, l, k, q, s, t);
  } else {
    if (t) hipLaunchKernelGGL((silu_mul_quant_kernel<false, true>), grid, dim3(kFThreads), 0, st, gp, up_, l, k, q, s, t);
    else hipLaunchKernelGGL((silu_mul_quant_kernel<false, false>), grid, dim3(kFThreads), 0, st, gp, up_, l, k, q, s, t);
  }
}

}  // namespace qoq
