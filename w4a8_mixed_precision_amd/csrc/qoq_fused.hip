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

constexpr int kFThreads = 256;           // up to 16 chunks x 8 values x 256 threads: K <= 32768

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

// Quantize the fp16 values y (CH register chunks per thread, fp16 bits) of one row,
// given their maximum magnitude (fp16 bits): s_X, the codes of this part's slots
// (slot c of every thread belongs to part c % gridDim.y), the code sum.
// The unfused pipeline's fp16 output instead (the value the fused kernels quantize):
// row-major [M, K] fp16.
template <int CH>
__device__ __forceinline__ void store_row_fp16(const uint4 (&y)[CH], int row, int K, __half *__restrict__ out) {
  const int nchunk = K >> 3;
  uint4 *o = reinterpret_cast<uint4 *>(out + static_cast<size_t>(row) * K);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = threadIdx.x + c * kFThreads;
    if (idx < nchunk) o[idx] = y[c];
  }
}

template <int CH, bool TILED, bool ROWSUM>
__device__ __forceinline__ void quantize_row(const uint4 (&y)[CH], unsigned amax, int row, int K,
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
  for (int c = 0; c < CH; ++c) {
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
// CH chunks of 8 values per thread hold the row (CH * 2048 >= K): the launcher
// picks the smallest, so short rows leave registers for more waves.
// ---------------------------------------------------------------------------
template <int CH, bool TILED, bool ROWSUM, bool OUT16 = false>
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
  uint4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {                 // every load first: all in flight together
    const int idx = threadIdx.x + c * kFThreads;
    v[c] = idx < nchunk ? xr[idx] : make_uint4(0u, 0u, 0u, 0u);
  }
  double ss = 0.0;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const unsigned w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double xv = static_cast<double>(half_bits_to_float((w[i >> 1] >> (16 * (i & 1))) & 0xffffu));
      ss += xv * xv;                             // each square is exact in fp64; zero chunks add 0
    }
  }
  const double sum = block_sum_f64(ss, dred);
  const float mean = static_cast<float>(sum / static_cast<double>(K));
  // IEEE square root: __builtin_sqrtf is correctly rounded here (HIP's __fsqrt_rn
  // maps to the approximate native instruction unless the library's rounded
  // operations are selected, and differed in the last bit)
  const float inv = __fdiv_rn(1.0f, __builtin_sqrtf(__fadd_rn(mean, eps)));

  unsigned amax = 0;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = threadIdx.x + c * kFThreads;
    const uint4 gc = idx < nchunk ? gr[idx] : make_uint4(0u, 0u, 0u, 0u);   // L2-resident, shared by rows
    const unsigned w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
    const unsigned gw[4] = {gc.x, gc.y, gc.z, gc.w};
    unsigned o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = half_bits_to_float(w[i] & 0xffffu), x1 = half_bits_to_float(w[i] >> 16);
      const float g0 = half_bits_to_float(gw[i] & 0xffffu), g1 = half_bits_to_float(gw[i] >> 16);
      float t0 = x0 * inv, t1 = x1 * inv;
      __asm__ volatile("" : "+v"(t0), "+v"(t1));   // fp32(x * inv) is rounded before the gamma product
      o[i] = pack_half2(mul_round_half(t0, g0), mul_round_half(t1, g1));
    }
    v[c] = make_uint4(o[0], o[1], o[2], o[3]);   // past the row: x = 0, gamma = 0 -> 0
    amax = absmax_bits8(v[c], amax);
  }
  if (OUT16) {                                   // qx carries the fp16 output
    store_row_fp16<CH>(v, row, K, reinterpret_cast<__half *>(qx));
    return;
  }
  amax = block_max_u32(amax, ured);
  quantize_row<CH, TILED, ROWSUM>(v, amax, row, K, qx, sx, tx, ired);
}

// ---------------------------------------------------------------------------
// SiLU(gate) * up + quantization.  gate and up rows have stride ld (elements).
// h = fp16 of the exact gate * up / (1 + exp(-gate)).  Each value is first formed
// in fp32, h32 = (gate * up) * rcp(1 + e^(-gate)): gate * up is exact (two 11-bit
// significands) and the rest costs a few ulps, well under 2^-20 relative.  If
// h32 - e and h32 + e (e = 2^-20 |h32|) round to the same fp16, so does the exact
// value (rounding is monotone).  Otherwise the two fp16 candidates are adjacent
// and the exact value is compared with their midpoint in fp64 (gate * up / (1 +
// exp(-gate)) in fp64; for gate != 0 it is irrational, so it never equals the
// midpoint), in a branch the wave takes only when one of its lanes needs it.  The
// fp16 value is therefore RN16 of the fp64 expression, like the oracle's.
// ---------------------------------------------------------------------------
// e^(-g) for an fp16 value g, as 2^t with t = -g log2(e) split into n + f (n the
// nearest integer, |f| <= 1/2), so the hardware base-2 exponential sees only a small
// argument: -g * kLog2eHi is exact (kLog2eHi = 2955 / 2048 has 12 significant bits,
// g at most 11), the rest of log2(e) enters through one fma, and 2^n is an exact
// scaling.  Relative error about 2^-22.5 (the hardware 2^f and two roundings), well
// inside the 2^-20 the exact-rounding test below allows for.  |t| stays below 2^17
// for finite fp16 g; beyond the fp32 range the scaling gives 0 or infinity, as e^(-g)
// rounds there.
constexpr float kLog2eHi = 1.44287109375f;
constexpr float kLog2eLo = static_cast<float>(1.4426950408889634 - 1.44287109375);

__device__ __forceinline__ float exp_neg(float g) {
  const float th = -g * kLog2eHi;
  const float n = __builtin_rintf(th);
  const float f = __builtin_fmaf(-g, kLog2eLo, th - n);
  return __builtin_ldexpf(__builtin_amdgcn_exp2f(f), static_cast<int>(n));
}

__device__ __forceinline__ float silu_mul_fast(float gf, float uf) {
  return (gf * uf) * __builtin_amdgcn_rcpf(1.0f + exp_neg(gf));
}

// fp16 bits of RN16(h) for h within e of h32, or 0xffffffff when undecided
__device__ __forceinline__ unsigned round_h16(float h32) {
  const float e = fabsf(h32) * 0x1p-20f;
  const unsigned lo = __half_as_ushort(__float2half_rn(h32 - e));
  const unsigned hi = __half_as_ushort(__float2half_rn(h32 + e));
  return lo == hi ? lo : 0xffffffffu;
}

// the undecided case: compare the fp64 value with the midpoint of the two
// candidates RN16(h32 - e) < RN16(h32 + e)
__device__ __noinline__ unsigned decide_h16(float gf, float uf, float h32) {
  const float e = fabsf(h32) * 0x1p-20f;
  const __half lo = __float2half_rn(h32 - e), hi = __float2half_rn(h32 + e);
  const double mid = 0.5 * (static_cast<double>(__half2float(lo)) + static_cast<double>(__half2float(hi)));
  const double gd = static_cast<double>(gf);
  const double h = gd * static_cast<double>(uf) / (1.0 + exp(-gd));
  const unsigned lb = __half_as_ushort(lo), hb = __half_as_ushort(hi);
  if (h < mid) return lb;
  if (h > mid) return hb;
  return (lb & 1u) ? hb : lb;                      // a tie (only in principle): to even
}

// fp16 bits of SiLU(gate) * up for the 8 values of a chunk (every lane of the wave
// calls it: the rare exact decision is a wave-uniform branch)
__device__ __forceinline__ uint4 silu_chunk8(uint4 gv, uint4 uv) {
  const unsigned gw[4] = {gv.x, gv.y, gv.z, gv.w};
  const unsigned uw[4] = {uv.x, uv.y, uv.z, uv.w};
  float gf[8], uf[8], h[8];
  unsigned r[8];
  bool open = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const unsigned sh = 16 * (i & 1);
    gf[i] = half_bits_to_float((gw[i >> 1] >> sh) & 0xffffu);
    uf[i] = half_bits_to_float((uw[i >> 1] >> sh) & 0xffffu);
    h[i] = silu_mul_fast(gf[i], uf[i]);
    r[i] = round_h16(h[i]);
    open |= r[i] == 0xffffffffu;
  }
  if (__ballot(open) != 0) {                       // uniform: rare
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (r[i] == 0xffffffffu) r[i] = decide_h16(gf[i], uf[i], h[i]);
  }
  return make_uint4(r[0] | (r[1] << 16), r[2] | (r[3] << 16), r[4] | (r[5] << 16), r[6] | (r[7] << 16));
}

template <int CH, bool TILED, bool ROWSUM, bool OUT16 = false>
__global__ __launch_bounds__(kFThreads) void silu_mul_quant_kernel(const __half *__restrict__ gate,
                                                                   const __half *__restrict__ up, int ld, int K,
                                                                   int8_t *__restrict__ qx,
                                                                   __half *__restrict__ sx,
                                                                   int *__restrict__ tx) {
  __shared__ unsigned ured[kFThreads / 64];
  __shared__ int ired[kFThreads / 64];
  const int row = blockIdx.x;
  const int nchunk = K >> 3;
  const uint4 *gr = reinterpret_cast<const uint4 *>(gate + static_cast<size_t>(row) * ld);
  const uint4 *ur = reinterpret_cast<const uint4 *>(up + static_cast<size_t>(row) * ld);
  uint4 a[CH], b[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = threadIdx.x + c * kFThreads;
    a[c] = idx < nchunk ? gr[idx] : make_uint4(0u, 0u, 0u, 0u);
    b[c] = idx < nchunk ? ur[idx] : make_uint4(0u, 0u, 0u, 0u);
  }
  unsigned amax = 0;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    a[c] = silu_chunk8(a[c], b[c]);
    amax = absmax_bits8(a[c], amax);               // past the row: gate = up = 0 -> 0
  }
  if (OUT16) {
    store_row_fp16<CH>(a, row, K, reinterpret_cast<__half *>(qx));
    return;
  }
  amax = block_max_u32(amax, ured);
  quantize_row<CH, TILED, ROWSUM>(a, amax, row, K, qx, sx, tx, ired);
}

// ---------------------------------------------------------------------------
// A few rows with a long K, split without repetition: the kernel above spreads a
// row over several workgroups that each form the whole row (every part needs the
// row maximum), which makes one decode row of Qwen-72B's down projection a
// vector-ALU job for one compute unit.  Here the row is cut into slices of
// kSliceChunks chunks (2048 values); pass 1 forms each slice's values and writes
// their maximum magnitude (fp16 bits) to ws[row * slices + slice]; pass 2 takes the
// row maximum from those, forms its slice's values again and quantizes them (the
// same routines, so the codes are identical).  Two launches instead of one.
// ---------------------------------------------------------------------------
constexpr int kSliceChunks = kFThreads;             // one chunk of 8 values per thread

__global__ __launch_bounds__(kFThreads) void silu_slice_max_kernel(const __half *__restrict__ gate,
                                                                   const __half *__restrict__ up, int ld, int K,
                                                                   unsigned *__restrict__ ws) {
  __shared__ unsigned ured[kFThreads / 64];
  const int row = blockIdx.x, slice = blockIdx.y, slices = gridDim.y;
  const int nchunk = K >> 3, idx = slice * kSliceChunks + threadIdx.x;
  const uint4 *gr = reinterpret_cast<const uint4 *>(gate + static_cast<size_t>(row) * ld);
  const uint4 *ur = reinterpret_cast<const uint4 *>(up + static_cast<size_t>(row) * ld);
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  const uint4 y = silu_chunk8(idx < nchunk ? gr[idx] : zero, idx < nchunk ? ur[idx] : zero);
  const unsigned amax = block_max_u32(absmax_bits8(y, 0u), ured);
  if (threadIdx.x == 0) ws[static_cast<size_t>(row) * slices + slice] = amax;
}

template <bool TILED>
__global__ __launch_bounds__(kFThreads) void silu_slice_quant_kernel(const __half *__restrict__ gate,
                                                                     const __half *__restrict__ up, int ld, int K,
                                                                     const unsigned *__restrict__ ws,
                                                                     int8_t *__restrict__ qx,
                                                                     __half *__restrict__ sx) {
  __shared__ unsigned ured[kFThreads / 64];
  const int row = blockIdx.x, slice = blockIdx.y, slices = gridDim.y;
  const int nchunk = K >> 3, idx = slice * kSliceChunks + threadIdx.x;
  const uint4 *gr = reinterpret_cast<const uint4 *>(gate + static_cast<size_t>(row) * ld);
  const uint4 *ur = reinterpret_cast<const uint4 *>(up + static_cast<size_t>(row) * ld);
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  const uint4 gv = idx < nchunk ? gr[idx] : zero, uv = idx < nchunk ? ur[idx] : zero;
  unsigned part = 0;
  for (int i = threadIdx.x; i < slices; i += kFThreads) part = max(part, ws[static_cast<size_t>(row) * slices + i]);
  const unsigned amax = block_max_u32(part, ured);
  const uint4 y = silu_chunk8(gv, uv);
  const __half sh = sym_scale(amax, static_cast<float>(kXQmax));
  if (threadIdx.x == 0 && slice == 0) sx[row] = sh;
  const float s = __half2float(sh);
  if (idx < nchunk) store_codes<TILED>(qx, row, K, idx, quant_chunk8(y, s, act_rcp(s)));
}

// workgroups per row: as for the standalone quantizer (a few tokens spread a row
// over up to one workgroup per register slot); one when the code sum is wanted
unsigned fused_row_parts(int64_t M, int64_t K, bool rowsum) {
  if (rowsum) return 1;
  const int64_t slots = (K / 8 + kFThreads - 1) / kFThreads;
  return static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>(slots, 256 / M)));
}

// register chunks per thread: the smallest power of two that holds the row
int fused_chunks(int64_t K) {
  const int64_t slots = (K / 8 + kFThreads - 1) / kFThreads;
  int ch = 1;
  while (ch < slots) ch *= 2;
  return ch;
}

template <int CH>
void launch_rmsnorm_ch(const __half *x, const __half *g, float eps, int K, bool tiled, int8_t *q, __half *s, int *t,
                       dim3 grid, hipStream_t st, bool out16) {
  if (out16) {
    hipLaunchKernelGGL((rmsnorm_quant_kernel<CH, false, false, true>), grid, dim3(kFThreads), 0, st, x, g, eps, K, q, s, t);
    return;
  }
  if (tiled) {
    if (t) hipLaunchKernelGGL((rmsnorm_quant_kernel<CH, true, true>), grid, dim3(kFThreads), 0, st, x, g, eps, K, q, s, t);
    else hipLaunchKernelGGL((rmsnorm_quant_kernel<CH, true, false>), grid, dim3(kFThreads), 0, st, x, g, eps, K, q, s, t);
  } else {
    if (t) hipLaunchKernelGGL((rmsnorm_quant_kernel<CH, false, true>), grid, dim3(kFThreads), 0, st, x, g, eps, K, q, s, t);
    else hipLaunchKernelGGL((rmsnorm_quant_kernel<CH, false, false>), grid, dim3(kFThreads), 0, st, x, g, eps, K, q, s, t);
  }
}

template <int CH>
void launch_silu_ch(const __half *g, const __half *u, int ld, int K, bool tiled, int8_t *q, __half *s, int *t,
                    dim3 grid, hipStream_t st, bool out16) {
  if (out16) {
    hipLaunchKernelGGL((silu_mul_quant_kernel<CH, false, false, true>), grid, dim3(kFThreads), 0, st, g, u, ld, K, q, s, t);
    return;
  }
  if (tiled) {
    if (t) hipLaunchKernelGGL((silu_mul_quant_kernel<CH, true, true>), grid, dim3(kFThreads), 0, st, g, u, ld, K, q, s, t);
    else hipLaunchKernelGGL((silu_mul_quant_kernel<CH, true, false>), grid, dim3(kFThreads), 0, st, g, u, ld, K, q, s, t);
  } else {
    if (t) hipLaunchKernelGGL((silu_mul_quant_kernel<CH, false, true>), grid, dim3(kFThreads), 0, st, g, u, ld, K, q, s, t);
    else hipLaunchKernelGGL((silu_mul_quant_kernel<CH, false, false>), grid, dim3(kFThreads), 0, st, g, u, ld, K, q, s, t);
  }
}

}  // namespace

int silu_split_slices(int64_t M, int64_t K) {
  if (M > kSiluSplitMaxM) return 0;
  const int64_t slices = (K / 8 + kSliceChunks - 1) / kSliceChunks;
  return slices > 1 ? static_cast<int>(slices) : 0;
}

size_t silu_split_workspace(int64_t M, int64_t K) {
  return static_cast<size_t>(M) * silu_split_slices(M, K) * sizeof(unsigned);
}

void launch_silu_mul_quantize_split(const void *gate, const void *up, int64_t ld, int64_t M, int64_t K, bool tiled,
                                    void *qx, void *sx, void *ws, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(M), static_cast<unsigned>(silu_split_slices(M, K)));
  const __half *gp = static_cast<const __half *>(gate), *upp = static_cast<const __half *>(up);
  const int k = static_cast<int>(K), l = static_cast<int>(ld);
  hipLaunchKernelGGL(silu_slice_max_kernel, grid, dim3(kFThreads), 0, st, gp, upp, l, k, static_cast<unsigned *>(ws));
  if (tiled)
    hipLaunchKernelGGL(silu_slice_quant_kernel<true>, grid, dim3(kFThreads), 0, st, gp, upp, l, k,
                       static_cast<const unsigned *>(ws), static_cast<int8_t *>(qx), static_cast<__half *>(sx));
  else
    hipLaunchKernelGGL(silu_slice_quant_kernel<false>, grid, dim3(kFThreads), 0, st, gp, upp, l, k,
                       static_cast<const unsigned *>(ws), static_cast<int8_t *>(qx), static_cast<__half *>(sx));
}


// tiled == -1: the fp16 output of the normalization itself into qx (no quantization)
void launch_rmsnorm_quantize(const void *x, const void *gamma, float eps, int64_t M, int64_t K, int tiled,
                             void *qx, void *sx, void *tx, hipStream_t st) {
  const bool out16 = tiled < 0;
  const dim3 grid(static_cast<unsigned>(M), out16 ? 1u : fused_row_parts(M, K, tx != nullptr));
  const __half *xp = static_cast<const __half *>(x);
  const __half *gp = static_cast<const __half *>(gamma);
  int8_t *q = static_cast<int8_t *>(qx);
  __half *s = static_cast<__half *>(sx);
  int *t = static_cast<int *>(tx);
  const int k = static_cast<int>(K);
  switch (fused_chunks(K)) {
    case 1: launch_rmsnorm_ch<1>(xp, gp, eps, k, tiled > 0, q, s, t, grid, st, out16); break;
    case 2: launch_rmsnorm_ch<2>(xp, gp, eps, k, tiled > 0, q, s, t, grid, st, out16); break;
    case 4: launch_rmsnorm_ch<4>(xp, gp, eps, k, tiled > 0, q, s, t, grid, st, out16); break;
    case 8: launch_rmsnorm_ch<8>(xp, gp, eps, k, tiled > 0, q, s, t, grid, st, out16); break;
    default: launch_rmsnorm_ch<16>(xp, gp, eps, k, tiled > 0, q, s, t, grid, st, out16); break;
  }
}

// tiled == -1: the fp16 activation itself into qx (no quantization)
void launch_silu_mul_quantize(const void *gate, const void *up, int64_t ld, int64_t M, int64_t K, int tiled,
                              void *qx, void *sx, void *tx, hipStream_t st) {
  const bool out16 = tiled < 0;
  const dim3 grid(static_cast<unsigned>(M), out16 ? 1u : fused_row_parts(M, K, tx != nullptr));
  const __half *gp = static_cast<const __half *>(gate);
  const __half *up_ = static_cast<const __half *>(up);
  int8_t *q = static_cast<int8_t *>(qx);
  __half *s = static_cast<__half *>(sx);
  int *t = static_cast<int *>(tx);
  const int k = static_cast<int>(K), l = static_cast<int>(ld);
  switch (fused_chunks(K)) {
    case 1: launch_silu_ch<1>(gp, up_, l, k, tiled > 0, q, s, t, grid, st, out16); break;
    case 2: launch_silu_ch<2>(gp, up_, l, k, tiled > 0, q, s, t, grid, st, out16); break;
    case 4: launch_silu_ch<4>(gp, up_, l, k, tiled > 0, q, s, t, grid, st, out16); break;
    case 8: launch_silu_ch<8>(gp, up_, l, k, tiled > 0, q, s, t, grid, st, out16); break;
    default: launch_silu_ch<16>(gp, up_, l, k, tiled > 0, q, s, t, grid, st, out16); break;
  }
}

}  // namespace qoq
