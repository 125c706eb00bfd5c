// Per-token INT8 activation quantizer and offline QoQ weight packer (gfx950).
//
// Activation side: per-token symmetric INT8 ("QServe: W4A8KV4 Quantization and
// System Co-design ..." summary, the s_X factor of the epilogue; symmetric
// quantizer of "01 inference papers and experiments" §4.1).
// Weight side: progressive group quantization with the protective range
// ("QServe ..." summary, sections on progressive group quantization and the
// protective quantization range; "QServe：把 W4A8KV4 ..." review §3.1) and the
// compute-order storage layout (review §3.2), bytes as described in include/qoq.h.
#include "qoq_device.h"
#include "qoq_internal.h"

#include <algorithm>

namespace qoq {

// ---------------------------------------------------------------------------
// activation quantizer: 256-thread workgroups, gridDim.y of them per token row.
// Each thread keeps up to kActChunks 16-byte chunks of the row in registers so the
// row is read from HBM once; longer rows re-read the remainder (L2-resident) in the
// second pass.  With few tokens a row is split over gridDim.y workgroups: each
// reads the whole row for the maximum (the other reads hit L2) and quantizes and
// stores only the register slots c with c % gridDim.y == blockIdx.y, so the work of
// a long row is not left to one compute unit.
// ---------------------------------------------------------------------------
constexpr int kActThreads = 256;
constexpr int kActChunks = 16;   // 16 x 8 halves x 256 threads = rows up to K = 32768

// sum of the 8 signed codes of a chunk (v_dot4_i32_i8 against ones)
__device__ __forceinline__ int code_sum8(uint2 q) {
  return __builtin_amdgcn_sdot4(static_cast<int>(q.x), 0x01010101, 0, false) +
         __builtin_amdgcn_sdot4(static_cast<int>(q.y), 0x01010101, 0, false);
}

// ROWSUM: also t[row] = sum_k qx[row, k] (the activation term of the per-channel
// epilogue, "QServe ..." summary, per-channel fast dequantization: t_X is computed
// by the memory-bound kernel that precedes the GEMM)
// TILED: codes stored in the tiled layout of the few-token GEMM (tiled_offset)
// instead of row-major.
template <bool ROWSUM, bool TILED = false>
__global__ __launch_bounds__(kActThreads) void quantize_act_kernel(const __half *__restrict__ x, int K,
                                                                   int8_t *__restrict__ qx,
                                                                   __half *__restrict__ sx,
                                                                   int *__restrict__ tx) {
  __shared__ unsigned red[kActThreads / 64];
  __shared__ int tred[kActThreads / 64];
  const int row = blockIdx.x;
  const int nchunk = K >> 3;
  const uint4 *xr = reinterpret_cast<const uint4 *>(x + static_cast<size_t>(row) * K);
  uint2 *qr = reinterpret_cast<uint2 *>(qx + static_cast<size_t>(row) * K);

  // every load is issued before any value is used, so they are in flight together
  // (a use right after each load would wait for it, one memory latency per chunk);
  // chunks past the row are zero and leave the maximum unchanged
  uint4 v[kActChunks];
#pragma unroll
  for (int c = 0; c < kActChunks; ++c) {
    int idx = threadIdx.x + c * kActThreads;
    v[c] = idx < nchunk ? xr[idx] : make_uint4(0u, 0u, 0u, 0u);
  }
  unsigned amax = 0;
#pragma unroll
  for (int c = 0; c < kActChunks; ++c) amax = absmax_bits8(v[c], amax);
  for (int idx = threadIdx.x + kActChunks * kActThreads; idx < nchunk; idx += kActThreads)
    amax = absmax_bits8(xr[idx], amax);

  amax = wave_max_u32(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kActThreads / 64; ++w) amax = max(amax, red[w]);

  const __half sh = sym_scale(amax, static_cast<float>(kXQmax));
  const float s = __half2float(sh);
  const float rcp = act_rcp(s);
  const int part = blockIdx.y, parts = gridDim.y;
  if (threadIdx.x == 0 && part == 0) sx[row] = sh;

  auto store = [&](int idx, uint2 q) {
    if (TILED)
      *reinterpret_cast<uint2 *>(qx + tiled_offset(row, 8 * idx, K)) = q;
    else
      qr[idx] = q;
  };
  int tsum = 0;
#pragma unroll
  for (int c = 0; c < kActChunks; ++c) {
    int idx = threadIdx.x + c * kActThreads;
    if (idx < nchunk && c % parts == part) {
      const uint2 q = quant_chunk8(v[c], s, rcp);
      store(idx, q);
      if (ROWSUM) tsum += code_sum8(q);
    }
  }
  // the remainder of rows longer than the register budget (launched with one part)
  for (int idx = threadIdx.x + kActChunks * kActThreads; idx < nchunk; idx += kActThreads) {
    const uint2 q = quant_chunk8(xr[idx], s, rcp);
    store(idx, q);
    if (ROWSUM) tsum += code_sum8(q);
  }
  if (ROWSUM) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) tsum += __shfl_xor(tsum, off, 64);
    if ((threadIdx.x & 63) == 0) tred[threadIdx.x >> 6] = tsum;
    __syncthreads();
    if (threadIdx.x == 0) {
      int t = 0;
#pragma unroll
      for (int w = 0; w < kActThreads / 64; ++w) t += tred[w];
      tx[row] = t;
    }
  }
}

// Many short rows: one wave per row, four rows per workgroup, the row held in
// registers (up to kRowChunks 16-byte chunks per lane) and its maximum taken within
// the wave, with no LDS and no barrier.  For thousands of rows of a few KB a
// 256-thread workgroup per row spends more on its setup and barrier than on its
// data.  Same arithmetic as quantize_act_kernel, row-major codes.
constexpr int kRowChunks = 8;                       // rows up to K = 64 x 8 x 8 = 4096
constexpr int64_t kRowKernelMinRows = 1024;

template <bool ROWSUM>
__global__ __launch_bounds__(256) void quantize_act_rows_kernel(const __half *__restrict__ x, int M, int K,
                                                                int8_t *__restrict__ qx, __half *__restrict__ sx,
                                                                int *__restrict__ tx) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;                             // whole waves; no barrier below
  const int nchunk = K >> 3;
  const uint4 *xr = reinterpret_cast<const uint4 *>(x + static_cast<size_t>(row) * K);
  uint2 *qr = reinterpret_cast<uint2 *>(qx + static_cast<size_t>(row) * K);
  uint4 v[kRowChunks];
#pragma unroll
  for (int c = 0; c < kRowChunks; ++c) {
    const int idx = lane + 64 * c;
    v[c] = idx < nchunk ? xr[idx] : make_uint4(0u, 0u, 0u, 0u);
  }
  unsigned amax = 0;
#pragma unroll
  for (int c = 0; c < kRowChunks; ++c) amax = absmax_bits8(v[c], amax);
  amax = wave_max_u32(amax);
  const __half sh = sym_scale(amax, static_cast<float>(kXQmax));
  const float s = __half2float(sh);
  const float rcp = act_rcp(s);
  if (lane == 0) sx[row] = sh;
  int tsum = 0;
#pragma unroll
  for (int c = 0; c < kRowChunks; ++c) {
    const int idx = lane + 64 * c;
    if (idx < nchunk) {
      const uint2 q = quant_chunk8(v[c], s, rcp);
      qr[idx] = q;
      if (ROWSUM) tsum += code_sum8(q);
    }
  }
  if (ROWSUM) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) tsum += __shfl_xor(tsum, off, 64);
    if (lane == 0) tx[row] = tsum;
  }
}

static bool use_rows_kernel(int64_t M, int64_t K) { return M >= kRowKernelMinRows && K <= 64 * 8 * kRowChunks; }

// workgroups per row: enough to give a few rows about 256 workgroups, at most one
// per register slot in use; one when the row does not fit the registers
unsigned row_parts(int64_t M, int64_t K) {
  const int64_t slots = (K / 8 + kActThreads - 1) / kActThreads;
  if (slots > kActChunks) return 1;
  return static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>(slots, 256 / M)));
}

void launch_quantize_activations(const void *x, int64_t M, int64_t K, void *qx, void *sx,
                                 hipStream_t stream) {
  if (use_rows_kernel(M, K)) {
    hipLaunchKernelGGL(quantize_act_rows_kernel<false>, dim3(static_cast<unsigned>((M + 3) / 4)), dim3(256), 0,
                       stream, static_cast<const __half *>(x), static_cast<int>(M), static_cast<int>(K),
                       static_cast<int8_t *>(qx), static_cast<__half *>(sx), nullptr);
    return;
  }
  hipLaunchKernelGGL(quantize_act_kernel<false>, dim3(static_cast<unsigned>(M), row_parts(M, K)),
                     dim3(kActThreads), 0, stream, static_cast<const __half *>(x), static_cast<int>(K),
                     static_cast<int8_t *>(qx), static_cast<__half *>(sx), nullptr);
}

void launch_quantize_activations_tiled(const void *x, int64_t M, int64_t K, void *qx, void *sx,
                                       hipStream_t stream) {
  hipLaunchKernelGGL((quantize_act_kernel<false, true>), dim3(static_cast<unsigned>(M), row_parts(M, K)),
                     dim3(kActThreads), 0, stream, static_cast<const __half *>(x), static_cast<int>(K),
                     static_cast<int8_t *>(qx), static_cast<__half *>(sx), nullptr);
}

// one part per row: the code sum needs every code of the row
void launch_quantize_activations_rowsum_tiled(const void *x, int64_t M, int64_t K, void *qx, void *sx, void *tx,
                                              hipStream_t stream) {
  hipLaunchKernelGGL((quantize_act_kernel<true, true>), dim3(static_cast<unsigned>(M)), dim3(kActThreads), 0, stream,
                     static_cast<const __half *>(x), static_cast<int>(K), static_cast<int8_t *>(qx),
                     static_cast<__half *>(sx), static_cast<int *>(tx));
}

void launch_quantize_activations_rowsum(const void *x, int64_t M, int64_t K, void *qx, void *sx, void *tx,
                                        hipStream_t stream) {
  if (use_rows_kernel(M, K)) {
    hipLaunchKernelGGL(quantize_act_rows_kernel<true>, dim3(static_cast<unsigned>((M + 3) / 4)), dim3(256), 0,
                       stream, static_cast<const __half *>(x), static_cast<int>(M), static_cast<int>(K),
                       static_cast<int8_t *>(qx), static_cast<__half *>(sx), static_cast<int *>(tx));
    return;
  }
  hipLaunchKernelGGL(quantize_act_kernel<true>, dim3(static_cast<unsigned>(M)), dim3(kActThreads), 0, stream,
                     static_cast<const __half *>(x), static_cast<int>(K), static_cast<int8_t *>(qx),
                     static_cast<__half *>(sx), static_cast<int *>(tx));
}

// ---------------------------------------------------------------------------
// weight packer: one wave per output channel n (four channels per workgroup).
//   pass 1: absmax of the row -> s_W[n]
//   pass 2: per group of 128: level-0 codes (two per lane), wave min/max, level-1
//           scale / zero / codes, then the bytes of the storage layout.
// Lane l holds k = 2l, 2l+1 of the group.  For l < 32 those are the low-nibble
// codes of bytes i = 2l mod 16, i+1 in slot h = l / 8; lane l + 32 holds the
// matching high-nibble codes (k + 64).
// ---------------------------------------------------------------------------
// Store one group's codes of channel c of strip b: lane l holds the codes of k = 2l,
// 2l+1 of the group.  For l < 32 those are the low-nibble codes of bytes i = 2l mod
// 16, i+1 in slot h = l / 8; lane l + 32 holds the matching high-nibble codes (k + 64).
__device__ __forceinline__ void store_group_codes(unsigned u0, unsigned u1, int lane, uint8_t *__restrict__ packed,
                                                  int b, int G, int j, int c) {
  const unsigned two = u0 | (u1 << 8);                                  // low nibbles
  const unsigned upper = static_cast<unsigned>(__shfl_down(static_cast<int>(two), 32, 64));
  const unsigned bytes2 = two | (upper << 4);                           // valid for lane < 32
  const unsigned next = static_cast<unsigned>(__shfl_down(static_cast<int>(bytes2), 1, 64));
  if (lane < 32 && (lane & 1) == 0) {
    const int h = lane >> 3;
    const int i = (2 * lane) & 15;                                      // 0, 4, 8, 12
    const size_t off = (static_cast<size_t>(b * G + j) * 64 + 16 * h + c) * 16 + i;
    *reinterpret_cast<unsigned *>(packed + off) = (bytes2 & 0xffffu) | (next << 16);
  }
}

__device__ __forceinline__ int w_code(unsigned half_bits, float s) {
  return sym_code(half_bits_to_float(half_bits), s, kWQmax);
}

__global__ __launch_bounds__(256) void pack_weights_kernel(const __half *__restrict__ w, int N, int K,
                                                           uint8_t *__restrict__ packed,
                                                           uint16_t *__restrict__ meta,
                                                           __half *__restrict__ sw) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const __half *wr = w + static_cast<size_t>(n) * K;

  unsigned amax = 0;
  for (int k = lane * 8; k < K; k += 64 * 8)
    amax = absmax_bits8(*reinterpret_cast<const uint4 *>(wr + k), amax);
  amax = wave_max_u32(amax);
  const __half sh = sym_scale(amax, static_cast<float>(kWQmax));
  const float s = __half2float(sh);
  if (lane == 0) sw[n] = sh;

  const int G = K / kGroup;
  const int b = n >> 4, c = n & 15;
  for (int j = 0; j < G; ++j) {
    unsigned pair = *reinterpret_cast<const unsigned *>(wr + kGroup * j + 2 * lane);
    int q0 = w_code(pair & 0xffffu, s);
    int q1 = w_code(pair >> 16, s);
    int lo = wave_min_i32(min(min(q0, q1), 0));
    int hi = wave_max_i32(max(max(q0, q1), 0));
    int su = max(1, (hi - lo + 14) / 15);            // ceil((hi - lo) / 15), at least 1
    int z = min(max(rne_div(-lo, su), 0), 15);
    unsigned u0 = static_cast<unsigned>(min(max(z + rne_div(q0, su), 0), 15));
    unsigned u1 = static_cast<unsigned>(min(max(z + rne_div(q1, su), 0), 15));
    store_group_codes(u0, u1, lane, packed, b, G, j, c);
    if (lane == 0) meta[static_cast<size_t>(b * G + j) * 16 + c] = static_cast<uint16_t>(su | (z << 8));
  }
}

// ---------------------------------------------------------------------------
// per-channel packer: one wave per output channel n.
//   pass 1: min / max of the row (widened to contain 0) -> s_W[n] (fp16), z[n]
//   pass 2: per group of 128 the codes q = clamp(z + rint(w / s_W), 0, 15), in the
//           same storage layout as the per-group packer.
// ("QServe ..." summary, integer quantization (asymmetric, zero point) with one
// scale and zero per output channel; per-channel fast dequantization)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_weights_pc_kernel(const __half *__restrict__ w, int N, int K,
                                                              uint8_t *__restrict__ packed,
                                                              uint8_t *__restrict__ zeros,
                                                              __half *__restrict__ sw) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const __half *wr = w + static_cast<size_t>(n) * K;

  float lo = 0.0f, hi = 0.0f;                                         // the range contains 0
  for (int k = lane * 8; k < K; k += 64 * 8) {
    const uint4 v = *reinterpret_cast<const uint4 *>(wr + k);
    const unsigned u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = half_bits_to_float(u[i] & 0xffffu), b = half_bits_to_float(u[i] >> 16);
      lo = fminf(lo, fminf(a, b));
      hi = fmaxf(hi, fmaxf(a, b));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, off, 64));
    hi = fmaxf(hi, __shfl_xor(hi, off, 64));
  }
  float q = __fdiv_rn(hi - lo, 15.0f);
  __asm__ volatile("" : "+v"(q));       // the fp32 quotient is rounded before narrowing
  const __half sh = __float2half_rn(q);
  const float s = __half2float(sh);
  const int z = s == 0.0f ? 0 : static_cast<int>(fminf(fmaxf(rintf(__fdiv_rn(-lo, s)), 0.0f), 15.0f));
  if (lane == 0) {
    sw[n] = sh;
    zeros[n] = static_cast<uint8_t>(z);
  }

  const int G = K / kGroup;
  const int b = n >> 4, c = n & 15;
  for (int j = 0; j < G; ++j) {
    const unsigned pair = *reinterpret_cast<const unsigned *>(wr + kGroup * j + 2 * lane);
    unsigned u[2] = {0u, 0u};
    if (s != 0.0f) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float r = rintf(__fdiv_rn(half_bits_to_float((pair >> (16 * e)) & 0xffffu), s));
        u[e] = static_cast<unsigned>(fminf(fmaxf(static_cast<float>(z) + r, 0.0f), 15.0f));
      }
    }
    store_group_codes(u[0], u[1], lane, packed, b, G, j, c);
  }
}

void launch_quantize_pack_weights_pc(const void *w, int64_t N, int64_t K, void *packed, void *zeros, void *sw,
                                     hipStream_t stream) {
  hipLaunchKernelGGL(pack_weights_pc_kernel, dim3(static_cast<unsigned>((N + 3) / 4)), dim3(256), 0, stream,
                     static_cast<const __half *>(w), static_cast<int>(N), static_cast<int>(K),
                     static_cast<uint8_t *>(packed), static_cast<uint8_t *>(zeros), static_cast<__half *>(sw));
}

void launch_quantize_pack_weights(const void *w, int64_t N, int64_t K, void *packed, void *meta, void *sw,
                                  hipStream_t stream) {
  unsigned blocks = static_cast<unsigned>((N + 3) / 4);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const __half *>(w),
                     static_cast<int>(N), static_cast<int>(K), static_cast<uint8_t *>(packed),
                     static_cast<uint16_t *>(meta), static_cast<__half *>(sw));
}

}  // namespace qoq
