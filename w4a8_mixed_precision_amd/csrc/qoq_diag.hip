// Diagnostic kernels: in-register dequantization to memory (verifies the GEMM's
// own dequantization routine), a streaming copy (bandwidth ceiling and the
// reference for hardware byte counters) and a one-instruction MFMA probe (pins the
// operand / result lane layout of v_mfma_i32_16x16x64_i8).
#include "qoq_device.h"
#include "qoq_internal.h"

namespace qoq {

// one wave per (strip, group) chunk: lane l = 16 h + c holds column 16 b + c and
// codes k = 128 j + 16 h + i (low nibbles) and k + 64 (high nibbles), i = 0..15
__global__ __launch_bounds__(256) void dequant_packed_kernel(const uint4 *__restrict__ packed,
                                                             const uint16_t *__restrict__ meta, int N, int K,
                                                             int8_t *__restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int G = K >> 7;
  const long chunk = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (chunk >= static_cast<long>(N >> 4) * G) return;
  const int b = static_cast<int>(chunk / G), j = static_cast<int>(chunk % G);
  const int c = lane & 15, h = lane >> 4;
  const uint4 p = packed[chunk * 64 + lane];
  const unsigned md = meta[chunk * 16 + c];
  v4i b0, b1;
  dequant_lane(p, group_consts(md), b0, b1);
  int8_t *row = w + static_cast<size_t>(16 * b + c) * K + 128 * j + 16 * h;
  *reinterpret_cast<v4i *>(row) = b0;
  *reinterpret_cast<v4i *>(row + 64) = b1;
}

void launch_dequantize_packed(const void *packed, const void *meta, int64_t N, int64_t K, void *w_i8,
                              hipStream_t stream) {
  const long chunks = (N / 16) * (K / 128);
  hipLaunchKernelGGL(dequant_packed_kernel, dim3(static_cast<unsigned>((chunks + 3) / 4)), dim3(256), 0, stream,
                     static_cast<const uint4 *>(packed), static_cast<const uint16_t *>(meta), static_cast<int>(N),
                     static_cast<int>(K), static_cast<int8_t *>(w_i8));
}

__global__ __launch_bounds__(256) void stream_copy_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                          size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

void launch_stream_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n16);
}

// read-only stream: each thread loads U 16-byte words per iteration (all issued
// before any is used) and folds them into a checksum that is stored only if it
// equals a value the data never produces, so the loads cannot be dropped
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ src, size_t n16,
                                                          unsigned *__restrict__ sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  unsigned acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

void launch_stream_read(const void *src, size_t bytes, void *sink, int unroll, int blocks, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const dim3 g(static_cast<unsigned>(blocks)), b(256);
  const uint4 *s = static_cast<const uint4 *>(src);
  unsigned *k = static_cast<unsigned *>(sink);
  if (unroll >= 8)
    hipLaunchKernelGGL(stream_read_kernel<8>, g, b, 0, stream, s, n16, k);
  else if (unroll >= 4)
    hipLaunchKernelGGL(stream_read_kernel<4>, g, b, 0, stream, s, n16, k);
  else
    hipLaunchKernelGGL(stream_read_kernel<1>, g, b, 0, stream, s, n16, k);
}

// MFMA-only loop: each wave runs `iters` rounds of 8 independent
// v_mfma_i32_16x16x64_i8 chains on register operands (the practical INT8 matrix
// throughput); the accumulators are folded and stored only in a case that does not
// occur for the operands used, so the work cannot be dropped
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, int seed, int *__restrict__ sink) {
  v4i a = {seed, seed + 1, seed + 2, seed + 3};
  v4i b = {seed ^ 0x5a5a5a5a, seed + 7, seed - 3, seed * 5};
  // 32x32x32: on gfx950 the 16x16x64 INT8 instruction delivers about half the ops
  // per cycle of this one (2.9 against 4.9 POPS measured), so this is the ceiling
  v16i acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = v16i{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = mfma32x32x32(a, b, acc[i]);
  }
  int x = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) x ^= acc[i][0] ^ acc[i][5] ^ acc[i][10] ^ acc[i][15];
  if (x == 0x7fffffff) sink[0] = x;
}

// The same loop on operands taken from memory: lane l of wave w of block b loads
// eight A and eight B fragments (16 bytes each) from a and b at positions spread
// over the buffers, then runs iters rounds of eight MFMAs cycling through them, so
// the matrix units see the toggling of real data (the chip's clock under MFMA load
// depends on it: constant operands let it run faster than GEMM data does).
__global__ __launch_bounds__(256) void mfma_peak_operands_kernel(const v4i *__restrict__ a, size_t na,
                                                                 const v4i *__restrict__ b, size_t nb, int iters,
                                                                 int *__restrict__ sink) {
  const size_t t = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  v4i fa[8], fb[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    fa[i] = a[(t * 8 + i * 131 + 17) % na];
    fb[i] = b[(t * 8 + i * 257 + 5) % nb];
  }
  v16i acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = v16i{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i & 3] = mfma32x32x32(fa[i], fb[(i * 5 + 3) & 7], acc[i & 3]);
  }
  int x = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) x ^= acc[i][0] ^ acc[i][5] ^ acc[i][10] ^ acc[i][15];
  if (x == 0x7fffffff) sink[0] = x;
}

void launch_mfma_peak_operands(const void *a, size_t a_bytes, const void *b, size_t b_bytes, int iters, int blocks,
                               void *sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_peak_operands_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<const v4i *>(a), a_bytes / 16, static_cast<const v4i *>(b), b_bytes / 16, iters,
                     static_cast<int *>(sink));
}

void launch_mfma_peak(int iters, int blocks, void *sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, iters, 3,
                     static_cast<int *>(sink));
}

__global__ __launch_bounds__(64) void mfma_probe_kernel(const v4i *__restrict__ a, const v4i *__restrict__ b,
                                                        v4i *__restrict__ d) {
  const int l = threadIdx.x;
  d[l] = mfma16x16x64(a[l], b[l], v4i{0, 0, 0, 0});
}

__global__ __launch_bounds__(64) void mfma_probe32_kernel(const v4i *__restrict__ a, const v4i *__restrict__ b,
                                                          v16i *__restrict__ d) {
  const int l = threadIdx.x;
  d[l] = mfma32x32x32(a[l], b[l], v16i{});
}

void launch_mfma_probe32(const void *a, const void *b, void *d, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe32_kernel, dim3(1), dim3(64), 0, stream, static_cast<const v4i *>(a),
                     static_cast<const v4i *>(b), static_cast<v16i *>(d));
}

void launch_mfma_probe(const void *a, const void *b, void *d, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(1), dim3(64), 0, stream, static_cast<const v4i *>(a),
                     static_cast<const v4i *>(b), static_cast<v4i *>(d));
}

}  // namespace qoq
