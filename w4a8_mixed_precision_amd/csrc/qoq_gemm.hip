// W4A8 per-group GEMM on INT8 MFMA (gfx950 / CDNA4).
//
// acc[m,n] = sum_k qx[m,k] * w_hat[n,k],  w_hat = (q_u4 - z) * s_u8  (exact INT32)
// out[m,n] = fp16( float(acc) * (float(s_X[m]) * float(s_W[n])) )
//
// Method: "QServe: W4A8KV4 Quantization and System Co-design ..." summary, per-group
// W4A8 GEMM fast dequantization (multiply-then-subtract in registers, all products
// on the INT8 matrix path) and the epilogue O = (Q_X Q_W) ⊙ (s_W x s_X); review
// "QServe：把 W4A8KV4 ..." §3.2 (compute-order weight layout, 128-bit loads, split-k
// for small batches) and §4 step 3 (main loop: load, unpack, dequantize, INT8 MMA,
// epilogue).  The tilings below are this library's own, sized for 64-lane waves,
// the 16x16x64 INT8 MFMA and the 160 KB LDS of a CDNA4 compute unit.
//
// MFMA operand mapping used throughout (v_mfma_i32_16x16x64_i8): lane l supplies
// row (l % 16) of A and column (l % 16) of B, each as 16 bytes covering the k
// indices 16*(l / 16) .. +15 of a 64-wide k block; A and B use the same mapping, so
// the sum over k is correct whatever order the unit walks the 64 products in.
// Result: lane l, register i holds D[4*(l / 16) + i][l % 16].
#include "qoq_device.h"
#include "qoq_internal.h"

#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

namespace qoq {

namespace {

__device__ __forceinline__ void store_result(void *out, int out_kind, size_t idx, int acc, float scale) {
  if (out_kind == 0)
    static_cast<__half *>(out)[idx] = mul_round_half(static_cast<float>(acc), scale);
  else
    static_cast<int *>(out)[idx] = acc;
}

// ---------------------------------------------------------------------------
// Skinny regime (a few tokens: the weight stream from HBM is the whole cost).
//   workgroup = WAVES waves; it owns NBW strips of 16 output columns and 16*MT
//   token rows, and its waves split the K groups round-robin (split-K): wave w
//   takes groups w, w + WAVES, w + 2*WAVES, ...  A wave works through its groups in
//   batches of U: every load of a batch (one 128-bit packed-code load per lane per
//   strip, one metadata load, the activation fragments) is issued before any
//   of them is consumed.  Batches live in a ring of R register sets: batch b + R - 1
//   is issued before batch b is computed, so R - 1 batches are in flight while one
//   is computed, and the wait for batch b leaves the later ones in flight.  The
//   ring is indexed by compile-time slots (the loop is unrolled by R): a copy from
//   one register set to another at the loop edge would wait for every load in
//   flight.  Slots past the wave's last group get zero activations and add nothing.
//   AT: the activation codes are in the tiled layout (tiled_offset), so each
//   fragment load is 1 KB of consecutive bytes (row-major codes: 16 rows, 16 cache
//   lines, per load).  Partial sums of the waves are added through LDS; the
//   epilogue follows.
// ---------------------------------------------------------------------------
// The metadata word of column col of a chunk is loaded as the aligned 32-bit pair
// (columns col & ~1, col | 1) and shifted at its use (meta_of): a 16-bit load is
// widened right where it lands, and when that point is the merge after a
// conditional load, the widening waits for every load issued before it.
__device__ __forceinline__ unsigned meta_pair(const uint16_t *__restrict__ meta, size_t chunk, int col) {
  return reinterpret_cast<const unsigned *>(meta)[chunk * 8 + (col >> 1)];
}

__device__ __forceinline__ unsigned meta_of(unsigned pair, int col) { return pair >> (16 * (col & 1)); }

// A packed-code load.  NT (streaming): the load carries the non-temporal hint, so
// the caches keep these lines only briefly.  Few tokens read every weight once, and
// on the long weight streams this raises the rate HBM delivers them at (Qwen-72B
// gate+up, 248 MB: 5.4 -> 5.8 TB/s measured); on short streams the hint costs a
// little latency, so both forms are configurations and the measured table chooses.
template <bool NT>
__device__ __forceinline__ uint4 load_codes(const uint4 *__restrict__ p) {
  if constexpr (NT) {
    typedef unsigned u4v_nt __attribute__((ext_vector_type(4)));
    const u4v_nt v = __builtin_nontemporal_load(reinterpret_cast<const u4v_nt *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *p;
  }
}

template <int MT, int NBW, int U>
struct SkinnyBatch {
  uint4 p[U][NBW];
  unsigned md[U][NBW];
  v4i a0[U][MT];
  v4i a1[U][MT];
};

// Issues every load of batch b (groups t = b*U .. b*U+U-1 of this wave).  Only
// scalars come in, so no pointer array can end up in private (scratch) memory.
template <int MT, int NBW, int WAVES, int U, bool PC, bool AT, bool NT>
__device__ __forceinline__ void skinny_load(SkinnyBatch<MT, NBW, U> &B, int b, int ngroups, int wave,
                                            const uint4 *__restrict__ packed, const uint16_t *__restrict__ meta,
                                            const int8_t *__restrict__ qx, int strip0, int NS, int G, int K,
                                            int M, int m0, int lane) {
  const int col = lane & 15, kq = lane >> 4;
  const v4i zero4 = {0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = b * U + u;
    const bool ok = t < ngroups;
    // a slot past the wave's last group reloads its first group's weights (in
    // bounds) and zero activations, so it adds nothing; the weight loads stay
    // unconditional (a value merged from a conditional load is consumed at the
    // merge, which would wait for every load issued before it)
    const int j = wave + WAVES * (ok ? t : 0);
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      // strips past the end repeat the last one; their results are dropped at the store
      const size_t chunk = static_cast<size_t>(min(strip0 + nb, NS - 1)) * G + j;
      B.p[u][nb] = load_codes<NT>(packed + chunk * 64 + lane);
      B.md[u][nb] = PC ? 0u : meta_pair(meta, chunk, col);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = m0 + 16 * mt + col;
      const bool oka = ok && r < M;
      // row-major codes: a lane reads 16 bytes of its own row (16 rows per load);
      // tiled codes: the two 1 KB blocks (k blocks 2j, 2j + 1) of the row block
      const int8_t *a = AT ? qx + ((static_cast<size_t>((m0 >> 4) + mt) * (K >> 6) + 2 * j) * 64 + lane) * 16
                           : qx + static_cast<size_t>(oka ? r : 0) * K + 128 * j + 16 * kq;
      B.a0[u][mt] = oka ? *reinterpret_cast<const v4i *>(a) : zero4;
      B.a1[u][mt] = oka ? *reinterpret_cast<const v4i *>(a + (AT ? 1024 : 64)) : zero4;
    }
  }
}

template <int MT, int NBW, int U, bool PC>
__device__ __forceinline__ void skinny_compute(const SkinnyBatch<MT, NBW, U> &B, v4i (&acc)[MT][NBW], int col) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      v4i b0, b1;
      weights_lane<PC>(B.p[u][nb], meta_of(B.md[u][nb], col), b0, b1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt][nb] = mfma16x16x64(B.a0[u][mt], b0, acc[mt][nb]);
        acc[mt][nb] = mfma16x16x64(B.a1[u][mt], b1, acc[mt][nb]);
      }
    }
}

template <int MT, int NBW, int WAVES, int U, int R, int OUT, bool PC, bool AT = false, bool NT = false>
__global__ __launch_bounds__(64 * WAVES) void gemm_skinny_kernel(
    const int8_t *__restrict__ qx, const __half *__restrict__ sx, const uint4 *__restrict__ packed,
    const uint16_t *__restrict__ meta, const __half *__restrict__ sw, const uint8_t *__restrict__ zp,
    const int *__restrict__ trow, void *__restrict__ out, int M, int N,
    int K, int, int *) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = K >> 7;
  const int NS = N >> 4;
  const int col = lane & 15;
  const int kq = lane >> 4;
  const int strip0 = blockIdx.x * NBW;
  const int m0 = blockIdx.y * (16 * MT);

  v4i acc[MT][NBW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[mt][nb] = v4i{0, 0, 0, 0};

  const int ngroups = wave < G ? (G - wave + WAVES - 1) / WAVES : 0;   // groups of this wave
  const int nbatch = (ngroups + U - 1) / U;

  SkinnyBatch<MT, NBW, U> ring[R];
#pragma unroll
  for (int r = 0; r < R - 1; ++r)
    if (r < nbatch)
      skinny_load<MT, NBW, WAVES, U, PC, AT, NT>(ring[r], r, ngroups, wave, packed, meta, qx, strip0, NS, G, K, M, m0,
                                             lane);
  for (int b0 = 0; b0 < nbatch; b0 += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int b = b0 + r;
      if (b >= nbatch) break;
      if (b + R - 1 < nbatch)
        skinny_load<MT, NBW, WAVES, U, PC, AT, NT>(ring[(r + R - 1) % R], b + R - 1, ngroups, wave, packed, meta, qx,
                                               strip0, NS, G, K, M, m0, lane);
      skinny_compute<MT, NBW, U, PC>(ring[r], acc, col);
    }
  }

  constexpr int T = MT * NBW;   // 16x16 tiles per wave
  if constexpr (WAVES > 1) {
    __shared__ int red[WAVES][T * 4][64];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][(mt * NBW + nb) * 4 + i][lane] = acc[mt][nb][i];
    __syncthreads();
    for (int e = threadIdx.x; e < T * 256; e += 64 * WAVES) {
      const int ln = e & 63;
      const int ti = e >> 6;
      int sum = 0;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) sum += red[w][ti][ln];
      const int t = ti >> 2, i = ti & 3;
      const int mt = t / NBW, nb = t % NBW;
      const int m = m0 + 16 * mt + 4 * (ln >> 4) + i;
      const int strip = strip0 + nb;
      if (m < M && strip < NS) {
        const int n = strip * 16 + (ln & 15);
        float scale = 0.0f;
        if (OUT == 0) scale = __half2float(sx[m]) * __half2float(sw[n]);
        if (PC) sum -= static_cast<int>(zp[n]) * trow[m];
        store_result(out, OUT, static_cast<size_t>(m) * N + n, sum, scale);
      }
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + 16 * mt + 4 * kq + i;
          const int strip = strip0 + nb;
          if (m < M && strip < NS) {
            const int n = strip * 16 + col;
            float scale = 0.0f;
            if (OUT == 0) scale = __half2float(sx[m]) * __half2float(sw[n]);
            const int v = acc[mt][nb][i] - (PC ? static_cast<int>(zp[n]) * trow[m] : 0);
            store_result(out, OUT, static_cast<size_t>(m) * N + n, v, scale);
          }
        }
  }
}

// ---------------------------------------------------------------------------
// Skinny regime on 32x32x32 MFMAs (17..64 tokens).  On gfx950 the 16x16x64 INT8
// instruction delivers about 60 % of the ops per cycle of v_mfma_i32_32x32x32_i8,
// so row blocks of 32 halve the matrix-core time of the few-token kernel where it
// shows (64 tokens).  Same split of the K groups over the waves, same batches and
// ring as above; a workgroup owns NP pairs of strips (32 columns each) and 32*MT2
// rows.  B operand of one pair (lane l: column l % 32, k = 16*(l / 32) + i of a
// 32-wide k block): slots 16*(l / 32) + c and 16*(l / 32) + 32 + c of the strip
// holding column l % 32 (c = l % 16) give, from their low and high nibbles, the four
// 32-wide k blocks of the group.  A operand (row l % 32 of the block, same k): 16
// bytes per lane per k block, from the tiled layout (two 16-row blocks) or the row.
// Result: lane l, register i holds D[8*(i / 4) + 4*(l / 32) + i % 4][l % 32].
// ---------------------------------------------------------------------------
template <int MT2, int NP, int U>
struct Skinny32Batch {
  uint4 p0[U][NP], p1[U][NP];
  unsigned md[U][NP];
  v4i a[U][MT2][4];
};

template <int MT2, int NP, int WAVES, int U, bool PC, bool AT, bool NT>
__device__ __forceinline__ void skinny32_load(Skinny32Batch<MT2, NP, U> &B, int b, int ngroups, int wave,
                                              const uint4 *__restrict__ packed, const uint16_t *__restrict__ meta,
                                              const int8_t *__restrict__ qx, int strip0, int NS, int G, int K,
                                              int M, int m0, int lane) {
  const int c32 = lane & 31, hi = lane >> 5, col = lane & 15;
  const v4i zero4 = {0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = b * U + u;
    const bool ok = t < ngroups;
    // past the wave's last group: in-bounds weight reload, zero activations
    const int j = wave + WAVES * (ok ? t : 0);
#pragma unroll
    for (int np = 0; np < NP; ++np) {
      const size_t chunk = static_cast<size_t>(min(strip0 + 2 * np + (c32 >> 4), NS - 1)) * G + j;
      B.p0[u][np] = load_codes<NT>(packed + chunk * 64 + 16 * hi + col);
      B.p1[u][np] = load_codes<NT>(packed + chunk * 64 + 16 * hi + 32 + col);
      B.md[u][np] = PC ? 0u : meta_pair(meta, chunk, col);
    }
#pragma unroll
    for (int mt = 0; mt < MT2; ++mt) {
      const int r = m0 + 32 * mt + c32;
      const bool oka = ok && r < M;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int8_t *a =
            AT ? qx + ((static_cast<size_t>(r >> 4) * (K >> 6) + 2 * j + (kb >> 1)) * 64 + ((2 * kb + hi) & 3) * 16 +
                       (r & 15)) * 16
               : qx + static_cast<size_t>(oka ? r : 0) * K + 128 * j + 32 * kb + 16 * hi;
        B.a[u][mt][kb] = oka ? *reinterpret_cast<const v4i *>(a) : zero4;
      }
    }
  }
}

template <int MT2, int NP, int U, bool PC>
__device__ __forceinline__ void skinny32_compute(const Skinny32Batch<MT2, NP, U> &B, v16i (&acc)[MT2][NP],
                                                 int col) {
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int np = 0; np < NP; ++np) {
      v4i b[4];
      weights_lane<PC>(B.p0[u][np], meta_of(B.md[u][np], col), b[0], b[2]);
      weights_lane<PC>(B.p1[u][np], meta_of(B.md[u][np], col), b[1], b[3]);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt) acc[mt][np] = mfma32x32x32(B.a[u][mt][kb], b[kb], acc[mt][np]);
    }
}

template <int MT2, int NP, int WAVES, int U, int R, int OUT, bool PC, bool AT = false, bool NT = false>
__global__ __launch_bounds__(64 * WAVES) void gemm_skinny32_kernel(
    const int8_t *__restrict__ qx, const __half *__restrict__ sx, const uint4 *__restrict__ packed,
    const uint16_t *__restrict__ meta, const __half *__restrict__ sw, const uint8_t *__restrict__ zp,
    const int *__restrict__ trow, void *__restrict__ out, int M, int N, int K, int, int *) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = K >> 7;
  const int NS = N >> 4;
  const int col = lane & 15;
  const int strip0 = blockIdx.x * 2 * NP;
  const int m0 = blockIdx.y * (32 * MT2);

  v16i acc[MT2][NP];
#pragma unroll
  for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
    for (int np = 0; np < NP; ++np) acc[mt][np] = v16i{};

  const int ngroups = wave < G ? (G - wave + WAVES - 1) / WAVES : 0;
  const int nbatch = (ngroups + U - 1) / U;

  Skinny32Batch<MT2, NP, U> ring[R];
#pragma unroll
  for (int r = 0; r < R - 1; ++r)
    if (r < nbatch)
      skinny32_load<MT2, NP, WAVES, U, PC, AT, NT>(ring[r], r, ngroups, wave, packed, meta, qx, strip0, NS, G, K, M,
                                               m0, lane);
  for (int b0 = 0; b0 < nbatch; b0 += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int b = b0 + r;
      if (b >= nbatch) break;
      if (b + R - 1 < nbatch)
        skinny32_load<MT2, NP, WAVES, U, PC, AT, NT>(ring[(r + R - 1) % R], b + R - 1, ngroups, wave, packed, meta, qx,
                                                 strip0, NS, G, K, M, m0, lane);
      skinny32_compute<MT2, NP, U, PC>(ring[r], acc, col);
    }
  }

  constexpr int T = MT2 * NP;   // 32x32 tiles per wave
  if constexpr (WAVES > 1) {
    __shared__ int red[WAVES][T * 16][64];
#pragma unroll
    for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
      for (int np = 0; np < NP; ++np)
#pragma unroll
        for (int i = 0; i < 16; ++i) red[wave][(mt * NP + np) * 16 + i][lane] = acc[mt][np][i];
    __syncthreads();
    for (int e = threadIdx.x; e < T * 1024; e += 64 * WAVES) {
      const int ln = e & 63;
      const int ti = e >> 6;
      int sum = 0;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) sum += red[w][ti][ln];
      const int t = ti >> 4, i = ti & 15;
      const int mt = t / NP, np = t % NP;
      const int m = m0 + 32 * mt + 8 * (i >> 2) + 4 * (ln >> 5) + (i & 3);
      const int c = ln & 31;
      const int strip = strip0 + 2 * np + (c >> 4);
      if (m < M && strip < NS) {
        const int n = strip * 16 + (c & 15);
        float scale = 0.0f;
        if (OUT == 0) scale = __half2float(sx[m]) * __half2float(sw[n]);
        if (PC) sum -= static_cast<int>(zp[n]) * trow[m];
        store_result(out, OUT, static_cast<size_t>(m) * N + n, sum, scale);
      }
    }
  } else {
    const int c = lane & 31;
#pragma unroll
    for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
      for (int np = 0; np < NP; ++np)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = m0 + 32 * mt + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          const int strip = strip0 + 2 * np + (c >> 4);
          if (m < M && strip < NS) {
            const int n = strip * 16 + (c & 15);
            float scale = 0.0f;
            if (OUT == 0) scale = __half2float(sx[m]) * __half2float(sw[n]);
            const int v = acc[mt][np][i] - (PC ? static_cast<int>(zp[n]) * trow[m] : 0);
            store_result(out, OUT, static_cast<size_t>(m) * N + n, v, scale);
          }
        }
  }
}

// ---------------------------------------------------------------------------
// Few tokens with the activation quantization fused in (the linear entry point,
// few rows x K).  The workgroup quantizes the token rows itself, with the routines
// of the standalone quantizer (per-token absmax, fp16 scale, codes), so codes and
// scales are identical to it, into LDS rows of K + 16 bytes (the 16-byte skew puts
// the 16 rows one A-fragment read touches in distinct banks), while its first batch
// of packed weights is in flight; then the skinny main loop runs with A fragments
// read from LDS.  All threads share the quantization (row absmax by LDS atomics).
// Every workgroup repeats it, so the fused kernel serves only shapes where that
// costs less than a launch of its own.  Rows past M are never stored.
// LDS: 16 fp32 token scales and their reciprocals, then M code rows; the same space
// holds the partial sums of the waves once the main loop is done.
// ---------------------------------------------------------------------------
constexpr int kXqMaxK = 8192;                   // the rule's limit (16 code rows of K + 16 bytes)
constexpr int kXqCodeBytes = 16 * (kXqMaxK + 16);   // LDS for the code rows: M * (K + 16) at most
constexpr int kXqHead = 128;                    // LDS: 16 token scales and reciprocals
constexpr int kXqPerThread = 8;                 // chunks per thread: M * K / 8 <= 8 * threads

template <int NBW, int U>
struct SkinnyWBatch {
  uint4 p[U][NBW];
  unsigned md[U][NBW];
};

template <int NBW, int WAVES, int U, bool NT>
__device__ __forceinline__ void skinny_wload(SkinnyWBatch<NBW, U> &B, int b, int ngroups, int wave,
                                             const uint4 *__restrict__ packed, const uint16_t *__restrict__ meta,
                                             int strip0, int NS, int G, int lane) {
  const int col = lane & 15;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = b * U + u;
    const int j = wave + WAVES * (t < ngroups ? t : 0);   // past the end: in-bounds reload, zero activations
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const size_t chunk = static_cast<size_t>(min(strip0 + nb, NS - 1)) * G + j;
      B.p[u][nb] = load_codes<NT>(packed + chunk * 64 + lane);
      B.md[u][nb] = meta_pair(meta, chunk, col);
    }
  }
}

template <int NBW, int WAVES, int U>
constexpr int skinny_xq_red_bytes() {
  return WAVES * NBW * 4 * 64 * 4;
}

template <int NBW, int WAVES, int U, int R, bool NT = false>
__global__ __launch_bounds__(64 * WAVES) void gemm_skinny_xq_kernel(
    const __half *__restrict__ x, __half *__restrict__ sx_out, const uint4 *__restrict__ packed,
    const uint16_t *__restrict__ meta, const __half *__restrict__ sw, __half *__restrict__ out, int M, int N,
    int K) {
  extern __shared__ __attribute__((aligned(16))) int8_t lds[];
  float *sxl = reinterpret_cast<float *>(lds);             // 16 token scales
  float *rcpl = sxl + 16;                                   // their reciprocals (act_rcp)
  int8_t *qa = lds + kXqHead;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = K >> 7;
  const int NS = N >> 4;
  const int col = lane & 15;
  const int kq = lane >> 4;
  const int strip0 = blockIdx.x * NBW;
  const int pitch = K + 16;

  const int ngroups = wave < G ? (G - wave + WAVES - 1) / WAVES : 0;
  const int nbatch = (ngroups + U - 1) / U;
  // weight batches in a ring of R register sets, as in the skinny kernel
  SkinnyWBatch<NBW, U> ring[R];
#pragma unroll
  for (int r = 0; r < R - 1; ++r)
    if (r < nbatch) skinny_wload<NBW, WAVES, U, NT>(ring[r], r, ngroups, wave, packed, meta, strip0, NS, G, lane);

  // per-token quantization of the M rows into LDS, shared by all threads: chunk c
  // (8 halves) of the M x K/8 chunks goes to thread c mod T, kept in registers
  // between the absmax and the quantization (M * K / 8 <= kXqPerThread * T)
  constexpr int T = 64 * WAVES;
  const int nchunk = K >> 3;
  const int total = M * nchunk;
  unsigned *rowmax = reinterpret_cast<unsigned *>(lds);          // 16 words, then reused for scales
  if (threadIdx.x < 16) rowmax[threadIdx.x] = 0u;
  __syncthreads();
  uint4 v[kXqPerThread];
#pragma unroll
  for (int i = 0; i < kXqPerThread; ++i) {      // every load first, so they are in flight together
    const int c = static_cast<int>(threadIdx.x) + T * i;
    if (c < total) {
      const int r = c / nchunk;
      v[i] = reinterpret_cast<const uint4 *>(x + static_cast<size_t>(r) * K)[c - r * nchunk];
    }
  }
#pragma unroll
  for (int i = 0; i < kXqPerThread; ++i) {
    const int c = static_cast<int>(threadIdx.x) + T * i;
    if (c < total) atomicMax(&rowmax[c / nchunk], absmax_bits8(v[i], 0u));
  }
  __syncthreads();
  if (threadIdx.x < static_cast<unsigned>(M)) {
    const __half sh = sym_scale(rowmax[threadIdx.x], static_cast<float>(kXQmax));
    if (blockIdx.x == 0 && sx_out) sx_out[threadIdx.x] = sh;
    sxl[threadIdx.x] = __half2float(sh);                        // overwrites this row's max
    rcpl[threadIdx.x] = act_rcp(__half2float(sh));
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kXqPerThread; ++i) {
    const int c = static_cast<int>(threadIdx.x) + T * i;
    if (c < total) {
      const int r = c / nchunk;
      *reinterpret_cast<uint2 *>(qa + r * pitch + 8 * (c - r * nchunk)) = quant_chunk8(v[i], sxl[r], rcpl[r]);
    }
  }
  __syncthreads();

  v4i acc[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) acc[nb] = v4i{0, 0, 0, 0};
  const int8_t *arow = qa + min(col, M - 1) * pitch + 16 * kq;   // rows past M repeat row M-1 (never stored)
  for (int b0 = 0; b0 < nbatch; b0 += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int b = b0 + r;
      if (b >= nbatch) break;
      if (b + R - 1 < nbatch)
        skinny_wload<NBW, WAVES, U, NT>(ring[(r + R - 1) % R], b + R - 1, ngroups, wave, packed, meta, strip0, NS, G,
                                    lane);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = b * U + u;
        const bool ok = t < ngroups;                          // uniform: slots past the end add zero
        const int j = wave + WAVES * (ok ? t : 0);
        const v4i zero4 = {0, 0, 0, 0};
        const v4i a0 = ok ? *reinterpret_cast<const v4i *>(arow + 128 * j) : zero4;
        const v4i a1 = ok ? *reinterpret_cast<const v4i *>(arow + 128 * j + 64) : zero4;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          v4i w0, w1;
          dequant_lane(ring[r].p[u][nb], group_consts(meta_of(ring[r].md[u][nb], col)), w0, w1);
          acc[nb] = mfma16x16x64(a0, w0, acc[nb]);
          acc[nb] = mfma16x16x64(a1, w1, acc[nb]);
        }
      }
    }
  }

  // partial sums of the waves, added through LDS (the code rows are done with)
  __syncthreads();
  int *red = reinterpret_cast<int *>(lds + kXqHead);
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wave * NBW + nb) * 4 + i) * 64 + lane] = acc[nb][i];
  __syncthreads();
  for (int e = threadIdx.x; e < NBW * 256; e += 64 * WAVES) {
    const int ln = e & 63;
    const int ti = e >> 6;                        // nb * 4 + i
    int sum = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += red[(w * NBW * 4 + ti) * 64 + ln];
    const int nb = ti >> 2, i = ti & 3;
    const int m = 4 * (ln >> 4) + i;
    const int strip = strip0 + nb;
    if (m < M && strip < NS) {
      const int n = strip * 16 + (ln & 15);
      out[static_cast<size_t>(m) * N + n] = mul_round_half(static_cast<float>(sum), sxl[m] * __half2float(sw[n]));
    }
  }
}

// ---------------------------------------------------------------------------
// Large-M regime (many tokens: INT8 MFMA throughput is the bound), on the 32x32x32
// INT8 MFMA (the shape that sustains the matrix cores with few accumulators).
//   workgroup = 4 waves side by side along N: wave w owns 32*TN output columns (TN
//   pairs of 16-column strips) and all BM = 32*TM rows of the tile, so every weight
//   is dequantized by exactly one wave and stays in its registers.  One K step =
//   one group of 128; the A tile (BM x 128 INT8) is staged through LDS and read by
//   all four waves.
//   32x32x32 operands: lane l supplies row / column (l % 32) and the 16 bytes
//   k = 16*(l / 32) .. +15 of a 32-wide k block.  From the packed layout a lane of
//   tile column tn reads, for its column (strip s0 + 2*tn + (l % 32) / 16, c = l % 16),
//   slot h = l / 32 (low nibbles: k block 0, high nibbles: k block 2) and slot
//   h = 2 + l / 32 (k blocks 1 and 3): two 16-byte loads per lane per group.
//   Result: register r of lane l holds D[8*(r / 4) + 4*(l / 32) + r % 4][l % 32].
//   Tile order: the grid is 1-D.  Workgroup b runs on XCD b % 8, so ids are first
//   renumbered to give each XCD a contiguous range of tiles, then ranges are walked
//   kTileGroupRows row-tiles at a time (row index fastest), so the workgroups
//   resident on one XCD cover a compact block of rows x columns and share both
//   operands in its L2.
// ---------------------------------------------------------------------------
constexpr int kLdsRow = 144;   // bytes per staged A row (128 + 16 padding)
constexpr int kXcds = 8;
constexpr int kTileGroupRows = 8;

// workgroup id -> position in an order where each XCD owns a contiguous range
__device__ __forceinline__ int xcd_order(int bid, int total) {
  return total % kXcds == 0 ? (bid % kXcds) * (total / kXcds) + bid / kXcds : bid;
}

// position -> tile (x = column tile, y = row tile), walking kTileGroupRows row
// tiles at a time
__device__ __forceinline__ void tile_walk(int t, int nx, int ny, int &x, int &y) {
  const int group = kTileGroupRows * nx;
  const int g = t / group;
  const int first = g * kTileGroupRows;
  const int rows = min(ny - first, kTileGroupRows);
  const int r = t - g * group;
  y = first + r % rows;
  x = r / rows;
}

__device__ __forceinline__ void tile_coords(int bid, int nx, int ny, int &x, int &y) {
  tile_walk(xcd_order(bid, nx * ny), nx, ny, x, y);
}

// ---------------------------------------------------------------------------
// Split-K.  When the output tiles alone would leave compute units idle (few tiles,
// long K), the K groups of every tile are divided among `splits` workgroups:
// split s takes groups [s*G/splits, (s+1)*G/splits) and stores its INT32 partial
// tile, row-major, into slice s of the workspace (splits x M x N INT32).  A second
// kernel (split_reduce_kernel) adds the slices (exact integer sums) and applies the
// epilogue; the kernel boundary orders the two, so no workgroup waits on another.
// Workgroups are ordered split-major within each XCD's contiguous range, so the
// tiles resident on one XCD read the same K range of A and of the weights.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split_coords(int bid, int nx, int ny, int splits, int &x, int &y, int &split) {
  const int tiles = nx * ny;
  const int t = xcd_order(bid, tiles * splits);
  split = t / tiles;
  tile_walk(t - split * tiles, nx, ny, x, y);
}

// ---------------------------------------------------------------------------
// Epilogue of the 32x32x32 kernels.  fp16: each 32-row block of a wave's tile goes
// through a wave-private LDS scratch (32 rows x 32*TN fp16, rows padded by 16 bytes)
// so the global writes are 16-byte row segments (whole cache lines) instead of
// 2-byte scattered stores; INT32 (verification path): direct stores.
// lds_wave: this wave's scratch, at least 32 * (64*TN + 16) bytes, free to use.
// PC (per-channel weights): acc - z[n] * t[m] first (the zero point, moved out of
// the main loop; "QServe ..." summary, per-channel fast dequantization).
template <int TM, int TN, int OUT, bool PC = false>
__device__ __forceinline__ void epilogue32(const v16i (&acc)[TM][TN], int8_t *__restrict__ lds_wave, int lane,
                                           int m0, int n0, int M, int N, const __half *__restrict__ sx,
                                           const __half *__restrict__ sw, void *__restrict__ out,
                                           const uint8_t *__restrict__ zp = nullptr,
                                           const int *__restrict__ trow = nullptr) {
  const int c32 = lane & 31, hi = lane >> 5;
  int zn[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) zn[tn] = PC ? static_cast<int>(zp[min(n0 + 32 * tn + c32, N - 1)]) : 0;
  if (OUT == 1) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int n = n0 + 32 * tn + c32;
      if (n >= N) continue;
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + 32 * tm + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (m < M)
            static_cast<int *>(out)[static_cast<size_t>(m) * N + n] = acc[tm][tn][r] - (PC ? zn[tn] * trow[m] : 0);
        }
    }
    return;
  }
  constexpr int ROW = 64 * TN + 16;                  // bytes per staged row
  constexpr int SEGS = 4 * TN;                       // 16-byte segments per row
  float swn[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) swn[tn] = __half2float(sw[min(n0 + 32 * tn + c32, N - 1)]);
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lr = 8 * (r >> 2) + 4 * hi + (r & 3);
      const int mrow = min(m0 + 32 * tm + lr, M - 1);
      const float sxm = __half2float(sx[mrow]);
      const int tm_ = PC ? trow[mrow] : 0;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        *reinterpret_cast<__half *>(lds_wave + lr * ROW + 2 * (32 * tn + c32)) =
            mul_round_half(static_cast<float>(acc[tm][tn][r] - zn[tn] * tm_), sxm * swn[tn]);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int e = lane; e < 32 * SEGS; e += 64) {
      const int lr = e / SEGS, sg = e % SEGS;
      const int m = m0 + 32 * tm + lr, n = n0 + 8 * sg;
      const uint4 v = *reinterpret_cast<const uint4 *>(lds_wave + lr * ROW + 16 * sg);
      if (m < M && n < N) *reinterpret_cast<uint4 *>(static_cast<__half *>(out) + static_cast<size_t>(m) * N + n) = v;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// ---------------------------------------------------------------------------
// Large-M regime, A staged by the waves, two-group register prefetch.  The A tile
// is double buffered in LDS with rows padded to kLdsRow = 144 bytes, so the rows a
// 16-lane phase reads fall in distinct banks.  A prefetched value is never
// copied between registers (a copy must wait for the load): the loop is unrolled
// by two and uses two register sets, so group j+2's A chunks and packed codes land
// in the set group j just released and are consumed in place two groups later.
// Per group j (set q = j & 1): dequantize B(j) from set q; issue the loads of
// group j+2 into set q; MFMAs of group j from LDS buffer q; write A(j+1) (set 1-q,
// loaded a group earlier) into LDS buffer 1-q; barrier.  Group indices past the
// end clamp to the last group (redundant in-bounds loads, never used).
// ---------------------------------------------------------------------------
template <int CH, int TN>
struct W2Set {
  v4i a[CH];
  uint4 p0[TN], p1[TN];
  unsigned md[TN];
};

template <int CH, int TN, bool PC>
__device__ __forceinline__ void w2_load(W2Set<CH, TN> &S, const int8_t *const (&ag)[CH], const uint4 *__restrict__ packed,
                                        const uint16_t *__restrict__ meta, const unsigned (&boff)[TN],
                                        const unsigned (&moff)[TN], int j) {
#pragma unroll
  for (int c = 0; c < CH; ++c) S.a[c] = *reinterpret_cast<const v4i *>(ag[c] + 128 * j);
  const uint4 *pj = packed + static_cast<size_t>(j) * 64;
  const uint16_t *mj = meta + static_cast<size_t>(j) * 16;
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    S.p0[tn] = pj[boff[tn]];
    S.p1[tn] = pj[boff[tn] + 32];
    S.md[tn] = PC ? 0u : mj[moff[tn]];
  }
}

template <int TM, int TN, int CH, int Q, bool PC>
__device__ __forceinline__ void w2_step(int j, int G, W2Set<CH, TN> &cur, W2Set<CH, TN> &oth, int8_t (*As)[32 * TM * kLdsRow],
                                        const int (&alds)[CH], int arow, const int8_t *const (&ag)[CH],
                                        const uint4 *__restrict__ packed, const uint16_t *__restrict__ meta,
                                        const unsigned (&boff)[TN], const unsigned (&moff)[TN],
                                        v16i (&acc)[TM][TN]) {
  v4i b[4][TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    weights_lane<PC>(cur.p0[tn], cur.md[tn], b[0][tn], b[2][tn]);
    weights_lane<PC>(cur.p1[tn], cur.md[tn], b[1][tn], b[3][tn]);
  }
  // cur's A chunks went to LDS a group ago and its codes are consumed: reuse it.
  // The scheduling fences keep these loads at the top of the group and the LDS
  // writes at its end, so each load has two groups of work to land in.
  __builtin_amdgcn_sched_barrier(0);
  w2_load<CH, TN, PC>(cur, ag, packed, meta, boff, moff, min(j + 2, G - 1));
  __builtin_amdgcn_sched_barrier(0);
  const int8_t *abuf = &As[Q][arow];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const v4i a = *reinterpret_cast<const v4i *>(abuf + tm * 32 * kLdsRow + 32 * kb);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = mfma32x32x32(a, b[kb][tn], acc[tm][tn]);
    }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < CH; ++c) *reinterpret_cast<v4i *>(&As[Q ^ 1][alds[c]]) = oth.a[c];
  __syncthreads();
}

template <int TM, int TN, int OUT, bool PC>
__global__ __launch_bounds__(256, 2) void gemm_wide2_kernel(const int8_t *__restrict__ qx,
                                                            const __half *__restrict__ sx,
                                                            const uint4 *__restrict__ packed,
                                                            const uint16_t *__restrict__ meta,
                                                            const __half *__restrict__ sw, const uint8_t *__restrict__ zp,
    const int *__restrict__ trow, void *__restrict__ out,
                                                            int M, int N, int K, int splits, int *__restrict__ ws) {
  constexpr int BM = 32 * TM;
  constexpr int CH = BM * 8 / 256;
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, hi = lane >> 5;
  const int Gs = K >> 7;
  const int NS = N >> 4;
  const int nx = (NS + 8 * TN - 1) / (8 * TN);
  const int ny = (M + BM - 1) / BM;
  int tx, ty, split;
  split_coords(blockIdx.x, nx, ny, splits, tx, ty, split);
  const int g0 = split * Gs / splits;
  const int G = (split + 1) * Gs / splits - g0;   // groups of this split (>= 1)
  const int m0 = ty * BM;
  const int s0 = (tx * 4 + wave) * 2 * TN;

  // A staging: chunk e = tid + 256*c -> row e / 8, 16-byte column e % 8 (rows past M
  // re-read row M-1; their results are never stored)
  const int8_t *ag[CH];
  int alds[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e = tid + 256 * c;
    const int r = e >> 3, cc = e & 7;
    ag[c] = qx + static_cast<size_t>(min(m0 + r, M - 1)) * K + 128 * g0 + 16 * cc;
    alds[c] = r * kLdsRow + 16 * cc;
  }
  unsigned boff[TN], moff[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const unsigned strip = static_cast<unsigned>(min(s0 + 2 * tn + (c32 >> 4), NS - 1));
    boff[tn] = (strip * static_cast<unsigned>(Gs) + g0) * 64u + 16u * hi + (lane & 15);
    moff[tn] = (strip * static_cast<unsigned>(Gs) + g0) * 16u + (lane & 15);
  }

  v16i acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = v16i{};

  W2Set<CH, TN> s0set, s1set;
  w2_load<CH, TN, PC>(s0set, ag, packed, meta, boff, moff, 0);
  w2_load<CH, TN, PC>(s1set, ag, packed, meta, boff, moff, min(1, G - 1));
#pragma unroll
  for (int c = 0; c < CH; ++c) *reinterpret_cast<v4i *>(&As[0][alds[c]]) = s0set.a[c];
  __syncthreads();

  const int arow = c32 * kLdsRow + 16 * hi;
  int j = 0;
  for (; j + 1 < G; j += 2) {
    w2_step<TM, TN, CH, 0, PC>(j, G, s0set, s1set, As, alds, arow, ag, packed, meta, boff, moff, acc);
    w2_step<TM, TN, CH, 1, PC>(j + 1, G, s1set, s0set, As, alds, arow, ag, packed, meta, boff, moff, acc);
  }
  if (j < G) w2_step<TM, TN, CH, 0, PC>(j, G, s0set, s1set, As, alds, arow, ag, packed, meta, boff, moff, acc);

  static_assert(4 * 32 * (64 * TN + 16) <= 2 * BM * kLdsRow, "epilogue scratch exceeds the A buffers");
  if (splits > 1) {   // partial sums of this split -> workspace slice
    epilogue32<TM, TN, 1>(acc, nullptr, lane, m0, 16 * s0, M, N, nullptr, nullptr,
                          ws + static_cast<size_t>(split) * M * N);
    return;
  }
  epilogue32<TM, TN, OUT, PC>(acc, &As[0][0] + wave * 32 * (64 * TN + 16), lane, m0, 16 * s0, M, N, sx, sw, out,
                              zp, trow);
}

// ---------------------------------------------------------------------------
// Copy-engine helpers: global -> LDS copies (global_load_lds) count in vmcnt like
// loads, so a wave waits for the copies it needs with a vmcnt-only wait.
// The rule every such wait follows: copies retire in issue order among
// themselves, but not in order with register loads.  A wait for copy c may
// therefore leave in flight only copies issued after c: the count is the number
// of copies issued after c (register loads issued after c are then waited for as
// well, which costs time but not correctness).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// vmcnt-only wait (expcnt and lgkmcnt left at their maxima): gfx9 encoding
#define QOQ_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | (7 << 4) | (15 << 8))
// lgkmcnt(0) only (LDS writes of this wave done; vmcnt and expcnt at their maxima)
#define QOQ_WAIT_LGKMCNT0() __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4))

// ---------------------------------------------------------------------------
// Large-M regime, A by copy engine and B by two register sets (32x32x32 MFMA).
// Four waves side by side along N as above.  A (BM rows x 128 per group) is copied
// global -> LDS with global_load_lds into a 3-stage ring, so it costs no registers
// and no LDS-write instructions.  The 16-byte chunks of row r are stored at
// position chunk ^ ((r >> 1) & 7): the LDS serves 16 lanes x 16 bytes per cycle
// over 64 banks, two 128-byte rows per bank row, so the 16 rows one phase of an
// A-operand read touches land in 16 distinct bank groups.  The packed codes of group j+2
// are loaded into the register set group j just consumed (loop unrolled by two; a
// prefetched register is never copied, so the compiler can wait for exactly the
// loads it needs).  A fragments are read one k block ahead of the MFMAs that use
// them.  Per group j: dequantize B(j); copy A(j+2) and load B(j+2); MFMAs of j;
// wait for A(j+1)'s copies; barrier.  The copies and the register loads share
// vmcnt; the waits follow the copy rule above.
// ---------------------------------------------------------------------------
template <int TN>
struct DBSet {
  uint4 p0[TN], p1[TN];
  unsigned md[TN];
};

template <int TM, int TN, int Q, bool PC>
__device__ __forceinline__ void dma2_step(int j, int G, DBSet<TN> &cur, int8_t *__restrict__ lds,
                                          const int8_t *const (&asrc)[TM], int wave, int lane,
                                          const uint4 *__restrict__ packed, const uint16_t *__restrict__ meta,
                                          const unsigned (&boff)[TN], const unsigned (&moff)[TN],
                                          v16i (&acc)[TM][TN]) {
  constexpr int STAGE = 32 * TM * 128;
  // dequantize this group's codes (set Q, loaded two groups ago)
  v4i b[4][TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    weights_lane<PC>(cur.p0[tn], cur.md[tn], b[0][tn], b[2][tn]);
    weights_lane<PC>(cur.p1[tn], cur.md[tn], b[1][tn], b[3][tn]);
  }
  // The codes die here.  The empty volatile asm consumes every dequantized value,
  // so instruction selection cannot move any of the dequantization below the loads
  // that refill the same set; otherwise the allocator keeps old and new codes in
  // different registers and copies them at the loop edge, which makes the wave wait
  // for those loads there.
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) asm volatile("" ::"v"(b[kb][tn]));
  __builtin_amdgcn_sched_barrier(0);
  // group j+2: A copies into ring stage (j+2) % 3 (held group j-1, finished before
  // the last barrier), then the codes into the set just consumed
  {
    const int jn = min(j + 2, G - 1);
    int8_t *st = lds + ((j + 2) % 3) * STAGE;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      __builtin_amdgcn_global_load_lds((glb_void_t *)(asrc[i] + 128 * jn), (lds_void_t *)(st + 1024 * (wave * TM + i)),
                                       16, 0, 0);
    const uint4 *pj = packed + static_cast<size_t>(jn) * 64;
    const uint16_t *mj = meta + static_cast<size_t>(jn) * 16;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      cur.p0[tn] = pj[boff[tn]];
      cur.p1[tn] = pj[boff[tn] + 32];
      cur.md[tn] = PC ? 0u : mj[moff[tn]];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // MFMAs of group j, A fragments read one k block ahead
  const int8_t *stage = lds + (j % 3) * STAGE;
  const int r = lane & 31, hi = lane >> 5;
  v4i af[2][TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int row = 32 * tm + r;
    af[0][tm] = *reinterpret_cast<const v4i *>(stage + row * 128 + 16 * ((0 + hi) ^ ((row >> 1) & 7)));
  }
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    if (kb + 1 < 4) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int row = 32 * tm + r;
        af[(kb + 1) & 1][tm] =
            *reinterpret_cast<const v4i *>(stage + row * 128 + 16 * ((2 * (kb + 1) + hi) ^ ((row >> 1) & 7)));
      }
    }
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = mfma32x32x32(af[kb & 1][tm], b[kb][tn], acc[tm][tn]);
  }
  __builtin_amdgcn_sched_barrier(0);
  // A(j+1) was copied one group ago.  The only copies issued after it are this
  // group's TM copies of A(j+2), so vmcnt(TM) guarantees A(j+1) is in LDS (the
  // copy rule above); B(j+2)'s register loads, issued after those copies, are
  // partly waited for as well.
  QOQ_WAIT_VMCNT(TM);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <int TM, int TN, int OUT, bool PC>
__global__ __launch_bounds__(256, 2) void gemm_dma2_kernel(const int8_t *__restrict__ qx,
                                                           const __half *__restrict__ sx,
                                                           const uint4 *__restrict__ packed,
                                                           const uint16_t *__restrict__ meta,
                                                           const __half *__restrict__ sw, const uint8_t *__restrict__ zp,
    const int *__restrict__ trow, void *__restrict__ out,
                                                           int M, int N, int K, int splits, int *__restrict__ ws) {
  constexpr int BM = 32 * TM;
  constexpr int STAGE = BM * 128;
  __shared__ __attribute__((aligned(1024))) int8_t lds[3 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, hi = lane >> 5;
  const int Gs = K >> 7;
  const int NS = N >> 4;
  const int nx = (NS + 8 * TN - 1) / (8 * TN);
  const int ny = (M + BM - 1) / BM;
  int tx, ty, split;
  split_coords(blockIdx.x, nx, ny, splits, tx, ty, split);
  const int g0 = split * Gs / splits;
  const int G = (split + 1) * Gs / splits - g0;   // groups of this split (>= 1)
  const int m0 = ty * BM;
  const int s0 = (tx * 4 + wave) * 2 * TN;

  const int8_t *asrc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = 8 * (wave * TM + i) + (lane >> 3);
    asrc[i] = qx + static_cast<size_t>(min(m0 + row, M - 1)) * K + 128 * g0 + 16 * ((lane & 7) ^ ((row >> 1) & 7));
  }
  unsigned boff[TN], moff[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const unsigned strip = static_cast<unsigned>(min(s0 + 2 * tn + (c32 >> 4), NS - 1));
    boff[tn] = (strip * static_cast<unsigned>(Gs) + g0) * 64u + 16u * hi + (lane & 15);
    moff[tn] = (strip * static_cast<unsigned>(Gs) + g0) * 16u + (lane & 15);
  }

  v16i acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = v16i{};

  // prologue: A(0), A(1) copies; B(0), B(1) into the two sets
  DBSet<TN> set0, set1;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int jg = min(g, G - 1);
#pragma unroll
    for (int i = 0; i < TM; ++i)
      __builtin_amdgcn_global_load_lds((glb_void_t *)(asrc[i] + 128 * jg),
                                       (lds_void_t *)(lds + g * STAGE + 1024 * (wave * TM + i)), 16, 0, 0);
  }
  {
    const uint16_t *m1 = meta + static_cast<size_t>(min(1, G - 1)) * 16;
    const uint4 *p1 = packed + static_cast<size_t>(min(1, G - 1)) * 64;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      set0.p0[tn] = packed[boff[tn]];
      set0.p1[tn] = packed[boff[tn] + 32];
      set0.md[tn] = PC ? 0u : meta[moff[tn]];
    }
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      set1.p0[tn] = p1[boff[tn]];
      set1.p1[tn] = p1[boff[tn] + 32];
      set1.md[tn] = PC ? 0u : m1[moff[tn]];
    }
  }
  // A(0) resident (one wait for everything the prologue issued)
  QOQ_WAIT_VMCNT(0);
  __builtin_amdgcn_s_barrier();

  int j = 0;
  for (; j + 1 < G; j += 2) {
    dma2_step<TM, TN, 0, PC>(j, G, set0, lds, asrc, wave, lane, packed, meta, boff, moff, acc);
    dma2_step<TM, TN, 1, PC>(j + 1, G, set1, lds, asrc, wave, lane, packed, meta, boff, moff, acc);
  }
  if (j < G) dma2_step<TM, TN, 0, PC>(j, G, set0, lds, asrc, wave, lane, packed, meta, boff, moff, acc);
  QOQ_WAIT_VMCNT(0);                            // no copy outlives the kernel
  __syncthreads();
  static_assert(4 * 32 * (64 * TN + 16) <= 3 * STAGE, "epilogue scratch exceeds the ring");
  if (splits > 1) {   // partial sums of this split -> workspace slice
    epilogue32<TM, TN, 1>(acc, nullptr, lane, m0, 16 * s0, M, N, nullptr, nullptr,
                          ws + static_cast<size_t>(split) * M * N);
    return;
  }
  epilogue32<TM, TN, OUT, PC>(acc, lds + wave * 32 * (64 * TN + 16), lane, m0, 16 * s0, M, N, sx, sw, out, zp,
                              trow);
}

// ---------------------------------------------------------------------------
// Large-M regime, shared dequantization (32x32x32 INT8 MFMA).  The dequantization
// work per MFMA falls with the number of rows that reuse each dequantized weight;
// the register budget of two waves per SIMD caps a wave's tile, so here the rows
// are spread over waves and the weights are dequantized once per workgroup and
// shared through LDS:
//   workgroup = 8 waves (two per SIMD), tile 128*TM rows x 256 columns; wave w
//   computes rows 32*TM*(w & 3) .. +32*TM-1 and columns 128*(w >> 2) .. +127 (TM
//   blocks of 32 rows, TN = 4) and dequantizes column block w (32 columns, two
//   strips) for the whole workgroup, writing its B fragments to LDS in MFMA operand
//   order (bbuf[block][k block][lane], 16 bytes each: every read and write is 64
//   lanes x 16 contiguous bytes).  TM = 2 (256-row tiles) for large batches; TM = 1
//   (128-row tiles) for mid-size ones, where it copies A half as often per weight
//   byte as the 128-column tile kernels.
//   A (128*TM x 128 per group) comes by copy engine into an AS-stage ring with the
//   row-pair XOR swizzle; each wave reads only its own 32*TM rows.
//   Per group j: load the codes of j+3 (three register sets, group g in set g % 3);
//   dequantize j+1 (codes loaded two groups earlier) into B buffer (j+1) & 1; copy
//   A(j+AS-1); MFMAs of j from A stage j % AS and B buffer j & 1; wait for A(j+1);
//   barrier (which also publishes B(j+1)).
// ---------------------------------------------------------------------------
template <int TM>
constexpr int sd_stage_a() {                     // A bytes per stage (128 * TM rows)
  return 128 * TM * 128;
}
constexpr int kSdBufB = 8 * 4 * 1024;            // dequantized B bytes per group

template <int AS, int TM>
constexpr int sd_lds_bytes() {
  return AS * sd_stage_a<TM>() + 2 * kSdBufB;
}

struct SdCodes {
  uint4 p0, p1;
  unsigned md;
};

template <bool PC>
__device__ __forceinline__ void sd_load_codes(SdCodes &c, const uint4 *__restrict__ packed,
                                              const uint16_t *__restrict__ meta, unsigned boff, unsigned moff,
                                              int j) {
  const uint4 *pj = packed + static_cast<size_t>(j) * 64;
  c.p0 = pj[boff];
  c.p1 = pj[boff + 32];
  c.md = PC ? 0u : meta[static_cast<size_t>(j) * 16 + moff];
}

// Copies written as inline asm: the compiler does not see them, so it adds no wait
// of its own for them (it would otherwise wait for every copy in flight before the
// next LDS read of a wave that reads LDS first); the kernel's explicit vmcnt waits
// order them.  Safe next to the compiler's own waits for register loads: a wait that
// leaves k operations in flight cannot end while a load is pending that has k
// register loads after it (those are pending too), so hidden copies only make such
// a wait later.  The address registers are read when the copy issues; the copy
// writes no register.  M0 is reserved: the compiler sets it right before each
// instruction of its own that reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_hidden(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int AS, int TM>
__device__ __forceinline__ void sd_copy_a(int j, int8_t *__restrict__ lds, const int8_t *const (&asrc)[2 * TM],
                                          int wave) {
  const uint32_t st = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t *)lds)) +
                      static_cast<uint32_t>((j % AS) * sd_stage_a<TM>());
#pragma unroll
  for (int i = 0; i < 2 * TM; ++i) copy16_hidden(asrc[i] + 128 * j, st + 1024 * (wave * 2 * TM + i));
}

template <int Q, bool PC>
__device__ __forceinline__ void sd_dequant(int8_t *__restrict__ bbuf, int wave, int lane, const SdCodes &cur) {
  v4i b[4];
  weights_lane<PC>(cur.p0, cur.md, b[0], b[2]);
  weights_lane<PC>(cur.p1, cur.md, b[1], b[3]);
  int8_t *dst = bbuf + (Q ^ 1) * kSdBufB + wave * 4096 + 16 * lane;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) *reinterpret_cast<v4i *>(dst + 1024 * kb) = b[kb];
}

template <int AS, int Q, int TM>
__device__ __forceinline__ void sd_mfma(int j, const int8_t *__restrict__ lds, int wave, int lane,
                                        v16i (&acc)[TM][4]) {
  const int8_t *stage = lds + (j % AS) * sd_stage_a<TM>();
  const int8_t *bj = lds + AS * sd_stage_a<TM>() + Q * kSdBufB + (wave >> 2) * 4 * 4096 + 16 * lane;
  const int r = lane & 31, hi = lane >> 5;
  const int rbase = 32 * TM * (wave & 3);
  auto read_a = [&](int kb, v4i (&a)[TM]) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int row = rbase + 32 * tm + r;
      a[tm] = *reinterpret_cast<const v4i *>(stage + row * 128 + 16 * ((2 * kb + hi) ^ ((row >> 1) & 7)));
    }
  };
  v4i a[2][TM], bf[4];
  read_a(0, a[0]);
#pragma unroll
  for (int tn = 0; tn < 4; ++tn) bf[tn] = *reinterpret_cast<const v4i *>(bj + tn * 4096);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    if (kb + 1 < 4) read_a(kb + 1, a[(kb + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) acc[tm][tn] = mfma32x32x32(a[kb & 1][tm], bf[tn], acc[tm][tn]);
      if (kb + 1 < 4) bf[tn] = *reinterpret_cast<const v4i *>(bj + tn * 4096 + 1024 * (kb + 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// One group.  Waves w and w + 4 share a SIMD and meet at the same barriers, so
// they run the step's two phases in opposite orders (MF = MFMAs first for waves
// 4..7): while one dequantizes (vector ALU) the other issues MFMAs, and the two
// units work side by side.  A wave raises its issue priority for its MFMA phase, so
// when both waves of the SIMD have an instruction ready the matrix unit is fed
// first and the dequantization fills the gaps.
template <int AS, int Q, bool MF, bool PC, int TM>
__device__ __forceinline__ void sd_step(int j, int G, int8_t *__restrict__ lds, int wave, int lane,
                                        const int8_t *const (&asrc)[2 * TM], const SdCodes &deq, SdCodes &fill,
                                        const uint4 *__restrict__ packed, const uint16_t *__restrict__ meta,
                                        unsigned boff, unsigned moff, v16i (&acc)[TM][4]) {
  int8_t *bbuf = lds + AS * sd_stage_a<TM>();
  // group j+3's codes go out first, into the set that held group j (dequantized a
  // group ago): the copy wait at the bottom cannot leave register loads issued after
  // the copies in flight, so codes loaded there would be waited for at once
  sd_load_codes<PC>(fill, packed, meta, boff, moff, min(j + 3, G - 1));
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (MF) {
    __builtin_amdgcn_s_setprio(1);
    sd_mfma<AS, Q, TM>(j, lds, wave, lane, acc);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // group j+1 is dequantized (codes loaded two groups ago) into B buffer (j+1) & 1,
  // which every wave finished reading before the last barrier; then group j+AS-1's
  // A copies are issued (its stage held group j-1)
  sd_dequant<Q, PC>(bbuf, wave, lane, deq);
  __builtin_amdgcn_sched_barrier(0);
  sd_copy_a<AS, TM>(min(j + AS - 1, G - 1), lds, asrc, wave);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!MF) {
    __builtin_amdgcn_s_setprio(1);
    sd_mfma<AS, Q, TM>(j, lds, wave, lane, acc);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // A(j+1) must be resident.  By the copy rule above the count may include only
  // the copies issued after A(j+1)'s: AS == 3, this step's 2 * TM copies of A(j+2);
  // AS == 2, none (A(j+1) is this step's copy).
  QOQ_WAIT_VMCNT(AS == 3 ? 2 * TM : 0);
  QOQ_WAIT_LGKMCNT0();                          // this wave's B(j+1) fragments are in LDS
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// code set g % 3 holds group g: the loop is unrolled by six (B buffer j & 1, sets j % 3)
template <int AS, bool MF, bool PC, int TM>
__device__ __forceinline__ void sd_loop(int G, int8_t *__restrict__ lds, int wave, int lane,
                                        const int8_t *const (&asrc)[2 * TM], SdCodes &s0, SdCodes &s1, SdCodes &s2,
                                        const uint4 *__restrict__ packed, const uint16_t *__restrict__ meta,
                                        unsigned boff, unsigned moff, v16i (&acc)[TM][4]) {
  int j = 0;
  for (; j + 5 < G; j += 6) {
    sd_step<AS, 0, MF, PC, TM>(j, G, lds, wave, lane, asrc, s1, s0, packed, meta, boff, moff, acc);
    sd_step<AS, 1, MF, PC, TM>(j + 1, G, lds, wave, lane, asrc, s2, s1, packed, meta, boff, moff, acc);
    sd_step<AS, 0, MF, PC, TM>(j + 2, G, lds, wave, lane, asrc, s0, s2, packed, meta, boff, moff, acc);
    sd_step<AS, 1, MF, PC, TM>(j + 3, G, lds, wave, lane, asrc, s1, s0, packed, meta, boff, moff, acc);
    sd_step<AS, 0, MF, PC, TM>(j + 4, G, lds, wave, lane, asrc, s2, s1, packed, meta, boff, moff, acc);
    sd_step<AS, 1, MF, PC, TM>(j + 5, G, lds, wave, lane, asrc, s0, s2, packed, meta, boff, moff, acc);
  }
  if (j < G) sd_step<AS, 0, MF, PC, TM>(j, G, lds, wave, lane, asrc, s1, s0, packed, meta, boff, moff, acc);
  if (j + 1 < G) sd_step<AS, 1, MF, PC, TM>(j + 1, G, lds, wave, lane, asrc, s2, s1, packed, meta, boff, moff, acc);
  if (j + 2 < G) sd_step<AS, 0, MF, PC, TM>(j + 2, G, lds, wave, lane, asrc, s0, s2, packed, meta, boff, moff, acc);
  if (j + 3 < G) sd_step<AS, 1, MF, PC, TM>(j + 3, G, lds, wave, lane, asrc, s1, s0, packed, meta, boff, moff, acc);
  if (j + 4 < G) sd_step<AS, 0, MF, PC, TM>(j + 4, G, lds, wave, lane, asrc, s2, s1, packed, meta, boff, moff, acc);
}

template <int AS, int TM, int OUT, bool PC>
__global__ __launch_bounds__(512, 1) void gemm_sd_kernel(const int8_t *__restrict__ qx,
                                                        const __half *__restrict__ sx,
                                                        const uint4 *__restrict__ packed,
                                                        const uint16_t *__restrict__ meta,
                                                        const __half *__restrict__ sw, const uint8_t *__restrict__ zp,
    const int *__restrict__ trow, void *__restrict__ out,
                                                        int M, int N, int K, int splits, int *__restrict__ ws) {
  static_assert(AS == 2 || AS == 3, "two or three A stages");
  static_assert(TM == 1 || TM == 2, "tiles of 128 or 256 rows");
  constexpr int BM = 128 * TM;                  // tile rows
  extern __shared__ __attribute__((aligned(1024))) int8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31, hi = lane >> 5;
  const int Gs = K >> 7;
  const int NS = N >> 4;
  const int nx = (NS + 15) / 16;
  const int ny = (M + BM - 1) / BM;
  int tx, ty, split;
  split_coords(blockIdx.x, nx, ny, splits, tx, ty, split);
  const int g0 = split * Gs / splits;
  const int G = (split + 1) * Gs / splits - g0;   // groups of this split (>= 1)
  const int m0 = ty * BM;

  // A copies: wave w moves rows 8*(2*TM*w + i) .. +7 of the stage
  const int8_t *asrc[2 * TM];
#pragma unroll
  for (int i = 0; i < 2 * TM; ++i) {
    const int row = 8 * (wave * 2 * TM + i) + (lane >> 3);
    asrc[i] = qx + static_cast<size_t>(min(m0 + row, M - 1)) * K + 128 * g0 + 16 * ((lane & 7) ^ ((row >> 1) & 7));
  }
  // codes of column block `wave`: strip 16*tx + 2*wave + (c32 >> 4), slots 16*hi + c
  // (k blocks 0, 2) and 32 + 16*hi + c (k blocks 1, 3); strips past N repeat the last
  const unsigned strip = static_cast<unsigned>(min(16 * tx + 2 * wave + (c32 >> 4), NS - 1));
  const unsigned boff = (strip * static_cast<unsigned>(Gs) + g0) * 64u + 16u * hi + (lane & 15);
  const unsigned moff = (strip * static_cast<unsigned>(Gs) + g0) * 16u + (lane & 15);

  v16i acc[TM][4];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = v16i{};

  // prologue: A(0) .. A(AS-2); codes 0, 1, 2 into sets 0, 1, 2; dequantize group 0
  // into B buffer 0
  for (int g = 0; g < AS - 1; ++g) sd_copy_a<AS, TM>(min(g, G - 1), lds, asrc, wave);
  SdCodes set0, set1, set2;
  sd_load_codes<PC>(set0, packed, meta, boff, moff, 0);
  sd_load_codes<PC>(set1, packed, meta, boff, moff, min(1, G - 1));
  sd_load_codes<PC>(set2, packed, meta, boff, moff, min(2, G - 1));
  {
    v4i b[4];
    weights_lane<PC>(set0.p0, set0.md, b[0], b[2]);
    weights_lane<PC>(set0.p1, set0.md, b[1], b[3]);
    int8_t *dst = lds + AS * sd_stage_a<TM>() + wave * 4096 + 16 * lane;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) *reinterpret_cast<v4i *>(dst + 1024 * kb) = b[kb];
  }
  QOQ_WAIT_VMCNT(0);
  __syncthreads();

  if (wave < 4)
    sd_loop<AS, false, PC, TM>(G, lds, wave, lane, asrc, set0, set1, set2, packed, meta, boff, moff, acc);
  else
    sd_loop<AS, true, PC, TM>(G, lds, wave, lane, asrc, set0, set1, set2, packed, meta, boff, moff, acc);
  QOQ_WAIT_VMCNT(0);                            // no copy outlives the kernel
  __syncthreads();
  const int wm0 = m0 + 32 * TM * (wave & 3);
  const int wn0 = 16 * (16 * tx + 8 * (wave >> 2));   // first column of this wave
  if (splits > 1) {                             // partial sums of this split -> workspace slice
    epilogue32<TM, 4, 1>(acc, nullptr, lane, wm0, wn0, M, N, nullptr, nullptr,
                        ws + static_cast<size_t>(split) * M * N);
    return;
  }
  static_assert(8 * 32 * (64 * 4 + 16) <= sd_lds_bytes<AS, TM>(), "epilogue scratch exceeds the LDS in use");
  epilogue32<TM, 4, OUT, PC>(acc, lds + wave * 32 * (64 * 4 + 16), lane, wm0, wn0, M, N, sx, sw, out, zp, trow);
}

// ---------------------------------------------------------------------------
// Second pass of split-K: out[m, n] = epilogue(sum_s part[s][m][n]).  Each thread
// takes 8 consecutive columns of one row (N % 16 == 0, so they never cross a row):
// two 16-byte loads per slice, one 16-byte fp16 store (or two INT32 stores).
// ---------------------------------------------------------------------------
template <int OUT, bool PC>
__global__ __launch_bounds__(256) void split_reduce_kernel(const int *__restrict__ part, int splits, int M, int N,
                                                           const __half *__restrict__ sx,
                                                           const __half *__restrict__ sw,
                                                           const uint8_t *__restrict__ zp,
                                                           const int *__restrict__ trow, void *__restrict__ out) {
  const size_t MN = static_cast<size_t>(M) * N;
  const size_t e = (static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (e >= MN) return;
  v4i lo = *reinterpret_cast<const v4i *>(part + e);
  v4i hi = *reinterpret_cast<const v4i *>(part + e + 4);
  for (int s = 1; s < splits; ++s) {
    const int *p = part + static_cast<size_t>(s) * MN + e;
    lo += *reinterpret_cast<const v4i *>(p);
    hi += *reinterpret_cast<const v4i *>(p + 4);
  }
  const int m = static_cast<int>(e / N), n = static_cast<int>(e % N);
  if (PC) {                                    // zero point of the per-channel weights
    const int t = trow[m];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] -= static_cast<int>(zp[n + i]) * t;
      hi[i] -= static_cast<int>(zp[n + 4 + i]) * t;
    }
  }
  if (OUT == 1) {
    *reinterpret_cast<v4i *>(static_cast<int *>(out) + e) = lo;
    *reinterpret_cast<v4i *>(static_cast<int *>(out) + e + 4) = hi;
    return;
  }
  const float sxm = __half2float(sx[m]);
  const int acc[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  __align__(16) __half h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = mul_round_half(static_cast<float>(acc[i]), sxm * __half2float(sw[n + i]));
  *reinterpret_cast<uint4 *>(static_cast<__half *>(out) + e) = *reinterpret_cast<const uint4 *>(h);
}

// ---------------------------------------------------------------------------
// Measurement overrides of the planner (results never depend on them, only the
// speed does): a configuration forced for every shape, a split-K factor, the
// few-token or the tile regime, the linear entry point's fused configuration.
// They are taken from the environment once per process (QOQ_GEMM_CONFIG,
// QOQ_GEMM_SPLITS, QOQ_GEMM_REGIME, QOQ_LINEAR_CONFIG) and replaced through
// qoq_set_plan_override; the launch path copies them under a mutex.
// ---------------------------------------------------------------------------
struct Overrides {
  int config = -1;          // index into kConfigs, -1: none
  int splits = 0;           // 0: none
  int regime = 0;           // 0: none, 1: few-token kernels, 2: tile kernels
  int linear = -2;          // -2: none, -1: unfused, >= 0: index into kXqConfigs
};
Overrides current_overrides();

// ---------------------------------------------------------------------------
// planning: which kernel and launch shape for (M, N, K)
// ---------------------------------------------------------------------------
typedef void (*GemmKernel)(const int8_t *, const __half *, const uint4 *, const uint16_t *, const __half *,
                           const uint8_t *, const int *, void *, int, int, int, int, int *);

struct Config {
  int kind;                 // 0 skinny, 7 skinny on 32x32 blocks, 4 wide2, 5 dma2, 6 shared dequantization
  int a, b, c, d, e;        // skinny: MT, NBW, WAVES, U, R   skinny32: MT2, NP, WAVES, U, R
                            // wide2 / dma2: TM, TN   sd: A stages, 1 for 128-row tiles
  GemmKernel k[2][2];       // [per-group, per-channel][fp16 epilogue, INT32 epilogue]
  const char *name;
  int lds = 0;              // dynamic LDS bytes
  // few-token kernels on tiled activation codes: [per-group, per-channel][fp16, INT32]
  GemmKernel kt[2][2] = {{nullptr, nullptr}, {nullptr, nullptr}};
  int nt = 0;               // few-token kernels: packed codes loaded with the streaming hint
};

#define QOQ_K4(...) {{__VA_ARGS__, 0, false>, __VA_ARGS__, 1, false>}, {__VA_ARGS__, 0, true>, __VA_ARGS__, 1, true>}}
// skinny names carry the ring depth only when it is not 2
#define QOQ_KT(...) \
  {{__VA_ARGS__, 0, false, true>, __VA_ARGS__, 1, false, true>}, {__VA_ARGS__, 0, true, true>, __VA_ARGS__, 1, true, true>}}
// the same with streaming code loads (names end in "_nt")
#define QOQ_K4NT(...)                                                                         \
  {{__VA_ARGS__, 0, false, false, true>, __VA_ARGS__, 1, false, false, true>},                 \
   {__VA_ARGS__, 0, true, false, true>, __VA_ARGS__, 1, true, false, true>}}
#define QOQ_KTNT(...)                                                                         \
  {{__VA_ARGS__, 0, false, true, true>, __VA_ARGS__, 1, false, true, true>},                   \
   {__VA_ARGS__, 0, true, true, true>, __VA_ARGS__, 1, true, true, true>}}
#define QOQ_SKINNY(MT, NBW, W, U)                                                                      \
  {0, MT, NBW, W, U, 2, QOQ_K4(gemm_skinny_kernel<MT, NBW, W, U, 2), "skinny_mt" #MT "_nb" #NBW "_w" #W "_u" #U, \
   0, QOQ_KT(gemm_skinny_kernel<MT, NBW, W, U, 2)},
#define QOQ_SKINNY_R(MT, NBW, W, U, R)                                                      \
  {0, MT, NBW, W, U, R, QOQ_K4(gemm_skinny_kernel<MT, NBW, W, U, R),                          \
   "skinny_mt" #MT "_nb" #NBW "_w" #W "_u" #U "_r" #R, 0, QOQ_KT(gemm_skinny_kernel<MT, NBW, W, U, R)},
#define QOQ_SKINNY32(MT2, NP, W, U, R)                                                                  \
  {7, MT2, NP, W, U, R, QOQ_K4(gemm_skinny32_kernel<MT2, NP, W, U, R),                                   \
   "skinny32_mt" #MT2 "_np" #NP "_w" #W "_u" #U "_r" #R, 0, QOQ_KT(gemm_skinny32_kernel<MT2, NP, W, U, R)},
#define QOQ_SKINNY_NT(MT, NBW, W, U)                                                                  \
  {0, MT, NBW, W, U, 2, QOQ_K4NT(gemm_skinny_kernel<MT, NBW, W, U, 2),                                  \
   "skinny_mt" #MT "_nb" #NBW "_w" #W "_u" #U "_nt", 0, QOQ_KTNT(gemm_skinny_kernel<MT, NBW, W, U, 2), 1},
#define QOQ_SKINNY_RNT(MT, NBW, W, U, R)                                                              \
  {0, MT, NBW, W, U, R, QOQ_K4NT(gemm_skinny_kernel<MT, NBW, W, U, R),                                  \
   "skinny_mt" #MT "_nb" #NBW "_w" #W "_u" #U "_r" #R "_nt", 0, QOQ_KTNT(gemm_skinny_kernel<MT, NBW, W, U, R), 1},
#define QOQ_SKINNY32_NT(MT2, NP, W, U, R)                                                             \
  {7, MT2, NP, W, U, R, QOQ_K4NT(gemm_skinny32_kernel<MT2, NP, W, U, R),                               \
   "skinny32_mt" #MT2 "_np" #NP "_w" #W "_u" #U "_r" #R "_nt", 0,                                     \
   QOQ_KTNT(gemm_skinny32_kernel<MT2, NP, W, U, R), 1},
#define QOQ_WIDE2(TM, TN) {4, TM, TN, 0, 0, 0, QOQ_K4(gemm_wide2_kernel<TM, TN), "wide2_tm" #TM "_tn" #TN},
#define QOQ_DMA2(TM, TN) {5, TM, TN, 0, 0, 0, QOQ_K4(gemm_dma2_kernel<TM, TN), "dma2_tm" #TM "_tn" #TN},
#define QOQ_SD(AS) {6, AS, 0, 0, 0, 0, QOQ_K4(gemm_sd_kernel<AS, 2), "sd_as" #AS, sd_lds_bytes<AS, 2>()},
// 128-row tiles (each wave 32 rows x 128 columns): half the A copies per weight byte
// of the 128 x 128 tile kernels for mid-size batches
#define QOQ_SD128(AS) {6, AS, 1, 0, 0, 0, QOQ_K4(gemm_sd_kernel<AS, 1), "sd_m128_as" #AS, sd_lds_bytes<AS, 1>()},

const Config kConfigs[] = {
    // the configurations the measured dispatch table uses (qoq_plan_table.inc): the
    // profiling sweep times 58, and keeps the fewest that are near-best (within 3 %)
    // at every profiled point
    QOQ_SKINNY_NT(1, 1, 8, 2) QOQ_SKINNY_R(1, 2, 16, 1, 4)
    QOQ_SKINNY_NT(1, 2, 16, 2) QOQ_SKINNY_NT(1, 4, 8, 2) QOQ_SKINNY_NT(3, 2, 8, 2)
    QOQ_SKINNY_R(2, 2, 8, 1, 3) QOQ_SKINNY_RNT(2, 2, 8, 1, 3)
    QOQ_SKINNY32(1, 2, 8, 1, 2) QOQ_SKINNY32_NT(1, 2, 8, 1, 2) QOQ_SKINNY32(2, 2, 8, 1, 2) QOQ_SKINNY32_NT(2, 2, 8, 1, 2)
    QOQ_WIDE2(2, 1) QOQ_WIDE2(2, 2)
    QOQ_DMA2(2, 1) QOQ_DMA2(4, 1)
    QOQ_SD(3) QOQ_SD(2) QOQ_SD128(3)
#ifdef QOQ_ALL_CONFIGS
    // the rest of the profiling sweep's candidates (build.py --all-configs): none is
    // needed for the table, so the product build leaves them out
    QOQ_SKINNY(1, 1, 8, 2) QOQ_SKINNY_RNT(1, 2, 16, 1, 4) QOQ_WIDE2(4, 1) QOQ_SD128(2)
    QOQ_SKINNY(1, 1, 8, 4) QOQ_SKINNY(1, 2, 8, 4) QOQ_SKINNY(1, 1, 4, 4) QOQ_SKINNY(1, 2, 4, 4)
    QOQ_SKINNY(1, 1, 16, 2) QOQ_SKINNY(2, 1, 8, 4) QOQ_SKINNY(2, 2, 8, 2) QOQ_SKINNY(2, 1, 8, 2)
    QOQ_SKINNY(3, 1, 8, 2) QOQ_SKINNY(4, 1, 8, 2) QOQ_SKINNY(4, 2, 8, 2) QOQ_SKINNY(4, 2, 8, 1)
    QOQ_SKINNY(4, 4, 8, 1) QOQ_SKINNY(1, 2, 16, 2) QOQ_SKINNY(3, 2, 8, 2) QOQ_SKINNY(1, 4, 8, 2)
    QOQ_SKINNY_R(1, 2, 8, 2, 3) QOQ_SKINNY_R(2, 2, 8, 2, 3) QOQ_SKINNY_R(1, 1, 8, 2, 3)
    QOQ_SKINNY_R(2, 2, 8, 1, 4) QOQ_SKINNY_R(4, 2, 8, 1, 3) QOQ_SKINNY_R(4, 2, 8, 1, 4)
    QOQ_SKINNY_R(4, 4, 8, 1, 3) QOQ_SKINNY_R(1, 1, 16, 2, 3)
    QOQ_SKINNY32(2, 1, 8, 1, 2) QOQ_SKINNY32(2, 1, 8, 1, 3) QOQ_SKINNY32(1, 1, 8, 2, 2)
    QOQ_DMA2(2, 2) QOQ_DMA2(4, 2)
    QOQ_SKINNY_NT(2, 2, 8, 2) QOQ_SKINNY_NT(4, 4, 8, 1) QOQ_SKINNY_NT(2, 1, 8, 2) QOQ_SKINNY_NT(4, 2, 8, 1)
    QOQ_SKINNY_RNT(1, 1, 16, 2, 3) QOQ_SKINNY_RNT(4, 2, 8, 1, 3) QOQ_SKINNY32_NT(2, 1, 8, 1, 2)
#endif
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

const Config *find_config(int kind, int a, int b, int c, int d, int e = 0, bool nt = false) {
  if (kind == 0 && e == 0) e = 2;
  for (int i = 0; i < kNumConfigs; ++i) {
    const Config &cf = kConfigs[i];
    if (cf.kind == kind && cf.a == a && cf.b == b && cf.c == c && cf.d == d && cf.e == e && (cf.nt != 0) == nt)
      return &cf;
  }
  return nullptr;
}

struct Plan {
  const Config *cfg;
  dim3 grid, block;
  int splits;           // split-K factor (tile kernels: kinds 4, 5 and 6)
  size_t ws_bytes;      // workspace the launch needs (0 without split-K)
};

// Split-K factor: about kTargetWorkgroups workgroups (two per compute unit), each
// split keeping at least kMinSplitGroups groups of 128 so the loop prologue stays
// amortized.
constexpr int64_t kTargetWorkgroups = 512;
constexpr int64_t kMinSplitGroups = 4;
constexpr int64_t kMaxSplits = 16;

int choose_splits(int64_t tiles, int64_t G, int forced) {
  int64_t s = (kTargetWorkgroups + tiles / 2) / tiles;   // rounded
  if (forced >= 1) return static_cast<int>(std::min<int64_t>(std::min<int64_t>(forced, kMaxSplits), G));
  s = std::min<int64_t>(s, std::max<int64_t>(1, G / kMinSplitGroups));
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(s, kMaxSplits)));
}

// ---------------------------------------------------------------------------
// The measured dispatch table ("ADAngel" page: an offline policy map from the
// profiled shape to the fastest kernel, looked up at run time): one row per
// (N, K, activation-code layout, M) of the workloads' layer shapes, naming the
// configuration (and split-K factor) that was fastest on MI355X in the profiling
// sweep (`bench.py --profile-plan`, which writes qoq_plan_table.inc).  A shape the
// table covers takes the row with the nearest M (nearest in ratio); other shapes
// fall back to the rules below.
// ---------------------------------------------------------------------------
struct PlanRow {
  int64_t N, K;
  int tiled;
  int64_t M;
  const char *config;
  int splits;
};
const PlanRow kPlanRows[] = {
#define QOQ_PLAN_ROW(N, K, T, M, C, S) {N, K, T, M, C, S},
#include "qoq_plan_table.inc"
#undef QOQ_PLAN_ROW
    {0, 0, 0, 0, nullptr, 0}};   // end marker
constexpr int kNumPlanRows = sizeof(kPlanRows) / sizeof(kPlanRows[0]) - 1;

struct PlanIndex {
  const Config *cfg[kNumPlanRows + 1];
  struct Range {
    int64_t N, K;
    int tiled, begin, end;      // rows [begin, end), sorted by M
  } ranges[64];
  int nranges = 0;
};
PlanIndex g_plan_index;
std::once_flag g_plan_once;

void build_plan_index() {
  PlanIndex &ix = g_plan_index;
  for (int i = 0; i < kNumPlanRows; ++i) {
    ix.cfg[i] = nullptr;
    for (int c = 0; c < kNumConfigs; ++c)
      if (strcmp(kConfigs[c].name, kPlanRows[i].config) == 0 && (!kPlanRows[i].tiled || kConfigs[c].kt[0][0]))
        ix.cfg[i] = &kConfigs[c];
    const PlanRow &r = kPlanRows[i];
    const bool same = ix.nranges > 0 && ix.ranges[ix.nranges - 1].N == r.N && ix.ranges[ix.nranges - 1].K == r.K &&
                      ix.ranges[ix.nranges - 1].tiled == r.tiled;
    if (same) {
      ix.ranges[ix.nranges - 1].end = i + 1;
    } else if (ix.nranges < 64) {
      ix.ranges[ix.nranges++] = {r.N, r.K, r.tiled, i, i + 1};
    }
  }
}

// the table's configuration for this shape (nullptr when the table does not cover
// it); splits receives the row's split-K factor
const Config *table_plan(int64_t M, int64_t N, int64_t K, bool tiled_a, int &splits) {
  std::call_once(g_plan_once, build_plan_index);
  const PlanIndex &ix = g_plan_index;
  for (int r = 0; r < ix.nranges; ++r) {
    const auto &rg = ix.ranges[r];
    if (rg.N != N || rg.K != K || rg.tiled != static_cast<int>(tiled_a)) continue;
    int best = rg.begin;
    for (int i = rg.begin + 1; i < rg.end; ++i) {
      // between rows a < b: M is nearer to a in ratio iff M * M < a * b
      if (kPlanRows[i].M <= M || M * M >= kPlanRows[i - 1].M * kPlanRows[i].M) best = i;
      else break;
    }
    if (!ix.cfg[best]) return nullptr;
    splits = kPlanRows[best].splits;
    return ix.cfg[best];
  }
  return nullptr;
}

// split-K factor of a tile plan: the override, else the table's row, else the
// rule (when the rules allow splitting)
int plan_splits(int64_t tiles, int64_t G, int forced, int table_splits, bool split_k) {
  if (forced > 0) return choose_splits(tiles, G, forced);
  if (table_splits > 0) return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>({table_splits, kMaxSplits, G})));
  return split_k ? choose_splits(tiles, G, 0) : 1;
}

// tiled_a: the activation codes are in the tiled layout (M <= kTiledMaxM), which
// only the few-token kernels read
Plan make_plan(int64_t M, int64_t N, int64_t K, bool tiled_a = false) {
  const int64_t NS = N / 16;
  const int64_t G = K / 128;
  const Overrides ov = current_overrides();
  const Config *cfg = nullptr;
  if (ov.config >= 0 && (!tiled_a || kConfigs[ov.config].kt[0][0])) cfg = &kConfigs[ov.config];
  const int64_t t256 = ((NS + 15) / 16) * ((M + 127) / 128);   // 128 x 256 tiles
  const int64_t t128 = ((NS + 7) / 8) * ((M + 127) / 128);     // 128 x 128 tiles
  bool split_k = true;   // may the plan split K (tile kernels)
  int table_splits = 0;  // split-K factor of the table's row (0: no row)
  if (!cfg && ov.regime == 0) cfg = table_plan(M, N, K, tiled_a, table_splits);
  if (!cfg) {
    // 49..64 tokens on a wide layer: 64-row MFMA tiles beat the split-K-by-wave
    // skinny kernel (the weights are read once either way)
    bool tiled = M > 64 || (M > 48 && NS >= 1024);
    if (ov.regime == 1) tiled = false;
    if (ov.regime == 2) tiled = true;
    if (tiled_a) tiled = false;
    if (!tiled) {
      // shapes outside the measured table (rules distilled from the same sweeps):
      //  M <= 16: one 16-row block, streaming code loads; wide layers with short K
      //           (and weights under 8 MiB) one strip per workgroup with 8 K-split
      //           waves, the rest two strips and 16 waves
      //  streaming code loads past 16 tokens once the weights pass 8 MiB
      //  17..64 tokens: 32-row blocks on the 32x32x32 MFMA (about 60 % more INT8 ops
      //           per cycle than 16x16x64), two strip pairs per workgroup, one 32-row
      //           block up to 32 tokens and two beyond
      const bool nt = static_cast<int64_t>(N) * K / 2 >= (8 << 20);
      if (M <= 16) {
        cfg = (!nt || (NS >= 640 && G <= 64)) ? find_config(0, 1, 1, 8, 2, 2, true)
                                              : find_config(0, 1, 2, 16, 2, 2, true);
      } else {
        cfg = find_config(7, M <= 32 ? 1 : 2, 2, 8, 1, 2, nt);
      }
    } else {
      // measured on MI355X over the layer shapes of the workloads: the largest tile
      // that still gives enough workgroups to fill the chip; when no tile size does
      // (few columns, long K), split K over about 512 workgroups
      split_k = true;
      const int64_t t64 = ((NS + 7) / 8) * ((M + 63) / 64);   // 64 x 128 tiles
      if (t256 >= 384) {
        cfg = find_config(6, 3, 0, 0, 0);       // 256 x 256, shared dequantization
        split_k = false;
      } else if (t256 >= 192 && G >= 96) {
        cfg = find_config(6, 3, 0, 0, 0);       // 256 x 256, long K: split in two
      } else if (t128 >= 320) {
        cfg = find_config(5, 4, 1, 0, 0);       // 128 x 128, A by the copy engine
        split_k = false;
      } else if (M <= 64) {
        cfg = find_config(4, 2, 1, 0, 0);       // 64 x 128
        split_k = t64 < 192;
      } else if (t256 >= 96) {
        cfg = find_config(6, 3, 0, 0, 0);       // 256 x 256, split K
      } else {
        cfg = find_config(5, 4, 1, 0, 0);       // 128 x 128, split K
      }
    }
  }
  if (!cfg) cfg = find_config(0, 1, 1, 8, 2, 2, true);   // present in kConfigs; never reached by the rules above
  Plan p;
  p.cfg = cfg;
  p.splits = 1;
  p.ws_bytes = 0;
  if (cfg->kind == 0) {
    const int mt = cfg->a, nbw = cfg->b, waves = cfg->c;
    p.grid = dim3(static_cast<unsigned>((NS + nbw - 1) / nbw), static_cast<unsigned>((M + 16 * mt - 1) / (16 * mt)));
    p.block = dim3(64 * waves);
  } else if (cfg->kind == 7) {
    const int mt2 = cfg->a, np = cfg->b, waves = cfg->c;
    p.grid = dim3(static_cast<unsigned>((NS + 2 * np - 1) / (2 * np)),
                  static_cast<unsigned>((M + 32 * mt2 - 1) / (32 * mt2)));
    p.block = dim3(64 * waves);
  } else if (cfg->kind == 6) {   // 256 (or 128) x 256 tiles, 8 waves
    const int64_t bm = cfg->b == 1 ? 128 : 256;
    const int64_t tiles = ((NS + 15) / 16) * ((M + bm - 1) / bm);
    p.splits = plan_splits(tiles, G, ov.splits, table_splits, split_k);
    if (p.splits > 1) p.ws_bytes = sizeof(int) * static_cast<size_t>(p.splits) * M * N;
    p.grid = dim3(static_cast<unsigned>(tiles * p.splits));
    p.block = dim3(512);
  } else {   // wide2 / dma2: 32-row blocks, 4 waves x 2*TN strips
    const int tm = cfg->a, tn = cfg->b;
    const int64_t nx = (NS + 8 * tn - 1) / (8 * tn), ny = (M + 32 * tm - 1) / (32 * tm);
    const int64_t tiles = nx * ny;
    p.splits = plan_splits(tiles, G, ov.splits, table_splits, split_k);
    if (p.splits > 1) p.ws_bytes = sizeof(int) * static_cast<size_t>(p.splits) * M * N;
    p.grid = dim3(static_cast<unsigned>(tiles * p.splits));
    p.block = dim3(256);
  }
  return p;
}

}  // namespace

// Kernels with more than 64 KB of dynamic LDS are granted their size once per
// process (the attribute is kept per kernel).
std::once_flag g_lds_once[kNumConfigs][2][2];

void ensure_lds_attribute(const Config *cfg, int pc, int out_kind) {
  if (cfg->lds <= 65536) return;
  const int idx = static_cast<int>(cfg - kConfigs);
  std::call_once(g_lds_once[idx][pc][out_kind], [cfg, pc, out_kind] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(cfg->k[pc][out_kind]),
                              hipFuncAttributeMaxDynamicSharedMemorySize, cfg->lds);
  });
}

void launch_gemm_any(const void *qx, const void *sx, const void *packed, const void *meta, const void *sw,
                     const void *zp, const void *tx, void *out, int pc, int out_kind, int64_t M, int64_t N, int64_t K,
                     void *ws, hipStream_t st) {
  const Plan p = make_plan(M, N, K);
  ensure_lds_attribute(p.cfg, pc, out_kind);
  hipLaunchKernelGGL(p.cfg->k[pc][out_kind], p.grid, p.block, p.cfg->lds, st, static_cast<const int8_t *>(qx),
                     static_cast<const __half *>(sx), static_cast<const uint4 *>(packed),
                     static_cast<const uint16_t *>(meta), static_cast<const __half *>(sw),
                     static_cast<const uint8_t *>(zp), static_cast<const int *>(tx), out, static_cast<int>(M),
                     static_cast<int>(N), static_cast<int>(K), p.splits,
                     static_cast<int *>(p.splits > 1 ? ws : nullptr));
  if (p.splits > 1) {
    const size_t threads = static_cast<size_t>(M) * N / 8;
    const dim3 g(static_cast<unsigned>((threads + 255) / 256));
    using RK = void (*)(const int *, int, int, int, const __half *, const __half *, const uint8_t *, const int *,
                        void *);
    const RK rk[2][2] = {{split_reduce_kernel<0, false>, split_reduce_kernel<1, false>},
                         {split_reduce_kernel<0, true>, split_reduce_kernel<1, true>}};
    hipLaunchKernelGGL(rk[pc][out_kind], g, dim3(256), 0, st, static_cast<const int *>(ws), p.splits,
                       static_cast<int>(M), static_cast<int>(N), static_cast<const __half *>(sx),
                       static_cast<const __half *>(sw), static_cast<const uint8_t *>(zp),
                       static_cast<const int *>(tx), out);
  }
}

void launch_w4a8_gemm(const void *qx, const void *sx, const void *packed, const void *meta, const void *sw,
                      void *out, int out_kind, int64_t M, int64_t N, int64_t K, void *ws, hipStream_t st) {
  launch_gemm_any(qx, sx, packed, meta, sw, nullptr, nullptr, out, 0, out_kind, M, N, K, ws, st);
}

void launch_w4a8_gemm_pc(const void *qx, const void *sx, const void *tx, const void *packed, const void *zeros,
                         const void *sw, void *out, int out_kind, int64_t M, int64_t N, int64_t K, void *ws,
                         hipStream_t st) {
  launch_gemm_any(qx, sx, packed, nullptr, sw, zeros, tx, out, 1, out_kind, M, N, K, ws, st);
}

void launch_w4a8_gemm_tiled(const void *qx, const void *sx, const void *packed, const void *meta, const void *sw,
                            void *out, int out_kind, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const Plan p = make_plan(M, N, K, true);
  hipLaunchKernelGGL(p.cfg->kt[0][out_kind], p.grid, p.block, 0, st, static_cast<const int8_t *>(qx),
                     static_cast<const __half *>(sx), static_cast<const uint4 *>(packed),
                     static_cast<const uint16_t *>(meta), static_cast<const __half *>(sw), nullptr, nullptr, out,
                     static_cast<int>(M), static_cast<int>(N), static_cast<int>(K), 1, nullptr);
}

// per-channel weights on tiled codes: the same plan, the kernels' per-channel instances
void launch_w4a8_gemm_pc_tiled(const void *qx, const void *sx, const void *tx, const void *packed, const void *zeros,
                               const void *sw, void *out, int out_kind, int64_t M, int64_t N, int64_t K,
                               hipStream_t st) {
  const Plan p = make_plan(M, N, K, true);
  hipLaunchKernelGGL(p.cfg->kt[1][out_kind], p.grid, p.block, 0, st, static_cast<const int8_t *>(qx),
                     static_cast<const __half *>(sx), static_cast<const uint4 *>(packed), nullptr,
                     static_cast<const __half *>(sw), static_cast<const uint8_t *>(zeros),
                     static_cast<const int *>(tx), out, static_cast<int>(M), static_cast<int>(N), static_cast<int>(K),
                     1, nullptr);
}

const char *gemm_tiled_plan_name(int64_t M, int64_t N, int64_t K) { return make_plan(M, N, K, true).cfg->name; }

size_t gemm_workspace_need(int64_t M, int64_t N, int64_t K) { return make_plan(M, N, K).ws_bytes; }

int gemm_plan_splits(int64_t M, int64_t N, int64_t K) { return make_plan(M, N, K).splits; }

const char *gemm_plan_name(int64_t M, int64_t N, int64_t K) { return make_plan(M, N, K).cfg->name; }

// ---------------------------------------------------------------------------
// linear = per-token quantization + GEMM.  A few tokens (xq_plan): one fused kernel;
// otherwise the standalone quantizer writes the codes and s_X into the workspace
// (tiled codes up to kTiledMaxM tokens, read by a few-token kernel; row-major codes
// and the GEMM plan beyond).
// ---------------------------------------------------------------------------
typedef void (*XqKernel)(const __half *, __half *, const uint4 *, const uint16_t *, const __half *, __half *, int,
                         int, int);

struct XqConfig {
  int nbw, waves;
  XqKernel k;
  const char *name;
  int red;                  // LDS bytes of the partial-sum reduction
};

#define QOQ_XQ(NBW, W, U)                                                                              \
  {NBW, W, gemm_skinny_xq_kernel<NBW, W, U, 2>, "skinny_xq_nb" #NBW "_w" #W "_u" #U, \
   skinny_xq_red_bytes<NBW, W, U>()},
#define QOQ_XQ_R(NBW, W, U, R)                                                                         \
  {NBW, W, gemm_skinny_xq_kernel<NBW, W, U, R>, "skinny_xq_nb" #NBW "_w" #W "_u" #U "_r" #R, \
   skinny_xq_red_bytes<NBW, W, U>()},
// streaming code loads, as the few-token GEMM's "_nt" configurations
#define QOQ_XQ_NT(NBW, W, U)                                                                           \
  {NBW, W, gemm_skinny_xq_kernel<NBW, W, U, 2, true>, "skinny_xq_nb" #NBW "_w" #W "_u" #U "_nt", \
   skinny_xq_red_bytes<NBW, W, U>()},

// The fused configurations the measured linear table uses (qoq_linear_table.inc);
// the first is the one the rule below falls back to for shapes outside the table
const XqConfig kXqConfigs[] = {
    QOQ_XQ(2, 8, 2) QOQ_XQ(1, 8, 2) QOQ_XQ_NT(2, 16, 1) QOQ_XQ_NT(4, 8, 1)
#ifdef QOQ_ALL_CONFIGS
    QOQ_XQ(2, 16, 1) QOQ_XQ(4, 8, 1)
    QOQ_XQ_R(2, 8, 1, 3) QOQ_XQ_R(2, 8, 2, 3) QOQ_XQ_R(2, 16, 1, 3)
    QOQ_XQ_NT(2, 8, 2) QOQ_XQ_NT(1, 8, 2)
#endif
};
constexpr int kNumXq = sizeof(kXqConfigs) / sizeof(kXqConfigs[0]);
std::once_flag g_xq_once[kNumXq];

// The measured linear table: for the decode shapes of the workloads, whether one
// fused kernel (and which) or the quantizer + GEMM pair was fastest at M tokens
// (bench.py --profile-plan, real activations, weights rotated; "unfused" names the
// pair).  A covered (N, K) takes the row with the nearest M up to the largest
// profiled M, and the pair beyond it.
struct LinearRow {
  int64_t N, K, M;
  const char *config;
};
const LinearRow kLinearRows[] = {
#define QOQ_LINEAR_ROW(N, K, M, C) {N, K, M, C},
#include "qoq_linear_table.inc"
#undef QOQ_LINEAR_ROW
    {0, 0, 0, nullptr}};   // end marker
constexpr int kNumLinearRows = sizeof(kLinearRows) / sizeof(kLinearRows[0]) - 1;

int xq_index(const char *name) {
  for (int i = 0; i < kNumXq; ++i)
    if (strcmp(kXqConfigs[i].name, name) == 0) return i;
  return -1;
}

// covered: whether the table has rows for (N, K); the result: the row's fused
// configuration, or nullptr for the pair (or past the largest profiled M)
const XqConfig *linear_table_plan(int64_t M, int64_t N, int64_t K, bool &covered) {
  covered = false;
  int first = -1, last = -1;
  for (int i = 0; i < kNumLinearRows; ++i)
    if (kLinearRows[i].N == N && kLinearRows[i].K == K) {
      if (first < 0) first = i;
      last = i;
    }
  if (first < 0) return nullptr;
  covered = true;
  if (M > kLinearRows[last].M) return nullptr;
  int best = first;
  for (int i = first + 1; i <= last; ++i) {
    // between rows a < b: M is nearer to a in ratio iff M * M < a * b
    if (kLinearRows[i].M <= M || M * M >= kLinearRows[i - 1].M * kLinearRows[i].M) best = i;
    else break;
  }
  const int idx = xq_index(kLinearRows[best].config);
  return idx >= 0 ? &kXqConfigs[idx] : nullptr;
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

constexpr int64_t kXqMaxM = 2;               // measured: beyond two rows the repeated
constexpr int64_t kXqMaxRepeat = 32 << 20;    // quantization costs more than a launch

bool xq_fits(const XqConfig *c, int64_t M, int64_t K) { return M * (K / 8) <= int64_t{kXqPerThread} * 64 * c->waves; }

const XqConfig *xq_plan(int64_t M, int64_t N, int64_t K) {
  if (M > 16 || M * (K + 16) > kXqCodeBytes) return nullptr;      // the kernel's own limits (LDS code rows)
  const Overrides ov = current_overrides();
  if (ov.linear == -1) return nullptr;
  if (ov.linear >= 0) return xq_fits(&kXqConfigs[ov.linear], M, K) ? &kXqConfigs[ov.linear] : nullptr;
  if (ov.config < 0 && ov.regime == 0) {
    bool covered = false;
    const XqConfig *t = linear_table_plan(M, N, K, covered);
    if (covered) return t && xq_fits(t, M, K) ? t : nullptr;
  }
  // shapes outside the table: the first configuration up to two tokens and K = 8192,
  // while the quantization every workgroup repeats stays bounded
  if (M > kXqMaxM || K > kXqMaxK) return nullptr;
  // fused only while the quantization every workgroup repeats (workgroups x M x K
  // elements) stays bounded
  const int64_t NS = N / 16;
  const XqConfig *c = &kXqConfigs[0];
  if ((NS + c->nbw - 1) / c->nbw * M * K > kXqMaxRepeat) return nullptr;
  return xq_fits(c, M, K) ? c : nullptr;
}



int xq_lds_bytes(const XqConfig *c, int64_t M, int64_t K) {
  return kXqHead + std::max(static_cast<int>(M * (K + 16)), c->red);
}

// Unfused linear: up to kTiledMaxM tokens the quantizer writes the tiled layout and
// a few-token kernel reads it; beyond, row-major codes and the GEMM plan.
bool linear_tiled(int64_t M) { return M <= kTiledMaxM; }

size_t linear_qx_bytes(int64_t M, int64_t K) {
  return align256(static_cast<size_t>(linear_tiled(M) ? (M + 15) / 16 * 16 : M) * K);
}

size_t linear_workspace_need(int64_t M, int64_t N, int64_t K) {
  if (xq_plan(M, N, K)) return 0;
  return linear_qx_bytes(M, K) + align256(2 * static_cast<size_t>(M)) +
         (linear_tiled(M) ? 0 : gemm_workspace_need(M, N, K));
}

const char *linear_plan_name(int64_t M, int64_t N, int64_t K) {
  const XqConfig *c = xq_plan(M, N, K);
  if (c) return c->name;
  return linear_tiled(M) ? gemm_tiled_plan_name(M, N, K) : gemm_plan_name(M, N, K);
}

void launch_w4a8_linear(const void *x, const void *packed, const void *meta, const void *sw, void *out, void *sx_out,
                        int64_t M, int64_t N, int64_t K, void *ws, hipStream_t st) {
  if (const XqConfig *c = xq_plan(M, N, K)) {
    const int idx = static_cast<int>(c - kXqConfigs);
    const int lds = xq_lds_bytes(c, M, K);
    std::call_once(g_xq_once[idx], [c] {
      (void)hipFuncSetAttribute(reinterpret_cast<const void *>(c->k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                kXqHead + kXqCodeBytes);
    });
    const int64_t NS = N / 16;
    hipLaunchKernelGGL(c->k, dim3(static_cast<unsigned>((NS + c->nbw - 1) / c->nbw)), dim3(64 * c->waves), lds, st,
                       static_cast<const __half *>(x), static_cast<__half *>(sx_out),
                       static_cast<const uint4 *>(packed), static_cast<const uint16_t *>(meta),
                       static_cast<const __half *>(sw), static_cast<__half *>(out), static_cast<int>(M),
                       static_cast<int>(N), static_cast<int>(K));
    return;
  }
  int8_t *qx = static_cast<int8_t *>(ws);
  void *sx = sx_out ? sx_out : static_cast<void *>(qx + linear_qx_bytes(M, K));
  if (linear_tiled(M)) {
    launch_quantize_activations_tiled(x, M, K, qx, sx, st);
    launch_w4a8_gemm_tiled(qx, sx, packed, meta, sw, out, 0, M, N, K, st);
    return;
  }
  void *gws = qx + linear_qx_bytes(M, K) + align256(2 * static_cast<size_t>(M));
  launch_quantize_activations(x, M, K, qx, sx, st);
  launch_w4a8_gemm(qx, sx, packed, meta, sw, out, 0, M, N, K, gws, st);
}

// ---------------------------------------------------------------------------
// Static scratch of qoq_w4a8_linear_noalloc: a file-scope device array, one copy
// on every GPU the code object is loaded on.  Host code never uses the array's
// name as an address (on the host it names a stand-in, not device memory): the
// device address comes from hipGetSymbolAddress, once per device, with that
// device current, and is kept per device.
// ---------------------------------------------------------------------------
__device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t linear_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void *p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  if (!g_scratch_ptr[dev]) return hipErrorInvalidSymbol;
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

const char *linear_config_name(int index) {
  return (index >= 0 && index < kNumXq) ? kXqConfigs[index].name : nullptr;
}

const char *gemm_config_name(int index) {
  return (index >= 0 && index < kNumConfigs) ? kConfigs[index].name : nullptr;
}

namespace {

std::mutex g_override_mu;
std::once_flag g_override_env_once;
Overrides g_override;

int config_index(const char *name) {
  for (int i = 0; i < kNumConfigs; ++i)
    if (strcmp(kConfigs[i].name, name) == 0) return i;
  return -1;
}

int linear_index(const char *name) {
  if (strcmp(name, "unfused") == 0) return -1;
  for (int i = 0; i < kNumXq; ++i)
    if (strcmp(kXqConfigs[i].name, name) == 0) return i;
  return -3;
}

// 1 / 2 for the two regime names, 0 for none, -1 for anything else
int regime_code(const char *r) {
  if (!r || !r[0]) return 0;
  if (strcmp(r, "skinny") == 0) return 1;
  if (strcmp(r, "tiled") == 0) return 2;
  return -1;
}

// the environment's values, taken once (unknown names are ignored)
void read_env_overrides() {
  Overrides o;
  if (const char *c = getenv("QOQ_GEMM_CONFIG")) o.config = config_index(c);
  if (const char *f = getenv("QOQ_GEMM_SPLITS")) o.splits = static_cast<int>(std::max(0L, strtol(f, nullptr, 10)));
  if (const char *r = getenv("QOQ_GEMM_REGIME")) o.regime = std::max(0, regime_code(r));
  if (const char *l = getenv("QOQ_LINEAR_CONFIG")) {
    const int v = linear_index(l);
    o.linear = v >= -1 ? v : -2;
  }
  std::lock_guard<std::mutex> lk(g_override_mu);
  g_override = o;
}

Overrides current_overrides() {
  std::call_once(g_override_env_once, read_env_overrides);
  std::lock_guard<std::mutex> lk(g_override_mu);
  return g_override;
}

}  // namespace

int set_plan_override(const char *gemm_config, int splits, const char *regime, const char *linear_config) {
  Overrides o;
  if (gemm_config && gemm_config[0]) {
    o.config = config_index(gemm_config);
    if (o.config < 0) return -1;
  }
  if (splits < 0) return -1;
  o.splits = splits;
  o.regime = regime_code(regime);
  if (o.regime < 0) return -1;
  if (linear_config && linear_config[0]) {
    o.linear = linear_index(linear_config);
    if (o.linear < -1) return -1;
  }
  std::call_once(g_override_env_once, read_env_overrides);   // the environment never overwrites it later
  std::lock_guard<std::mutex> lk(g_override_mu);
  g_override = o;
  return 0;
}

}  // namespace qoq
