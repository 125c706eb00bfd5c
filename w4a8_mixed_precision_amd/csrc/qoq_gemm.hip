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

#include <stdio.h>

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
//   token rows, and its waves split the K groups round-robin (split-K), so at each
//   step the workgroup reads WAVES consecutive 1 KB weight chunks of a strip.
//   Each wave: per group and strip, one 128-bit load per lane of packed codes and
//   one 16-bit metadata load, dequantize in registers, two MFMAs per row block.
//   The next group's loads are issued before the current group is consumed.
//   Partial sums of the waves are added through LDS; the epilogue follows.
// ---------------------------------------------------------------------------
template <int MT, int NBW, int WAVES, int OUT>
__global__ __launch_bounds__(64 * WAVES) void gemm_skinny_kernel(
    const int8_t *__restrict__ qx, const __half *__restrict__ sx, const uint4 *__restrict__ packed,
    const uint16_t *__restrict__ meta, const __half *__restrict__ sw, void *__restrict__ out, int M, int N,
    int K) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = K >> 7;
  const int NS = N >> 4;
  const int col = lane & 15;
  const int kq = lane >> 4;
  const int strip0 = blockIdx.x * NBW;
  const int m0 = blockIdx.y * (16 * MT);

  const uint4 *pb[NBW];
  const uint16_t *mb[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int s = min(strip0 + nb, NS - 1);      // strips past the end repeat the last; dropped at store
    pb[nb] = packed + static_cast<size_t>(s) * G * 64 + lane;
    mb[nb] = meta + static_cast<size_t>(s) * G * 16 + col;
  }
  const int8_t *ab[MT];
  bool av[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = m0 + 16 * mt + col;
    av[mt] = r < M;
    ab[mt] = qx + static_cast<size_t>(av[mt] ? r : 0) * K + 16 * kq;
  }

  v4i acc[MT][NBW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[mt][nb] = v4i{0, 0, 0, 0};

  uint4 p[NBW];
  unsigned md[NBW];
  v4i a0[MT], a1[MT];
  const v4i zero4 = {0, 0, 0, 0};

  int j = wave;
  if (j < G) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      p[nb] = pb[nb][static_cast<size_t>(j) * 64];
      md[nb] = mb[nb][static_cast<size_t>(j) * 16];
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      a0[mt] = av[mt] ? *reinterpret_cast<const v4i *>(ab[mt] + 128 * j) : zero4;
      a1[mt] = av[mt] ? *reinterpret_cast<const v4i *>(ab[mt] + 128 * j + 64) : zero4;
    }
  }
  while (j < G) {
    const int jn = j + WAVES;
    uint4 pn[NBW];
    unsigned mdn[NBW];
    v4i a0n[MT], a1n[MT];
    if (jn < G) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        pn[nb] = pb[nb][static_cast<size_t>(jn) * 64];
        mdn[nb] = mb[nb][static_cast<size_t>(jn) * 16];
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        a0n[mt] = av[mt] ? *reinterpret_cast<const v4i *>(ab[mt] + 128 * jn) : zero4;
        a1n[mt] = av[mt] ? *reinterpret_cast<const v4i *>(ab[mt] + 128 * jn + 64) : zero4;
      }
    }
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      v4i b0, b1;
      dequant_lane(p[nb], group_consts(md[nb]), b0, b1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt][nb] = mfma16x16x64(a0[mt], b0, acc[mt][nb]);
        acc[mt][nb] = mfma16x16x64(a1[mt], b1, acc[mt][nb]);
      }
    }
    if (jn < G) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        p[nb] = pn[nb];
        md[nb] = mdn[nb];
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        a0[mt] = a0n[mt];
        a1[mt] = a1n[mt];
      }
    }
    j = jn;
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
            store_result(out, OUT, static_cast<size_t>(m) * N + n, acc[mt][nb][i], scale);
          }
        }
  }
}

// ---------------------------------------------------------------------------
// Large-M regime (many tokens: INT8 MFMA throughput is the bound).
//   workgroup = 4 waves in a 2 x 2 arrangement; wave tile (16*TM) x (16*TN),
//   workgroup tile BM x BN = (32*TM) x (32*TN); one K step = one group of 128.
//   A (INT8 activations) is staged through LDS, double buffered, rows padded to
//   144 bytes so the 16 rows a 16-lane phase reads fall in distinct banks.
//   B (packed weights) goes global -> registers one step ahead and is dequantized
//   by each wave for its own TN strips (the two wave rows sharing a strip each
//   dequantize it; the MFMA work per dequantized weight is 16*TM products).
// ---------------------------------------------------------------------------
constexpr int kLdsRow = 144;   // bytes per staged A row (128 + 16 padding)

template <int TM, int TN, int OUT>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(const int8_t *__restrict__ qx,
                                                         const __half *__restrict__ sx,
                                                         const uint4 *__restrict__ packed,
                                                         const uint16_t *__restrict__ meta,
                                                         const __half *__restrict__ sw, void *__restrict__ out,
                                                         int M, int N, int K) {
  constexpr int BM = 32 * TM;
  constexpr int CH = BM * 8 / 256;           // 16-byte A chunks per thread per step
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int col = lane & 15, kq = lane >> 4;
  const int G = K >> 7;
  const int NS = N >> 4;
  const int m0 = blockIdx.y * BM;
  const int strip0 = blockIdx.x * (2 * TN) + wn * TN;

  // A staging: chunk e = tid + 256*c -> row e / 8, 16-byte column e % 8
  const int8_t *ag[CH];
  bool agv[CH];
  int alds[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int e = tid + 256 * c;
    const int r = e >> 3, cc = e & 7;
    agv[c] = (m0 + r) < M;
    ag[c] = qx + static_cast<size_t>(agv[c] ? m0 + r : 0) * K + 16 * cc;
    alds[c] = r * kLdsRow + 16 * cc;
  }
  const uint4 *pb[TN];
  const uint16_t *mb[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int s = min(strip0 + tn, NS - 1);
    pb[tn] = packed + static_cast<size_t>(s) * G * 64 + lane;
    mb[tn] = meta + static_cast<size_t>(s) * G * 16 + col;
  }

  v4i acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = v4i{0, 0, 0, 0};

  const v4i zero4 = {0, 0, 0, 0};
  v4i ar[CH];
  uint4 p[TN];
  unsigned md[TN];

  // prologue: group 0 into LDS buffer 0 and registers
#pragma unroll
  for (int c = 0; c < CH; ++c) ar[c] = agv[c] ? *reinterpret_cast<const v4i *>(ag[c]) : zero4;
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    p[tn] = pb[tn][0];
    md[tn] = mb[tn][0];
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) *reinterpret_cast<v4i *>(&As[0][alds[c]]) = ar[c];
  __syncthreads();

  const int arow = (wm * 16 * TM + col) * kLdsRow + 16 * kq;
  for (int j = 0; j < G; ++j) {
    const int buf = j & 1;
    const bool more = (j + 1) < G;
    uint4 pn[TN];
    unsigned mdn[TN];
    if (more) {
#pragma unroll
      for (int c = 0; c < CH; ++c)
        ar[c] = agv[c] ? *reinterpret_cast<const v4i *>(ag[c] + 128 * (j + 1)) : zero4;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        pn[tn] = pb[tn][static_cast<size_t>(j + 1) * 64];
        mdn[tn] = mb[tn][static_cast<size_t>(j + 1) * 16];
      }
    }
    v4i b0[TN], b1[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) dequant_lane(p[tn], group_consts(md[tn]), b0[tn], b1[tn]);
    const int8_t *abuf = &As[buf][arow];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const v4i a0 = *reinterpret_cast<const v4i *>(abuf + tm * 16 * kLdsRow);
      const v4i a1 = *reinterpret_cast<const v4i *>(abuf + tm * 16 * kLdsRow + 64);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        acc[tm][tn] = mfma16x16x64(a0, b0[tn], acc[tm][tn]);
        acc[tm][tn] = mfma16x16x64(a1, b1[tn], acc[tm][tn]);
      }
    }
    if (more) {
#pragma unroll
      for (int c = 0; c < CH; ++c) *reinterpret_cast<v4i *>(&As[buf ^ 1][alds[c]]) = ar[c];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        p[tn] = pn[tn];
        md[tn] = mdn[tn];
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int strip = strip0 + tn;
      if (strip >= NS) continue;
      const int n = strip * 16 + col;
      const float swn = (OUT == 0) ? __half2float(sw[n]) : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 16 * TM + 16 * tm + 4 * kq + i;
        if (m < M) {
          const float scale = (OUT == 0) ? __half2float(sx[m]) * swn : 0.0f;
          store_result(out, OUT, static_cast<size_t>(m) * N + n, acc[tm][tn][i], scale);
        }
      }
    }
}

// ---------------------------------------------------------------------------
// planning: which kernel and launch shape for (M, N, K)
// ---------------------------------------------------------------------------
struct Plan {
  int kind;     // 0 skinny, 1 tiled
  int mt, nbw, waves;
  int tm, tn;
  dim3 grid, block;
  const char *name;
};

#define QOQ_SKINNY_NAME(MT, NBW, W) "skinny_mt" #MT "_nb" #NBW "_w" #W
#define QOQ_TILED_NAME(TM, TN) "tiled_tm" #TM "_tn" #TN

Plan make_plan(int64_t M, int64_t N, int64_t K) {
  Plan p{};
  const int64_t NS = N / 16;
  const int64_t G = K / 128;
  const char *force = getenv("QOQ_GEMM_REGIME");   // measurement override: "skinny" or "tiled"
  bool tiled = M > 64;
  if (force && force[0] == 's') tiled = false;
  if (force && force[0] == 't') tiled = true;
  if (!tiled) {
    p.kind = 0;
    p.mt = static_cast<int>(M >= 64 ? 4 : (M + 15) / 16);
    if (p.mt < 1) p.mt = 1;
    p.nbw = NS >= 2048 ? 2 : 1;
    p.waves = G >= 16 ? 8 : 4;
    p.grid = dim3(static_cast<unsigned>((NS + p.nbw - 1) / p.nbw), static_cast<unsigned>((M + 16 * p.mt - 1) / (16 * p.mt)));
    p.block = dim3(64 * p.waves);
  } else {
    p.kind = 1;
    p.tm = M >= 256 ? 8 : 4;
    p.tn = 4;
    p.grid = dim3(static_cast<unsigned>((NS + 2 * p.tn - 1) / (2 * p.tn)),
                  static_cast<unsigned>((M + 32 * p.tm - 1) / (32 * p.tm)));
    p.block = dim3(256);
  }
  return p;
}

template <int MT, int NBW, int W>
void launch_skinny_t(const Plan &p, int out_kind, const void *qx, const void *sx, const void *packed,
                     const void *meta, const void *sw, void *out, int M, int N, int K, hipStream_t st) {
  if (out_kind == 0)
    hipLaunchKernelGGL((gemm_skinny_kernel<MT, NBW, W, 0>), p.grid, p.block, 0, st,
                       static_cast<const int8_t *>(qx), static_cast<const __half *>(sx),
                       static_cast<const uint4 *>(packed), static_cast<const uint16_t *>(meta),
                       static_cast<const __half *>(sw), out, M, N, K);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<MT, NBW, W, 1>), p.grid, p.block, 0, st,
                       static_cast<const int8_t *>(qx), static_cast<const __half *>(sx),
                       static_cast<const uint4 *>(packed), static_cast<const uint16_t *>(meta),
                       static_cast<const __half *>(sw), out, M, N, K);
}

template <int MT, int NBW>
void launch_skinny_w(const Plan &p, int ok, const void *a, const void *b, const void *c, const void *d,
                     const void *e, void *o, int M, int N, int K, hipStream_t st) {
  if (p.waves == 8)
    launch_skinny_t<MT, NBW, 8>(p, ok, a, b, c, d, e, o, M, N, K, st);
  else
    launch_skinny_t<MT, NBW, 4>(p, ok, a, b, c, d, e, o, M, N, K, st);
}

template <int MT>
void launch_skinny_n(const Plan &p, int ok, const void *a, const void *b, const void *c, const void *d,
                     const void *e, void *o, int M, int N, int K, hipStream_t st) {
  if (p.nbw == 2)
    launch_skinny_w<MT, 2>(p, ok, a, b, c, d, e, o, M, N, K, st);
  else
    launch_skinny_w<MT, 1>(p, ok, a, b, c, d, e, o, M, N, K, st);
}

template <int TM, int TN>
void launch_tiled_t(const Plan &p, int out_kind, const void *qx, const void *sx, const void *packed,
                    const void *meta, const void *sw, void *out, int M, int N, int K, hipStream_t st) {
  if (out_kind == 0)
    hipLaunchKernelGGL((gemm_tiled_kernel<TM, TN, 0>), p.grid, p.block, 0, st, static_cast<const int8_t *>(qx),
                       static_cast<const __half *>(sx), static_cast<const uint4 *>(packed),
                       static_cast<const uint16_t *>(meta), static_cast<const __half *>(sw), out, M, N, K);
  else
    hipLaunchKernelGGL((gemm_tiled_kernel<TM, TN, 1>), p.grid, p.block, 0, st, static_cast<const int8_t *>(qx),
                       static_cast<const __half *>(sx), static_cast<const uint4 *>(packed),
                       static_cast<const uint16_t *>(meta), static_cast<const __half *>(sw), out, M, N, K);
}

}  // namespace

void launch_w4a8_gemm(const void *qx, const void *sx, const void *packed, const void *meta, const void *sw,
                      void *out, int out_kind, int64_t M64, int64_t N64, int64_t K64, hipStream_t st) {
  const Plan p = make_plan(M64, N64, K64);
  const int M = static_cast<int>(M64), N = static_cast<int>(N64), K = static_cast<int>(K64);
  if (p.kind == 0) {
    switch (p.mt) {
      case 1: launch_skinny_n<1>(p, out_kind, qx, sx, packed, meta, sw, out, M, N, K, st); break;
      case 2: launch_skinny_n<2>(p, out_kind, qx, sx, packed, meta, sw, out, M, N, K, st); break;
      case 3: launch_skinny_n<3>(p, out_kind, qx, sx, packed, meta, sw, out, M, N, K, st); break;
      default: launch_skinny_n<4>(p, out_kind, qx, sx, packed, meta, sw, out, M, N, K, st); break;
    }
  } else {
    if (p.tm == 8)
      launch_tiled_t<8, 4>(p, out_kind, qx, sx, packed, meta, sw, out, M, N, K, st);
    else
      launch_tiled_t<4, 4>(p, out_kind, qx, sx, packed, meta, sw, out, M, N, K, st);
  }
}

const char *gemm_plan_name(int64_t M, int64_t N, int64_t K) {
  const Plan p = make_plan(M, N, K);
  if (p.kind == 1) return p.tm == 8 ? QOQ_TILED_NAME(8, 4) : QOQ_TILED_NAME(4, 4);
  static const char *names[4][2][2] = {
      {{QOQ_SKINNY_NAME(1, 1, 4), QOQ_SKINNY_NAME(1, 1, 8)}, {QOQ_SKINNY_NAME(1, 2, 4), QOQ_SKINNY_NAME(1, 2, 8)}},
      {{QOQ_SKINNY_NAME(2, 1, 4), QOQ_SKINNY_NAME(2, 1, 8)}, {QOQ_SKINNY_NAME(2, 2, 4), QOQ_SKINNY_NAME(2, 2, 8)}},
      {{QOQ_SKINNY_NAME(3, 1, 4), QOQ_SKINNY_NAME(3, 1, 8)}, {QOQ_SKINNY_NAME(3, 2, 4), QOQ_SKINNY_NAME(3, 2, 8)}},
      {{QOQ_SKINNY_NAME(4, 1, 4), QOQ_SKINNY_NAME(4, 1, 8)}, {QOQ_SKINNY_NAME(4, 2, 4), QOQ_SKINNY_NAME(4, 2, 8)}}};
  return names[p.mt - 1][p.nbw == 2][p.waves == 8];
}

}  // namespace qoq
