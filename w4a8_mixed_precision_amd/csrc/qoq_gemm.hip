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
//   strip, one 16-bit metadata load, the activation fragments) is issued before any
//   of them is consumed, and the next batch is issued before the current one is
//   computed, so each wave keeps up to 2*U KB of weights in flight per strip.
//   Slots past the wave's last group are zero-filled: zero codes with zero
//   metadata dequantize to 0 and add nothing.  Partial sums of the waves are added
//   through LDS; the epilogue follows.
// ---------------------------------------------------------------------------
template <int MT, int NBW, int U>
struct SkinnyBatch {
  uint4 p[U][NBW];
  unsigned md[U][NBW];
  v4i a0[U][MT];
  v4i a1[U][MT];
};

// Issues every load of batch b (groups t = b*U .. b*U+U-1 of this wave).  Only
// scalars come in, so no pointer array can end up in private (scratch) memory.
template <int MT, int NBW, int WAVES, int U>
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
    const int j = wave + WAVES * t;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      // strips past the end repeat the last one; their results are dropped at the store
      const size_t chunk = static_cast<size_t>(min(strip0 + nb, NS - 1)) * G + j;
      B.p[u][nb] = ok ? packed[chunk * 64 + lane] : make_uint4(0u, 0u, 0u, 0u);
      B.md[u][nb] = ok ? static_cast<unsigned>(meta[chunk * 16 + col]) : 0u;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = m0 + 16 * mt + col;
      const bool oka = ok && r < M;
      const int8_t *a = qx + static_cast<size_t>(oka ? r : 0) * K + 128 * (ok ? j : 0) + 16 * kq;
      B.a0[u][mt] = oka ? *reinterpret_cast<const v4i *>(a) : zero4;
      B.a1[u][mt] = oka ? *reinterpret_cast<const v4i *>(a + 64) : zero4;
    }
  }
}

template <int MT, int NBW, int WAVES, int U, int OUT>
__global__ __launch_bounds__(64 * WAVES) void gemm_skinny_kernel(
    const int8_t *__restrict__ qx, const __half *__restrict__ sx, const uint4 *__restrict__ packed,
    const uint16_t *__restrict__ meta, const __half *__restrict__ sw, void *__restrict__ out, int M, int N,
    int K) {
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

  SkinnyBatch<MT, NBW, U> cur, nxt;
  if (nbatch > 0)
    skinny_load<MT, NBW, WAVES, U>(cur, 0, ngroups, wave, packed, meta, qx, strip0, NS, G, K, M, m0, lane);
  for (int b = 0; b < nbatch; ++b) {
    if (b + 1 < nbatch)
      skinny_load<MT, NBW, WAVES, U>(nxt, b + 1, ngroups, wave, packed, meta, qx, strip0, NS, G, K, M, m0, lane);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        v4i b0, b1;
        dequant_lane(cur.p[u][nb], group_consts(cur.md[u][nb]), b0, b1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          acc[mt][nb] = mfma16x16x64(cur.a0[u][mt], b0, acc[mt][nb]);
          acc[mt][nb] = mfma16x16x64(cur.a1[u][mt], b1, acc[mt][nb]);
        }
      }
    if (b + 1 < nbatch) cur = nxt;
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
//   workgroup = 4 waves side by side along N: wave w owns TN strips (16*TN output
//   columns) and all BM = 16*TM rows of the tile, so every weight is dequantized by
//   exactly one wave and stays in that wave's registers (no LDS traffic for B).
//   One K step = one group of 128.  The A tile (BM x 128 INT8) is staged through
//   LDS, double buffered, and read by all four waves; its rows are padded to 144
//   bytes so the rows a 16-lane phase reads fall in distinct banks.  The next
//   group's A chunks and packed weights are fetched into registers before the
//   current group is consumed.
//   Tile order: the grid is 1-D.  Workgroup b runs on XCD b % 8, so ids are first
//   renumbered to give each XCD a contiguous range of tiles, then ranges are walked
//   GY row-tiles at a time (row index fastest), so the workgroups resident on one
//   XCD cover a compact block of rows x columns and share both operands in its L2.
// ---------------------------------------------------------------------------
constexpr int kLdsRow = 144;   // bytes per staged A row (128 + 16 padding)
constexpr int kXcds = 8;
constexpr int kTileGroupRows = 8;

__device__ __forceinline__ void tile_coords(int bid, int nx, int ny, int &x, int &y) {
  const int total = nx * ny;
  int t = bid;
  if (total % kXcds == 0) t = (bid % kXcds) * (total / kXcds) + bid / kXcds;
  const int group = kTileGroupRows * nx;
  const int g = t / group;
  const int first = g * kTileGroupRows;
  const int rows = min(ny - first, kTileGroupRows);
  const int r = t - g * group;
  y = first + r % rows;
  x = r / rows;
}

template <int TM, int TN, int OUT>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(const int8_t *__restrict__ qx,
                                                         const __half *__restrict__ sx,
                                                         const uint4 *__restrict__ packed,
                                                         const uint16_t *__restrict__ meta,
                                                         const __half *__restrict__ sw, void *__restrict__ out,
                                                         int M, int N, int K) {
  constexpr int BM = 16 * TM;
  constexpr int CH = BM * 8 / 256;           // 16-byte A chunks per thread per group
  static_assert(CH >= 1, "tile too small");
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int G = K >> 7;
  const int NS = N >> 4;
  const int nx = (NS + 4 * TN - 1) / (4 * TN);
  const int ny = (M + BM - 1) / BM;
  int tx, ty;
  tile_coords(blockIdx.x, nx, ny, tx, ty);
  const int m0 = ty * BM;
  const int strip0 = tx * (4 * TN) + wave * TN;

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
    const int s = min(strip0 + tn, NS - 1);   // strips past the end repeat the last; dropped at store
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

  const int arow = col * kLdsRow + 16 * kq;
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
  for (int tn = 0; tn < TN; ++tn) {
    const int strip = strip0 + tn;
    if (strip >= NS) continue;
    const int n = strip * 16 + col;
    const float swn = (OUT == 0) ? __half2float(sw[n]) : 0.0f;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 16 * tm + 4 * kq + i;
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
typedef void (*GemmKernel)(const int8_t *, const __half *, const uint4 *, const uint16_t *, const __half *,
                           void *, int, int, int);

struct Config {
  int kind;                 // 0 skinny, 1 tiled
  int a, b, c, d;           // skinny: MT, NBW, WAVES, U    tiled: TM, TN, -, -
  GemmKernel k[2];          // fp16 epilogue, INT32 epilogue
  const char *name;
};

#define QOQ_SKINNY(MT, NBW, W, U)                                                                   \
  {0, MT, NBW, W, U, {gemm_skinny_kernel<MT, NBW, W, U, 0>, gemm_skinny_kernel<MT, NBW, W, U, 1>}, \
   "skinny_mt" #MT "_nb" #NBW "_w" #W "_u" #U},
#define QOQ_TILED(TM, TN) \
  {1, TM, TN, 0, 0, {gemm_tiled_kernel<TM, TN, 0>, gemm_tiled_kernel<TM, TN, 1>}, "tiled_tm" #TM "_tn" #TN},

const Config kConfigs[] = {
    QOQ_SKINNY(1, 1, 8, 4) QOQ_SKINNY(1, 2, 8, 4) QOQ_SKINNY(1, 4, 8, 2) QOQ_SKINNY(1, 1, 4, 4)
    QOQ_SKINNY(1, 2, 4, 4) QOQ_SKINNY(1, 1, 8, 2) QOQ_SKINNY(1, 1, 16, 2) QOQ_SKINNY(1, 2, 16, 2)
    QOQ_SKINNY(2, 1, 8, 4) QOQ_SKINNY(2, 2, 8, 2) QOQ_SKINNY(2, 1, 8, 2)
    QOQ_SKINNY(3, 1, 8, 2) QOQ_SKINNY(3, 2, 8, 2)
    QOQ_SKINNY(4, 1, 8, 2) QOQ_SKINNY(4, 2, 8, 2) QOQ_SKINNY(4, 4, 8, 1) QOQ_SKINNY(4, 2, 8, 1)
    QOQ_TILED(4, 2) QOQ_TILED(4, 4) QOQ_TILED(8, 2) QOQ_TILED(8, 4) QOQ_TILED(16, 2)
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

const Config *find_config(int kind, int a, int b, int c, int d) {
  for (int i = 0; i < kNumConfigs; ++i) {
    const Config &cf = kConfigs[i];
    if (cf.kind == kind && cf.a == a && cf.b == b && (kind == 1 || (cf.c == c && cf.d == d))) return &cf;
  }
  return nullptr;
}

struct Plan {
  const Config *cfg;
  dim3 grid, block;
};

Plan make_plan(int64_t M, int64_t N, int64_t K) {
  const int64_t NS = N / 16;
  const int64_t G = K / 128;
  // measurement overrides (not needed for correct use): QOQ_GEMM_REGIME=skinny|tiled,
  // QOQ_GEMM_CONFIG=<name of a configuration in kConfigs>
  const Config *cfg = nullptr;
  if (const char *name = getenv("QOQ_GEMM_CONFIG")) {
    for (int i = 0; i < kNumConfigs; ++i)
      if (strcmp(kConfigs[i].name, name) == 0) cfg = &kConfigs[i];
  }
  if (!cfg) {
    const char *force = getenv("QOQ_GEMM_REGIME");
    bool tiled = M > 64;
    if (force && force[0] == 's') tiled = false;
    if (force && force[0] == 't') tiled = true;
    if (!tiled) {
      // measured on MI355X (config sweep over the layer shapes of the workloads):
      //  M <= 16: one 16-row block; wide layers with short K stream one strip per
      //           workgroup with 8 K-split waves, the rest two strips and 16 waves
      //  M <= 64: long K (>= 64 groups): at most two row blocks per workgroup;
      //           short K: all row blocks in one workgroup, 4 strips once N is wide
      const int mt = static_cast<int>(M >= 64 ? 4 : (M + 15) / 16);   // grid.y covers rows past 64
      if (mt <= 1) {
        cfg = (NS >= 640 && G <= 64) ? find_config(0, 1, 1, 8, 2) : find_config(0, 1, 2, 16, 2);
      } else if (G >= 64) {
        cfg = find_config(0, 2, 2, 8, 2);
      } else if (mt == 4) {
        cfg = NS >= 1024 ? find_config(0, 4, 4, 8, 1) : find_config(0, 4, 2, 8, 1);
      } else {
        cfg = find_config(0, mt, 2, 8, 2);
      }
    } else {
      // 128 x 128 workgroup tiles; 64-row tiles when that is needed for >= 512 tiles
      const int64_t tiles128 = ((NS + 7) / 8) * ((M + 127) / 128);
      cfg = tiles128 >= 512 ? find_config(1, 8, 2, 0, 0) : find_config(1, 4, 2, 0, 0);
    }
  }
  if (!cfg) cfg = find_config(0, 1, 1, 8, 2);   // present in kConfigs; never reached by the rules above
  Plan p;
  p.cfg = cfg;
  if (cfg->kind == 0) {
    const int mt = cfg->a, nbw = cfg->b, waves = cfg->c;
    p.grid = dim3(static_cast<unsigned>((NS + nbw - 1) / nbw), static_cast<unsigned>((M + 16 * mt - 1) / (16 * mt)));
    p.block = dim3(64 * waves);
  } else {
    const int tm = cfg->a, tn = cfg->b;
    const int64_t nx = (NS + 4 * tn - 1) / (4 * tn), ny = (M + 16 * tm - 1) / (16 * tm);
    p.grid = dim3(static_cast<unsigned>(nx * ny));
    p.block = dim3(256);
  }
  return p;
}

}  // namespace

void launch_w4a8_gemm(const void *qx, const void *sx, const void *packed, const void *meta, const void *sw,
                      void *out, int out_kind, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const Plan p = make_plan(M, N, K);
  hipLaunchKernelGGL(p.cfg->k[out_kind], p.grid, p.block, 0, st, static_cast<const int8_t *>(qx),
                     static_cast<const __half *>(sx), static_cast<const uint4 *>(packed),
                     static_cast<const uint16_t *>(meta), static_cast<const __half *>(sw), out,
                     static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
}

const char *gemm_plan_name(int64_t M, int64_t N, int64_t K) { return make_plan(M, N, K).cfg->name; }

const char *gemm_config_name(int index) {
  return (index >= 0 && index < kNumConfigs) ? kConfigs[index].name : nullptr;
}

}  // namespace qoq
