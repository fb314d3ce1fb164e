// Decode step of one tensor-parallel rank: one new token per sequence against
// the rank's share of the KV cache.
//
// What is computed: "Megatron-LM: GPU-Cluster Training Parallelism", section
// "Paper 1: QKV Column-Parallel Splitting in Detail", inference-time
// behaviour: generation keeps the training split; each rank appends the K and
// V of its own heads for the new token to its local cache shard, and the
// layer's two g sums then cover one row per sequence. The layer is the pre-LN
// layer of the forward kernels restricted to that row; the new token attends
// to cache rows 0..pos (itself included).
//
// Every step of decode is bound by HBM reads of data used once: the weights
// (a [B, K] x [K, N] product with B of at most 128 rows) and the cached K and
// V rows. The kernels are built for streaming, not for reuse:
//   gemv_kernel     : B rows against a 64-column weight strip, the K range
//                     split over workgroups so that the whole chip streams
//                     the matrix; fp16 MFMA 16x16x32 (bf16 weights converted
//                     at the LDS store) with the weight tile read back
//                     transposed by ds_read_b64_tr_b16. The split-K partials
//                     are summed in split order by gemv_finish_kernel, which
//                     runs the fused epilogue: bias + K/V append into the
//                     cache (QKV), bias + GeLU (FC1), bias + residual (W_o,
//                     FC2).
//   dec_attn_kernel : one wave per (sequence, head, slice of the cache);
//                     64-key blocks staged in LDS, scores with one lane per
//                     key, online softmax in the log2 domain, P V with one
//                     lane per pair of head dims. dec_combine_kernel merges
//                     the slices of each (sequence, head).
// The partial sums are merged by the next launch in the stream, not by the
// last workgroup to arrive: on gfx950 that needs a device-scope release per
// workgroup (an L2 write-back), which costs far more than a launch.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace tpl {

namespace {

constexpr int kStrip = 64;      // weight columns per workgroup of the fp32 path

__device__ __forceinline__ float ld_dt(const void* p, int dt, size_t i) {
  if (dt == DT_F32) return ((const float*)p)[i];
  if (dt == DT_BF16) return bf2f(((const bf16*)p)[i]);
  return (float)((const f16*)p)[i];
}
__device__ __forceinline__ void st_dt(void* p, int dt, size_t i, float v) {
  if (dt == DT_F32) ((float*)p)[i] = v;
  else if (dt == DT_BF16) ((bf16*)p)[i] = f2bf(v);
  else ((f16*)p)[i] = (f16)v;
}

// One output element of a decode GEMV: v is the full K sum.
__device__ __forceinline__ void gemv_epilogue(const GemvArgs& g, int m, int n, float v) {
  if (g.bias) v += ld_dt(g.bias, g.bias_dt, n);
  const size_t mn = (size_t)m * g.N + n;
  if (g.epi == GEMV_EPI_OUT) {
    if (g.resid) v += ld_dt(g.resid, g.resid_dt, mn);
    st_dt(g.out, g.out_dt, mn, v);
  } else {  // GEMV_EPI_GELU
    st_dt(g.out, g.out_dt, mn, gelu_f(v, g.gelu_tanh));
  }
}

// Shared tail: R[m][c] (m < M, LDS, pitch kStrip) holds this workgroup's sum
// over its K range for columns n0 + c. Without a split (and unless the caller
// consumes raw partials) it goes straight to the epilogue; otherwise it is
// stored as partial `ks`, summed by the next launch in the stream.
__device__ __forceinline__ void gemv_tail(const GemvArgs& g, const float* R, int tile, int ks) {
  const int tid = threadIdx.x, col = tid & (kStrip - 1), n = tile * kStrip + col;
  const int M = g.M, N = g.N;
  if (n >= N) return;
  if (g.nsplit == 1 && !g.raw) {
    for (int m = tid >> 6; m < M; m += 4) gemv_epilogue(g, m, n, R[m * kStrip + col]);
    return;
  }
  for (int m = tid >> 6; m < M; m += 4)
    g.part[((size_t)ks * M + m) * N + n] = R[m * kStrip + col];
}

// Sum of the split-K partials in split order (8 independent loads at a
// time), then the epilogue; one thread per output element.
__global__ __launch_bounds__(256) void gemv_finish_kernel(GemvArgs g) {
  const size_t total = (size_t)g.M * g.N;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int m = (int)(i / g.N), n = (int)(i % g.N);
  const int ns = g.nsplit;
  const float* p = g.part + i;
  float v = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 8) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = p[(size_t)min(s0 + u, ns - 1) * total];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < ns) v += x[u];
  }
  gemv_epilogue(g, m, n, v);
}

// One staged chunk of the fp16 path, held in registers between its load and
// its LDS store: the CH x STRIP weight chunk (16-byte pieces, CH*STRIP/2048
// per thread) and the row tile [16*MB][CH]. Out-of-range rows and columns
// load as zero (addresses clamped inside the matrices).
template <int MB, int STRIP, int CH>
struct GemvStage {
  static constexpr int kWRow = STRIP / 8;               // pieces per weight row
  static constexpr int kWPer = CH * kWRow / 256;
  static constexpr int kXRow = CH / 8;                  // pieces per row-tile row
  static constexpr int kXAll = 16 * MB * kXRow;
  static constexpr int kXPer = (kXAll + 255) / 256;
  static_assert(kWPer >= 1 && CH * kWRow % 256 == 0, "weight chunk / threads");
  uint4 wr[kWPer], xr[kXPer];
  __device__ __forceinline__ void load(const bf16* __restrict__ W, const f16* __restrict__ X,
                                       int M, int N, int K, int n0, int k0, int kend, int tid) {
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
      const int c = tid + 256 * i, r = c / kWRow, nn = n0 + 8 * (c % kWRow);
      const bool ok = (k0 + r < kend) & (nn < N);
      const uint4 v = *reinterpret_cast<const uint4*>(
          W + (size_t)min(k0 + r, K - 1) * N + min(nn, N - 8));
      wr[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int c = tid + 256 * i, m = c / kXRow, kk = k0 + 8 * (c % kXRow);
      const bool ok = (kXAll % 256 == 0 || c < kXAll) & (m < M) & (kk < kend);
      const uint4 v = *reinterpret_cast<const uint4*>(
          X + (size_t)min(m, M - 1) * K + min(kk, K - 8));
      xr[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
  }
  template <int WP, int XP>
  __device__ __forceinline__ void store(f16* Wl, f16* Xl, int tid) const {
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<uint4*>(Wl + (c / kWRow) * WP + 8 * (c % kWRow)) = bf16x8_to_f16x8(wr[i]);
    }
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
      const int c = tid + 256 * i;
      if (kXAll % 256 == 0 || c < kXAll)
        *reinterpret_cast<uint4*>(Xl + (c / kXRow) * XP + 8 * (c % kXRow)) = xr[i];
    }
  }
};

// fp16 MFMA path: X fp16 [M, K], W bf16 [K, N]; M <= 16 * MB. A workgroup
// owns a STRIP-column strip and kc rows of K, staged CH rows at a time; wave
// w owns columns [w*STRIP/4, (w+1)*STRIP/4) in 16-column MFMA tiles. The LDS
// pitches keep the transposing reads of the weight tile (4 rows x 32 bytes
// per 16 lanes) and the 16-byte row-tile reads free of bank conflicts.
template <int MB, int STRIP, int CH>
__global__ __launch_bounds__(256) void gemv_f16_kernel(GemvArgs g) {
  constexpr int WP = STRIP == 64 ? 72 : STRIP + 16;
  constexpr int XP = CH + 8;
  constexpr int NB = STRIP / 64;  // 16-column tiles per wave
  static_assert((CH * WP + 16 * MB * XP) * 2 <= 65536, "LDS");
  __shared__ __align__(16) f16 Wl[CH * WP];
  __shared__ __align__(16) f16 Xl[16 * MB * XP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = blockIdx.x, ks = blockIdx.y;
  const int M = g.M, N = g.N, K = g.K;
  const int n0 = tile * STRIP;
  const int kbeg = ks * g.kc, kend = min(K, kbeg + g.kc);
  const bf16* W = (const bf16*)g.W;
  const f16* X = (const f16*)g.X;

  GemvStage<MB, STRIP, CH> st;
  f32x4 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[i][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int g4 = lane >> 4, L16 = lane & 15;

  st.load(W, X, M, N, K, n0, kbeg, kend, tid);
  for (int k0 = kbeg; k0 < kend; k0 += CH) {
    __syncthreads();  // the previous chunk's LDS reads are done
    st.template store<WP, XP>(Wl, Xl, tid);
    __syncthreads();
    if (k0 + CH < kend) st.load(W, X, M, N, K, n0, k0 + CH, kend, tid);  // streams during the MFMAs
#pragma unroll
    for (int kk = 0; kk < CH; kk += 32) {
      f16x8 bop[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int c0 = 16 * (w * NB + b);
        const uint2 b0 = tr4(Wl, WP, kk + 8 * g4, c0, L16);
        const uint2 b1 = tr4(Wl, WP, kk + 8 * g4 + 4, c0, L16);
        bop[b] = __builtin_bit_cast(f16x8, make_uint4(b0.x, b0.y, b1.x, b1.y));
      }
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const f16x8 aop = *reinterpret_cast<const f16x8*>(Xl + (16 * i + L16) * XP + kk + 8 * g4);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[b], acc[i][b], 0, 0, 0);
      }
    }
  }
  // accumulator lane layout: rows 4*(lane/16) + r of block i, column lane%16
  // of tile b; straight to the epilogue, or to partial ks
  float* part = g.part + (size_t)ks * M * N;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int n = n0 + 16 * (w * NB + b) + L16;
    if (n < N) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 16 * i + 4 * g4 + r;
          if (m < M) {
            if (g.nsplit == 1 && !g.raw) gemv_epilogue(g, m, n, acc[i][b][r]);
            else part[(size_t)m * N + n] = acc[i][b][r];
          }
        }
    }
  }
}

// fp32 path: X fp32 [M, K], W fp32 [K, N]; thread (column, quarter of the
// rows) FMA, the quarters summed through LDS. Rows in blocks of 16.
template <int MB>
__global__ __launch_bounds__(256) void gemv_f32_kernel(GemvArgs g) {
  __shared__ float red[4][16][kStrip];
  __shared__ float R[16 * MB * kStrip];
  const int tid = threadIdx.x, col = tid & 63, q4 = tid >> 6;
  const int tile = blockIdx.x, ks = blockIdx.y;
  const int M = g.M, N = g.N, K = g.K;
  const int n = tile * kStrip + col;
  const int kbeg = ks * g.kc, kend = min(K, kbeg + g.kc);
  const float* W = (const float*)g.W;
  const float* X = (const float*)g.X;
  const int nc = min(n, N - 1);
  for (int m0 = 0; m0 < 16 * MB; m0 += 16) {
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    if (m0 < M) {
      for (int k = kbeg + q4; k < kend; k += 4) {
        const float wv = W[(size_t)k * N + nc];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[i] += X[(size_t)min(m0 + i, M - 1) * K + k] * wv;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) red[q4][i][col] = acc[i];
    __syncthreads();
    for (int i = q4; i < 16; i += 4)
      R[(m0 + i) * kStrip + col] = red[0][i][col] + red[1][i][col] + red[2][i][col] + red[3][i][col];
    __syncthreads();
  }
  gemv_tail(g, R, tile, ks);
}

// ---------------------------------------------------------------------------
// Decode attention
// ---------------------------------------------------------------------------
template <typename T> struct CacheVec;
template <> struct CacheVec<f16> {
  static constexpr int kPer = 8;  // elements per 16 bytes
  static __device__ __forceinline__ void to_f32(uint4 u, float* v) {
    const f16x8 h = __builtin_bit_cast(f16x8, u);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
  }
  static __device__ __forceinline__ void pair(const f16* p, float* a, float* b) {
    const f16x2 h = *reinterpret_cast<const f16x2*>(p);
    *a = (float)h[0];
    *b = (float)h[1];
  }
  static __device__ __forceinline__ void put_pair(f16* p, float a, float b) {
    *reinterpret_cast<f16x2*>(p) = f16x2{(f16)a, (f16)b};
  }
};
template <> struct CacheVec<float> {
  static constexpr int kPer = 4;
  static __device__ __forceinline__ void to_f32(uint4 u, float* v) {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
  }
  static __device__ __forceinline__ void pair(const float* p, float* a, float* b) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    *a = v.x;
    *b = v.y;
  }
  static __device__ __forceinline__ void put_pair(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
  }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// 64 rows (r0 .. r0+nr-1 valid, nr >= 1) of D elements of a cache slice,
// contiguous from `src`, into registers; rows >= nr read as zero.
template <typename T, int D>
struct CacheRows {
  static constexpr int kCpr = D / CacheVec<T>::kPer;  // 16-byte pieces per row
  uint4 st[kCpr];
  __device__ __forceinline__ void load(const T* __restrict__ src, int nr, int lane) {
#pragma unroll
    for (int i = 0; i < kCpr; ++i) {
      const int c = lane + 64 * i, row = c / kCpr, cc = c % kCpr;
      const uint4 v = *reinterpret_cast<const uint4*>(
          src + (size_t)min(row, nr - 1) * D + cc * CacheVec<T>::kPer);
      st[i] = row < nr ? v : make_uint4(0, 0, 0, 0);
    }
  }
  template <int P>
  __device__ __forceinline__ void store(T* dst, int lane) const {
#pragma unroll
    for (int i = 0; i < kCpr; ++i) {
      const int c = lane + 64 * i, row = c / kCpr, cc = c % kCpr;
      *reinterpret_cast<uint4*>(dst + row * P + cc * CacheVec<T>::kPer) = st[i];
    }
  }
};

template <typename T, int D, bool SPLIT>
__global__ __launch_bounds__(64) void dec_attn_kernel(DecAttnArgs g) {
  constexpr int kPad = 16 / sizeof(T);
  constexpr int P = D + kPad;     // LDS row pitch (elements)
  constexpr int NP = (D / 2 + 63) / 64;  // head-dim pairs per lane
  // V is fetched together with K when both fit in registers, else after the
  // scores (the residual tile of split scores takes V's place)
  constexpr bool kEarlyV = !SPLIT && CacheRows<T, D>::kCpr <= 16;
  __shared__ __align__(16) T tile[64 * P];
  __shared__ __align__(16) f16 tlo[SPLIT ? 64 * (D + 8) : 8];
  __shared__ __align__(16) float qs[D];
  __shared__ __align__(16) float ps[64];

  const int lane = threadIdx.x;
  const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int Hl = g.Hl, L = g.cache_len;
  const int pos = g.pos[b];
  const int nk = min(max(pos + 1, 0), L);
  const int kb0 = s * g.chunk, kb1 = min(kb0 + g.chunk, nk);
  const size_t base = ((size_t)b * Hl + j) * L * D;
  T* Kc = (T*)g.kc + base;
  T* Vc = (T*)g.vc + base;

  // the first 64-key block is fetched before anything else; each later block
  // is fetched while the previous one is being used
  CacheRows<T, D> kr, vr;
  CacheRows<f16, D> lr;
  auto fetch = [&](int kb, bool with_v) {
    const int nr = min(64, kb1 - kb);
    kr.load(Kc + (size_t)kb * D, nr, lane);
    if constexpr (SPLIT) lr.load(g.klo + base + (size_t)kb * D, nr, lane);
    if (with_v) vr.load(Vc + (size_t)kb * D, nr, lane);
  };
  if (kb0 < kb1) fetch(kb0, kEarlyV);

  // the new token's q, k, v for head j: the QKV split partials summed in
  // split order, plus the bias (lane owns head-dim pairs 2*(lane + 64 i))
  float nq[NP][2], nkv[NP][2][2];
  {
    const size_t N3 = (size_t)3 * Hl * D, stride = (size_t)g.batch * N3;
    const float* qp = g.qkv_part + (size_t)b * N3 + (size_t)j * 3 * D;
    const int ns = g.qkv_ns;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int d = min(2 * (lane + 64 * i), D - 2);
      float2 a[3] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
      for (int s0 = 0; s0 < ns; s0 += 4) {
        float2 x[4][3];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int c = 0; c < 3; ++c)
            x[u][c] = *reinterpret_cast<const float2*>(qp + (size_t)min(s0 + u, ns - 1) * stride +
                                                       c * D + d);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (s0 + u < ns)
#pragma unroll
            for (int c = 0; c < 3; ++c) {
              a[c].x += x[u][c].x;
              a[c].y += x[u][c].y;
            }
      }
      const int col = j * 3 * D + d;
      nq[i][0] = a[0].x + ld_dt(g.b_qkv, g.bias_dt, col);
      nq[i][1] = a[0].y + ld_dt(g.b_qkv, g.bias_dt, col + 1);
      nkv[i][0][0] = a[1].x + ld_dt(g.b_qkv, g.bias_dt, col + D);
      nkv[i][0][1] = a[1].y + ld_dt(g.b_qkv, g.bias_dt, col + D + 1);
      nkv[i][1][0] = a[2].x + ld_dt(g.b_qkv, g.bias_dt, col + 2 * D);
      nkv[i][1][1] = a[2].y + ld_dt(g.b_qkv, g.bias_dt, col + 2 * D + 1);
    }
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int d = 2 * (lane + 64 * i);
    if (d < D) {
      qs[d] = nq[i][0] * g.scale_log2;
      qs[d + 1] = nq[i][1] * g.scale_log2;
    }
  }
  // the slice holding row pos appends the new K and V to the cache; every
  // later use reads the stored (cache-precision) values
  const bool own = pos >= kb0 && pos < kb1;
  if (own) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int d = 2 * (lane + 64 * i);
      if (d < D) {
        CacheVec<T>::put_pair(Kc + (size_t)pos * D + d, nkv[i][0][0], nkv[i][0][1]);
        CacheVec<T>::put_pair(Vc + (size_t)pos * D + d, nkv[i][1][0], nkv[i][1][1]);
        if constexpr (SPLIT) {
          const float r0 = nkv[i][0][0] - (float)(T)nkv[i][0][0];
          const float r1 = nkv[i][0][1] - (float)(T)nkv[i][0][1];
          CacheVec<f16>::put_pair(g.klo + base + (size_t)pos * D + d, r0, r1);
        }
      }
    }
  }

  float m = -INFINITY, lsum = 0.f;
  float o[NP][2];
#pragma unroll
  for (int i = 0; i < NP; ++i) o[i][0] = o[i][1] = 0.f;

  for (int kb = kb0; kb < kb1; kb += 64) {
    const int nr = min(64, kb1 - kb);
    __syncthreads();  // qs written; previous block's tile reads done
    kr.template store<P>(tile, lane);
    if constexpr (SPLIT) lr.template store<D + 8>(tlo, lane);
    if (own && pos < kb + 64) {  // the new row, as stored in the cache
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int d = 2 * (lane + 64 * i);
        if (d < D) {
          CacheVec<T>::put_pair(tile + (pos - kb) * P + d, nkv[i][0][0], nkv[i][0][1]);
          if constexpr (SPLIT) {
            const float r0 = nkv[i][0][0] - (float)(T)nkv[i][0][0];
            const float r1 = nkv[i][0][1] - (float)(T)nkv[i][0][1];
            CacheVec<f16>::put_pair(tlo + (pos - kb) * (D + 8) + d, r0, r1);
          }
        }
      }
    }
    __syncthreads();

    // scores, one lane per key, log2 domain
    float sc = 0.f;
#pragma unroll
    for (int d = 0; d < D; d += CacheVec<T>::kPer) {
      float kv[CacheVec<T>::kPer];
      CacheVec<T>::to_f32(*reinterpret_cast<const uint4*>(tile + lane * P + d), kv);
      if constexpr (SPLIT) {
#pragma unroll
        for (int h = 0; h < CacheVec<T>::kPer; h += 8) {
          float lv[8];
          CacheVec<f16>::to_f32(*reinterpret_cast<const uint4*>(tlo + lane * (D + 8) + d + h), lv);
#pragma unroll
          for (int i = 0; i < 8; ++i) kv[h + i] += lv[i];
        }
      }
#pragma unroll
      for (int i = 0; i < CacheVec<T>::kPer; i += 4) {
        const float4 qv = *reinterpret_cast<const float4*>(qs + d + i);
        sc += qv.x * kv[i] + qv.y * kv[i + 1] + qv.z * kv[i + 2] + qv.w * kv[i + 3];
      }
    }
    sc = lane < nr ? sc : -INFINITY;
    const float mn = fmaxf(m, wave_max(sc));
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    const float pk = __builtin_amdgcn_exp2f(sc - mn);
    lsum = lsum * alpha + wave_sum(pk);
    m = mn;
    ps[lane] = pk;
    if constexpr (!kEarlyV) vr.load(Vc + (size_t)kb * D, nr, lane);
    __syncthreads();  // score reads of the tile done; ps visible
    vr.template store<P>(tile, lane);
    if (own && pos < kb + 64) {
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int d = 2 * (lane + 64 * i);
        if (d < D) CacheVec<T>::put_pair(tile + (pos - kb) * P + d, nkv[i][1][0], nkv[i][1][1]);
      }
    }
    __syncthreads();
    if (kb + 64 < kb1) fetch(kb + 64, kEarlyV);  // in flight during P V

    // O += P V, lane owns head dims 2*(lane + 64 i), +1
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      o[i][0] *= alpha;
      o[i][1] *= alpha;
    }
    // all 64 rows: rows >= nr hold zeros and carry weight 0
#pragma unroll
    for (int k0 = 0; k0 < 64; k0 += 4) {
      const float4 pv = *reinterpret_cast<const float4*>(ps + k0);
      const float pw[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int d = 2 * (lane + 64 * i);
        if (d < D) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float v0, v1;
            CacheVec<T>::pair(tile + (k0 + u) * P + d, &v0, &v1);
            o[i][0] += pw[u] * v0;
            o[i][1] += pw[u] * v1;
          }
        }
      }
    }
  }

  const size_t orow = ((size_t)b * Hl + j) * D;
  if (g.nsplit == 1) {
    const float inv = 1.f / lsum;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int d = 2 * (lane + 64 * i);
      if (d < D) {
        st_dt(g.o, g.o_dt, orow + d, o[i][0] * inv);
        st_dt(g.o, g.o_dt, orow + d + 1, o[i][1] * inv);
      }
    }
    return;
  }
  // partial of this slice: unnormalised o, running max, running sum; the
  // slices are merged by dec_combine_kernel, the next launch in the stream
  const int pair = b * Hl + j;
  float* part = g.part + ((size_t)pair * g.nsplit + s) * (D + 2);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int d = 2 * (lane + 64 * i);
    if (d < D) {
      part[d] = o[i][0];
      part[d + 1] = o[i][1];
    }
  }
  if (lane == 0) {
    part[D] = m;
    part[D + 1] = lsum;
  }
}

// Merge of the cache slices of one (sequence, head): lane t < nsplit holds
// slice t's running max and sum; the slice weights 2^(m_t - M) go through LDS
// to every lane, which owns head-dim pairs and reads the slices' partial
// outputs 8 at a time (independent loads), summed in slice order.
template <int D>
__global__ __launch_bounds__(64) void dec_combine_kernel(DecAttnArgs g) {
  constexpr int NP = (D / 2 + 63) / 64;
  __shared__ float ws[64];
  const int lane = threadIdx.x;
  const int pair = blockIdx.y * g.Hl + blockIdx.x;
  const int ns = g.nsplit;
  const float* pp = g.part + (size_t)pair * ns * (D + 2);
  const float mt = lane < ns ? pp[(size_t)lane * (D + 2) + D] : -INFINITY;
  const float lt_ = lane < ns ? pp[(size_t)lane * (D + 2) + D + 1] : 0.f;
  const float M = wave_max(mt);
  const float wt = __builtin_amdgcn_exp2f(mt - M);
  const float lt = wave_sum(lt_ * wt);
  ws[lane] = wt;
  __syncthreads();
  float acc[NP][2];
#pragma unroll
  for (int i = 0; i < NP; ++i) acc[i][0] = acc[i][1] = 0.f;
  for (int t0 = 0; t0 < ns; t0 += 8) {
    float2 v[8][NP];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float* q = pp + (size_t)min(t0 + u, ns - 1) * (D + 2);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int d = min(2 * (lane + 64 * i), D - 2);
        v[u][i] = *reinterpret_cast<const float2*>(q + d);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (t0 + u < ns) {
        const float wgt = ws[t0 + u];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          acc[i][0] += v[u][i].x * wgt;
          acc[i][1] += v[u][i].y * wgt;
        }
      }
    }
  }
  const float inv = 1.f / lt;
  const size_t orow = (size_t)pair * D;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int d = 2 * (lane + 64 * i);
    if (d < D) {
      st_dt(g.o, g.o_dt, orow + d, acc[i][0] * inv);
      st_dt(g.o, g.o_dt, orow + d + 1, acc[i][1] * inv);
    }
  }
}

// Residual stream and LayerNorm of one decode row (the output projection's
// epilogue fused with the second LayerNorm): h_mid = sum_s part[s] + bias + x
// (split order, then bias, then x), written in fp32 for the FC2 residual,
// then y = LN(h_mid). One workgroup per row, the row held in registers.
template <typename Tx, typename T, typename To, int NT, int NV>
__global__ __launch_bounds__(NT) void dec_resid_ln_kernel(
    const float* __restrict__ part, int ns, size_t pstride, const T* __restrict__ bias,
    const Tx* __restrict__ x, float* __restrict__ h_mid, const T* __restrict__ gamma,
    const T* __restrict__ beta, To* __restrict__ y, int h, float eps) {
  __shared__ float red[16];
  const int row = blockIdx.x, tid = threadIdx.x, nvec = h >> 3;
  const size_t ro = (size_t)row * h;
  float v[NV][8];
  float acc[1] = {0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int jv = tid + i * NT;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
    if (jv < nvec) {
      const float* p = part + ro + 8 * jv;
#pragma unroll 4
      for (int s = 0; s < ns; ++s) {
        float t[8];
        Vec8<float>::load(p + (size_t)s * pstride, t);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] += t[e];
      }
      float bb[8], xx[8];
      Vec8<T>::load(bias + 8 * jv, bb);
      Vec8<Tx>::load(x + ro + 8 * jv, xx);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[i][e] = (v[i][e] + bb[e]) + xx[e];
        acc[0] += v[i][e];
      }
      Vec8<float>::store(h_mid + ro + 8 * jv, v[i]);
    }
  }
  block_sum<1>(acc, red);
  const float mu = acc[0] / (float)h;
  float sq[1] = {0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (tid + i * NT < nvec)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[i][e] - mu;
        sq[0] += d * d;
      }
  block_sum<1>(sq, red);
  const float rstd = 1.f / sqrtf(sq[0] / (float)h + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int jv = tid + i * NT;
    if (jv < nvec) {
      float gg[8], be[8], o[8];
      Vec8<T>::load(gamma + 8 * jv, gg);
      Vec8<T>::load(beta + 8 * jv, be);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = gg[e] * ((v[i][e] - mu) * rstd) + be[e];
      Vec8<To>::store(y + ro + 8 * jv, o);
    }
  }
}

// K, V (and K residual) of every token of a forward's fused qkv into a cache.
template <typename T>
__global__ __launch_bounds__(256) void kv_fill_kernel(const T* __restrict__ qkv,
                                                     const f16* __restrict__ qkv_lo, T* kc,
                                                     T* vc, f16* klo, int batch, int seq,
                                                     int Hl, int D, int L) {
  constexpr int V = CacheVec<T>::kPer;
  const int cpr = D / V;
  const size_t total = (size_t)batch * seq * Hl * cpr;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (size_t)gridDim.x * blockDim.x) {
    const int cc = (int)(c % cpr);
    size_t r = c / cpr;
    const int j = (int)(r % Hl);
    r /= Hl;
    const int s = (int)(r % seq);
    const int b = (int)(r / seq);
    const size_t src = ((size_t)b * seq + s) * 3 * Hl * D + (size_t)j * 3 * D + cc * V;
    const size_t dst = (((size_t)b * Hl + j) * L + s) * D + cc * V;
    *reinterpret_cast<uint4*>(kc + dst) = *reinterpret_cast<const uint4*>(qkv + src + D);
    *reinterpret_cast<uint4*>(vc + dst) = *reinterpret_cast<const uint4*>(qkv + src + 2 * D);
    if (klo) {
      // fp16 residuals: 8 per 16 bytes, V = 8 here (klo is only used with fp16 caches)
      *reinterpret_cast<uint4*>(klo + dst) = *reinterpret_cast<const uint4*>(qkv_lo + src + D);
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// Strip width, chunk depth and K split of a decode GEMV (measured on the
// decode shapes of the 1.2B, 8.3B and 1T shards). Wide strips read long
// contiguous row segments and pay off on large matrices (5.6-5.8 TB/s at 256
// columns against 4.8 at 64 on the 1T shard); small matrices are bound by
// launch and memory latency, where fewer, longer workgroups win (about one
// workgroup per 32 KB of weights, at least 256). The fp32 partials written
// and read back stay below a quarter of the weight bytes.
void gemv_plan(int math, int M, int N, int K, int* strip, int* chunk, int* kc, int* nsplit) {
  const double wbytes = 2.0 * K * N;
  int st = 64, ch = 128;
  if (math == DT_F16 && wbytes >= 128e6) {
    if (M <= 16 && N >= 16 * 256) {
      st = 256;
      ch = 64;
    } else if (M <= 64 && N >= 16 * 128) {
      st = 128;
    }
  }
  double target = wbytes / 32768.0;
  target = target < 256 ? 256 : target > 2048 ? 2048 : target;
  const int tiles = (N + st - 1) / st;
  const int chunks = (K + ch - 1) / ch;
  int ns = (int)((target + tiles - 1) / tiles);
  const int cap = (int)(0.0625 * K / (M > 0 ? M : 1));
  if (ns > cap) ns = cap;
  if (ns > chunks) ns = chunks;
  if (ns < 1) ns = 1;
  const int per = (chunks + ns - 1) / ns;
  *strip = st;
  *chunk = ch;
  *kc = per * ch;
  *nsplit = (K + *kc - 1) / *kc;
}

hipError_t gemv(const GemvArgs& g, int math, hipStream_t s) {
  if (g.M < 1 || g.M > 128 || g.N % 8 || g.K % 8 || g.kc % g.chunk) return hipErrorInvalidValue;
  const int mb = (g.M + 15) / 16;
  const int MB = mb <= 1 ? 1 : mb <= 2 ? 2 : mb <= 4 ? 4 : 8;
  auto finish = [&]() -> hipError_t {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.nsplit == 1 || g.raw) return e;
    const size_t total = (size_t)g.M * g.N;
    gemv_finish_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(g);
    return hipGetLastError();
  };
  if (math != DT_F16) {
    if (g.strip != 64) return hipErrorInvalidValue;
    const dim3 grid((g.N + 63) / 64, g.nsplit);
    switch (MB) {
      case 1: gemv_f32_kernel<1><<<grid, 256, 0, s>>>(g); break;
      case 2: gemv_f32_kernel<2><<<grid, 256, 0, s>>>(g); break;
      case 4: gemv_f32_kernel<4><<<grid, 256, 0, s>>>(g); break;
      default: gemv_f32_kernel<8><<<grid, 256, 0, s>>>(g); break;
    }
    return finish();
  }
  const dim3 grid((g.N + g.strip - 1) / g.strip, g.nsplit);
#define TPL_GEMV(MB_, ST_, CH_)                                  \
  if (MB == MB_ && g.strip == ST_ && g.chunk == CH_) {           \
    gemv_f16_kernel<MB_, ST_, CH_><<<grid, 256, 0, s>>>(g);      \
    return finish();                                             \
  }
  TPL_GEMV(1, 64, 128) TPL_GEMV(2, 64, 128) TPL_GEMV(4, 64, 128) TPL_GEMV(8, 64, 128)
  TPL_GEMV(1, 64, 64) TPL_GEMV(2, 64, 64) TPL_GEMV(4, 64, 64) TPL_GEMV(8, 64, 64)
  TPL_GEMV(1, 128, 128) TPL_GEMV(2, 128, 128) TPL_GEMV(4, 128, 128)
  TPL_GEMV(1, 128, 64) TPL_GEMV(2, 128, 64) TPL_GEMV(4, 128, 64)
  TPL_GEMV(1, 256, 64) TPL_GEMV(2, 256, 64)
#undef TPL_GEMV
  return hipErrorInvalidValue;
}

int dec_attn_split(int batch, int Hl, int cache_len, int* chunk) {
  const int pairs = batch * Hl;
  int ns = (kDecWaves + pairs - 1) / pairs;
  const int blocks = (cache_len + 63) / 64;
  if (ns > blocks) ns = blocks;
  if (ns > kDecMaxSplit) ns = kDecMaxSplit;
  if (ns < 1) ns = 1;
  const int per = (blocks + ns - 1) / ns;
  *chunk = per * 64;
  return (cache_len + *chunk - 1) / *chunk;
}

hipError_t dec_attn(int dtype, const DecAttnArgs& g, int D, int split, hipStream_t s) {
  const dim3 grid(g.nsplit, g.Hl, g.batch);
  auto combine = [&]() -> hipError_t {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.nsplit == 1) return e;
    const dim3 cg(g.Hl, g.batch);
    switch (D) {
      case 32: dec_combine_kernel<32><<<cg, 64, 0, s>>>(g); break;
      case 64: dec_combine_kernel<64><<<cg, 64, 0, s>>>(g); break;
      case 96: dec_combine_kernel<96><<<cg, 64, 0, s>>>(g); break;
      case 128: dec_combine_kernel<128><<<cg, 64, 0, s>>>(g); break;
      default: dec_combine_kernel<160><<<cg, 64, 0, s>>>(g); break;
    }
    return hipGetLastError();
  };
#define TPL_DA(T_, D_, S_)                                  \
  if (D == D_ && split == S_) {                             \
    dec_attn_kernel<T_, D_, S_><<<grid, 64, 0, s>>>(g);     \
    return combine();                                       \
  }
  if (dtype == DT_F16) {
    TPL_DA(f16, 32, false) TPL_DA(f16, 64, false) TPL_DA(f16, 96, false)
    TPL_DA(f16, 128, false) TPL_DA(f16, 160, false)
    TPL_DA(f16, 32, true) TPL_DA(f16, 64, true) TPL_DA(f16, 96, true)
    TPL_DA(f16, 128, true) TPL_DA(f16, 160, true)
  } else if (!split) {
    TPL_DA(float, 32, false) TPL_DA(float, 64, false) TPL_DA(float, 96, false)
    TPL_DA(float, 128, false) TPL_DA(float, 160, false)
  }
#undef TPL_DA
  return hipErrorInvalidValue;
}

hipError_t dec_resid_ln(int dtype, const float* part, int ns, const void* bias, const void* x,
                        float* h_mid, const void* gamma, const void* beta, void* y, int rows,
                        int h, float eps, hipStream_t s) {
  const int nvec = h / 8;
  int nt, nv;
  if (nvec <= 256) { nt = 256; nv = 1; }
  else if (nvec <= 512) { nt = 256; nv = 2; }
  else if (nvec <= 1024) { nt = 512; nv = 2; }
  else if (nvec <= 2048) { nt = 1024; nv = 2; }
  else if (nvec <= 4096) { nt = 1024; nv = 4; }
  else return hipErrorInvalidValue;
  const size_t pstride = (size_t)rows * h;
#define TPL_DRL(TX, TP, TO, NT_, NV_)                                                          \
  if (nt == NT_ && nv == NV_) {                                                               \
    dec_resid_ln_kernel<TX, TP, TO, NT_, NV_><<<rows, NT_, 0, s>>>(                          \
        part, ns, pstride, (const TP*)bias, (const TX*)x, h_mid, (const TP*)gamma,            \
        (const TP*)beta, (TO*)y, h, eps);                                                     \
    return hipGetLastError();                                                                 \
  }
#define TPL_DRL_ALL(TX, TP, TO) \
  TPL_DRL(TX, TP, TO, 256, 1) TPL_DRL(TX, TP, TO, 256, 2) TPL_DRL(TX, TP, TO, 512, 2) \
  TPL_DRL(TX, TP, TO, 1024, 2) TPL_DRL(TX, TP, TO, 1024, 4)
  if (dtype == DT_F16) {
    TPL_DRL_ALL(bf16, bf16, f16)
  } else {
    TPL_DRL_ALL(float, float, float)
  }
#undef TPL_DRL_ALL
#undef TPL_DRL
  return hipErrorInvalidValue;
}

hipError_t kv_fill(int dtype, const void* qkv, const void* qkv_lo, void* kc, void* vc, void* klo,
                   int batch, int seq, int Hl, int D, int cache_len, hipStream_t s) {
  const int per = dtype == DT_F16 ? 8 : 4;
  const size_t total = (size_t)batch * seq * Hl * (D / per);
  if (total == 0) return hipSuccess;
  const int blocks = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  if (dtype == DT_F16)
    kv_fill_kernel<f16><<<blocks, 256, 0, s>>>((const f16*)qkv, (const f16*)qkv_lo, (f16*)kc,
                                               (f16*)vc, (f16*)klo, batch, seq, Hl, D, cache_len);
  else
    kv_fill_kernel<float><<<blocks, 256, 0, s>>>((const float*)qkv, nullptr, (float*)kc,
                                                 (float*)vc, nullptr, batch, seq, Hl, D,
                                                 cache_len);
  return hipGetLastError();
}

}  // namespace tpl
