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
//                     are summed by the last workgroup of each strip to
//                     arrive (arrival counter), in split order, and the fused
//                     epilogue runs there: bias + K/V append into the cache
//                     (QKV), bias + GeLU (FC1), bias + residual (W_o, FC2).
//   dec_attn_kernel : one wave per (sequence, head, slice of the cache);
//                     64-key blocks staged in LDS, scores with one lane per
//                     key, online softmax in the log2 domain, P V with one
//                     lane per pair of head dims. Slices are merged by the
//                     last wave of each (sequence, head) to arrive.
// Arrival counters start at zero: the LayerNorm launch that opens each phase
// clears them, and the last arrival resets its own counter.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace tpl {

namespace {

constexpr int kStrip = 64;      // weight columns per workgroup
constexpr int kChunk = 128;     // K rows per staged chunk
constexpr int kWP = kStrip + 8; // LDS pitch of the fp16 weight tile (halves)
constexpr int kXP = kChunk + 8; // LDS pitch of the fp16 row tile (halves)

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

typedef short v4s __attribute__((ext_vector_type(4)));
#define DEC_LDS_V4S(p) ((__attribute__((address_space(3))) v4s*)(p))

// Four fp16 values of column mb + j of a row-major LDS tile T (pitch P),
// rows k0..k0+3, for lane j of each 16-lane group (ds_read_b64_tr_b16: lane L
// of the group addresses row k0 + L/4, columns mb + 4*(L%4) .. +3).
__device__ __forceinline__ uint2 tr4(const f16* T, int P, int k0, int mb, int L) {
  const f16* p = T + (k0 + (L >> 2)) * P + mb + 4 * (L & 3);
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(DEC_LDS_V4S(p)));
}

// One output element of a decode GEMV: v is the full K sum.
__device__ __forceinline__ void gemv_epilogue(const GemvArgs& g, int m, int n, float v) {
  if (g.bias) v += ld_dt(g.bias, g.bias_dt, n);
  const size_t mn = (size_t)m * g.N + n;
  if (g.epi == GEMV_EPI_OUT) {
    if (g.resid) v += ld_dt(g.resid, g.resid_dt, mn);
    st_dt(g.out, g.out_dt, mn, v);
  } else if (g.epi == GEMV_EPI_GELU) {
    st_dt(g.out, g.out_dt, mn, gelu_f(v, g.gelu_tanh));
  } else {  // GEMV_EPI_QKV: head-interleaved columns [q_j k_j v_j], width D each
    const int D = g.D;
    const int j = n / (3 * D), r = n - j * 3 * D, part = r / D, e = r - part * D;
    if (part == 0) {
      g.q[(size_t)m * g.Hl * D + j * D + e] = v;
    } else {
      const int p = g.pos[m];
      if (p >= 0 && p < g.cache_len) {
        const size_t idx = (((size_t)m * g.Hl + j) * g.cache_len + p) * D + e;
        if (part == 1) {
          st_dt(g.kcache, g.cache_dt, idx, v);
          if (g.klo) {
            const f16 hi = (f16)v;
            g.klo[idx] = (f16)(v - (float)hi);
          }
        } else {
          st_dt(g.vcache, g.cache_dt, idx, v);
        }
      }
    }
  }
}

// Shared tail: R[m][c] (m < M, LDS, pitch kStrip) holds this workgroup's sum
// over its K range for columns n0 + c. Without a split it goes straight to
// the epilogue; otherwise it becomes partial `ks`, and the last workgroup of
// the strip to arrive sums all partials in split order.
__device__ __forceinline__ void gemv_tail(const GemvArgs& g, const float* R, int tile, int ks) {
  __shared__ int s_last;
  const int tid = threadIdx.x, col = tid & (kStrip - 1), n = tile * kStrip + col;
  const int M = g.M, N = g.N;
  if (g.nsplit == 1) {
    if (n < N)
      for (int m = tid >> 6; m < M; m += 4) gemv_epilogue(g, m, n, R[m * kStrip + col]);
    return;
  }
  if (n < N)
    for (int m = tid >> 6; m < M; m += 4)
      g.part[((size_t)ks * M + m) * N + n] = R[m * kStrip + col];
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&g.count[tile], 1) == g.nsplit - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (n < N) {
    for (int m = tid >> 6; m < M; m += 4) {
      float v = 0.f;
      for (int s = 0; s < g.nsplit; ++s) v += g.part[((size_t)s * M + m) * N + n];
      gemv_epilogue(g, m, n, v);
    }
  }
  if (tid == 0) g.count[tile] = 0;
}

// One staged chunk of the fp16 path, held in registers between its load and
// its LDS store: the 128 x 64 weight chunk (1024 16-byte pieces, 4 per
// thread) and the row tile [16*MB][128] (256*MB pieces, MB per thread).
// Out-of-range rows and columns load as zero (addresses clamped inside).
template <int MB>
struct GemvStage {
  uint4 wr[4], xr[MB];
  __device__ __forceinline__ void load(const bf16* __restrict__ W, const f16* __restrict__ X,
                                       int M, int N, int K, int n0, int k0, int kend, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c >> 3, nn = n0 + 8 * (c & 7);
      const bool ok = (k0 + r < kend) & (nn < N);
      const uint4 v = *reinterpret_cast<const uint4*>(
          W + (size_t)min(k0 + r, K - 1) * N + min(nn, N - 8));
      wr[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int c = tid + 256 * i, m = c >> 4, kk = k0 + 8 * (c & 15);
      const bool ok = (m < M) & (kk < kend);
      const uint4 v = *reinterpret_cast<const uint4*>(
          X + (size_t)min(m, M - 1) * K + min(kk, K - 8));
      xr[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(f16* Wl, f16* Xl, int tid) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c >> 3;
      *reinterpret_cast<uint4*>(Wl + r * kWP + 8 * (c & 7)) = bf16x8_to_f16x8(wr[i]);
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int c = tid + 256 * i, m = c >> 4;
      *reinterpret_cast<uint4*>(Xl + m * kXP + 8 * (c & 15)) = xr[i];
    }
  }
};

// fp16 MFMA path: X fp16 [M, K], W bf16 [K, N]; M <= 16 * MB.
template <int MB>
__global__ __launch_bounds__(256) void gemv_f16_kernel(GemvArgs g) {
  constexpr int kWBytes = kChunk * kWP * 2;
  constexpr int kXBytes = 16 * MB * kXP * 2;
  constexpr int kRBytes = 16 * MB * kStrip * 4;
  constexpr int kBytes = (kWBytes + kXBytes) > kRBytes ? (kWBytes + kXBytes) : kRBytes;
  static_assert(kBytes <= 65536, "LDS");
  __shared__ __align__(16) char smem[kBytes];
  f16* Wl = reinterpret_cast<f16*>(smem);
  f16* Xl = reinterpret_cast<f16*>(smem + kWBytes);
  float* R = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = blockIdx.x, ks = blockIdx.y;
  const int M = g.M, N = g.N, K = g.K;
  const int n0 = tile * kStrip;
  const int kbeg = ks * g.kc, kend = min(K, kbeg + g.kc);
  const bf16* W = (const bf16*)g.W;
  const f16* X = (const f16*)g.X;

  GemvStage<MB> st;
  f32x4 acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int g4 = lane >> 4, L16 = lane & 15;

  st.load(W, X, M, N, K, n0, kbeg, kend, tid);
  for (int k0 = kbeg; k0 < kend; k0 += kChunk) {
    __syncthreads();  // the previous chunk's LDS reads are done
    st.store(Wl, Xl, tid);
    __syncthreads();
    if (k0 + kChunk < kend) st.load(W, X, M, N, K, n0, k0 + kChunk, kend, tid);  // streams during the MFMAs
#pragma unroll
    for (int kk = 0; kk < kChunk; kk += 32) {
      const uint2 b0 = tr4(Wl, kWP, kk + 8 * g4, 16 * w, L16);
      const uint2 b1 = tr4(Wl, kWP, kk + 8 * g4 + 4, 16 * w, L16);
      const f16x8 bop = __builtin_bit_cast(f16x8, make_uint4(b0.x, b0.y, b1.x, b1.y));
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const f16x8 aop = *reinterpret_cast<const f16x8*>(Xl + (16 * i + L16) * kXP + kk + 8 * g4);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, acc[i], 0, 0, 0);
      }
    }
  }
  __syncthreads();
  // accumulator lane layout: rows 4*(lane/16) + r of block i, column lane%16
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) R[(16 * i + 4 * g4 + r) * kStrip + 16 * w + L16] = acc[i][r];
  __syncthreads();
  gemv_tail(g, R, tile, ks);
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
  const T* Kc = (const T*)g.kc + base;
  const T* Vc = (const T*)g.vc + base;

  for (int e = lane; e < D; e += 64) qs[e] = g.q[((size_t)b * Hl + j) * D + e] * g.scale_log2;

  float m = -INFINITY, lsum = 0.f;
  float o[NP][2];
#pragma unroll
  for (int i = 0; i < NP; ++i) o[i][0] = o[i][1] = 0.f;

  for (int kb = kb0; kb < kb1; kb += 64) {
    const int nr = min(64, kb1 - kb);
    CacheRows<T, D> kr, vr;
    kr.load(Kc + (size_t)kb * D, nr, lane);
    CacheRows<f16, D> lr;
    if constexpr (SPLIT) lr.load(g.klo + base + (size_t)kb * D, nr, lane);
    if constexpr (kEarlyV) vr.load(Vc + (size_t)kb * D, nr, lane);
    __syncthreads();  // qs written; previous block's tile reads done
    kr.template store<P>(tile, lane);
    if constexpr (SPLIT) lr.template store<D + 8>(tlo, lane);
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
    __syncthreads();

    // O += P V, lane owns head dims 2*(lane + 64 i), +1
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      o[i][0] *= alpha;
      o[i][1] *= alpha;
    }
    for (int k = 0; k < nr; ++k) {
      const float pv = ps[k];
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int d = 2 * (lane + 64 * i);
        if (d < D) {
          float v0, v1;
          CacheVec<T>::pair(tile + k * P + d, &v0, &v1);
          o[i][0] += pv * v0;
          o[i][1] += pv * v1;
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
  // partial of this slice: unnormalised o, running max, running sum
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
  __threadfence();
  __syncthreads();
  __shared__ int s_last;
  if (lane == 0) s_last = atomicAdd(&g.count[pair], 1) == g.nsplit - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float* pp = g.part + (size_t)pair * g.nsplit * (D + 2);
  float M = -INFINITY;
  for (int t = 0; t < g.nsplit; ++t) M = fmaxf(M, pp[(size_t)t * (D + 2) + D]);
  float lt = 0.f;
  float acc[NP][2];
#pragma unroll
  for (int i = 0; i < NP; ++i) acc[i][0] = acc[i][1] = 0.f;
  for (int t = 0; t < g.nsplit; ++t) {
    const float* q = pp + (size_t)t * (D + 2);
    const float wgt = __builtin_amdgcn_exp2f(q[D] - M);
    lt += q[D + 1] * wgt;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int d = 2 * (lane + 64 * i);
      if (d < D) {
        acc[i][0] += q[d] * wgt;
        acc[i][1] += q[d + 1] * wgt;
      }
    }
  }
  const float inv = 1.f / lt;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int d = 2 * (lane + 64 * i);
    if (d < D) {
      st_dt(g.o, g.o_dt, orow + d, acc[i][0] * inv);
      st_dt(g.o, g.o_dt, orow + d + 1, acc[i][1] * inv);
    }
  }
  if (lane == 0) g.count[pair] = 0;
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
void gemv_plan(int M, int N, int K, int* kc, int* nsplit) {
  const int tiles = (N + kStrip - 1) / kStrip;
  const int chunks = (K + kChunk - 1) / kChunk;
  // enough workgroups to stream from every CU (about 2048), while the fp32
  // partials written and read back stay below a quarter of the weight bytes
  int ns = (2048 + tiles - 1) / tiles;
  const int cap = (int)(0.0625 * K / (M > 0 ? M : 1));
  if (ns > cap) ns = cap;
  if (ns > chunks) ns = chunks;
  if (ns < 1) ns = 1;
  const int per = (chunks + ns - 1) / ns;
  *kc = per * kChunk;
  *nsplit = (K + *kc - 1) / *kc;
}

hipError_t gemv(const GemvArgs& g, int math, hipStream_t s) {
  if (g.M < 1 || g.M > 128 || g.N % 8 || g.K % 8) return hipErrorInvalidValue;
  const dim3 grid((g.N + kStrip - 1) / kStrip, g.nsplit);
  const int mb = (g.M + 15) / 16;
  const int MB = mb <= 1 ? 1 : mb <= 2 ? 2 : mb <= 4 ? 4 : 8;
#define TPL_GEMV(KER, MB_)                       \
  if (MB == MB_) {                               \
    KER<MB_><<<grid, 256, 0, s>>>(g);            \
    return hipGetLastError();                    \
  }
  if (math == DT_F16) {
    TPL_GEMV(gemv_f16_kernel, 1) TPL_GEMV(gemv_f16_kernel, 2)
    TPL_GEMV(gemv_f16_kernel, 4) TPL_GEMV(gemv_f16_kernel, 8)
  } else {
    TPL_GEMV(gemv_f32_kernel, 1) TPL_GEMV(gemv_f32_kernel, 2)
    TPL_GEMV(gemv_f32_kernel, 4) TPL_GEMV(gemv_f32_kernel, 8)
  }
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
#define TPL_DA(T_, D_, S_)                                  \
  if (D == D_ && split == S_) {                             \
    dec_attn_kernel<T_, D_, S_><<<grid, 64, 0, s>>>(g);     \
    return hipGetLastError();                               \
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
