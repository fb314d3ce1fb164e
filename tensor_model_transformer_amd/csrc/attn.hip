// Causal / padding-masked softmax attention over one rank's local heads,
// forward and backward.
//
// What is computed: "Megatron-LM: GPU-Cluster Training Parallelism", section
// "Paper 1: QKV Column-Parallel Splitting in Detail" (each rank runs complete
// heads on its own Q, K, V; no exchange inside attention) and section
// "Fused Transformer Kernels" (scale-mask-softmax with general or causal
// masks; Q, K, V read in place from the fused projection output, no transpose
// kernels). S = Q K^T / sqrt(dh), masked keys excluded, P = row softmax,
// O = P V. The tiled, online-softmax evaluation that never materialises the
// s x s matrix is the memory-efficient attention the megatron-core package
// description names (FlashAttention); it changes rounding only.
//
// 16-bit path (fp16 operands on the gfx950 MFMA 32x32x16 f16, fp32
// accumulate; the layer's internal activations are fp16). The forward runs
// transposed (S^T = K Q^T and O^T = V^T P^T) so that each lane owns one query:
// the running max / sum of the online softmax stay in registers and the
// 32x32 accumulator of S^T feeds the P^T operand of the next MFMA directly.
// Within each 16-key slice the accumulator holds keys in the order
// {4h..4h+3, 8+4h..8+4h+3} for lane half h; the V^T operand is read in that
// same order straight from the row-major V tile with ds_read_b64_tr_b16
// (gfx950's transposing LDS read), so no transposed copy is ever built.
// Scores are kept in the log2 domain (scale * log2(e) folded into S) and the
// per-row normaliser is saved as lse2 = max + log2(sum).
//
// Backward (deterministic, no atomics): delta = rowsum(dO * O); one kernel
// owns a block of keys and sweeps the queries (dK, dV); another owns a block
// of queries and sweeps the keys (dQ). P is recomputed from lse2.
//
// fp32 path: one thread per query (forward, dQ) or key (dK, dV) with exact
// fp32 arithmetic.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace tpl {

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 2^x with the hardware exponential (v_exp_f32, about 1 ulp; results below
// the fp32 normal range flush to zero, which is below anything the softmax
// can resolve next to its row maximum).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f16x8 ld8(const f16* p) {
  return *reinterpret_cast<const f16x8*>(p);
}

__device__ __forceinline__ f16x8 pack8(const float* v) {
  uint4 u;
  u.x = pack2h(v[0], v[1]);
  u.y = pack2h(v[2], v[3]);
  u.z = pack2h(v[4], v[5]);
  u.w = pack2h(v[6], v[7]);
  return __builtin_bit_cast(f16x8, u);
}

// 8 consecutive accumulator values starting at `off` (0 or 8), packed to fp16.
__device__ __forceinline__ f16x8 pack8v(const f32x16& a, int off) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = a[off + i];
  return pack8(v);
}

// Register staging for a [R][D] row-major slice of global memory (row stride
// ld), rows >= nrows read as zero; stored into an LDS tile of pitch P. The
// address is clamped to the last row (nrows >= 1) and the value selected.
template <int R, int D, int NT>
struct RowTile {
  static constexpr int kChunks = R * (D / 8);
  static constexpr int kPer = (kChunks + NT - 1) / NT;
  uint4 st[kPer];
  __device__ __forceinline__ void load(const f16* __restrict__ src, long ld, int r0, int nrows,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / 8), dc = c % (D / 8);
      const bool ok = (kChunks % NT == 0 || c < kChunks) & (r0 + row < nrows);
      const int rr = min(r0 + row, nrows - 1);
      const int cc = (kChunks % NT == 0 || c < kChunks) ? dc : 0;
      const uint4 v = *reinterpret_cast<const uint4*>(src + (size_t)rr * ld + 8 * cc);
      st[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(f16* dst, int P, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * NT;
      const int row = c / (D / 8), dc = c % (D / 8);
      if (kChunks % NT == 0 || c < kChunks)
        *reinterpret_cast<uint4*>(dst + row * P + 8 * dc) = st[i];
    }
  }
};

// Workgroup barrier that leaves global loads in flight: this wave's LDS
// traffic is drained (lgkmcnt(0)) but vmcnt is not waited, so tiles fetched
// into registers for later blocks keep streaming across it. The empty asm
// statements keep the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// K and V (and the K residual) tiles of one 64-key block, staged in registers.
template <int D, bool SPLIT>
struct KVRegs {
  RowTile<64, D, 256> k, v, kl;
  __device__ __forceinline__ void load(const f16* Kp, const f16* Vp, const f16* Klp, long ldq,
                                       int r0, int seq, int tid) {
    k.load(Kp, ldq, r0, seq, tid);
    v.load(Vp, ldq, r0, seq, tid);
    if constexpr (SPLIT) kl.load(Klp, ldq, r0, seq, tid);
  }
  __device__ __forceinline__ void store(f16* base, int P, int TILE, int tid) const {
    k.store(base, P, tid);
    v.store(base + TILE, P, tid);
    if constexpr (SPLIT) kl.store(base + 2 * TILE, P, tid);
  }
};

// Block pipeline shared by the kernels that stream 64-row tiles through two
// LDS buffers. Memory latency on this part runs to microseconds, longer than
// one block's MFMA work, so when registers allow (DEEP) the tile of block
// ib+1 is fetched two blocks ahead, at ib-2, into one of two register
// stages; otherwise one block ahead. `fetch(stage, blk)` issues the global
// loads, `put(stage, buf)` writes a staged tile to LDS buffer `buf`, and
// `compute(ib)` consumes LDS buffer ib & 1.
template <bool DEEP, typename Stage, typename Fetch, typename Put, typename Compute>
__device__ __forceinline__ void block_pipeline(int nblk, Stage& sa, Stage& sb, Fetch fetch, Put put,
                                               Compute compute) {
  if (nblk <= 0) return;
  fetch(sa, 0);
  put(sa, 0);
  if constexpr (DEEP) {
    if (nblk > 1) fetch(sa, 1);
    if (nblk > 2) fetch(sb, 2);
    lds_barrier();
    auto step = [&](int ib, Stage& st) {
      compute(ib);
      if (ib + 1 < nblk) put(st, (ib + 1) & 1);
      if (ib + 3 < nblk) fetch(st, ib + 3);
      lds_barrier();
    };
    for (int ib = 0; ib < nblk; ib += 2) {
      step(ib, sa);
      if (ib + 1 < nblk) step(ib + 1, sb);
    }
  } else {
    lds_barrier();
    for (int ib = 0; ib < nblk; ++ib) {
      if (ib + 1 < nblk) fetch(sa, ib + 1);
      compute(ib);
      if (ib + 1 < nblk) put(sa, (ib + 1) & 1);
      lds_barrier();
    }
  }
}

// Waves per SIMD requested from the compiler: two where the registers fit
// without spilling (forward and dQ up to head dim 96, dK/dV up to 64, without
// the split-score residuals), else no constraint.
template <int D, bool SPLIT>
constexpr int kAttnWaves = (D <= 96 && !SPLIT) ? 2 : 1;
template <int D, bool SPLIT>
constexpr int kDkdvWaves = (D <= 64 && !SPLIT) ? 2 : 1;

// ============================================================================
// fp16 forward
// ============================================================================
// A workgroup owns 128 queries (32 per wave) of one (sequence, head) and
// sweeps 64-key blocks; K and V tiles are double-buffered in LDS through
// registers (the next block's loads are in flight during the current MFMAs).
template <int D, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kAttnWaves<D, SPLIT>))) void attn_fwd_f16_kernel(
    const f16* __restrict__ qkv, const f16* __restrict__ qkv_lo, f16* __restrict__ o,
    float* __restrict__ lse2, const int* __restrict__ valid_len, int seq, int Hl, int causal,
    float sl2) {
  constexpr int KB = 64, P = D + 8, TILE = KB * P, NT = SPLIT ? 3 : 2;
  extern __shared__ __align__(16) unsigned char smem[];
  f16* lds = reinterpret_cast<f16*>(smem);  // [2][K tile, V tile (, K residual tile)]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int qb = causal ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
  const int head = blockIdx.y, b = blockIdx.z;
  const int qw0 = qb * 128 + w * 32;
  const int q = qw0 + l32;
  const long ldq = 3L * Hl * D, ldo = (long)Hl * D;
  const size_t tok0 = (size_t)b * seq;
  const f16* Qp = qkv + tok0 * ldq + (size_t)head * 3 * D;
  const f16* Kp = Qp + D;
  const f16* Vp = Qp + 2 * D;
  const f16* Qlp = SPLIT ? qkv_lo + tok0 * ldq + (size_t)head * 3 * D : nullptr;
  const f16* Klp = SPLIT ? Qlp + D : nullptr;
  const int L = causal ? seq : min(max(valid_len[b], 0), seq);
  const int kv_end = causal ? min(seq, qb * 128 + 128) : L;
  const int lim = causal ? min(q + 1, seq) : L;  // this lane's keys are [0, lim)

  f16x8 qf[D / 16], ql[SPLIT ? D / 16 : 1];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (q < seq) v = *reinterpret_cast<const uint4*>(Qp + (size_t)q * ldq + 16 * ks + 8 * hh);
    qf[ks] = __builtin_bit_cast(f16x8, v);
    if constexpr (SPLIT) {
      uint4 r = make_uint4(0, 0, 0, 0);
      if (q < seq) r = *reinterpret_cast<const uint4*>(Qlp + (size_t)q * ldq + 16 * ks + 8 * hh);
      ql[ks] = __builtin_bit_cast(f16x8, r);
    }
  }
  f32x16 O[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) O[t][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int nblk = (kv_end + KB - 1) / KB;
  KVRegs<D, SPLIT> sa, sb;
  auto fetch = [&](KVRegs<D, SPLIT>& st, int blk) {
    st.load(Kp, Vp, Klp, ldq, blk * KB, seq, tid);
  };
  auto put = [&](const KVRegs<D, SPLIT>& st, int buf) { st.store(lds + buf * NT * TILE, P, TILE, tid); };
  auto compute = [&](int ib) {
    const int kb0 = ib * KB;
    const f16* Ks = lds + (ib & 1) * NT * TILE;
    const f16* Vs = Ks + TILE;
    const f16* Kls = Ks + 2 * TILE;  // residual tile (SPLIT only)
    if (!(causal && kb0 > qw0 + 31)) {  // some key of this block precedes a query of this wave
      f32x16 S[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int e = 0; e < 16; ++e) S[st][e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const int off = (32 * st + l32) * P + 16 * ks + 8 * hh;
          const f16x8 kh = ld8(Ks + off);
          S[st] = mfma32(kh, qf[ks], S[st]);
          if constexpr (SPLIT) {
            S[st] = mfma32(ld8(Kls + off), qf[ks], S[st]);
            S[st] = mfma32(kh, ql[ks], S[st]);
          }
        }
      }
      // S[st][4*jj+ii]: key kb0 + 32*st + 8*jj + 4*hh + ii, query q. Raw
      // scores: the scale sl2 > 0 is applied inside the exponent's FMA. Only
      // blocks that cross this wave's causal diagonal or the padding limit
      // need the mask (a wave-uniform test).
      const bool need_mask = causal ? kb0 + KB - 1 > qw0 : kb0 + KB > L;
      float mx = -INFINITY;
      if (need_mask) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kb0 + 32 * st + 8 * (e >> 2) + 4 * hh + (e & 3);
            S[st][e] = key < lim ? S[st][e] : -INFINITY;
            mx = fmaxf(mx, S[st][e]);
          }
      } else {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, S[st][e]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // Lazy rescaling: the reference point m_run (log2 domain) moves only
      // when this block's maximum exceeds it by more than kSlack, so p stays
      // below 2^kSlack (exact in fp32, and well inside fp16 for the P operand)
      // and most blocks skip the rescale of O. The result is independent of
      // the reference point up to rounding; lse2 = m_run + log2(l_run).
      constexpr float kSlack = 8.f;
      const float m_blk = mx * sl2;
      if (__builtin_amdgcn_ballot_w64(m_blk > m_run + kSlack)) {
        const float m_new = m_blk > m_run + kSlack ? m_blk : m_run;
        const float alpha = exp2_fast(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) O[t][e] *= alpha;
      }
      float ls = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2_fast(__builtin_fmaf(S[st][e], sl2, -m_run));
          S[st][e] = p;
          ls += p;
        }
      ls += __shfl_xor(ls, 32, 64);
      l_run += ls;
      // O^T[d][q] += sum_key V[key][d] P[q][key]; 16 keys per MFMA, slot order
      // {4h..4h+3, 8+4h..8+4h+3} within the 16 (the accumulator's row order)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f16x8 pf = pack8v(S[c >> 1], 8 * (c & 1));
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
          O[t] = mfma32(tr_frag(Vs, P, 32 * t, 16 * c + 4 * hh, 16 * c + 8 + 4 * hh, lane), pf,
                        O[t]);
      }
    }
  };
  block_pipeline<(D <= 128)>(nblk, sa, sb, fetch, put, compute);

  if (q < seq) {
    const float inv = 1.f / l_run;
    f16* op = o + (tok0 + q) * ldo + (size_t)head * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float v[4] = {O[t][4 * jj] * inv, O[t][4 * jj + 1] * inv, O[t][4 * jj + 2] * inv,
                      O[t][4 * jj + 3] * inv};
        Vec4<f16>::store(op + 32 * t + 8 * jj + 4 * hh, v);
      }
    if (hh == 0) lse2[((size_t)b * Hl + head) * seq + q] = m_run + log2f(l_run);
  }
}

// ============================================================================
// delta = rowsum(dO * O) per (token, head), fp32
// ============================================================================
template <typename T>
// Delta = rowsum(dO * O) per (token, head). One wave per token row: lanes
// read the row's 16-byte chunks of O and dO (coalesced) and sum each chunk's
// products; the chunk sums go through LDS and one lane per head adds its
// head's chunks in order.
__global__ __launch_bounds__(64) void attn_delta_kernel(const T* __restrict__ o,
                                                        const T* __restrict__ dO,
                                                        float* __restrict__ delta, int seq,
                                                        int Hl, int D) {
  constexpr int V = 16 / sizeof(T);  // elements per chunk
  extern __shared__ float csum[];    // [Hl * D / V]
  const int lane = threadIdx.x;
  const long tok = blockIdx.x;
  const int C = Hl * D / V;
  const T* a = o + tok * Hl * D;
  const T* g = dO + tok * Hl * D;
  for (int c = lane; c < C; c += 64) {
    float x[8], y[8];
    if constexpr (V == 8) {
      Vec8<T>::load(a + 8 * c, x);
      Vec8<T>::load(g + 8 * c, y);
    } else {
      Vec4<T>::load(a + 4 * c, x);
      Vec4<T>::load(g + 4 * c, y);
    }
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < V; ++e) acc += x[e] * y[e];
    csum[c] = acc;
  }
  __syncthreads();
  const long b = tok / seq, q = tok % seq;
  const int per = D / V;
  for (int hd = lane; hd < Hl; hd += 64) {
    float acc = 0.f;
    for (int i = 0; i < per; ++i) acc += csum[hd * per + i];
    delta[(b * Hl + hd) * seq + q] = acc;
  }
}

// ============================================================================
// fp16 backward: dK, dV (a workgroup owns 128 keys, 32 per wave)
// ============================================================================
// Sweeps 64-query blocks (two 32-query halves per MFMA step); Q and dO tiles
// are double-buffered in LDS through registers. Q^T and dO^T operands are
// read from the row-major tiles with transposing LDS reads.
template <int D, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kDkdvWaves<D, SPLIT>))) void attn_bwd_dkdv_f16_kernel(
    const f16* __restrict__ qkv, const f16* __restrict__ qkv_lo, const f16* __restrict__ dO,
    const float* __restrict__ lse2, const float* __restrict__ delta, f16* __restrict__ dqkv,
    const int* __restrict__ valid_len, int seq, int Hl, int causal, float sl2, float scale) {
  constexpr int QB = 64, P = D + 8, TILE = QB * P, NT = SPLIT ? 3 : 2;
  extern __shared__ __align__(16) unsigned char smem[];
  f16* lds = reinterpret_cast<f16*>(smem);                          // [2][Q, dO (, Q residual)]
  float* ls = reinterpret_cast<float*>(lds + 2 * NT * TILE);        // [2][QB]
  float* dl = ls + 2 * QB;                                          // [2][QB]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int kblk = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int kw0 = kblk * 128 + w * 32;
  const int key = kw0 + l32;
  const long ldq = 3L * Hl * D, ldo = (long)Hl * D;
  const size_t tok0 = (size_t)b * seq;
  const f16* Qp = qkv + tok0 * ldq + (size_t)head * 3 * D;
  const f16* Kp = Qp + D;
  const f16* Vp = Qp + 2 * D;
  const f16* dOp = dO + tok0 * ldo + (size_t)head * D;
  const f16* Qlp = SPLIT ? qkv_lo + tok0 * ldq + (size_t)head * 3 * D : nullptr;
  const float* lsp = lse2 + ((size_t)b * Hl + head) * seq;
  const float* dlp = delta + ((size_t)b * Hl + head) * seq;
  const int L = causal ? seq : min(max(valid_len[b], 0), seq);

  f16x8 kf[D / 16], vf[D / 16], kl[SPLIT ? D / 16 : 1];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (key < seq) {
      kv = *reinterpret_cast<const uint4*>(Kp + (size_t)key * ldq + 16 * ks + 8 * hh);
      vv = *reinterpret_cast<const uint4*>(Vp + (size_t)key * ldq + 16 * ks + 8 * hh);
    }
    kf[ks] = __builtin_bit_cast(f16x8, kv);
    vf[ks] = __builtin_bit_cast(f16x8, vv);
    if constexpr (SPLIT) {
      uint4 r = make_uint4(0, 0, 0, 0);
      if (key < seq)
        r = *reinterpret_cast<const uint4*>(Qlp + D + (size_t)key * ldq + 16 * ks + 8 * hh);
      kl[ks] = __builtin_bit_cast(f16x8, r);
    }
  }
  f32x16 dK[D / 32], dV[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) dK[t][e] = dV[t][e] = 0.f;

  const bool wave_keys_valid = kw0 < (causal ? seq : L);
  const int q_begin = causal ? kblk * 128 : 0;
  const int nblk = (seq - q_begin + QB - 1) / QB;
  struct QGRegs {
    RowTile<QB, D, 256> q, g, ql;
    float ls, dl;
  };
  QGRegs sa, sb;
  auto fetch = [&](QGRegs& st, int blk) {
    const int q0 = q_begin + blk * QB;
    st.q.load(Qp, ldq, q0, seq, tid);
    st.g.load(dOp, ldo, q0, seq, tid);
    if constexpr (SPLIT) st.ql.load(Qlp, ldq, q0, seq, tid);
    if (tid < QB) {
      const int qq = q0 + tid;
      st.ls = qq < seq ? lsp[qq] : 0.f;
      st.dl = qq < seq ? dlp[qq] : 0.f;
    }
  };
  auto put = [&](const QGRegs& st, int buf) {
    f16* base = lds + buf * NT * TILE;
    st.q.store(base, P, tid);
    st.g.store(base + TILE, P, tid);
    if constexpr (SPLIT) st.ql.store(base + 2 * TILE, P, tid);
    if (tid < QB) {
      ls[buf * QB + tid] = st.ls;
      dl[buf * QB + tid] = st.dl;
    }
  };
  auto compute = [&](int ib) {
    const int q0 = q_begin + ib * QB;
    const f16* Qs = lds + (ib & 1) * NT * TILE;
    const f16* Gs = Qs + TILE;
    const f16* Qls = Qs + 2 * TILE;  // residual tile (SPLIT only)
    const float* lsb = ls + (ib & 1) * QB;
    const float* dlb = dl + (ib & 1) * QB;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int qh0 = q0 + 32 * qs;  // first query of this half
      if (!wave_keys_valid || (causal && qh0 + 31 < kw0)) continue;
      f32x16 S, dP;
#pragma unroll
      for (int e = 0; e < 16; ++e) S[e] = dP[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int off = (32 * qs + l32) * P + 16 * ks + 8 * hh;
        const f16x8 qh = ld8(Qs + off);
        S = mfma32(qh, kf[ks], S);
        if constexpr (SPLIT) {
          S = mfma32(ld8(Qls + off), kf[ks], S);
          S = mfma32(qh, kl[ks], S);
        }
        dP = mfma32(ld8(Gs + off), vf[ks], dP);
      }
      // element e: query qh0 + 8*(e>>2) + 4*hh + (e&3), key = this lane's key.
      // The lse / delta of those rows come as 4 vector reads; every element
      // is evaluated and masked by a select, so the loop has no branches.
      float lsv[16], dlv[16];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float4 a = *reinterpret_cast<const float4*>(lsb + 32 * qs + 8 * jj + 4 * hh);
        const float4 b = *reinterpret_cast<const float4*>(dlb + 32 * qs + 8 * jj + 4 * hh);
        lsv[4 * jj] = a.x; lsv[4 * jj + 1] = a.y; lsv[4 * jj + 2] = a.z; lsv[4 * jj + 3] = a.w;
        dlv[4 * jj] = b.x; dlv[4 * jj + 1] = b.y; dlv[4 * jj + 2] = b.z; dlv[4 * jj + 3] = b.w;
      }
      float Pv[16], dS[16];
      // every (query, key) of this half allowed: no mask (a wave-uniform
      // test; the unmasked copy is left out where its registers would spill)
      constexpr bool kFast = !(D >= 160 && SPLIT);
      const bool need_mask = !kFast | (qh0 + 31 >= seq) | (kw0 + 31 >= L) | (causal & (kw0 + 31 > qh0));
      if (need_mask) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int qq = qh0 + 8 * (e >> 2) + 4 * hh + (e & 3);
          // bitwise & / |: no short-circuit, hence no branch per element
          const bool ok = (qq < seq) & (key < L) & (!causal | (key <= qq));
          const float p = exp2_fast(ok ? __builtin_fmaf(S[e], sl2, -lsv[e]) : -INFINITY);
          Pv[e] = p;
          dS[e] = p * (dP[e] - dlv[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2_fast(__builtin_fmaf(S[e], sl2, -lsv[e]));
          Pv[e] = p;
          dS[e] = p * (dP[e] - dlv[e]);
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const f16x8 pf = pack8(Pv + 8 * c);
        const f16x8 sf = pack8(dS + 8 * c);
        const int kA = 32 * qs + 16 * c + 4 * hh, kB = kA + 8;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          dV[t] = mfma32(tr_frag(Gs, P, 32 * t, kA, kB, lane), pf, dV[t]);
          dK[t] = mfma32(tr_frag(Qs, P, 32 * t, kA, kB, lane), sf, dK[t]);
        }
      }
    }
  };
  block_pipeline<(D <= 96 || (D <= 128 && !SPLIT))>(nblk, sa, sb, fetch, put, compute);

  if (key < seq) {
    f16* dk = dqkv + (tok0 + key) * ldq + (size_t)head * 3 * D + D;
    f16* dv = dk + D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float a[4], c[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = dK[t][4 * jj + e] * scale;
          c[e] = dV[t][4 * jj + e];
        }
        Vec4<f16>::store(dk + 32 * t + 8 * jj + 4 * hh, a);
        Vec4<f16>::store(dv + 32 * t + 8 * jj + 4 * hh, c);
      }
  }
}

// ============================================================================
// fp16 backward: dQ (a workgroup owns 128 queries, 32 per wave)
// ============================================================================
template <int D, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kAttnWaves<D, SPLIT>))) void attn_bwd_dq_f16_kernel(
    const f16* __restrict__ qkv, const f16* __restrict__ qkv_lo, const f16* __restrict__ dO,
    const float* __restrict__ lse2, const float* __restrict__ delta, f16* __restrict__ dqkv,
    const int* __restrict__ valid_len, int seq, int Hl, int causal, float sl2, float scale) {
  constexpr int KB = 64, P = D + 8, TILE = KB * P, NT = SPLIT ? 3 : 2;
  extern __shared__ __align__(16) unsigned char smem[];
  f16* lds = reinterpret_cast<f16*>(smem);  // [2][K tile, V tile (, K residual tile)]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int qb = causal ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
  const int head = blockIdx.y, b = blockIdx.z;
  const int qw0 = qb * 128 + w * 32;
  const int q = qw0 + l32;
  const long ldq = 3L * Hl * D, ldo = (long)Hl * D;
  const size_t tok0 = (size_t)b * seq;
  const f16* Qp = qkv + tok0 * ldq + (size_t)head * 3 * D;
  const f16* Kp = Qp + D;
  const f16* Vp = Qp + 2 * D;
  const f16* dOp = dO + tok0 * ldo + (size_t)head * D;
  const int L = causal ? seq : min(max(valid_len[b], 0), seq);
  const int kv_end = causal ? min(seq, qb * 128 + 128) : L;
  const int lim = causal ? min(q + 1, seq) : L;
  const bool qok = q < seq;
  const float lq = qok ? lse2[((size_t)b * Hl + head) * seq + q] : 0.f;
  const float dq_ = qok ? delta[((size_t)b * Hl + head) * seq + q] : 0.f;
  const f16* Qlp = SPLIT ? qkv_lo + tok0 * ldq + (size_t)head * 3 * D : nullptr;
  const f16* Klp = SPLIT ? Qlp + D : nullptr;

  f16x8 qf[D / 16], gf[D / 16], ql[SPLIT ? D / 16 : 1];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    uint4 a = make_uint4(0, 0, 0, 0), c = make_uint4(0, 0, 0, 0);
    if (qok) {
      a = *reinterpret_cast<const uint4*>(Qp + (size_t)q * ldq + 16 * ks + 8 * hh);
      c = *reinterpret_cast<const uint4*>(dOp + (size_t)q * ldo + 16 * ks + 8 * hh);
    }
    qf[ks] = __builtin_bit_cast(f16x8, a);
    gf[ks] = __builtin_bit_cast(f16x8, c);
    if constexpr (SPLIT) {
      uint4 r = make_uint4(0, 0, 0, 0);
      if (qok) r = *reinterpret_cast<const uint4*>(Qlp + (size_t)q * ldq + 16 * ks + 8 * hh);
      ql[ks] = __builtin_bit_cast(f16x8, r);
    }
  }
  f32x16 dQ[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) dQ[t][e] = 0.f;

  const int nblk = (kv_end + KB - 1) / KB;
  KVRegs<D, SPLIT> sa, sb;
  auto fetch = [&](KVRegs<D, SPLIT>& st, int blk) {
    st.load(Kp, Vp, Klp, ldq, blk * KB, seq, tid);
  };
  auto put = [&](const KVRegs<D, SPLIT>& st, int buf) { st.store(lds + buf * NT * TILE, P, TILE, tid); };
  auto compute = [&](int ib) {
    const int kb0 = ib * KB;
    const f16* Ks = lds + (ib & 1) * NT * TILE;
    const f16* Vs = Ks + TILE;
    const f16* Kls = Ks + 2 * TILE;  // residual tile (SPLIT only)
    if (!(causal && kb0 > qw0 + 31)) {
      float dS[2][16];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        f32x16 S, dP;
#pragma unroll
        for (int e = 0; e < 16; ++e) S[e] = dP[e] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const int off = (32 * st + l32) * P + 16 * ks + 8 * hh;
          const f16x8 kh = ld8(Ks + off);
          S = mfma32(kh, qf[ks], S);
          if constexpr (SPLIT) {
            S = mfma32(ld8(Kls + off), qf[ks], S);
            S = mfma32(kh, ql[ks], S);
          }
          dP = mfma32(ld8(Vs + off), gf[ks], dP);
        }
        // every (query, key) of this 32-key half allowed: no mask (a
        // wave-uniform test); otherwise masked elements get p = 0
        const int k0 = kb0 + 32 * st;
        const bool need_mask = (qw0 + 31 >= seq) | (causal ? k0 + 31 > qw0 : k0 + 32 > L);
        if (need_mask) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int k = k0 + 8 * (e >> 2) + 4 * hh + (e & 3);
            const float p = exp2_fast((qok & (k < lim)) ? __builtin_fmaf(S[e], sl2, -lq) : -INFINITY);
            dS[st][e] = p * (dP[e] - dq_);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float p = exp2_fast(__builtin_fmaf(S[e], sl2, -lq));
            dS[st][e] = p * (dP[e] - dq_);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f16x8 sf = pack8(&dS[c >> 1][8 * (c & 1)]);
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
          dQ[t] = mfma32(tr_frag(Ks, P, 32 * t, 16 * c + 4 * hh, 16 * c + 8 + 4 * hh, lane), sf,
                         dQ[t]);
      }
    }
  };
  block_pipeline<(D <= 128)>(nblk, sa, sb, fetch, put, compute);

  if (qok) {
    f16* dq = dqkv + (tok0 + q) * ldq + (size_t)head * 3 * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float a[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = dQ[t][4 * jj + e] * scale;
        Vec4<f16>::store(dq + 32 * t + 8 * jj + 4 * hh, a);
      }
  }
}

// ============================================================================
// fp32 kernels: one thread per query (forward, dQ) or per key (dK, dV)
// ============================================================================
template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(const float* __restrict__ qkv,
                                                         float* __restrict__ o,
                                                         float* __restrict__ lse2,
                                                         const int* __restrict__ valid_len,
                                                         int batch, int seq, int Hl, int causal,
                                                         float sl2) {
  const long idx = (long)blockIdx.x * 64 + threadIdx.x;
  if (idx >= (long)batch * Hl * seq) return;
  const int q = (int)(idx % seq);
  const int head = (int)((idx / seq) % Hl);
  const int b = (int)(idx / ((long)seq * Hl));
  const long ldq = 3L * Hl * D;
  const float* base = qkv + (size_t)b * seq * ldq + (size_t)head * 3 * D;
  const int lim = causal ? q + 1 : min(max(valid_len[b], 0), seq);
  float qv[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = base[(size_t)q * ldq + d];
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int k = 0; k < lim; ++k) {
    const float* kr = base + (size_t)k * ldq + D;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qv[d], kr[d], s);
    s *= sl2;
    const float mn = fmaxf(m, s);
    const float a = exp2f(m - mn), p = exp2f(s - mn);
    l = l * a + p;
    const float* vr = kr + D;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = acc[d] * a + p * vr[d];
    m = mn;
  }
  float* op = o + ((size_t)b * seq + q) * Hl * D + (size_t)head * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = acc[d] * inv;
  lse2[((size_t)b * Hl + head) * seq + q] = m + log2f(l);
}

template <int D>
__global__ __launch_bounds__(64) void attn_bwd_dq_f32_kernel(
    const float* __restrict__ qkv, const float* __restrict__ dO, const float* __restrict__ lse2,
    const float* __restrict__ delta, float* __restrict__ dqkv, const int* __restrict__ valid_len,
    int batch, int seq, int Hl, int causal, float sl2, float scale) {
  const long idx = (long)blockIdx.x * 64 + threadIdx.x;
  if (idx >= (long)batch * Hl * seq) return;
  const int q = (int)(idx % seq);
  const int head = (int)((idx / seq) % Hl);
  const int b = (int)(idx / ((long)seq * Hl));
  const long ldq = 3L * Hl * D, ldo = (long)Hl * D;
  const float* base = qkv + (size_t)b * seq * ldq + (size_t)head * 3 * D;
  const float* g = dO + ((size_t)b * seq + q) * ldo + (size_t)head * D;
  const size_t si = ((size_t)b * Hl + head) * seq + q;
  const float lq = lse2[si], dl = delta[si];
  const int lim = causal ? q + 1 : min(max(valid_len[b], 0), seq);
  float qv[D], gv[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = base[(size_t)q * ldq + d];
    gv[d] = g[d];
    acc[d] = 0.f;
  }
  for (int k = 0; k < lim; ++k) {
    const float* kr = base + (size_t)k * ldq + D;
    const float* vr = kr + D;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      s = fmaf(qv[d], kr[d], s);
      dp = fmaf(gv[d], vr[d], dp);
    }
    const float p = exp2f(s * sl2 - lq);
    const float ds = p * (dp - dl);
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, kr[d], acc[d]);
  }
  float* out = dqkv + ((size_t)b * seq + q) * ldq + (size_t)head * 3 * D;
#pragma unroll
  for (int d = 0; d < D; ++d) out[d] = acc[d] * scale;
}

template <int D>
__global__ __launch_bounds__(64) void attn_bwd_dkdv_f32_kernel(
    const float* __restrict__ qkv, const float* __restrict__ dO, const float* __restrict__ lse2,
    const float* __restrict__ delta, float* __restrict__ dqkv, const int* __restrict__ valid_len,
    int batch, int seq, int Hl, int causal, float sl2, float scale) {
  const long idx = (long)blockIdx.x * 64 + threadIdx.x;
  if (idx >= (long)batch * Hl * seq) return;
  const int k = (int)(idx % seq);
  const int head = (int)((idx / seq) % Hl);
  const int b = (int)(idx / ((long)seq * Hl));
  const long ldq = 3L * Hl * D, ldo = (long)Hl * D;
  const float* base = qkv + (size_t)b * seq * ldq + (size_t)head * 3 * D;
  const float* lsp = lse2 + ((size_t)b * Hl + head) * seq;
  const float* dlp = delta + ((size_t)b * Hl + head) * seq;
  const bool valid = causal ? true : k < min(valid_len[b], seq);
  float kv[D], vv[D], dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    kv[d] = base[(size_t)k * ldq + D + d];
    vv[d] = base[(size_t)k * ldq + 2 * D + d];
    dk[d] = dv[d] = 0.f;
  }
  if (valid) {
    for (int q = causal ? k : 0; q < seq; ++q) {
      const float* qr = base + (size_t)q * ldq;
      const float* g = dO + ((size_t)b * seq + q) * ldo + (size_t)head * D;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s = fmaf(qr[d], kv[d], s);
        dp = fmaf(g[d], vv[d], dp);
      }
      const float p = exp2f(s * sl2 - lsp[q]);
      const float ds = p * (dp - dlp[q]);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        dv[d] = fmaf(p, g[d], dv[d]);
        dk[d] = fmaf(ds, qr[d], dk[d]);
      }
    }
  }
  float* out = dqkv + ((size_t)b * seq + k) * ldq + (size_t)head * 3 * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    out[D + d] = dk[d] * scale;
    out[2 * D + d] = dv[d];
  }
}

// ============================================================================
// Host launchers
// ============================================================================
// Two buffers of two 64-row tiles (three with the score residuals).
template <int D, bool SPLIT>
static size_t fwd_lds() { return (size_t)(SPLIT ? 6 : 4) * 64 * (D + 8) * 2; }
template <int D, bool SPLIT>
static size_t dkdv_lds() { return (size_t)(SPLIT ? 6 : 4) * 64 * (D + 8) * 2 + 4 * 64 * 4; }
template <int D, bool SPLIT>
static size_t dq_lds() { return (size_t)(SPLIT ? 6 : 4) * 64 * (D + 8) * 2; }

template <typename K>
static hipError_t set_lds(K kern, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

template <int D, bool SPLIT>
static hipError_t fwd_f16(const void* qkv, const void* qkv_lo, void* o, float* lse2,
                          const int* vl, int batch, int seq, int Hl, int causal, float sl2,
                          hipStream_t s) {
  auto k = attn_fwd_f16_kernel<D, SPLIT>;
  const size_t lds = fwd_lds<D, SPLIT>();
  hipError_t e = set_lds(k, lds);
  if (e != hipSuccess) return e;
  dim3 grid((seq + 127) / 128, Hl, batch);
  hipLaunchKernelGGL(k, grid, dim3(256), lds, s, (const f16*)qkv,
                     (const f16*)qkv_lo, (f16*)o, lse2, vl, seq, Hl, causal, sl2);
  return hipGetLastError();
}

template <int D, bool SPLIT>
static hipError_t bwd_f16(const void* qkv, const void* qkv_lo, const void* dO, const float* lse2,
                          const float* delta, void* dqkv, const int* vl, int batch, int seq,
                          int Hl, int causal, float sl2, float scale, hipStream_t s) {
  auto k1 = attn_bwd_dkdv_f16_kernel<D, SPLIT>;
  auto k2 = attn_bwd_dq_f16_kernel<D, SPLIT>;
  const size_t lds1 = dkdv_lds<D, SPLIT>(), lds2 = dq_lds<D, SPLIT>();
  hipError_t e = set_lds(k1, lds1);
  if (e == hipSuccess) e = set_lds(k2, lds2);
  if (e != hipSuccess) return e;
  dim3 grid((seq + 127) / 128, Hl, batch);
  hipLaunchKernelGGL(k1, grid, dim3(256), lds1, s, (const f16*)qkv,
                     (const f16*)qkv_lo, (const f16*)dO, lse2, delta, (f16*)dqkv, vl, seq, Hl,
                     causal, sl2, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k2, grid, dim3(256), lds2, s, (const f16*)qkv,
                     (const f16*)qkv_lo, (const f16*)dO, lse2, delta, (f16*)dqkv, vl, seq, Hl,
                     causal, sl2, scale);
  return hipGetLastError();
}

template <int D>
static hipError_t fwd_d(int dtype, const void* qkv, const void* qkv_lo, void* o, float* lse2,
                        const int* vl, int batch, int seq, int Hl, int causal, float sl2,
                        hipStream_t s) {
  if (dtype == DT_F16) {
    if (qkv_lo) return fwd_f16<D, true>(qkv, qkv_lo, o, lse2, vl, batch, seq, Hl, causal, sl2, s);
    return fwd_f16<D, false>(qkv, nullptr, o, lse2, vl, batch, seq, Hl, causal, sl2, s);
  } else {
    const long n = (long)batch * Hl * seq;
    attn_fwd_f32_kernel<D><<<(unsigned)((n + 63) / 64), 64, 0, s>>>(
        (const float*)qkv, (float*)o, lse2, vl, batch, seq, Hl, causal, sl2);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t bwd_d(int dtype, const void* qkv, const void* qkv_lo, const void* dO,
                        const float* lse2, const float* delta, void* dqkv, const int* vl,
                        int batch, int seq, int Hl, int causal, float sl2, float scale,
                        hipStream_t s) {
  if (dtype == DT_F16) {
    if (qkv_lo)
      return bwd_f16<D, true>(qkv, qkv_lo, dO, lse2, delta, dqkv, vl, batch, seq, Hl, causal,
                              sl2, scale, s);
    return bwd_f16<D, false>(qkv, nullptr, dO, lse2, delta, dqkv, vl, batch, seq, Hl, causal,
                             sl2, scale, s);
  } else {
    const long n = (long)batch * Hl * seq;
    const unsigned g = (unsigned)((n + 63) / 64);
    attn_bwd_dkdv_f32_kernel<D><<<g, 64, 0, s>>>((const float*)qkv, (const float*)dO, lse2, delta,
                                                 (float*)dqkv, vl, batch, seq, Hl, causal, sl2,
                                                 scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    attn_bwd_dq_f32_kernel<D><<<g, 64, 0, s>>>((const float*)qkv, (const float*)dO, lse2, delta,
                                               (float*)dqkv, vl, batch, seq, Hl, causal, sl2,
                                               scale);
  }
  return hipGetLastError();
}

hipError_t attn_fwd(int dtype, const void* qkv, const void* qkv_lo, void* o, float* lse2,
                    const int* valid_len, int batch, int seq, int Hl, int D, int mask,
                    hipStream_t s) {
  if (batch == 0 || seq == 0 || Hl == 0) return hipSuccess;
  if (qkv_lo && dtype != DT_F16) return hipErrorInvalidValue;
  const int causal = mask == 0;
  const float sl2 = (float)(1.4426950408889634 / sqrt((double)D));
  switch (D) {
    case 32: return fwd_d<32>(dtype, qkv, qkv_lo, o, lse2, valid_len, batch, seq, Hl, causal, sl2, s);
    case 64: return fwd_d<64>(dtype, qkv, qkv_lo, o, lse2, valid_len, batch, seq, Hl, causal, sl2, s);
    case 96: return fwd_d<96>(dtype, qkv, qkv_lo, o, lse2, valid_len, batch, seq, Hl, causal, sl2, s);
    case 128: return fwd_d<128>(dtype, qkv, qkv_lo, o, lse2, valid_len, batch, seq, Hl, causal, sl2, s);
    case 160: return fwd_d<160>(dtype, qkv, qkv_lo, o, lse2, valid_len, batch, seq, Hl, causal, sl2, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t attn_bwd(int dtype, const void* qkv, const void* qkv_lo, const void* o, const void* dO,
                    const float* lse2, float* delta, void* dqkv, const int* valid_len, int batch,
                    int seq, int Hl, int D, int mask, hipStream_t s) {
  if (batch == 0 || seq == 0 || Hl == 0) return hipSuccess;
  if (qkv_lo && dtype != DT_F16) return hipErrorInvalidValue;
  if (dtype == DT_F16)
    attn_delta_kernel<f16><<<(unsigned)(batch * seq), 64, (size_t)Hl * D / 8 * 4, s>>>(
        (const f16*)o, (const f16*)dO, delta, seq, Hl, D);
  else
    attn_delta_kernel<float><<<(unsigned)(batch * seq), 64, (size_t)Hl * D / 4 * 4, s>>>(
        (const float*)o, (const float*)dO, delta, seq, Hl, D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int causal = mask == 0;
  const double sc = 1.0 / sqrt((double)D);
  const float sl2 = (float)(1.4426950408889634 * sc), scale = (float)sc;
  switch (D) {
    case 32: return bwd_d<32>(dtype, qkv, qkv_lo, dO, lse2, delta, dqkv, valid_len, batch, seq, Hl, causal, sl2, scale, s);
    case 64: return bwd_d<64>(dtype, qkv, qkv_lo, dO, lse2, delta, dqkv, valid_len, batch, seq, Hl, causal, sl2, scale, s);
    case 96: return bwd_d<96>(dtype, qkv, qkv_lo, dO, lse2, delta, dqkv, valid_len, batch, seq, Hl, causal, sl2, scale, s);
    case 128: return bwd_d<128>(dtype, qkv, qkv_lo, dO, lse2, delta, dqkv, valid_len, batch, seq, Hl, causal, sl2, scale, s);
    case 160: return bwd_d<160>(dtype, qkv, qkv_lo, dO, lse2, delta, dqkv, valid_len, batch, seq, Hl, causal, sl2, scale, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpl
