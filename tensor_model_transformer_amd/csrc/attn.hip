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
// Backward (deterministic, no atomics): a small kernel writes delta =
// rowsum(dO * O) per query first. Then one grid holds two kinds of
// workgroups: one owns a block of queries and sweeps the keys (dQ), the other
// owns a block of keys and sweeps the queries (dK, dV). P is recomputed from
// lse2.
//
// fp32 path: one thread per query (forward, dQ) or key (dK, dV) with exact
// fp32 arithmetic.
#include <math.h>

#include <algorithm>

#include "attn_sched.hpp"
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

// ---- 64-row LDS tiles loaded straight from HBM ------------------------------
// A tile holds 64 rows of D fp16 columns, unpadded (pitch D). The 16-byte
// chunk c of row r sits in slot c ^ tsw<D>(r), a swizzle that keeps both the
// row reads (8 columns of 32 rows, ds_read_b128) and the transposing reads
// (4 columns of 4 rows per 16 lanes, ds_read_b64_tr_b16) of the MFMA operands
// on distinct LDS banks. It only permutes chunks within an aligned group of
// 4 (D = 32, 96, 160), 8 (64) or 16 (128), so a row stays a row.
template <int D>
__device__ __forceinline__ int tsw(int r) {
  if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (r >> 2) & 3;
}
template <int D>
constexpr int kSwzMask = D == 64 ? 7 : D == 128 ? 15 : 3;

// Element offset of (row r, column col) in a swizzled tile; the chunk bits
// the swizzle leaves alone are added separately so that unrolled constant
// columns fold into the LDS instruction's immediate offset.
template <int D>
__device__ __forceinline__ int toff(int r, int col) {
  const int c = col >> 3;
  return r * D + 8 * (c & ~kSwzMask<D>) + 8 * ((c & kSwzMask<D>) ^ tsw<D>(r)) + (col & 7);
}

// Columns col .. col+7 (col a multiple of 8) of tile row r.
template <int D>
__device__ __forceinline__ f16x8 ld8s(const f16* T, int r, int col) {
  return ld8(T + toff<D>(r, col));
}

// tr_frag (common.hpp) on a swizzled tile: MFMA operand whose rows are the
// tile's columns m0 .. m0+31 and whose 8 reduction slots are tile rows
// kA + 0..3 then kB + 0..3.
template <int D>
__device__ __forceinline__ f16x8 tr_frag_s(const f16* T, int m0, int kA, int kB, int lane) {
  const int g = lane >> 4, L = lane & 15;
  const int col = m0 + 16 * (g & 1) + 4 * (L & 3);
  const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TPL_LDS_V4S(T + toff<D>(kA + (L >> 2), col)));
  const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(TPL_LDS_V4S(T + toff<D>(kB + (L >> 2), col)));
  const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  return __builtin_bit_cast(f16x8, make_uint4(ua.x, ua.y, ub.x, ub.y));
}

// Issues this wave's share, D/32 loads of 16 bytes per lane, of the tile whose
// row i is src[(r0 + i) * ld + 0 .. D-1]; the four waves of the workgroup
// together load the whole tile. Rows at or past `rows` (r0 < rows) read as
// zero: the buffer descriptor ends at the last valid row's last column.
// wid is the wave index 0..3 (wave-uniform); ld * 128 < 2^31.
template <int D>
__device__ __forceinline__ void tile_dtl(const f16* src, long ld, int r0, int rows, f16* tile,
                                         int wid, int lane) {
  constexpr int CPR = D / 8;  // chunks per row; the tile is CPR loads of 64 chunks
  static_assert(CPR % 4 == 0, "tile loads split evenly over four waves");
  const int nr = min(rows - r0, 64);
  const __amdgpu_buffer_rsrc_t rs =
      buffer_rsrc(src + (size_t)r0 * ld, (int)(((nr - 1) * ld + D) * 2));
  dma_guard();
#pragma unroll
  for (int t = 0; t < CPR / 4; ++t) {
    const int q = wid + 4 * t;
    const int p = 64 * q + lane;
    const int row = p / CPR, c = (p % CPR) ^ tsw<D>(row);
    dma16(rs, tile + 8 * 64 * q, (row * (int)ld + 8 * c) * 2);
  }
}

// One load per wave: 64 fp32 values src[r0 .. r0+63] into dst; entries at or
// past `rows` (r0 < rows) read as zero.
__device__ __forceinline__ void row_f32_dtl(const float* src, int r0, int rows, float* dst,
                                            int lane) {
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src + r0, min(rows - r0, 64) * 4);
  dma_guard();
  dma4(rs, dst, lane * 4);
}

// x and the value of lane l ^ 32, as the two outputs of v_permlane32_swap
// (gfx950: lanes 32-63 of the first operand trade places with lanes 0-31 of
// the second). Both operands hold x; the second is an opaque copy so that
// the compiler cannot treat the swap of one value with itself as a no-op.
// max(a, b) or a + b of the pair combines each lane with its partner in the
// other half without an LDS round trip.
__device__ __forceinline__ void pair32(float x, float* a, float* b) {
  unsigned y;
  asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(__builtin_bit_cast(unsigned, x)));
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), y, false, false);
  *a = __builtin_bit_cast(float, (unsigned)r[0]);
  *b = __builtin_bit_cast(float, (unsigned)r[1]);
}

// Workgroup coordinates (block along the sequence, head, sequence, role) of
// this workgroup in the rank-ordered job lists of attn_sched.hpp.
struct AttnWG {
  int blk, head, b, role;
};
__device__ __forceinline__ AttnWG attn_wg(int nblk, int Hl, int batch, int nroles, bool rev0,
                                          bool rev1) {
  const AttnJob jb = attn_job((int)blockIdx.x, nblk, Hl * batch, nroles, rev0, rev1);
  return AttnWG{jb.blk, jb.pair % Hl, jb.pair / Hl, jb.role};
}

// LDS stages: three when three stages of the workgroups that share a compute
// unit (one per wave per SIMD) fit its 160 KB, else two.
constexpr int attn_stages(int stage_bytes, int waves) {
  return 3 * stage_bytes * waves <= 160 * 1024 ? 3 : 2;
}

// Waves per SIMD requested from the compiler where the registers fit without
// spilling, else no constraint.
template <int D, bool SPLIT>
constexpr int kFwdWaves = (D <= 96 && !SPLIT) ? 3 : 1;
template <int D, bool SPLIT>
constexpr int kDqWaves = (D <= 96 && !SPLIT) ? 2 : 1;
template <int D, bool SPLIT>
constexpr int kDkdvWaves = (D <= 96 && !SPLIT) ? 2 : 1;

// Stage counts. The forward takes three where they fit (without a wave
// hint two workgroups per compute unit are assumed); the backward kernels
// measured faster with two than with three at head dim 96.
template <int D, bool SPLIT>
constexpr int kKvStageBytes = (SPLIT ? 3 : 2) * 64 * D * 2;  // K, V (, K residual)
template <int D, bool SPLIT>
constexpr int kQgStageBytes = (SPLIT ? 3 : 2) * 64 * D * 2 + 2 * 64 * 4;  // Q, dO (, Q res.), lse2, delta
template <int D, bool SPLIT>
constexpr int kFwdStages =
    attn_stages(kKvStageBytes<D, SPLIT>, kFwdWaves<D, SPLIT> > 1 ? kFwdWaves<D, SPLIT> : 2);
template <int D, bool SPLIT>
constexpr int kDqStages = 2;
template <int D, bool SPLIT>
constexpr int kDkdvStages = 2;

// ============================================================================
// fp16 forward
// ============================================================================
// A workgroup owns 128 queries (32 per wave) of one (sequence, head) and
// sweeps 64-key blocks; the K and V tiles of the next blocks load straight
// from HBM into LDS stages while the current block's MFMAs run.
template <int D, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kFwdWaves<D, SPLIT>))) void attn_fwd_f16_kernel(
    const f16* __restrict__ qkv, const f16* __restrict__ qkv_lo, f16* __restrict__ o,
    float* __restrict__ lse2, const int* __restrict__ valid_len, int batch, int seq, int Hl,
    int causal, float sl2) {
  constexpr int KB = 64, TILE = KB * D, NT = SPLIT ? 3 : 2;
  extern __shared__ __align__(16) unsigned char smem[];
  f16* lds = reinterpret_cast<f16*>(smem);  // [stages][K tile, V tile (, K residual tile)]

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const AttnWG wg = attn_wg((seq + 127) / 128, Hl, batch, 1, causal, false);
  if (wg.blk < 0) return;
  const int qb = wg.blk, head = wg.head, b = wg.b;
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
  auto load_regs = [&]() {
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
  };
  f32x16 O[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) O[t][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int nblk = (kv_end + KB - 1) / KB;
  auto issue = [&](int blk, int stg) {
    f16* base = lds + stg * NT * TILE;
    tile_dtl<D>(Kp, ldq, blk * KB, seq, base, w, lane);
    tile_dtl<D>(Vp, ldq, blk * KB, seq, base + TILE, w, lane);
    if constexpr (SPLIT) tile_dtl<D>(Klp, ldq, blk * KB, seq, base + 2 * TILE, w, lane);
  };
  auto compute = [&](int ib, int stg) {
    const int kb0 = ib * KB;
    const f16* Ks = lds + stg * NT * TILE;
    const f16* Vs = Ks + TILE;
    const f16* Kls = Ks + 2 * TILE;  // residual tile (SPLIT only)
    if (!(causal && kb0 > qw0 + 31)) {  // some key of this block precedes a query of this wave
      f32x16 S[2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) S[st][e] = 0.f;
      // With several waves per SIMD (head dim <= 96 without split scores)
      // each step's K fragments are read one step ahead and the two 32-key
      // halves alternate (1.2B shard: 48.9 -> 45.9 us); with one wave per SIMD
      // the register budget is better spent as the compiler schedules the
      // plain loop (that reordering measured 1.3 % slower at head dim 160).
      constexpr bool kPipe = kFwdWaves<D, SPLIT> > 1;
      f16x8 vf[2][D / 32];  // V^T fragments of a 16-key slice (kPipe)
      if constexpr (kPipe) {
        static_assert(!SPLIT, "several waves per SIMD only without split scores");
        f16x8 kh[2][2];  // [buffer][half]
#pragma unroll
        for (int st = 0; st < 2; ++st) kh[0][st] = ld8s<D>(Ks, 32 * st + l32, 8 * hh);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const int cur = ks & 1, nxt = cur ^ 1;
          if (ks + 1 < D / 16) {
#pragma unroll
            for (int st = 0; st < 2; ++st)
              kh[nxt][st] = ld8s<D>(Ks, 32 * st + l32, 16 * (ks + 1) + 8 * hh);
          }
#pragma unroll
          for (int st = 0; st < 2; ++st) S[st] = mfma32(kh[cur][st], qf[ks], S[st]);
        }
        // the first 16 keys' V^T fragments, read while the softmax runs
#pragma unroll
        for (int t = 0; t < D / 32; ++t) vf[0][t] = tr_frag_s<D>(Vs, 32 * t, 4 * hh, 8 + 4 * hh, lane);
      } else {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            const int r = 32 * st + l32, col = 16 * ks + 8 * hh;
            const f16x8 kh = ld8s<D>(Ks, r, col);
            S[st] = mfma32(kh, qf[ks], S[st]);
            if constexpr (SPLIT) {
              S[st] = mfma32(ld8s<D>(Kls, r, col), qf[ks], S[st]);
              S[st] = mfma32(kh, ql[ks], S[st]);
            }
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
      {
        float a, b;
        pair32(mx, &a, &b);
        mx = fmaxf(a, b);
      }
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
      {
        float a, b;
        pair32(ls, &a, &b);
        ls = a + b;
      }
      l_run += ls;
      // O^T[d][q] += sum_key V[key][d] P[q][key]; 16 keys per MFMA, slot order
      // {4h..4h+3, 8+4h..8+4h+3} within the 16 (the accumulator's row order)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f16x8 pf = pack8v(S[c >> 1], 8 * (c & 1));
        if constexpr (kPipe) {
          const int cur = c & 1, nxt = cur ^ 1;
          if (c + 1 < 4) {  // the next 16 keys' fragments ahead of this slice's MFMAs
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
              vf[nxt][t] = tr_frag_s<D>(Vs, 32 * t, 16 * (c + 1) + 4 * hh,
                                        16 * (c + 1) + 8 + 4 * hh, lane);
          }
#pragma unroll
          for (int t = 0; t < D / 32; ++t) O[t] = mfma32(vf[cur][t], pf, O[t]);
        } else {
#pragma unroll
          for (int t = 0; t < D / 32; ++t)
            O[t] = mfma32(tr_frag_s<D>(Vs, 32 * t, 16 * c + 4 * hh, 16 * c + 8 + 4 * hh, lane),
                          pf, O[t]);
        }
      }
    }
  };
  dtl_prologue<kFwdStages<D, SPLIT>>(nblk, issue);
  load_regs();
  wait_vm<0>();
  dtl_loop<kFwdStages<D, SPLIT>, NT * D / 32>(nblk, issue, compute);

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
// Sweeps 64-query blocks (two 32-query halves per MFMA step); the Q and dO
// tiles (with the blocks' lse2 and delta) of the next blocks load straight
// from HBM into LDS stages. Q^T and dO^T operands are read from the row-major
// tiles with transposing LDS reads.
template <int D, bool SPLIT>
__device__ __forceinline__ void attn_bwd_dkdv_f16(
    const f16* __restrict__ qkv, const f16* __restrict__ qkv_lo, const f16* __restrict__ dO,
    const float* __restrict__ lse2, const float* __restrict__ delta, f16* __restrict__ dqkv,
    const int* __restrict__ valid_len, int seq, int Hl, int causal, float sl2, float scale,
    const AttnWG wg, unsigned char* smem) {
  constexpr int QB = 64, TILE = QB * D, NT = SPLIT ? 3 : 2;
  constexpr int SE = kQgStageBytes<D, SPLIT> / 2;  // stage size in f16 elements
  // [stages][Q tile, dO tile (, Q residual tile), lse2[QB], delta[QB] (fp32)]
  f16* lds = reinterpret_cast<f16*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int kblk = wg.blk, head = wg.head, b = wg.b;
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
  auto load_regs = [&]() {
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
  };
  f32x16 dK[D / 32], dV[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) dK[t][e] = dV[t][e] = 0.f;

  const bool wave_keys_valid = kw0 < (causal ? seq : L);
  const int q_begin = causal ? kblk * 128 : 0;
  const int nblk = (seq - q_begin + QB - 1) / QB;
  // every wave issues the same loads per block: its share of each tile and
  // one 64-entry row, lse2 (even waves) or delta (odd waves)
  auto issue = [&](int blk, int stg) {
    const int q0 = q_begin + blk * QB;
    f16* base = lds + stg * SE;
    tile_dtl<D>(Qp, ldq, q0, seq, base, w, lane);
    tile_dtl<D>(dOp, ldo, q0, seq, base + TILE, w, lane);
    if constexpr (SPLIT) tile_dtl<D>(Qlp, ldq, q0, seq, base + 2 * TILE, w, lane);
    float* rows = reinterpret_cast<float*>(base + NT * TILE);
    row_f32_dtl((w & 1) ? dlp : lsp, q0, seq, rows + (w & 1) * QB, lane);
  };
  auto compute = [&](int ib, int stg) {
    const int q0 = q_begin + ib * QB;
    const f16* Qs = lds + stg * SE;
    const f16* Gs = Qs + TILE;
    const f16* Qls = Qs + 2 * TILE;  // residual tile (SPLIT only)
    const float* lsb = reinterpret_cast<const float*>(Qs + NT * TILE);
    const float* dlb = lsb + QB;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int qh0 = q0 + 32 * qs;  // first query of this half
      if (!wave_keys_valid || (causal && qh0 + 31 < kw0)) continue;
      f32x16 S, dP;
#pragma unroll
      for (int e = 0; e < 16; ++e) S[e] = dP[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int r = 32 * qs + l32, col = 16 * ks + 8 * hh;
        const f16x8 qh = ld8s<D>(Qs, r, col);
        S = mfma32(qh, kf[ks], S);
        if constexpr (SPLIT) {
          S = mfma32(ld8s<D>(Qls, r, col), kf[ks], S);
          S = mfma32(qh, kl[ks], S);
        }
        dP = mfma32(ld8s<D>(Gs, r, col), vf[ks], dP);
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
          dV[t] = mfma32(tr_frag_s<D>(Gs, 32 * t, kA, kB, lane), pf, dV[t]);
          dK[t] = mfma32(tr_frag_s<D>(Qs, 32 * t, kA, kB, lane), sf, dK[t]);
        }
      }
    }
  };
  dtl_prologue<kDkdvStages<D, SPLIT>>(nblk, issue);
  load_regs();
  wait_vm<0>();
  dtl_loop<kDkdvStages<D, SPLIT>, NT * D / 32 + 1>(nblk, issue, compute);

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
__device__ __forceinline__ void attn_bwd_dq_f16(
    const f16* __restrict__ qkv, const f16* __restrict__ qkv_lo, const f16* __restrict__ dO,
    const float* __restrict__ lse2, const float* __restrict__ delta, f16* __restrict__ dqkv,
    const int* __restrict__ valid_len, int seq, int Hl, int causal, float sl2, float scale,
    const AttnWG wg, unsigned char* smem) {
  constexpr int KB = 64, TILE = KB * D, NT = SPLIT ? 3 : 2;
  f16* lds = reinterpret_cast<f16*>(smem);  // [stages][K tile, V tile (, K residual tile)]

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int qb = wg.blk, head = wg.head, b = wg.b;
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
  float lq, dq_;
  const f16* Qlp = SPLIT ? qkv_lo + tok0 * ldq + (size_t)head * 3 * D : nullptr;
  const f16* Klp = SPLIT ? Qlp + D : nullptr;

  f16x8 qf[D / 16], gf[D / 16], ql[SPLIT ? D / 16 : 1];
  auto load_regs = [&]() {
  lq = qok ? lse2[((size_t)b * Hl + head) * seq + q] : 0.f;
  dq_ = qok ? delta[((size_t)b * Hl + head) * seq + q] : 0.f;
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
  };
  f32x16 dQ[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) dQ[t][e] = 0.f;

  const int nblk = (kv_end + KB - 1) / KB;
  auto issue = [&](int blk, int stg) {
    f16* base = lds + stg * NT * TILE;
    tile_dtl<D>(Kp, ldq, blk * KB, seq, base, w, lane);
    tile_dtl<D>(Vp, ldq, blk * KB, seq, base + TILE, w, lane);
    if constexpr (SPLIT) tile_dtl<D>(Klp, ldq, blk * KB, seq, base + 2 * TILE, w, lane);
  };
  auto compute = [&](int ib, int stg) {
    const int kb0 = ib * KB;
    const f16* Ks = lds + stg * NT * TILE;
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
          const int r = 32 * st + l32, col = 16 * ks + 8 * hh;
          const f16x8 kh = ld8s<D>(Ks, r, col);
          S = mfma32(kh, qf[ks], S);
          if constexpr (SPLIT) {
            S = mfma32(ld8s<D>(Kls, r, col), qf[ks], S);
            S = mfma32(kh, ql[ks], S);
          }
          dP = mfma32(ld8s<D>(Vs, r, col), gf[ks], dP);
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
          dQ[t] = mfma32(tr_frag_s<D>(Ks, 32 * t, 16 * c + 4 * hh, 16 * c + 8 + 4 * hh, lane), sf,
                         dQ[t]);
      }
    }
  };
  dtl_prologue<kDqStages<D, SPLIT>>(nblk, issue);
  load_regs();
  wait_vm<0>();
  dtl_loop<kDqStages<D, SPLIT>, NT * D / 32>(nblk, issue, compute);

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
// fp16 backward: one launch of both roles
// ============================================================================
// Workgroups of the dQ role and of the dK/dV role share one grid, in rank
// order per XCD (attn_sched.hpp): under the causal mask a 128-row block's work grows
// from 1 to nblk units along the sequence, and with one workgroup per compute
// unit (head dim 160) two separate launches each end on their longest blocks
// while most compute units idle; in one list the short blocks of either role
// fill in behind the long ones (1T shard: 20 heads x 16 blocks per role).
// delta = rowsum(dO * O) comes from attn_delta_kernel, launched before.
template <int D, bool SPLIT>
constexpr int kBwdWaves = kDqWaves<D, SPLIT> < kDkdvWaves<D, SPLIT> ? kDqWaves<D, SPLIT>
                                                                     : kDkdvWaves<D, SPLIT>;
template <int D, bool SPLIT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kBwdWaves<D, SPLIT>))) void attn_bwd_f16_kernel(
    const f16* __restrict__ qkv, const f16* __restrict__ qkv_lo, const f16* __restrict__ dO,
    const float* __restrict__ lse2, const float* __restrict__ delta, f16* __restrict__ dqkv,
    const int* __restrict__ valid_len, int batch, int seq, int Hl, int causal, float sl2,
    float scale) {
  extern __shared__ __align__(16) unsigned char smem[];
  const AttnWG wg = attn_wg((seq + 127) / 128, Hl, batch, 2, causal, false);
  if (wg.blk < 0) return;
  if (wg.role == 0)
    attn_bwd_dq_f16<D, SPLIT>(qkv, qkv_lo, dO, lse2, delta, dqkv, valid_len, seq, Hl, causal, sl2,
                              scale, wg, smem);
  else
    attn_bwd_dkdv_f16<D, SPLIT>(qkv, qkv_lo, dO, lse2, delta, dqkv, valid_len, seq, Hl, causal,
                                sl2, scale, wg, smem);
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
// Dynamic LDS: the kernels' stages of 64-row tiles.
template <int D, bool SPLIT>
static size_t fwd_lds() { return (size_t)kFwdStages<D, SPLIT> * kKvStageBytes<D, SPLIT>; }
template <int D, bool SPLIT>
static size_t dkdv_lds() { return (size_t)kDkdvStages<D, SPLIT> * kQgStageBytes<D, SPLIT>; }
template <int D, bool SPLIT>
static size_t dq_lds() { return (size_t)kDqStages<D, SPLIT> * kKvStageBytes<D, SPLIT>; }

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
  dim3 grid((unsigned)((seq + 127) / 128 * Hl * batch));
  hipLaunchKernelGGL(k, grid, dim3(256), lds, s, (const f16*)qkv,
                     (const f16*)qkv_lo, (f16*)o, lse2, vl, batch, seq, Hl, causal, sl2);
  return hipGetLastError();
}

// delta first (its own kernel), then both roles in one grid.
template <int D, bool SPLIT>
static hipError_t bwd_f16(const void* qkv, const void* qkv_lo, const void* dO, const float* lse2,
                          const float* delta, void* dqkv, const int* vl, int batch, int seq,
                          int Hl, int causal, float sl2, float scale, hipStream_t s) {
  auto k = attn_bwd_f16_kernel<D, SPLIT>;
  const size_t lds = std::max(dkdv_lds<D, SPLIT>(), dq_lds<D, SPLIT>());
  hipError_t e = set_lds(k, lds);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)(2 * ((seq + 127) / 128) * Hl * batch));
  hipLaunchKernelGGL(k, grid, dim3(256), lds, s, (const f16*)qkv, (const f16*)qkv_lo,
                     (const f16*)dO, lse2, delta, (f16*)dqkv, vl, batch, seq, Hl, causal, sl2,
                     scale);
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
static hipError_t bwd_d(int dtype, const void* qkv, const void* qkv_lo, const void* o,
                        const void* dO, const float* lse2, float* delta, void* dqkv,
                        const int* vl, int batch, int seq, int Hl, int causal, float sl2,
                        float scale, hipStream_t s) {
  if (dtype == DT_F16) {
    if (qkv_lo)
      return bwd_f16<D, true>(qkv, qkv_lo, dO, lse2, delta, dqkv, vl, batch, seq, Hl, causal, sl2,
                              scale, s);
    return bwd_f16<D, false>(qkv, nullptr, dO, lse2, delta, dqkv, vl, batch, seq, Hl, causal, sl2,
                             scale, s);
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
  // direct tile loads address 64 rows of the qkv row stride in 31 bits
  if (3L * Hl * D * 128 >= (1L << 31)) return hipErrorInvalidValue;
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
  if (3L * Hl * D * 128 >= (1L << 31)) return hipErrorInvalidValue;
  // delta = rowsum(dO * O) per (token, head), read by the dQ and dK/dV kernels
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
    case 32: return bwd_d<32>(dtype, qkv, qkv_lo, o, dO, lse2, delta, dqkv, valid_len, batch, seq, Hl, causal, sl2, scale, s);
    case 64: return bwd_d<64>(dtype, qkv, qkv_lo, o, dO, lse2, delta, dqkv, valid_len, batch, seq, Hl, causal, sl2, scale, s);
    case 96: return bwd_d<96>(dtype, qkv, qkv_lo, o, dO, lse2, delta, dqkv, valid_len, batch, seq, Hl, causal, sl2, scale, s);
    case 128: return bwd_d<128>(dtype, qkv, qkv_lo, o, dO, lse2, delta, dqkv, valid_len, batch, seq, Hl, causal, sl2, scale, s);
    case 160: return bwd_d<160>(dtype, qkv, qkv_lo, o, dO, lse2, delta, dqkv, valid_len, batch, seq, Hl, causal, sl2, scale, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tpl
