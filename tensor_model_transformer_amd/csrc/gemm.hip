// GEMMs of the layer shard: C[M,N] = A[M,K] @ B[K,N] with fused epilogues.
//
// The four projections of "Megatron-LM: GPU-Cluster Training Parallelism",
// section "Paper 1: The f/g Conjugate Operators" (column-parallel QKV and FC1,
// row-parallel output projection and FC2) and their data/weight gradients.
// Epilogue fusions follow section "Fused Transformer Kernels": bias + GeLU
// after FC1, bias + residual after the row-parallel GEMMs; backward adds the
// GeLU derivative to the FC2 data-gradient epilogue.
//
// 16-bit path: MFMA 32x32x16 on fp16 operands (v_mfma_f32_32x32x16_f16,
// fp32 accumulate; the same rate as bf16 on gfx950) on LDS double-buffered
// tiles. Both operands are fp16 in memory: internal activations are fp16, and
// the caller hands in fp16 copies of the bf16 tensors at the layer boundary
// (weights, the upstream gradient), made once per step. An operand tile keeps
// its HBM orientation in LDS: K-contiguous operands as rows of BK, operands
// that are contiguous along M or N (weights [in,out] in forward; both operands
// of a weight gradient) as k-lines of the tile's rows, whose MFMA fragments
// come from ds_read_b64_tr_b16, gfx950's transposing LDS read, so nothing is
// transposed in registers. The MFMA is issued with B as the first operand, so
// the accumulator holds C transposed: each lane owns one output row and 4
// consecutive columns per 32x32 tile, which the epilogue writes as one vector.
//
// When K is a whole number of K steps (every GEMM of the layer's shards), the
// operand tiles are loaded from HBM straight into LDS (buffer_load_dword*4
// ... lds): no staging registers and no LDS store instructions. Those loads
// write 64 consecutive 16-byte chunks per instruction, so the tiles are
// unpadded and their 16-byte chunks XOR-swizzled to keep the fragment reads
// free of bank conflicts. Other K take a register-staged kernel with padded
// tiles and bounds checks.
//
// fp32 path: a plain tiled FMA kernel (exact fp32 arithmetic).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace tpl {

// ----------------------------------------------------------------------------
// Epilogue on 4 consecutive columns n..n+3 of row m (N % 4 == 0).
// ----------------------------------------------------------------------------
// bias4, when given, holds bias[n .. n+3], already loaded; sc is *g.scale
// (1 without one), loaded once by the caller.
__device__ __forceinline__ void epilogue4(const GemmArgs& g, int m, int n, float v[4],
                                          const float* bias4, float sc) {
  if (m >= g.M || n >= g.N) return;
  if (g.scale) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= sc;
  }
  if (g.bias) {
    float b[4];
    if (bias4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) b[e] = bias4[e];
    } else {
      load4_dt(g.bias, g.bias_dtype, n, b);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += b[e];
  }
  if (g.resid) {
    float r[4];
    load4_dt(g.resid, g.resid_dtype, (size_t)m * g.ldr + n, r);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += r[e];
  }
  if (g.epi == EPI_BIAS_GELU) {
    // z = GeLU(v) to C2; C (if given) keeps GeLU'(v) for the backward
    float z[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) gelu_and_grad(v[e], g.gelu_tanh, &z[e], &v[e]);
    store4_dt(g.C2, g.c2_dtype, (size_t)m * g.ldc2 + n, z);
  } else if (g.epi == EPI_GELU_GRAD) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = gelu_grad_f(v[e], g.gelu_tanh);
  } else if (g.epi == EPI_DGELU) {
    float gp[4];
    load4_dt(g.aux, g.aux_dtype, (size_t)m * g.ldaux + n, gp);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= gp[e];
  } else if (g.epi == EPI_SPLIT16) {
    // hi = fp16(v) goes to C below (exactly representable, so stored as is);
    // lo = v - hi is exact in fp32 and rounded once more to fp16 in C2.
    float lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float hi = (float)(f16)v[e];
      lo[e] = v[e] - hi;
      v[e] = hi;
    }
    store4_dt(g.C2, DT_F16, (size_t)m * g.ldc2 + n, lo);
  }
  if (!g.C) return;  // only C2 wanted (the FC1 pre-activation is not kept)
  const size_t off = (size_t)m * g.ldc + n;
  if (g.accumulate && g.c_dtype == DT_F32) {
    float o[4];
    Vec4<float>::load((const float*)g.C + off, o);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += o[e];
  }
  if (g.stream_out && g.c_dtype == DT_F32) store4_f32_nt((float*)g.C + off, v);
  else store4_dt(g.C, g.c_dtype, off, v);
}

// Output tile of this workgroup. Workgroups are dealt to the 8 XCDs round
// robin (workgroup w runs on XCD w % 8), and each XCD has its own L2. The
// linear tile order is therefore regrouped so that XCD x receives the
// contiguous range [x*T/8, (x+1)*T/8) of a grouped order (bands of kGroupM
// tile rows, column by column inside a band): the tiles resident on one XCD
// at a time form a compact block that shares A row panels and B column
// panels in that XCD's L2.
constexpr int kXCDs = 8, kGroupM = 8;
__device__ __forceinline__ void tile_coords(int M, int N, int BM, int BN, int* tm, int* tn) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int total = tiles_m * tiles_n;
  int t = blockIdx.x;
  if (total % kXCDs == 0) t = (t % kXCDs) * (total / kXCDs) + t / kXCDs;
  const int band = kGroupM * tiles_n;
  const int b = t / band, r = t % band;
  const int rows = min(kGroupM, tiles_m - b * kGroupM);  // rows in this (maybe short) band
  *tm = b * kGroupM + r % rows;
  *tn = r / rows;
}

// Split-K partial (raw accumulator) store.
__device__ __forceinline__ void partial4(const GemmArgs& g, int split_idx, int m, int n,
                                         const float v[4]) {
  if (m >= g.M || n >= g.N) return;
  Vec4<float>::store(g.ws + ((size_t)split_idx * g.M + m) * g.N + n, v);
}

// ----------------------------------------------------------------------------
// fp16 MFMA GEMM
// ----------------------------------------------------------------------------
// LDS pitch (16-bit elements) of an operand tile: K-contiguous tiles are
// [ROWS][BK + 8] (16-byte MFMA fragment reads); row-contiguous tiles are
// [BK][ROWS + 32], read with ds_read_b64_tr_b16. Each half wave of such a
// read covers 4 tile rows x 64 bytes; the +32 pad (64 bytes) makes the row
// pitch 16 or 48 dwords modulo the 64 LDS banks, so the 4 rows fall on
// disjoint banks.
template <int ROWS, int BK, bool KMAJ>
struct TilePitch {
  static constexpr int P = KMAJ ? BK + 8 : ROWS + 32;
  static constexpr int kElems = KMAJ ? ROWS * (BK + 8) : BK * (ROWS + 32);
};

template <int ROWS, int BK, int NT, bool KMAJ>
struct TileLoader {
  // 16-byte chunks of 8 elements along the contiguous dimension:
  // K-contiguous source: chunk (row, 8 k); row-contiguous source: (k, 8 rows).
  static constexpr int kChunks = ROWS * BK / 8;
  static constexpr int kPer = (kChunks + NT - 1) / NT;
  static constexpr int kPerRow = KMAJ ? BK / 8 : ROWS / 8;  // chunks per contiguous line
  uint4 st[kPer];

  // src(row, k) = KMAJ ? p[row*ld + k] : p[k*ld + row]; 16-bit elements;
  // chunks outside the matrix read as zero. The loaded registers are consumed
  // only by store(), after the MFMAs of the current tile, so the global-load
  // latency overlaps the compute.
  __device__ __forceinline__ void load(const uint16_t* __restrict__ p, long ld, int row0, int nrows,
                                       int k0, int K, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * NT;
      const int line = c / kPerRow, w = c % kPerRow;
      // KMAJ: line = row, w = k chunk; else line = k, w = row chunk
      const int gr = KMAJ ? row0 + line : row0 + 8 * w;
      const int gk = KMAJ ? k0 + 8 * w : k0 + line;
      uint4 v = make_uint4(0, 0, 0, 0);
      if ((kChunks % NT == 0 || c < kChunks) && gr < nrows && gk < K)
        v = *reinterpret_cast<const uint4*>(
            p + (KMAJ ? (size_t)gr * ld + gk : (size_t)gk * ld + gr));
      st[i] = v;
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) {
    constexpr int P = TilePitch<ROWS, BK, KMAJ>::P;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * NT;
      if (kChunks % NT == 0 || c < kChunks)
        *reinterpret_cast<uint4*>(lds + (c / kPerRow) * P + 8 * (c % kPerRow)) = st[i];
    }
  }
};

// MFMA operand fragment of rows r0 .. r0+31 of an operand tile for K step
// ks (16 k), this lane's row r0 + lane%32 and k = 16 ks + 8 (lane/32) + 0..7.
template <int ROWS, int BK, bool KMAJ>
__device__ __forceinline__ f16x8 frag(const uint16_t* tile, int r0, int ks, int lane) {
  constexpr int P = TilePitch<ROWS, BK, KMAJ>::P;
  const int kA = 16 * ks + 8 * (lane >> 5);
  if constexpr (KMAJ) {
    return *reinterpret_cast<const f16x8*>(tile + (r0 + (lane & 31)) * P + kA);
  } else {
    return tr_frag(reinterpret_cast<const f16*>(tile), P, r0, kA, kA + 4, lane);
  }
}

// K not a multiple of the K step: register-staged loads with bounds checks
// into padded tiles.
template <int BM, int BN, int BK, int WM, int WN, bool AK, bool BKM>
__global__ __launch_bounds__(WM * WN * 64) void gemm_f16_kernel(GemmArgs g, int ktiles_per_split) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int AE = TilePitch<BM, BK, AK>::kElems, BE = TilePitch<BN, BK, BKM>::kElems;
  static_assert(TM >= 1 && TN >= 1 && BK % 16 == 0, "tile shape");

  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);       // [2][AE] fp16
  uint16_t* Bs = As + 2 * AE;                             // [2][BE] fp16

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / WN, wn = wid % WN;
  int tm, tn;
  tile_coords(g.M, g.N, BM, BN, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int split_idx = blockIdx.y;
  const int ktiles = (g.K + BK - 1) / BK;
  const int kt0 = split_idx * ktiles_per_split;
  const int kt1 = min(ktiles, kt0 + ktiles_per_split);

  const uint16_t* A = (const uint16_t*)g.A;
  const uint16_t* B = (const uint16_t*)g.B;
  TileLoader<BM, BK, NT, AK> la;
  TileLoader<BN, BK, NT, BKM> lb;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  if (kt0 < kt1) {
    la.load(A, g.lda, m0, g.M, kt0 * BK, g.K, tid);
    lb.load(B, g.ldb, n0, g.N, kt0 * BK, g.K, tid);
    la.store(As, tid);
    lb.store(Bs, tid);
    __syncthreads();
  }
  const int lrow = lane & 31;
  for (int kt = kt0; kt < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) {
      la.load(A, g.lda, m0, g.M, (kt + 1) * BK, g.K, tid);
      lb.load(B, g.ldb, n0, g.N, (kt + 1) * BK, g.K, tid);
    }
    const uint16_t* as = As + cur * AE;
    const uint16_t* bs = Bs + cur * BE;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      f16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = frag<BM, BK, AK>(as, wm * WTM + 32 * i, ks, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = frag<BN, BK, BKM>(bs, wn * WTN + 32 * j, ks, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      la.store(As + (cur ^ 1) * AE, tid);
      lb.store(Bs + (cur ^ 1) * BE, tid);
    }
    __syncthreads();
  }

  // Epilogue through LDS, one 32-row slice of the wave's tile at a time.
  // acc[i][j][4*jj + e] = C[m][n] with m = this lane's row and n = 8*jj +
  // 4*(lane/32) + e, i.e. each lane holds a column strip of one row. The
  // wave writes its slice to a private LDS region and then walks it row by
  // row, 4 consecutive columns per lane, so every output row segment is
  // written by adjacent lanes (coalesced) and acc is only ever indexed by
  // constants.
  constexpr int CP = WTN + 4;  // fp32 pitch of a slice row
  static_assert(2 * (AE + BE) * 2 >= WM * WN * 32 * CP * 4, "epilogue slices fit in LDS");
  float* cs = reinterpret_cast<float*>(smem) + wid * 32 * CP;
  const int half = lane >> 5;
  const float sc = g.scale ? g.scale[0] : 1.f;
  __syncthreads();  // every wave is done with the operand tiles
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<float4*>(cs + lrow * CP + j * 32 + 8 * jj + 4 * half) =
            make_float4(acc[i][j][4 * jj], acc[i][j][4 * jj + 1], acc[i][j][4 * jj + 2],
                        acc[i][j][4 * jj + 3]);
    constexpr int LPR = WTN / 4;  // lanes per slice row
#pragma unroll 1
    for (int r = lane / LPR; r < 32; r += 64 / LPR) {
      const int c = 4 * (lane % LPR);
      const float4 q = *reinterpret_cast<const float4*>(cs + r * CP + c);
      float v[4] = {q.x, q.y, q.z, q.w};
      const int m = m0 + wm * WTM + i * 32 + r, n = n0 + wn * WTN + c;
      if (gridDim.y > 1) partial4(g, split_idx, m, n, v);
      else epilogue4(g, m, n, v, nullptr, sc);
    }
  }
}

// ----------------------------------------------------------------------------
// HBM -> LDS direct loads, two stages of BK = 64
// ----------------------------------------------------------------------------
// One operand tile of ROWS (M or N) x BK in LDS, filled by direct loads.
//  K-contiguous source: ROWS lines of BK elements; 16-byte chunk position p
//    of line r holds source chunk p ^ ((r >> 1) & 7). A fragment read covers
//    16 consecutive lines at one chunk; line pairs share the 64 banks and the
//    XOR spreads the 8 pairs over distinct 4-bank groups.
//  Row-contiguous source: BK k-lines of ROWS elements; chunk position p of
//    k-line k holds source row chunk p ^ f(k). A half-wave transposing read
//    covers 4 k-lines x 4 chunks: with a line length that is a multiple of
//    256 bytes f(k) = 4 (k & 3); with 384-byte lines (ROWS = 192), which
//    already alternate between bank halves, f(k) = 4 ((k >> 1) & 1).
// Each wave issues kPerWave loads of 64 chunks per stage; when the count does
// not divide evenly, the last loads repeat chunks another wave also loads
// (same data to the same place), so every wave waits for the same count.
template <int ROWS, int BK, int NW, bool KMAJ>
struct DtlOperand {
  static constexpr int kChunks = ROWS * BK / 8;
  static constexpr int kInstr = kChunks / 64;
  static constexpr int kPerWave = (kInstr + NW - 1) / NW;
  static constexpr int kPerLine = KMAJ ? BK / 8 : ROWS / 8;
  static_assert(kChunks % 64 == 0 && kInstr >= NW, "direct-load chunking");
  static_assert(BK == 64, "swizzle written for 8 chunks per K-contiguous line");

  __device__ __forceinline__ static int swz(int line) {
    if constexpr (KMAJ) return (line >> 1) & 7;
    else return (ROWS * 2) % 256 == 0 ? 4 * (line & 3) : 4 * ((line >> 1) & 1);
  }

  // rs covers the whole operand; element (row, k) sits at row * ld + k
  // (K-contiguous) or k * ld + row; byte offsets fit 31 bits (host check).
  __device__ __forceinline__ static void load(__amdgpu_buffer_rsrc_t rs, int ld, int row0, int k0,
                                              uint16_t* stage, int wid, int lane) {
    dma_guard();
#pragma unroll
    for (int t = 0; t < kPerWave; ++t) {
      int q = wid + NW * t;
      if (q >= kInstr) q -= kInstr;
      const int p = 64 * q + lane;
      const int line = p / kPerLine, pos = p % kPerLine;
      const int c = pos ^ swz(line);
      const int off = KMAJ ? ((row0 + line) * ld + k0 + 8 * c) * 2
                           : ((k0 + line) * ld + row0 + 8 * c) * 2;
      dma16(rs, stage + 64 * q * 8, off);
    }
  }

  // MFMA operand of rows r0 .. r0+31 for K step ks (as frag() above).
  __device__ __forceinline__ static f16x8 frag(const uint16_t* st, int r0, int ks, int lane) {
    if constexpr (KMAJ) {
      const int r = r0 + (lane & 31);
      const int kc = 2 * ks + (lane >> 5);
      return *reinterpret_cast<const f16x8*>(st + r * BK + (kc ^ swz(r)) * 8);
    } else {
      const int gq = lane >> 4, L = lane & 15;
      const int row = r0 + 16 * (gq & 1) + 4 * (L & 3);
      const int kb = ks * 16 + 8 * (gq >> 1) + (L >> 2);
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          TPL_LDS_V4S(st + kb * ROWS + ((row >> 3) ^ swz(kb)) * 8 + (row & 7)));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          TPL_LDS_V4S(st + (kb + 4) * ROWS + ((row >> 3) ^ swz(kb + 4)) * 8 + (row & 7)));
      const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
      return __builtin_bit_cast(f16x8, make_uint4(a.x, a.y, b.x, b.y));
    }
  }
};

// LDS stages of the direct-load GEMM: two 64-deep K steps. A third stage of
// the 256-row tiles would need 168 KB (256x192) or 192 KB (256x256), more
// than the 160 KB of a compute unit.
constexpr int kGemmStages = 2;

// Same tiling and epilogue as gemm_f16_kernel, K steps streamed through
// kGemmStages LDS stages (dtl_prologue / dtl_loop): iteration j waits for
// this wave's loads of step j, a barrier publishes them (and ends every
// wave's reads of step j-1), the loads of step j+1 go into step j-1's
// stage, then the MFMAs of step j run.
//
// One call computes K steps [kt0, kt1) of the output tile at (m0, n0) and
// writes either the epilogue's result (pdst == null, no split), a split-K
// partial (split index split_idx, pdst == null, gridDim.y > 1) or the raw
// [BM][BN] accumulator tile to pdst (a stream-K segment). The caller must
// separate two calls on one workgroup with a barrier (the epilogue's LDS
// slices overlap the operand stages).
template <int BM, int BN, int WM, int WN, bool AK, bool BKM>
__device__ __forceinline__ void dtl_tile(const GemmArgs& g, int m0, int n0, int kt0, int kt1,
                                         int split_idx, float* pdst, unsigned char* smem) {
  constexpr int BK = 64, NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  using OA = DtlOperand<BM, BK, NW, AK>;
  using OB = DtlOperand<BN, BK, NW, BKM>;

  constexpr int S = kGemmStages;
  uint16_t* As = reinterpret_cast<uint16_t*>(smem);  // [S][BM * BK]
  uint16_t* Bs = As + S * BM * BK;                   // [S][BN * BK]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid / WN, wn = wid % WN;
  const int nk = kt1 - kt0;

  const int a_bytes = (int)((AK ? (long)g.M : (long)g.K) * g.lda * 2);
  const int b_bytes = (int)((BKM ? (long)g.N : (long)g.K) * g.ldb * 2);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.A), (short)0, a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.B), (short)0, b_bytes, 0x00020000);
  const int lda = (int)g.lda, ldb = (int)g.ldb;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto issue = [&](int j, int st) {
    OA::load(ra, lda, m0, (kt0 + j) * BK, As + st * BM * BK, wid, lane);
    OB::load(rb, ldb, n0, (kt0 + j) * BK, Bs + st * BN * BK, wid, lane);
  };
  // The operand fragments of K sub-step ks + 1 are read from LDS before the
  // MFMAs of sub-step ks issue (two fragment sets in registers); the
  // scheduling barriers keep the compiler from moving each read back next to
  // its MFMA, which left a full LDS latency before every other MFMA of a wave
  // (1T shard GEMMs 0.8 % faster in sum).
  auto compute = [&](int j, int st) {
    const uint16_t* as = As + st * BM * BK;
    const uint16_t* bs = Bs + st * BN * BK;
    f16x8 af[2][TM], bfr[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[0][i] = OA::frag(as, wm * WTM + 32 * i, 0, lane);
#pragma unroll
    for (int jj = 0; jj < TN; ++jj) bfr[0][jj] = OB::frag(bs, wn * WTN + 32 * jj, 0, lane);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < TM; ++i) af[nxt][i] = OA::frag(as, wm * WTM + 32 * i, ks + 1, lane);
#pragma unroll
        for (int jj = 0; jj < TN; ++jj)
          bfr[nxt][jj] = OB::frag(bs, wn * WTN + 32 * jj, ks + 1, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jj = 0; jj < TN; ++jj)
          acc[i][jj] =
              __builtin_amdgcn_mfma_f32_32x32x16_f16(bfr[cur][jj], af[cur][i], acc[i][jj], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  dtl_prologue<S>(nk, issue);
  dtl_loop<S, OA::kPerWave + OB::kPerWave>(nk, issue, compute);

  // Epilogue through LDS slices (see gemm_f16_kernel).
  const bool split = gridDim.y > 1;
  const bool plain = !pdst && !split && g.C && !g.accumulate;
  const bool pre_r = plain && g.resid && g.epi == EPI_STORE;
  const bool pre_a = plain && !g.resid && g.epi == EPI_DGELU;
  constexpr int CP = WTN + 4;
  float* cs = reinterpret_cast<float*>(smem) + wid * 32 * CP;
  const int lrow = lane & 31, half = lane >> 5;
  const float sc = g.scale ? g.scale[0] : 1.f;
  __syncthreads();  // every wave is done with the operand tiles
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<float4*>(cs + lrow * CP + j * 32 + 8 * jj + 4 * half) =
            make_float4(acc[i][j][4 * jj], acc[i][j][4 * jj + 1], acc[i][j][4 * jj + 2],
                        acc[i][j][4 * jj + 3]);
    constexpr int LPR = WTN / 4, RPI = 64 / LPR, NIT = 32 / RPI;
    if (pdst) {
      // stream-K segment: the raw accumulators, tile-local [BM][BN] rows
      const int c = 4 * (lane % LPR);
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int r = lane / LPR + it * RPI;
        const float4 q = *reinterpret_cast<const float4*>(cs + r * CP + c);
        *reinterpret_cast<float4*>(pdst + (size_t)(wm * WTM + i * 32 + r) * BN + wn * WTN + c) = q;
      }
      continue;
    }
    if (pre_r || pre_a) {
      // Plain store with a residual, or the product with the kept GeLU':
      // that operand (and the bias) for all NIT rows of this lane is loaded
      // before the row loop, so its memory latency is paid once per slice.
      // Same arithmetic, in the same order, as epilogue4.
      const int c = 4 * (lane % LPR), n = n0 + wn * WTN + c;
      const int mr = m0 + wm * WTM + i * 32 + lane / LPR;
      const void* src = pre_r ? g.resid : g.aux;
      const int sdt = pre_r ? g.resid_dtype : g.aux_dtype;
      const long sld = pre_r ? g.ldr : g.ldaux;
      float pp[NIT][4], bs[4] = {0.f, 0.f, 0.f, 0.f};
      if (g.bias && n < g.N) load4_dt(g.bias, g.bias_dtype, n, bs);
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int m = mr + it * RPI;
        if (m < g.M && n < g.N) load4_dt(src, sdt, (size_t)m * sld + n, pp[it]);
      }
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int m = mr + it * RPI;
        const float4 q = *reinterpret_cast<const float4*>(cs + (lane / LPR + it * RPI) * CP + c);
        float v[4] = {q.x, q.y, q.z, q.w};
        if (g.scale) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= sc;
        }
        if (g.bias) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += bs[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = pre_r ? v[e] + pp[it][e] : v[e] * pp[it][e];
        if (m < g.M && n < g.N) store4_dt(g.C, g.c_dtype, (size_t)m * g.ldc + n, v);
      }
      continue;
    }
    // a lane's columns, hence its bias values, are the same in every row
    const int c = 4 * (lane % LPR), n = n0 + wn * WTN + c;
    float bs[4] = {0.f, 0.f, 0.f, 0.f};
    if (g.bias && !split && n < g.N) load4_dt(g.bias, g.bias_dtype, n, bs);
#pragma unroll 1
    for (int r = lane / LPR; r < 32; r += RPI) {
      const float4 q = *reinterpret_cast<const float4*>(cs + r * CP + c);
      float v[4] = {q.x, q.y, q.z, q.w};
      const int m = m0 + wm * WTM + i * 32 + r;
      if (split) partial4(g, split_idx, m, n, v);
      else epilogue4(g, m, n, v, bs, sc);
    }
  }
}

template <int BM, int BN, int WM, int WN, bool AK, bool BKM>
__global__ __launch_bounds__(WM * WN * 64) void gemm_f16_dtl_kernel(GemmArgs g, int ktiles_per_split) {
  extern __shared__ __align__(16) unsigned char smem[];
  int tm, tn;
  tile_coords(g.M, g.N, BM, BN, &tm, &tn);
  const int split_idx = blockIdx.y;
  const int ktiles = g.K / 64;
  const int kt0 = split_idx * ktiles_per_split;
  const int kt1 = min(ktiles, kt0 + ktiles_per_split);
  dtl_tile<BM, BN, WM, WN, AK, BKM>(g, tm * BM, tn * BN, kt0, kt1, split_idx, nullptr, smem);
}

// ----------------------------------------------------------------------------
// Stream-K schedule for GEMMs whose tile grid leaves the last round of
// workgroups part empty (the 1T shard's M = 2048 GEMMs: 400 or 800 tiles on
// 256 compute units). A slot is Z = U x V workgroups on one XCD (workgroup w
// runs on XCD w mod 8): the U = ceil(M / BM) row tiles of V adjacent tile
// columns, a "unit" of V columns. The work, units x kI K steps, is split
// evenly over the S = 256 / Z slots: slot j takes the unit K steps
// [j T / S, (j+1) T / S) of the unit-major order (T = units * kI). The Z
// workgroups of a slot compute their tiles over the same K steps at the same
// time, so each K step of the unit's A row panels and B column panels is
// fetched into that XCD's L2 once and read by all of them. V = 32 / U (a
// slot is a whole XCD) shares the A panels across columns as a data-parallel
// grid does; V = 1 leaves no column idle when the columns do not divide by
// 32 / U. A unit a slot covers whole gets its epilogue at once; a unit split
// between slots has each piece's raw accumulators stored in the partial
// buffer ([S][2][Z][BM][BN]: a slot's first and last units) and
// gemm_sk_fixup_kernel sums the pieces in slot order (deterministic) and
// applies the epilogue. Columns past the last one in the last unit idle. No
// workgroup waits for another.
// ----------------------------------------------------------------------------
struct SkPlan {
  int U, V, Z, S, cols, units, kI;
  long T;
};

__device__ __forceinline__ long sk_begin(const SkPlan& p, int slot) {
  return (long)slot * p.T / p.S;
}

template <int BM, int BN, int WM, int WN, bool AK, bool BKM>
__global__ __launch_bounds__(WM * WN * 64) void gemm_f16_sk_kernel(GemmArgs g, SkPlan p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int xcd = blockIdx.x % kXCDs, local = blockIdx.x / kXCDs;
  const int per_xcd = p.S / kXCDs;  // slots per XCD (p.S = 256 / Z, Z divides 32)
  const int slot = xcd * per_xcd + local / p.Z, ls = local % p.Z;
  const int r = ls % p.U, v = ls / p.U;
  const long s0 = sk_begin(p, slot), s1 = sk_begin(p, slot + 1);
  if (s0 >= s1) return;
  const int u_first = (int)(s0 / p.kI), u_last = (int)((s1 - 1) / p.kI);
  bool first_tile = true;
  for (int u = u_first; u <= u_last; ++u) {
    const int c = u * p.V + v;
    if (c >= p.cols) continue;  // past the last column (uniform over the workgroup)
    const long ub = (long)u * p.kI;
    const int k0 = (int)(max(s0, ub) - ub), k1 = (int)(min(s1, ub + p.kI) - ub);
    float* pdst = nullptr;
    if (k1 - k0 < p.kI) {
      const int which = u == u_first ? 0 : 1;
      pdst = g.ws + ((size_t)(slot * 2 + which) * p.Z + ls) * (size_t)(BM * BN);
    }
    if (!first_tile) __syncthreads();  // the last epilogue's LDS reads are done
    first_tile = false;
    dtl_tile<BM, BN, WM, WN, AK, BKM>(g, r * BM, c * BN, k0, k1, 0, pdst, smem);
  }
}

// Units split between slots, and their slot range (host-computed).
constexpr int kSkMaxSplitCols = 64;
struct SkFix {
  int n;
  int col[kSkMaxSplitCols], j0[kSkMaxSplitCols], j1[kSkMaxSplitCols];  // col: the unit
};

// Sums the pieces of each split unit in slot order and applies the
// epilogue. Workgroup (q, ls, chunk): rows [chunk*32, chunk*32+32) of tile ls
// (row ls % U, column unit * V + ls / U) of split unit q; each thread owns NE
// float4 positions of those rows (4 consecutive columns each) and loads them
// from every piece before the epilogue, so NE loads per piece are in flight.
template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_sk_fixup_kernel(GemmArgs g, SkPlan p, SkFix f) {
  constexpr int RCH = BM / 32;
  constexpr int LPR = BN / 4;           // float4 per tile row
  constexpr int NE = 32 * LPR / 256;    // float4 per thread
  static_assert(32 * LPR % 256 == 0, "fix-up chunking");
  const int q = blockIdx.x / (p.Z * RCH);
  const int ls = (blockIdx.x / RCH) % p.Z, chunk = blockIdx.x % RCH;
  const int r = ls % p.U, u = f.col[q];
  const int c = u * p.V + ls / p.U;
  if (c >= p.cols) return;  // an idle column: no pieces
  const float sc = g.scale ? g.scale[0] : 1.f;
  float4 acc[NE];
#pragma unroll
  for (int it = 0; it < NE; ++it) acc[it] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = f.j0[q]; j <= f.j1[q]; ++j) {
    if (sk_begin(p, j) == sk_begin(p, j + 1)) continue;  // an empty slot wrote nothing
    const int which = (int)(sk_begin(p, j) / p.kI) == u ? 0 : 1;
    const float* src = g.ws + ((size_t)(j * 2 + which) * p.Z + ls) * (size_t)(BM * BN) +
                       (size_t)chunk * 32 * BN;
    float4 v[NE];
#pragma unroll
    for (int it = 0; it < NE; ++it) {
      const int e = threadIdx.x + it * 256;
      v[it] = *reinterpret_cast<const float4*>(src + (size_t)(e / LPR) * BN + 4 * (e % LPR));
    }
#pragma unroll
    for (int it = 0; it < NE; ++it) {
      acc[it].x += v[it].x; acc[it].y += v[it].y; acc[it].z += v[it].z; acc[it].w += v[it].w;
    }
  }
#pragma unroll
  for (int it = 0; it < NE; ++it) {
    const int e = threadIdx.x + it * 256;
    float o[4] = {acc[it].x, acc[it].y, acc[it].z, acc[it].w};
    epilogue4(g, r * BM + chunk * 32 + e / LPR, c * BN + 4 * (e % LPR), o, nullptr, sc);
  }
}

// ----------------------------------------------------------------------------
// fp32 FMA GEMM (64x64 tiles, 16-deep K steps, 4x4 outputs per thread)
// ----------------------------------------------------------------------------
template <bool AK, bool BKM>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g, int ktiles_per_split) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int tiles_n = (g.N + BN - 1) / BN;
  const int m0 = (blockIdx.x / tiles_n) * BM, n0 = (blockIdx.x % tiles_n) * BN;
  const int ktiles = (g.K + BK - 1) / BK;
  const int kt0 = blockIdx.y * ktiles_per_split;
  const int kt1 = min(ktiles, kt0 + ktiles_per_split);
  const float* A = (const float*)g.A;
  const float* B = (const float*)g.B;
  float acc[4][4] = {};
  for (int kt = kt0; kt < kt1; ++kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * 256;
      int r, k;
      if (AK) { r = e / BK; k = e % BK; } else { k = e / BM; r = e % BM; }
      const int gm = m0 + r, gk = k0 + k;
      float v = 0.f;
      if (gm < g.M && gk < g.K) v = AK ? A[(size_t)gm * g.lda + gk] : A[(size_t)gk * g.lda + gm];
      As[k][r] = v;
      int c;
      if (BKM) { c = e / BK; k = e % BK; } else { k = e / BN; c = e % BN; }
      const int gn = n0 + c;
      const int gk2 = k0 + k;
      float w = 0.f;
      if (gn < g.N && gk2 < g.K) w = BKM ? B[(size_t)gn * g.ldb + gk2] : B[(size_t)gk2 * g.ldb + gn];
      Bs[k][c] = w;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const float sc = g.scale ? g.scale[0] : 1.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[4] = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    if (gridDim.y > 1) partial4(g, blockIdx.y, m0 + ty * 4 + i, n0 + tx * 4, v);
    else epilogue4(g, m0 + ty * 4 + i, n0 + tx * 4, v, nullptr, sc);
  }
}

// Split-K reduction: C (+)= sum_s ws[s]  (fp32 output, plain store epilogue).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g) {
  const size_t nvec = (size_t)g.M * g.N / 4;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nvec) return;
  const size_t idx = 4 * i;
  const int m = (int)(idx / g.N), n = (int)(idx % g.N);
  float acc[4], v[4];
  Vec4<float>::load(g.ws + idx, acc);
  const size_t stride = (size_t)g.M * g.N;
  for (int s0 = 1; s0 < g.split; s0 += 4) {
    // 4 splits in flight, summed in split order
    float x[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      Vec4<float>::load(g.ws + (size_t)min(s0 + u, g.split - 1) * stride + idx, x[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s0 + u < g.split)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += x[u][e];
  }
  if (g.scale) {
    const float sc = g.scale[0];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= sc;
  }
  float* c = (float*)g.C + (size_t)m * g.ldc + n;
  if (g.accumulate) {
    Vec4<float>::load(c, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += v[e];
  }
  if (g.stream_out) store4_f32_nt(c, acc);
  else Vec4<float>::store(c, acc);
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
struct TileCfg {
  int bm, bn;
  int per_cu;       // workgroups resident per CU (LDS bound)
  double eff;       // relative MFMA efficiency of the tile shape
};
static constexpr TileCfg kBig = {256, 256, 1, 1.0};
static constexpr TileCfg kWide = {256, 192, 1, 0.95};
static constexpr TileCfg kSmall = {128, 128, 2, 0.8};
static constexpr int kCUs = 256;
// Time model constants: MACs per second of one CU inside a full round of the
// 256x256 kernel (about half the CU's dense fp16 MFMA rate, measured on the
// 1T shard's long-K GEMMs), and the HBM rate of the partial-sum traffic.
static constexpr double kMacPerCU = 2.4e12;
static constexpr double kPartialBW = 5.0e12;
static constexpr double kLaunch = 5e-6;  // one more launch and pipeline fills

static long ceil_div(long a, long b) { return (a + b - 1) / b; }

// Time model: rounds of resident workgroups times the work of one tile.
static double tile_cost(const TileCfg& t, int M, int N, int split) {
  const long tiles = ceil_div(M, t.bm) * ceil_div(N, t.bn) * split;
  const long rounds = ceil_div(tiles, (long)kCUs * t.per_cu);
  return (double)rounds * t.per_cu * t.bm * t.bn / t.eff;
}

static TileCfg choose_tile(int M, int N, int split) {
  TileCfg best = kBig;
  double bc = tile_cost(kBig, M, N, split);
  for (const TileCfg& t : {kWide, kSmall}) {
    const double c = tile_cost(t, M, N, split);
    if (c < bc) {
      bc = c;
      best = t;
    }
  }
  return best;
}

// Estimated seconds of a GEMM on tile t with a split-K factor s: rounds of
// resident workgroups times one workgroup's MACs, plus (s > 1) the fp32
// partials written by the main kernel and read by the reduce, and the reduce's
// output (read too when accumulating).
static double split_cost(const TileCfg& t, const GemmArgs& g, int s) {
  const long ktiles = ceil_div(g.K, 64);
  const long per = ceil_div(ktiles, s), real = ceil_div(ktiles, per);
  const long wgs = ceil_div(g.M, t.bm) * ceil_div(g.N, t.bn) * real;
  const long rounds = ceil_div(wgs, (long)kCUs * t.per_cu);
  double sec = (double)rounds * t.per_cu * t.bm * t.bn * (double)(per * 64) / t.eff / kMacPerCU;
  if (real > 1)
    sec += (2.0 * real + 1 + (g.accumulate ? 1 : 0)) * (double)g.M * g.N * 4 / kPartialBW + kLaunch;
  return sec;
}

// Split-K factor of a weight-gradient GEMM (few output tiles, long K): the
// factor with the lowest modelled time over the tile shapes, where a split
// costs its fp32 partial traffic (so a split that only rounds up the last
// round of a many-round grid is not taken).
int gemm_choose_split(const GemmArgs& g) {
  if (g.math != DT_F16) return 1;
  if (g.epi != EPI_STORE || g.bias || g.resid || g.c_dtype != DT_F32) return 1;
  const long ktiles = ceil_div(g.K, 64);
  int best = 1;
  double bc = 1e30;
  for (int s = 1; s <= 16; ++s) {
    if (s > 1 && ktiles / s < 8) break;  // keep >= 8 K-tiles per split
    for (const TileCfg& t : {kBig, kWide, kSmall}) {
      const double c = split_cost(t, g, s);
      if (c < bc * 0.98) {  // a split must win by more than the model's noise
        bc = c;
        best = s;
      }
    }
  }
  return best;
}

// ---- stream-K planning --------------------------------------------------------
// Slot shape for tile t: U = the row tiles (must divide the 32 CUs of an
// XCD), V columns per unit (V = 1, or 32 / U with `wide`).
static bool sk_shape(const GemmArgs& g, const TileCfg& t, int wide, SkPlan* p) {
  const long U = ceil_div(g.M, t.bm);
  if (t.per_cu != 1 || U > 32 || (32 % U) != 0) return false;
  p->U = (int)U;
  p->V = wide ? 32 / (int)U : 1;
  p->Z = p->U * p->V;
  p->S = kCUs / p->Z;
  p->cols = (int)ceil_div(g.N, t.bn);
  p->units = (int)ceil_div(p->cols, p->V);
  p->kI = g.K / 64;
  p->T = (long)p->units * p->kI;
  return true;
}

// The slot whose K-step range holds unit K step i: the largest j with
// j T / S <= i (empty slots, possible only when T < S, are skipped this way).
static int sk_slot_of(const SkPlan& p, long i) {
  return (int)(((i + 1) * p.S + p.T - 1) / p.T) - 1;
}

// The split units and, for each, the first and last slot covering it.
static void sk_fix(const SkPlan& p, SkFix* f) {
  f->n = 0;
  for (int j = 1; j < p.S; ++j) {
    const long b = (long)j * p.T / p.S;  // slot j starts here
    if (b % p.kI == 0 || b >= p.T) continue;  // on a unit edge: nothing split there
    const int u = (int)(b / p.kI);
    if (f->n && f->col[f->n - 1] == u) continue;
    if (f->n == kSkMaxSplitCols) {  // too many to list: the caller rejects the plan
      f->n = kSkMaxSplitCols + 1;
      return;
    }
    f->col[f->n] = u;
    f->j0[f->n] = sk_slot_of(p, (long)u * p.kI);
    f->j1[f->n] = sk_slot_of(p, (long)(u + 1) * p.kI - 1);
    ++f->n;
  }
}

// Modelled seconds: the slot's K steps, plus the pieces (at most two per
// slot and tile, written then read). Single-column units (V = 1) pay about 5 %
// per K step for fetching the A panels once per slot rather than once per XCD
// (the 1T shard's M = 2048 GEMMs).
static double sk_cost(const TileCfg& t, const SkPlan& p) {
  const long iters = ceil_div(p.T, p.S);
  const double shared = p.V == 1 && p.U < 32 ? 1.05 : 1.0;
  const double mac = (double)iters * t.bm * t.bn * 64 / t.eff * shared;
  const double part = 2.0 * 2.0 * p.S * p.Z * (double)t.bm * t.bn * 4;
  return mac / kMacPerCU + part / kPartialBW + kLaunch;
}

// Whether g runs stream-K (and on which tile and slot shape): K a whole
// number of long enough K steps (at least 128; 32 when M spans at most 8 row
// tiles, where a data-parallel grid's rounds are coarsest: the 1T shard's
// output projection, K = 3200, measured 444 -> 420 us, while shapes of 32
// row tiles gained nothing), no split-K, a partial buffer, and a modelled
// time at least 3 % below the best data-parallel grid's.
static bool sk_choose(const GemmArgs& g, TileCfg* tile, SkPlan* plan, bool need_ws) {
  if (g.math != DT_F16 || g.split > 1 || g.K % 64) return false;
  const long ksteps = g.K / 64;
  if (ksteps < 32 || (ksteps < 128 && ceil_div(g.M, 256) > 8)) return false;
  if (need_ws && !g.ws) return false;
  const TileCfg dp = choose_tile(g.M, g.N, 1);
  const double dp_cost = tile_cost(dp, g.M, g.N, 1) * (double)g.K / kMacPerCU;
  bool found = false;
  double best = dp_cost * 0.97;
  for (const TileCfg& t : {kBig, kWide}) {
    for (int wide = 0; wide < 2; ++wide) {
      SkPlan p;
      if (!sk_shape(g, t, wide, &p)) continue;
      const size_t need = (size_t)p.S * 2 * p.Z * t.bm * t.bn;
      if (need_ws && need > g.ws_floats) continue;
      SkFix f;
      sk_fix(p, &f);
      if (f.n > kSkMaxSplitCols) continue;
      const double c = sk_cost(t, p);
      if (c < best) {
        best = c;
        *tile = t;
        *plan = p;
        found = true;
      }
    }
  }
  return found;
}

size_t gemm_ws_floats(const GemmArgs& g) {
  size_t need = 0;
  const int split = g.split < 1 ? 1 : g.split;
  if (split > 1 && g.math == DT_F16) {
    const long ktiles = ceil_div(g.K, 64), per = ceil_div(ktiles, split);
    need = (size_t)ceil_div(ktiles, per) * g.M * g.N;
  }
  TileCfg t;
  SkPlan p;
  if (sk_choose(g, &t, &p, false)) need = std::max(need, (size_t)p.S * 2 * p.Z * t.bm * t.bn);
  return need;
}

template <int BM, int BN, int WM, int WN, bool AK, bool BKM>
static hipError_t launch_f16(const GemmArgs& g, int split, hipStream_t s,
                             const SkPlan* sk = nullptr) {
  constexpr int BK = 64;
  constexpr int NT = WM * WN * 64;
  const int ktiles = (int)ceil_div(g.K, BK);
  const int per = (int)ceil_div(ktiles, split);
  const int real_split = (int)ceil_div(ktiles, per);
  // The direct-load kernel takes every GEMM whose K is a whole number of
  // K steps and whose operand byte offsets (up to one tile past M and N) fit
  // 31 bits. Its loads have no bounds checks: the buffer descriptor returns
  // zero beyond an operand's last byte, and a partial tile's rows or columns
  // past M or N only ever reach outputs past M or N, which the epilogue
  // skips.
  const bool direct =
      g.K % BK == 0 &&
      ((size_t)(g.a_kmajor ? g.M + BM : g.K) * g.lda + BM) * 2 < (1u << 31) &&
      ((size_t)(g.b_kmajor ? g.N + BN : g.K) * g.ldb + BN) * 2 < (1u << 31);
  if (sk && !direct) return hipErrorInvalidValue;
  const size_t slices = (size_t)WM * WN * 32 * (BN / WN + 4) * sizeof(float);
  const size_t lds_pad = (size_t)2 *
                         (TilePitch<BM, BK, AK>::kElems + TilePitch<BN, BK, BKM>::kElems) *
                         sizeof(uint16_t);
  const size_t lds_ops = (size_t)kGemmStages * (BM + BN) * BK * sizeof(uint16_t);
  const size_t lds_dtl = lds_ops > slices ? lds_ops : slices;
  const size_t lds = direct ? lds_dtl : lds_pad;
  if (sk) {
    auto kern = gemm_f16_sk_kernel<BM, BN, WM, WN, AK, BKM>;
    static bool sk_attr = false;
    if (!sk_attr) {
      hipError_t e = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      sk_attr = true;
    }
    SkFix f;
    sk_fix(*sk, &f);
    GemmArgs a = g;
    a.split = 1;
    hipLaunchKernelGGL(kern, dim3((unsigned)(sk->S * sk->Z)), dim3(NT), lds, s, a, *sk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || f.n == 0) return e;
    hipLaunchKernelGGL((gemm_sk_fixup_kernel<BM, BN>), dim3((unsigned)(f.n * sk->Z * (BM / 32))),
                       dim3(256), 0, s, a, *sk, f);
    return hipGetLastError();
  }
  auto kern = direct ? gemm_f16_dtl_kernel<BM, BN, WM, WN, AK, BKM>
                       : gemm_f16_kernel<BM, BN, BK, WM, WN, AK, BKM>;
  static bool attr_set[2] = {false, false};  // per instantiation
  if (!attr_set[direct]) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set[direct] = true;
  }
  dim3 grid((unsigned)(ceil_div(g.M, BM) * ceil_div(g.N, BN)), (unsigned)real_split);
  GemmArgs a = g;
  a.split = real_split;
  hipLaunchKernelGGL(kern, grid, dim3(NT), lds, s, a, per);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || real_split == 1) return e;
  const size_t nvec = (size_t)g.M * g.N / 4;
  splitk_reduce_kernel<<<(unsigned)ceil_div((long)nvec, 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

template <bool AK, bool BKM>
static hipError_t dispatch_f16(const GemmArgs& g, int split, hipStream_t s) {
  TileCfg skt;
  SkPlan plan;
  if (split == 1 && sk_choose(g, &skt, &plan, true)) {
    if (skt.bn == 256) return launch_f16<256, 256, 4, 4, AK, BKM>(g, 1, s, &plan);
    return launch_f16<256, 192, 4, 3, AK, BKM>(g, 1, s, &plan);
  }
  const TileCfg t = choose_tile(g.M, g.N, split);
  if (t.bm == 256 && t.bn == 256) return launch_f16<256, 256, 4, 4, AK, BKM>(g, split, s);
  if (t.bm == 256) return launch_f16<256, 192, 4, 3, AK, BKM>(g, split, s);
  return launch_f16<128, 128, 2, 2, AK, BKM>(g, split, s);
}

template <bool AK, bool BKM>
static hipError_t launch_f32(const GemmArgs& g, int split, hipStream_t s) {
  const int ktiles = (int)ceil_div(g.K, 16);
  const int per = (int)ceil_div(ktiles, split);
  const int real_split = (int)ceil_div(ktiles, per);
  dim3 grid((unsigned)(ceil_div(g.M, 64) * ceil_div(g.N, 64)), (unsigned)real_split);
  GemmArgs a = g;
  a.split = real_split;
  gemm_f32_kernel<AK, BKM><<<grid, 256, 0, s>>>(a, per);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || real_split == 1) return e;
  const size_t nvec = (size_t)g.M * g.N / 4;
  splitk_reduce_kernel<<<(unsigned)ceil_div((long)nvec, 256), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t gemm(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.K < 0) return g.M == 0 || g.N == 0 ? hipSuccess : hipErrorInvalidValue;
  if (g.N % 4) return hipErrorInvalidValue;
  int split = g.split < 1 ? 1 : g.split;
  if (split > 1 && (!g.ws || g.epi != EPI_STORE || g.bias || g.resid || g.c_dtype != DT_F32))
    return hipErrorInvalidValue;
  if (split > 1 && g.math == DT_F16) {  // the partials must fit the scratch given
    GemmArgs q = g;
    q.split = split;
    if (gemm_ws_floats(q) > g.ws_floats) return hipErrorInvalidValue;
  }
  if (g.math == DT_F16) {
    if (g.a_dtype != DT_F16 || g.b_dtype != DT_F16) return hipErrorInvalidValue;
    // 16-byte operand chunks: the contiguous dimension must be a multiple of 8
    if (g.a_kmajor ? (g.K % 8) : (g.M % 8)) return hipErrorInvalidValue;
    if (g.b_kmajor ? (g.K % 8) : (g.N % 8)) return hipErrorInvalidValue;
    if (g.a_kmajor && g.b_kmajor) return dispatch_f16<true, true>(g, split, s);
    if (g.a_kmajor && !g.b_kmajor) return dispatch_f16<true, false>(g, split, s);
    if (!g.a_kmajor && !g.b_kmajor) return dispatch_f16<false, false>(g, split, s);
    return dispatch_f16<false, true>(g, split, s);
  }
  if (g.a_dtype != DT_F32 || g.b_dtype != DT_F32) return hipErrorInvalidValue;
  if (g.a_kmajor && g.b_kmajor) return launch_f32<true, true>(g, split, s);
  if (g.a_kmajor && !g.b_kmajor) return launch_f32<true, false>(g, split, s);
  if (!g.a_kmajor && !g.b_kmajor) return launch_f32<false, false>(g, split, s);
  return launch_f32<false, true>(g, split, s);
}

}  // namespace tpl
