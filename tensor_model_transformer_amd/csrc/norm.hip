// LayerNorm forward/backward, column reductions and the single-GPU exchange
// sum. All HBM-bound: one pass over each tensor (the LayerNorm backward of
// rows wider than 6144 elements reads its inputs twice), 16-byte vector
// accesses, fp32 statistics; column sums as block partials plus one
// reduction, in a fixed order (deterministic, no atomics).
//
// LayerNorm placement follows "Megatron-LM: GPU-Cluster Training Parallelism",
// section "Paper 1: BERT LayerNorm Rearrangement" (pre-LN: each sublayer reads
// LN of the residual stream, whose un-normalised value is carried forward).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace tpl {

template <typename T> struct DtOf;
template <> struct DtOf<float> { static constexpr int v = DT_F32; };
template <> struct DtOf<bf16> { static constexpr int v = DT_BF16; };
template <> struct DtOf<f16> { static constexpr int v = DT_F16; };

// ----------------------------------------------------------------------------
// LayerNorm forward: one workgroup per row, the row held in registers.
// ----------------------------------------------------------------------------
// Rows of 1024 threads x 4 vectors (hidden above 16384, 16-bit output) fit
// in 64 VGPRs without spilling, so two workgroups share a compute unit and
// one's reductions overlap the other's loads and stores.
template <typename To, int NT, int NV>
constexpr int kLnFwdWaves = (NT == 1024 && NV == 4 && sizeof(To) == 2) ? 8 : 1;

template <typename Tin, typename T, typename To, int NT, int NV>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(kLnFwdWaves<To, NT, NV>))) void ln_fwd_kernel(
    const Tin* __restrict__ x, const T* __restrict__ gamma, const T* __restrict__ beta,
    To* __restrict__ y, float* __restrict__ mean_out, float* __restrict__ rstd_out,
    float* __restrict__ x_copy, int h, float eps) {
  __shared__ float red[16];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nvec = h >> 3;
  const Tin* xr = x + (size_t)row * h;
  // Up to two vectors per thread, gamma and beta are loaded with the row,
  // ahead of the two reductions (wider rows have no registers to spare).
  constexpr bool kEarly = NV <= 2;
  float v[NV][8], gm[kEarly ? NV : 1][8], bt[kEarly ? NV : 1][8];
  float acc[1] = {0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = tid + i * NT;
    if (j < nvec) {
      if constexpr (kEarly) {
        Vec8<T>::load(gamma + 8 * j, gm[i]);
        Vec8<T>::load(beta + 8 * j, bt[i]);
      }
      Vec8<Tin>::load(xr + 8 * j, v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[0] += v[i][e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
    }
  }
  block_sum<1>(acc, red);
  const float mu = acc[0] / (float)h;
  float sq[1] = {0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = tid + i * NT;
    if (j < nvec) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[i][e] - mu;
        sq[0] += d * d;
      }
    }
  }
  block_sum<1>(sq, red);
  const float rstd = 1.f / sqrtf(sq[0] / (float)h + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = tid + i * NT;
    if (j < nvec) {
      float g[8], b[8], o[8];
      if constexpr (kEarly) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          g[e] = gm[i][e];
          b[e] = bt[i][e];
        }
      } else {
        Vec8<T>::load(gamma + 8 * j, g);
        Vec8<T>::load(beta + 8 * j, b);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = g[e] * ((v[i][e] - mu) * rstd) + b[e];
      Vec8<To>::store(y + (size_t)row * h + 8 * j, o);
      if (x_copy) Vec8<float>::store(x_copy + (size_t)row * h + 8 * j, v[i]);
    }
  }
  if (tid == 0 && mean_out) {
    mean_out[row] = mu;
    rstd_out[row] = rstd;
  }
}

// LayerNorm forward for rows of at most 4096 elements: one wave per row,
// the row in registers (NV 8-wide vectors per lane), both reductions by
// cross-lane shuffles, so no LDS round trip and no barrier; four rows per
// 256-thread workgroup. Same arithmetic per element as ln_fwd_kernel (the
// sums are taken in another order). At least four waves per SIMD are
// requested: six vectors per lane otherwise took 133 registers and three
// waves (8.3B and BERT shards: 63.8 -> 60.6 and 56.7 -> 54.1 us for both).
template <typename Tin, typename T, typename To, int NV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void ln_fwd_wave_kernel(
    const Tin* __restrict__ x, const T* __restrict__ gamma, const T* __restrict__ beta,
    To* __restrict__ y, float* __restrict__ mean_out, float* __restrict__ rstd_out,
    float* __restrict__ x_copy, int rows, int h, float eps) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform over the wave; no barrier follows
  const int nvec = h >> 3;
  const Tin* xr = x + (size_t)row * h;
  float v[NV][8];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = lane + 64 * i;
    if (j < nvec) {
      Vec8<Tin>::load(xr + 8 * j, v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[i][e];
    }
  }
  const float mu = wave_sum(s) / (float)h;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (lane + 64 * i < nvec) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[i][e] - mu;
        sq += d * d;
      }
    }
  }
  const float rstd = 1.f / sqrtf(wave_sum(sq) / (float)h + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = lane + 64 * i;
    if (j < nvec) {
      // gamma and beta (the same for every row, so cached) load after the
      // reductions: the registers go to more waves per SIMD instead
      float g[8], b[8], o[8];
      Vec8<T>::load(gamma + 8 * j, g);
      Vec8<T>::load(beta + 8 * j, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = g[e] * ((v[i][e] - mu) * rstd) + b[e];
      Vec8<To>::store(y + (size_t)row * h + 8 * j, o);
      if (x_copy) Vec8<float>::store(x_copy + (size_t)row * h + 8 * j, v[i]);
    }
  }
  if (lane == 0 && mean_out) {
    mean_out[row] = mu;
    rstd_out[row] = rstd;
  }
}

// Threads per row and 8-wide vectors per thread for a row of h elements.
static bool row_config(int h, int* nt, int* nv) {
  const int nvec = h / 8;
  if (nvec <= 256) { *nt = 256; *nv = 1; }
  else if (nvec <= 512) { *nt = 256; *nv = 2; }
  else if (nvec <= 1024) { *nt = 512; *nv = 2; }
  else if (nvec <= 2048) { *nt = 1024; *nv = 2; }
  else if (nvec <= 4096) { *nt = 1024; *nv = 4; }
  else return false;
  return true;
}

template <typename Tin, typename T, typename To>
static hipError_t ln_fwd_t(const void* x, const void* gamma, const void* beta, void* y,
                           float* mean, float* rstd, float* x_copy, int rows, int h,
                           float eps, hipStream_t s) {
  int nt, nv;
  if (!row_config(h, &nt, &nv)) return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  // rows of at most 4096 elements: a wave per row (vectors per lane: the
  // smallest instantiated count covering the row)
  const int wv = (h / 8 + 63) / 64;
  if (wv <= 8) {
    const unsigned grid = (unsigned)((rows + 3) / 4);
#define TPL_LNW(NV_)                                                                       \
  if (wv <= NV_) {                                                                         \
    ln_fwd_wave_kernel<Tin, T, To, NV_><<<grid, 256, 0, s>>>(                              \
        (const Tin*)x, (const T*)gamma, (const T*)beta, (To*)y, mean, rstd, x_copy, rows,  \
        h, eps);                                                                           \
    return hipGetLastError();                                                              \
  }
    TPL_LNW(1) TPL_LNW(2) TPL_LNW(3) TPL_LNW(4) TPL_LNW(6) TPL_LNW(8)
#undef TPL_LNW
  }
#define TPL_LNF(NT_, NV_)                                                                   \
  if (nt == NT_ && nv == NV_) {                                                             \
    ln_fwd_kernel<Tin, T, To, NT_, NV_><<<rows, NT_, 0, s>>>(                               \
        (const Tin*)x, (const T*)gamma, (const T*)beta, (To*)y, mean, rstd, x_copy, h, eps); \
    return hipGetLastError();                                                               \
  }
  TPL_LNF(256, 1) TPL_LNF(256, 2) TPL_LNF(512, 2) TPL_LNF(1024, 2) TPL_LNF(1024, 4)
#undef TPL_LNF
  return hipErrorInvalidValue;
}

hipError_t ln_fwd(int x_dtype, int p_dtype, int y_dtype, const void* x, const void* gamma,
                  const void* beta, void* y, float* mean, float* rstd, float* x_copy,
                  int rows, int h, float eps, hipStream_t s) {
  if (p_dtype == DT_BF16 && y_dtype == DT_F16) {
    if (x_dtype == DT_BF16)
      return ln_fwd_t<bf16, bf16, f16>(x, gamma, beta, y, mean, rstd, x_copy, rows, h, eps, s);
    if (x_dtype == DT_F32)
      return ln_fwd_t<float, bf16, f16>(x, gamma, beta, y, mean, rstd, x_copy, rows, h, eps, s);
  }
  if (p_dtype == DT_F32 && y_dtype == DT_F32 && x_dtype == DT_F32)
    return ln_fwd_t<float, float, float>(x, gamma, beta, y, mean, rstd, x_copy, rows, h, eps, s);
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------------------
// LayerNorm backward + residual-gradient add. A workgroup walks a block of
// rows; each thread owns the same columns in every row and accumulates the
// column sums (dgamma, dbeta, dx) for them, written once per block.
// ----------------------------------------------------------------------------
template <typename T, typename Tx, typename Tr, typename Ts, int NT, int NV, bool DSUM>
__global__ __launch_bounds__(NT) void ln_bwd_kernel(
    const float* __restrict__ dy, const Tx* __restrict__ x, const float* __restrict__ mean,
    const float* __restrict__ rstd, const T* __restrict__ gamma, const Tr* __restrict__ dres,
    float* __restrict__ dx_f32, Ts* __restrict__ dx_st, const float* __restrict__ st_scale,
    float* __restrict__ part, int rows_per_blk, int rows, int h) {
  __shared__ float red[32];
  const int tid = threadIdx.x;
  // power-of-two factor of the storage-dtype copy (exact; 1 when not given)
  const float sts = st_scale ? st_scale[0] : 1.f;
  const int nvec = h >> 3;
  const int r0 = blockIdx.x * rows_per_blk;
  const int r1 = min(rows, r0 + rows_per_blk);
  // Column sums over the block's rows: dgamma, dbeta and (DSUM) dx. Rows of
  // 1024 threads keep the dx sums in LDS, each thread its own entries (no
  // barrier needed), so the other two fit the registers.
  constexpr bool kLdsSum = DSUM && NT > 768;
  __shared__ float4 dsl[kLdsSum ? 2 * NV * NT : 1];
  float dg[NV][8], db[NV][8], ds[(DSUM && !kLdsSum) ? NV : 1][8];
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) dg[i][e] = db[i][e] = 0.f;
#pragma unroll
  for (int i = 0; i < ((DSUM && !kLdsSum) ? NV : 1); ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) ds[i][e] = 0.f;
  if constexpr (kLdsSum) {
#pragma unroll
    for (int i = 0; i < 2 * NV; ++i) dsl[i * NT + tid] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // Rows of up to 768 threads: row r + 1's inputs (with its mean and rstd)
  // are fetched while row r is reduced and written, and gamma is loaded once.
  // Wider rows (1024 threads) have no registers for the second copy and load
  // each row in turn.
  if constexpr (NT <= 768) {
  float nd[NV][8], nx[NV][8], nr[NV][8], gm[NV][8];
  float nmu = 0.f, nrs = 0.f;
#define TPL_LNB_FETCH(ROW)                                                     \
  {                                                                            \
    nmu = mean[ROW];                                                           \
    nrs = rstd[ROW];                                                           \
    _Pragma("unroll") for (int i = 0; i < NV; ++i) {                           \
      const int j = tid + i * NT;                                              \
      if (j < nvec) {                                                          \
        Vec8<float>::load(dy + (size_t)(ROW) * h + 8 * j, nd[i]);             \
        Vec8<Tx>::load(x + (size_t)(ROW) * h + 8 * j, nx[i]);                 \
        Vec8<Tr>::load(dres + (size_t)(ROW) * h + 8 * j, nr[i]);              \
      }                                                                        \
    }                                                                          \
  }
  if (r0 < r1) TPL_LNB_FETCH(r0)
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = tid + i * NT;
    if (j < nvec) Vec8<T>::load(gamma + 8 * j, gm[i]);
  }
  for (int row = r0; row < r1; ++row) {
    const float mu = nmu, rs = nrs;
    float d[NV][8], xv[NV][8], rv[NV][8];
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        d[i][e] = nd[i][e];
        xv[i][e] = nx[i][e];
        rv[i][e] = nr[i][e];
      }
    if (row + 1 < r1) TPL_LNB_FETCH(row + 1)
    float gy[NV][8], xh[NV][8];
    float sums[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = tid + i * NT;
      if (j < nvec) {
        const float* g = gm[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xh[i][e] = (xv[i][e] - mu) * rs;
          gy[i][e] = d[i][e] * g[e];
          sums[0] += gy[i][e];
          sums[1] += gy[i][e] * xh[i][e];
          dg[i][e] += d[i][e] * xh[i][e];
          db[i][e] += d[i][e];
        }
      }
    }
    block_sum<2>(sums, red);
    const float mg = sums[0] / (float)h, mgx = sums[1] / (float)h;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = tid + i * NT;
      if (j < nvec) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[e] = rs * (gy[i][e] - mg - xh[i][e] * mgx) + rv[i][e];
          if constexpr (DSUM) ds[i][e] += o[e];
        }
        if (dx_f32) Vec8<float>::store(dx_f32 + (size_t)row * h + 8 * j, o);
        if (dx_st) {
          float q[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) q[e] = o[e] * sts;
          Vec8<Ts>::store(dx_st + (size_t)row * h + 8 * j, q);
        }
      }
    }
  }
  } else {
  // Rows of 1024 threads (hidden above 16384): the column sums of up to 4
  // vectors per thread take 96 registers, which leaves no room to keep the
  // row between its reduction and its output (the first version did and
  // spilled). The row is read once for the two row sums and again, from
  // L2 or the last-level cache, for the output.
  for (int row = r0; row < r1; ++row) {
    const float mu = mean[row], rs = rstd[row];
    float sums[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = tid + i * NT;
      if (j < nvec) {
        float d[8], xv[8], g[8];
        Vec8<float>::load(dy + (size_t)row * h + 8 * j, d);
        Vec8<Tx>::load(x + (size_t)row * h + 8 * j, xv);
        Vec8<T>::load(gamma + 8 * j, g);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xh = (xv[e] - mu) * rs, gy = d[e] * g[e];
          sums[0] += gy;
          sums[1] += gy * xh;
          dg[i][e] += d[e] * xh;
          db[i][e] += d[e];
        }
      }
    }
    block_sum<2>(sums, red);
    const float mg = sums[0] / (float)h, mgx = sums[1] / (float)h;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int j = tid + i * NT;
      if (j < nvec) {
        float d[8], xv[8], g[8], r[8], o[8];
        Vec8<float>::load(dy + (size_t)row * h + 8 * j, d);
        Vec8<Tx>::load(x + (size_t)row * h + 8 * j, xv);
        Vec8<T>::load(gamma + 8 * j, g);
        Vec8<Tr>::load(dres + (size_t)row * h + 8 * j, r);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xh = (xv[e] - mu) * rs;
          o[e] = rs * (d[e] * g[e] - mg - xh * mgx) + r[e];
          if constexpr (DSUM && !kLdsSum) ds[i][e] += o[e];
        }
        if constexpr (kLdsSum) {
          float4 a = dsl[(2 * i) * NT + tid], b = dsl[(2 * i + 1) * NT + tid];
          a.x += o[0]; a.y += o[1]; a.z += o[2]; a.w += o[3];
          b.x += o[4]; b.y += o[5]; b.z += o[6]; b.w += o[7];
          dsl[(2 * i) * NT + tid] = a;
          dsl[(2 * i + 1) * NT + tid] = b;
        }
        if (dx_f32) Vec8<float>::store(dx_f32 + (size_t)row * h + 8 * j, o);
        if (dx_st) {
          float q[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) q[e] = o[e] * sts;
          Vec8<Ts>::store(dx_st + (size_t)row * h + 8 * j, q);
        }
      }
    }
  }
  }
#undef TPL_LNB_FETCH
  float* pb = part + (size_t)blockIdx.x * 3 * h;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = tid + i * NT;
    if (j < nvec) {
      Vec8<float>::store(pb + 8 * j, dg[i]);
      Vec8<float>::store(pb + h + 8 * j, db[i]);
      if constexpr (kLdsSum) {
        const float4 a = dsl[(2 * i) * NT + tid], b = dsl[(2 * i + 1) * NT + tid];
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        Vec8<float>::store(pb + 2 * h + 8 * j, v);
      } else if constexpr (DSUM) {
        Vec8<float>::store(pb + 2 * h + 8 * j, ds[i]);
      }
    }
  }
}

int ln_bwd_blocks(int rows, int h, int* rows_per_blk) {
  (void)h;
  const int rpb = rows <= 4096 ? 8 : 16;
  *rows_per_blk = rpb;
  return (rows + rpb - 1) / rpb;
}

template <typename T, typename Tx, typename Tr, typename Ts>
static hipError_t ln_bwd_t(const float* dy, const void* x, const float* mean,
                           const float* rstd, const void* gamma, const void* dres,
                           float* dx_f32, void* dx_st, const float* st_scale, float* part,
                           int rows_per_blk, int rows, int h, int want_dsum, hipStream_t s) {
  int nt, nv;
  if (!row_config(h, &nt, &nv)) return hipErrorInvalidValue;
  const int nblk = (rows + rows_per_blk - 1) / rows_per_blk;
  if (nblk == 0) return hipSuccess;
#define TPL_LNB(NT_, NV_)                                                                  \
  if (nt == NT_ && nv == NV_) {                                                            \
    if (want_dsum)                                                                         \
      ln_bwd_kernel<T, Tx, Tr, Ts, NT_, NV_, true><<<nblk, NT_, 0, s>>>(                   \
          dy, (const Tx*)x, mean, rstd, (const T*)gamma, (const Tr*)dres, dx_f32,          \
          (Ts*)dx_st, st_scale, part, rows_per_blk, rows, h);                              \
    else                                                                                   \
      ln_bwd_kernel<T, Tx, Tr, Ts, NT_, NV_, false><<<nblk, NT_, 0, s>>>(                  \
          dy, (const Tx*)x, mean, rstd, (const T*)gamma, (const Tr*)dres, dx_f32,          \
          (Ts*)dx_st, st_scale, part, rows_per_blk, rows, h);                              \
    return hipGetLastError();                                                              \
  }
  // rows of at most 768 vectors: one vector per thread, the workgroup as
  // wide as the row (rounded up to whole waves), so no thread idles on a
  // second, partly used vector (h = 3072: 384 threads, where 256 threads of
  // two vectors each left half the second vectors empty)
  if (h / 8 <= 768) {
    const int nt1 = (h / 8 + 63) / 64 * 64;
    if (want_dsum)
      ln_bwd_kernel<T, Tx, Tr, Ts, 768, 1, true><<<nblk, nt1, 0, s>>>(
          dy, (const Tx*)x, mean, rstd, (const T*)gamma, (const Tr*)dres, dx_f32, (Ts*)dx_st,
          st_scale, part, rows_per_blk, rows, h);
    else
      ln_bwd_kernel<T, Tx, Tr, Ts, 768, 1, false><<<nblk, nt1, 0, s>>>(
          dy, (const Tx*)x, mean, rstd, (const T*)gamma, (const Tr*)dres, dx_f32, (Ts*)dx_st,
          st_scale, part, rows_per_blk, rows, h);
    return hipGetLastError();
  }
  TPL_LNB(512, 2) TPL_LNB(1024, 2) TPL_LNB(1024, 4)
#undef TPL_LNB
  return hipErrorInvalidValue;
}

hipError_t ln_bwd(int p_dtype, const float* dy, int x_dtype, const void* x,
                  const float* mean, const float* rstd, const void* gamma, int dres_dtype,
                  const void* dres, float* dx_f32, int st_dtype, void* dx_st,
                  const float* st_scale, float* part, int rows_per_blk, int rows, int h,
                  int want_dsum, hipStream_t s) {
  if (p_dtype == DT_F32 && x_dtype == DT_F32 && dres_dtype == DT_F32 && st_dtype == DT_F32)
    return ln_bwd_t<float, float, float, float>(dy, x, mean, rstd, gamma, dres, dx_f32, dx_st,
                                                st_scale, part, rows_per_blk, rows, h, want_dsum,
                                                s);
  if (p_dtype != DT_BF16) return hipErrorInvalidValue;
  // LN2 backward: x = h_mid (fp32), dres = upstream gradient (bf16), dx -> fp32 + fp16
  if (x_dtype == DT_F32 && dres_dtype == DT_BF16 && st_dtype == DT_F16)
    return ln_bwd_t<bf16, float, bf16, f16>(dy, x, mean, rstd, gamma, dres, dx_f32, dx_st,
                                            st_scale, part, rows_per_blk, rows, h, want_dsum, s);
  // LN1 backward: x = layer input (bf16), dres = dh (fp32), dx -> bf16
  if (x_dtype == DT_BF16 && dres_dtype == DT_F32 && st_dtype == DT_BF16)
    return ln_bwd_t<bf16, bf16, float, bf16>(dy, x, mean, rstd, gamma, dres, dx_f32, dx_st,
                                             st_scale, part, rows_per_blk, rows, h, want_dsum, s);
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------------------
// Column partial sums (bias gradients): part[blk][c] = sum over the block's rows.
// ----------------------------------------------------------------------------
// With AMAX the workgroup also writes max|y| over its elements to
// amax[blockIdx.y * gridDim.x + blockIdx.x], and workgroup 0 zeroes the rest
// of the kAmaxFloats entries: the partial maxima of the upstream gradient,
// read in the same pass as its bias gradient's column sums.
template <typename T, bool AMAX = false>
__global__ __launch_bounds__(256) void colsum_kernel(const T* __restrict__ y, int rows,
                                                     int cols, int ld, float* __restrict__ part,
                                                     int rows_per_blk, float* __restrict__ amax) {
  const int j = blockIdx.x * 256 + threadIdx.x;  // vector index (8 columns)
  const bool active = 8 * j < cols;
  if (!AMAX && !active) return;
  float m = 0.f;
  if (active) {
    const int r0 = blockIdx.y * rows_per_blk;
    const int r1 = min(rows, r0 + rows_per_blk);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int r = r0;
    // 8 rows in flight at a time, summed in row order
    for (; r + 8 <= r1; r += 8) {
      float v[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) Vec8<T>::load(y + (size_t)(r + u) * ld + 8 * j, v[u]);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc[e] += v[u][e];
          if constexpr (AMAX) m = fmaxf(m, fabsf(v[u][e]));
        }
    }
    for (; r < r1; ++r) {
      float v[8];
      Vec8<T>::load(y + (size_t)r * ld + 8 * j, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[e] += v[e];
        if constexpr (AMAX) m = fmaxf(m, fabsf(v[e]));
      }
    }
    Vec8<float>::store(part + (size_t)blockIdx.y * cols + 8 * j, acc);
  }
  if constexpr (AMAX) {
    // the entries past the grid's workgroups hold zero (no effect on the maximum)
    const int nwg = gridDim.x * gridDim.y;
    if (blockIdx.x == 0 && blockIdx.y == 0)
      for (int i = nwg + threadIdx.x; i < kAmaxFloats; i += 256) amax[i] = 0.f;
    __shared__ float red[4];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0)
      amax[blockIdx.y * gridDim.x + blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  }
}

int colsum_blocks(int rows, int cols, int* rows_per_blk) {
  const int gx = (cols / 8 + 255) / 256;
  int nblk = (512 + gx - 1) / gx;  // aim for ~512 workgroups
  int rpb = (rows + nblk - 1) / nblk;
  if (rpb < 16) rpb = 16;
  *rows_per_blk = rpb;
  return (rows + rpb - 1) / rpb;
}

hipError_t colsum_partial(int y_dtype, const void* y, int rows, int cols, int ld, float* part,
                          int rows_per_blk, hipStream_t s) {
  const int nblk = (rows + rows_per_blk - 1) / rows_per_blk;
  if (nblk == 0 || cols == 0) return hipSuccess;
  dim3 grid((cols / 8 + 255) / 256, nblk);
  if (y_dtype == DT_BF16)
    colsum_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)y, rows, cols, ld, part, rows_per_blk,
                                             nullptr);
  else if (y_dtype == DT_F16)
    colsum_kernel<f16><<<grid, 256, 0, s>>>((const f16*)y, rows, cols, ld, part, rows_per_blk,
                                            nullptr);
  else
    colsum_kernel<float><<<grid, 256, 0, s>>>((const float*)y, rows, cols, ld, part,
                                              rows_per_blk, nullptr);
  return hipGetLastError();
}

hipError_t colsum_amax_partial(const void* y, int rows, int cols, int ld, float* part,
                               int rows_per_blk, float* amax_part, hipStream_t s) {
  const int nblk = (rows + rows_per_blk - 1) / rows_per_blk;
  const int gx = (cols / 8 + 255) / 256;
  if (cols % 8 || (long)gx * nblk > kAmaxFloats) return hipErrorInvalidValue;
  if (nblk == 0 || cols == 0) return hipErrorInvalidValue;
  colsum_kernel<bf16, true><<<dim3(gx, nblk), 256, 0, s>>>((const bf16*)y, rows, cols, ld, part,
                                                          rows_per_blk, amax_part);
  return hipGetLastError();
}

// out_k[j] (+)= sum_b part[b][k][j] in one launch. A workgroup of 1024
// threads takes 64 consecutive columns of the [nblk][total] partials; its 16
// row groups each sum a contiguous range of block rows in row order (16 loads
// in flight per thread), and one thread per column adds the 16 group sums in
// group order, so the result does not depend on timing. (Two launches, a
// grouped stage and a final one, cost about 8.6 us per reduction on the
// 8.3B shard against 4 us for one.)
constexpr int kRedCols = 64, kRedGroups = 16, kRedUnroll = 16;

__global__ __launch_bounds__(1024) void reduce_partials_kernel(
    const float* __restrict__ part, int nblk, int nout, int width, float* out0, float* out1,
    float* out2, const float* scale, int accumulate) {
  __shared__ float sums[kRedGroups][kRedCols];
  const int total = nout * width;
  const int c = threadIdx.x % kRedCols, grp = threadIdx.x / kRedCols;
  const int idx = blockIdx.x * kRedCols + c;
  const int per = (nblk + kRedGroups - 1) / kRedGroups;
  const int b0 = grp * per, b1 = min(nblk, b0 + per);
  float acc = 0.f;
  if (idx < total) {
    int b = b0;
    for (; b + kRedUnroll <= b1; b += kRedUnroll) {
      float x[kRedUnroll];
#pragma unroll
      for (int u = 0; u < kRedUnroll; ++u) x[u] = part[(size_t)(b + u) * total + idx];
#pragma unroll
      for (int u = 0; u < kRedUnroll; ++u) acc += x[u];
    }
    for (; b < b1; ++b) acc += part[(size_t)b * total + idx];
  }
  sums[grp][c] = acc;
  __syncthreads();
  if (grp != 0 || idx >= total) return;
  float t = 0.f;
#pragma unroll
  for (int q = 0; q < kRedGroups; ++q) t += sums[q][c];
  if (scale) t *= scale[0];
  const int k = idx / width, j = idx - k * width;
  float* o = k == 0 ? out0 : (k == 1 ? out1 : out2);
  if (!o) return;
  o[j] = accumulate ? o[j] + t : t;
}

size_t reduce_scratch_floats(int nblk, int nout, int width) {
  return (size_t)nblk * nout * width;
}

hipError_t reduce_partials(const float* part, int nblk, int nout, int width, float* out0,
                           float* out1, float* out2, int accumulate, hipStream_t s,
                           const float* scale) {
  const int total = nout * width;
  if (total == 0) return hipSuccess;
  reduce_partials_kernel<<<(total + kRedCols - 1) / kRedCols, kRedCols * kRedGroups, 0, s>>>(
      part, nblk, nout, width, out0, out1, out2, scale, accumulate);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Exchange sum (single-GPU stand-in for the all-reduce of fp32 partials).
// ----------------------------------------------------------------------------
struct PartPtrs {
  const float* p[16];
};

template <typename T>
__global__ __launch_bounds__(256) void exchange_sum_kernel(T* __restrict__ dst, PartPtrs parts,
                                                           int nparts, size_t nvec) {
  const size_t j = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= nvec) return;
  float acc[8], v[8];
  Vec8<float>::load(parts.p[0] + 8 * j, acc);
  for (int p = 1; p < nparts; ++p) {
    Vec8<float>::load(parts.p[p] + 8 * j, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += v[e];
  }
  Vec8<T>::store(dst + 8 * j, acc);
}

template <typename T>
__global__ void exchange_sum_tail_kernel(T* dst, PartPtrs parts, int nparts, size_t begin,
                                         size_t count) {
  const size_t i = begin + threadIdx.x;
  if (i >= count) return;
  float acc = parts.p[0][i];
  for (int p = 1; p < nparts; ++p) acc += parts.p[p][i];
  if constexpr (DtOf<T>::v == DT_BF16) dst[i] = f2bf(acc);
  else dst[i] = acc;
}

hipError_t exchange_sum(void* dst, int dst_dtype, const float* const* parts, int nparts,
                        size_t count, hipStream_t s) {
  if (nparts < 1 || nparts > 16) return hipErrorInvalidValue;
  PartPtrs pp = {};
  for (int p = 0; p < nparts; ++p) pp.p[p] = parts[p];
  const size_t nvec = count / 8, tail = count - nvec * 8;
  if (nvec) {
    const unsigned grid = (unsigned)((nvec + 255) / 256);
    if (dst_dtype == DT_BF16)
      exchange_sum_kernel<bf16><<<grid, 256, 0, s>>>((bf16*)dst, pp, nparts, nvec);
    else
      exchange_sum_kernel<float><<<grid, 256, 0, s>>>((float*)dst, pp, nparts, nvec);
  }
  if (tail) {
    if (dst_dtype == DT_BF16)
      exchange_sum_tail_kernel<bf16><<<1, 64, 0, s>>>((bf16*)dst, pp, nparts, nvec * 8, count);
    else
      exchange_sum_tail_kernel<float><<<1, 64, 0, s>>>((float*)dst, pp, nparts, nvec * 8, count);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// bf16 -> fp16 copies of up to 4 tensors in one launch (the weights and the
// upstream gradient the fp16 MFMA GEMMs read). Round to nearest even; every
// bf16 value inside fp16's normal range converts exactly. 8 elements per
// thread per step, grid-stride; tails (count % 8) element by element.
//
// With amax_part (the upstream gradient), the copy is multiplied by a power
// of two S = 2^-e, e = floor(log2(max|x|)) clamped to [-126, 126], taken from
// the kAmaxBlocks partial maxima of amax_kernel: max|S x| lies in [1, 2), so
// the fp16 gradient chain keeps its range and precision whatever the scale
// of the bf16 gradient (bf16 has fp32's exponent range, fp16 only 2^-24 ..
// 65504). Multiplying by S is exact; block 0 writes S and 1/S to scale_out.
// ----------------------------------------------------------------------------
constexpr int kAmaxBlocks = kAmaxFloats;  // one partial maximum per workgroup
static_assert(kAmaxBlocks % 256 == 0, "pow2_scale reduces the partials with a 256-thread block");

struct CvtSegs {
  const bf16* src[4];
  f16* dst[4];
  size_t n[4];
  size_t start[5];  // prefix sums of the vector counts
  int nseg;
  const float* amax_part;  // [kAmaxBlocks] or null
  float* scale_out;        // [2]: S, 1/S (with amax_part)
};

// Partial maxima of |x| over a bf16 tensor of n elements: part[b] for each of
// the kAmaxBlocks workgroups (grid-stride over 8-element vectors).
__global__ __launch_bounds__(256) void amax_kernel(const bf16* __restrict__ x, size_t n,
                                                   float* __restrict__ part) {
  __shared__ float red[4];
  const size_t nvec = n / 8, stride = (size_t)gridDim.x * 256;
  float m = 0.f;
  size_t v = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; v + 3 * stride < nvec; v += 4 * stride) {  // four 16-byte loads in flight
    float f[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) Vec8<bf16>::load(x + 8 * (v + u * stride), f[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(f[u][e]));
  }
  for (; v < nvec; v += stride) {
    float f[8];
    Vec8<bf16>::load(x + 8 * v, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(f[e]));
  }
  if (blockIdx.x == 0)
    for (size_t i = 8 * nvec + threadIdx.x; i < n; i += 256) m = fmaxf(m, fabsf(bf2f(x[i])));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// S from the partial maxima (every block of the conversion computes it).
__device__ float pow2_scale(const float* part, float* red) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < kAmaxBlocks / 256; ++i) m = fmaxf(m, part[i * 256 + threadIdx.x]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  if (!(m > 0.f) || !(m <= 3.4028235e38f)) return 1.f;  // zero, inf or NaN: no scaling
  int e = (int)((__float_as_uint(m) >> 23) & 0xff) - 127;  // floor(log2 m) for normal m
  e = e < -126 ? -126 : (e > 126 ? 126 : e);
  return __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
}

__global__ __launch_bounds__(256) void to_f16_kernel(CvtSegs c) {
  __shared__ float red[4];
  float sc = 1.f;
  if (c.amax_part) {
    sc = pow2_scale(c.amax_part, red);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      c.scale_out[0] = sc;
      c.scale_out[1] = 1.f / sc;  // exact: sc is a power of two in [2^-126, 2^126]
    }
  }
  const size_t total = c.start[c.nseg];
  for (size_t v = (size_t)blockIdx.x * 256 + threadIdx.x; v < total;
       v += (size_t)gridDim.x * 256) {
    int sg = 0;
    while (sg + 1 < c.nseg && v >= c.start[sg + 1]) ++sg;
    const size_t i = 8 * (v - c.start[sg]);
    const bf16* src = c.src[sg] + i;
    f16* dst = c.dst[sg] + i;
    if (i + 8 <= c.n[sg]) {
      float f[8];
      Vec8<bf16>::load(src, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= sc;
      Vec8<f16>::store(dst, f);
    } else {
      for (size_t e = i; e < c.n[sg]; ++e) c.dst[sg][e] = (f16)(bf2f(c.src[sg][e]) * sc);
    }
  }
}

// The unscaled copies (the weights): one 8-element vector per thread and a
// grid covering every vector, so each thread has one load and one store in
// flight and no workgroup loops (a grid-stride loop over a capped grid ran
// these copies at 5.15 TB/s where a plain fp32 copy reaches 5.8).
__global__ __launch_bounds__(256) void to_f16_flat_kernel(CvtSegs c) {
  const size_t v = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= c.start[c.nseg]) return;
  int sg = 0;
  while (sg + 1 < c.nseg && v >= c.start[sg + 1]) ++sg;
  const size_t i = 8 * (v - c.start[sg]);
  if (i + 8 <= c.n[sg]) {
    // the bf16 source is read once and the copy is far larger than the
    // caches: both sides stream (non-temporal), which leaves the LayerNorm
    // input that follows in the last-level cache (1T shard: LN forward
    // 125 -> 109 us, the copies themselves within 1 %)
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(c.src[sg] + i));
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack2h(__uint_as_float(w[q] << 16), __uint_as_float(w[q] & 0xffff0000u));
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(c.dst[sg] + i));
  } else {
    for (size_t e = i; e < c.n[sg]; ++e) c.dst[sg][e] = (f16)bf2f(c.src[sg][e]);
  }
}

hipError_t to_f16(const void* const* src, void* const* dst, const size_t* count, int nseg,
                  hipStream_t s, float* amax_part, float* scale_out, bool amax_ready) {
  if (nseg < 1 || nseg > 4) return hipErrorInvalidValue;
  if ((amax_part == nullptr) != (scale_out == nullptr)) return hipErrorInvalidValue;
  CvtSegs c = {};
  c.nseg = nseg;
  c.start[0] = 0;
  for (int i = 0; i < nseg; ++i) {
    c.src[i] = (const bf16*)src[i];
    c.dst[i] = (f16*)dst[i];
    c.n[i] = count[i];
    c.start[i + 1] = c.start[i] + (count[i] + 7) / 8;
  }
  c.amax_part = amax_part;
  c.scale_out = scale_out;
  if (amax_part) {
    // the maximum over every segment, one launch per segment (the upstream
    // gradient is a single segment); amax_ready: colsum_amax_partial has
    // written the partial maxima already
    if (nseg != 1) return hipErrorInvalidValue;
    if (!amax_ready) {
      amax_kernel<<<kAmaxBlocks, 256, 0, s>>>((const bf16*)src[0], count[0], amax_part);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const size_t total = c.start[nseg];
  if (!total && !amax_part) return hipSuccess;  // (with a scale, one block still writes it)
  if (!amax_part) {
    to_f16_flat_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(c);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)std::max<size_t>(1, std::min<size_t>((total + 255) / 256, 8192));
  to_f16_kernel<<<grid, 256, 0, s>>>(c);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// out = a + bias (per column) + r over a [rows, h] block: the bias and
// residual that the sequence-parallel layout adds after a reduce-scatter.
// a is fp32; bias, r and out take the dtype codes. 8 elements per thread.
// ----------------------------------------------------------------------------
template <typename TB, typename TR, typename TO>
__global__ __launch_bounds__(256) void residual_add_kernel(const float* __restrict__ a,
                                                           const TB* __restrict__ bias,
                                                           const TR* __restrict__ r,
                                                           TO* __restrict__ out, size_t nvec,
                                                           int h) {
  const size_t j = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= nvec) return;
  const int col = (int)((8 * j) % (size_t)h);
  float v[8], b[8], x[8];
  Vec8<float>::load(a + 8 * j, v);
  Vec8<TB>::load(bias + col, b);
  Vec8<TR>::load(r + 8 * j, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] += b[e] + x[e];
  Vec8<TO>::store(out + 8 * j, v);
}

hipError_t residual_add(const float* a, int bias_dtype, const void* bias, int r_dtype,
                        const void* r, int out_dtype, void* out, int rows, int h,
                        hipStream_t s) {
  if (h % 8) return hipErrorInvalidValue;
  const size_t nvec = (size_t)rows * h / 8;
  if (!nvec) return hipSuccess;
  const unsigned grid = (unsigned)((nvec + 255) / 256);
#define TPL_RA(TB, TR, TO)                                                                  \
  residual_add_kernel<TB, TR, TO><<<grid, 256, 0, s>>>(a, (const TB*)bias, (const TR*)r,  \
                                                       (TO*)out, nvec, h);                 \
  return hipGetLastError();
  if (bias_dtype == DT_F32 && r_dtype == DT_F32 && out_dtype == DT_F32) { TPL_RA(float, float, float) }
  if (bias_dtype == DT_BF16 && r_dtype == DT_BF16 && out_dtype == DT_F32) { TPL_RA(bf16, bf16, float) }
  if (bias_dtype == DT_BF16 && r_dtype == DT_F32 && out_dtype == DT_BF16) { TPL_RA(bf16, float, bf16) }
#undef TPL_RA
  return hipErrorInvalidValue;
}

}  // namespace tpl
