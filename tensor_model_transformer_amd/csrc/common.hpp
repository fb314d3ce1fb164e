// Shared device helpers for the gfx950 (CDNA4) kernels of the TP layer shard.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpl {

typedef uint16_t bf16;  // storage of bfloat16 values (upper half of an fp32)
typedef _Float16 f16;   // IEEE binary16 (internal activations of the bf16 path)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16 v) {
  return __uint_as_float(((uint32_t)v) << 16);
}
// Round to nearest even (gfx950 has a hardware conversion for this).
__device__ __forceinline__ bf16 f2bf(float v) {
  return __builtin_bit_cast(bf16, (__bf16)v);
}
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// Two floats to packed fp16, round to nearest even.
__device__ __forceinline__ uint32_t pack2h(float lo, float hi) {
  f16x2 h = {(f16)lo, (f16)hi};
  return __builtin_bit_cast(uint32_t, h);
}
// 8 bf16 values to 8 fp16 values, rounded to nearest even as the weight
// copies of the training path are. Every normal bf16 value inside the fp16
// range is exactly representable; values beyond 65504 become infinite (a
// weight outside fp16's range shows as a non-finite result, never as a
// saturated finite one), values below the normal range round to subnormals.
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack2h(__uint_as_float(w[i] << 16), __uint_as_float(w[i] & 0xffff0000u));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---- 8-element vector I/O for float, bf16 and fp16 storage -------------------
template <typename T> struct Vec8;
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float v[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float v[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};
template <> struct Vec8<bf16> {
  static __device__ __forceinline__ void load(const bf16* p, float v[8]) {
    uint4 a = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16* p, const float v[8]) {
    uint4 a;
    a.x = pack2(v[0], v[1]);
    a.y = pack2(v[2], v[3]);
    a.z = pack2(v[4], v[5]);
    a.w = pack2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = a;
  }
};

template <> struct Vec8<f16> {
  static __device__ __forceinline__ void load(const f16* p, float v[8]) {
    f16x8 a = *reinterpret_cast<const f16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
  }
  static __device__ __forceinline__ void store(f16* p, const float v[8]) {
    uint4 a;
    a.x = pack2h(v[0], v[1]);
    a.y = pack2h(v[2], v[3]);
    a.z = pack2h(v[4], v[5]);
    a.w = pack2h(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = a;
  }
};

// 4-element vector I/O (epilogues write 4 consecutive columns per lane).
template <typename T> struct Vec4;
template <> struct Vec4<float> {
  static __device__ __forceinline__ void load(const float* p, float v[4]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
  static __device__ __forceinline__ void store(float* p, const float v[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct Vec4<bf16> {
  static __device__ __forceinline__ void load(const bf16* p, float v[4]) {
    uint2 a = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(a.x << 16);
    v[1] = __uint_as_float(a.x & 0xffff0000u);
    v[2] = __uint_as_float(a.y << 16);
    v[3] = __uint_as_float(a.y & 0xffff0000u);
  }
  static __device__ __forceinline__ void store(bf16* p, const float v[4]) {
    uint2 a;
    a.x = pack2(v[0], v[1]);
    a.y = pack2(v[2], v[3]);
    *reinterpret_cast<uint2*>(p) = a;
  }
};

template <> struct Vec4<f16> {
  static __device__ __forceinline__ void load(const f16* p, float v[4]) {
    uint2 a = *reinterpret_cast<const uint2*>(p);
    f16x2 x = __builtin_bit_cast(f16x2, a.x), y = __builtin_bit_cast(f16x2, a.y);
    v[0] = (float)x[0]; v[1] = (float)x[1]; v[2] = (float)y[0]; v[3] = (float)y[1];
  }
  static __device__ __forceinline__ void store(f16* p, const float v[4]) {
    uint2 a;
    a.x = pack2h(v[0], v[1]);
    a.y = pack2h(v[2], v[3]);
    *reinterpret_cast<uint2*>(p) = a;
  }
};

// Runtime-typed 4-element access (dtype codes of kernels.hpp: 0 f32, 1 bf16, 2 f16).
__device__ __forceinline__ void load4_dt(const void* base, int dt, size_t off, float v[4]) {
  if (dt == 0) Vec4<float>::load((const float*)base + off, v);
  else if (dt == 1) Vec4<bf16>::load((const bf16*)base + off, v);
  else Vec4<f16>::load((const f16*)base + off, v);
}
// Four fp32 values with a non-temporal (streaming) vector store.
__device__ __forceinline__ void store4_f32_nt(float* p, const float v[4]) {
  typedef float f32x4_nt __attribute__((ext_vector_type(4)));
  const f32x4_nt q = {v[0], v[1], v[2], v[3]};
  __builtin_nontemporal_store(q, reinterpret_cast<f32x4_nt*>(p));
}

__device__ __forceinline__ void store4_dt(void* base, int dt, size_t off, const float v[4]) {
  if (dt == 0) Vec4<float>::store((float*)base + off, v);
  else if (dt == 1) Vec4<bf16>::store((bf16*)base + off, v);
  else Vec4<f16>::store((f16*)base + off, v);
}

// ---- transposing LDS reads (ds_read_b64_tr_b16, gfx950) ----------------------
typedef short v4s __attribute__((ext_vector_type(4)));
#define TPL_LDS_V4S(p) ((__attribute__((address_space(3))) v4s*)(p))

// Four 16-bit values of one column of a row-major LDS tile T (pitch P
// elements), read transposed with ds_read_b64_tr_b16: within each 16-lane
// group, lane j receives T[k0 + i][mb + j] for i = 0..3 when input lane L
// points at T[k0 + L/4][mb + 4*(L%4)].
__device__ __forceinline__ uint2 tr4(const f16* T, int P, int k0, int mb, int L) {
  const f16* p = T + (k0 + (L >> 2)) * P + mb + 4 * (L & 3);
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(TPL_LDS_V4S(p)));
}

// MFMA operand whose rows are columns m0 .. m0+31 of the row-major tile T
// (this lane's column m0 + lane%32) and whose 8 reduction slots are the tile
// rows kA + 0..3 then kB + 0..3, with (kA, kB) given for lane half h.
__device__ __forceinline__ f16x8 tr_frag(const f16* T, int P, int m0, int kA, int kB, int lane) {
  const int g = lane >> 4, L = lane & 15;
  const int mb = m0 + 16 * (g & 1);
  const uint2 a = tr4(T, P, kA, mb, L), b = tr4(T, P, kB, mb, L);
  return __builtin_bit_cast(f16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// ---- reductions ---------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Sum of NV values over the whole block (blockDim.x a multiple of 64, at
// most 1024). `red` must hold 16*NV floats. All threads get the result.
template <int NV>
__device__ __forceinline__ void block_sum(float (&v)[NV], float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = wave_sum(v[i]);
  __syncthreads();  // `red` may still be read by a previous call
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) red[wid * NV + i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += red[w * NV + i];
    v[i] = s;
  }
}

// ---- waits and barriers for loads that stay in flight ----------------------------
// s_waitcnt vmcnt(N), other counters not waited.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// vmcnt(n * L) for a wave-uniform n in 0..3: wait until at most n groups of
// L loads issued after the one waited for are still in flight.
template <int L>
__device__ __forceinline__ void wait_groups(int n) {
  if (n >= 3) wait_vm<3 * L>();
  else if (n == 2) wait_vm<2 * L>();
  else if (n == 1) wait_vm<L>();
  else wait_vm<0>();
}

// Workgroup barrier after this wave's LDS operations completed (lgkmcnt(0));
// global loads (including loads into LDS) may stay in flight, unlike
// __syncthreads(). The empty asm statements keep the compiler from moving
// memory operations across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Buffer descriptor over `bytes` bytes from p: loads past the end read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

// buffer_load_dwordx4 ... lds (16 bytes per lane from the buffer into LDS at
// lds + 16 * lane) written as inline asm. Issued through the builtin, the
// compiler makes every later LDS read that carries no alias information (the
// transposing reads among them) wait for all loads into LDS still in flight,
// which would put each prefetch back in series with the MFMAs. The kernels
// order these loads themselves: wait_groups / wait_vm, then a barrier, before
// a stage is read. Call dma_guard() before a group of these loads.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, const void* lds, int voff) {
  const unsigned a = (unsigned)(size_t)(const __attribute__((address_space(3))) void*)lds;
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(a)
               : "memory");
}
// buffer_load_dword ... lds (4 bytes per lane into lds + 4 * lane), as dma16.
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rs, const void* lds, int voff) {
  const unsigned a = (unsigned)(size_t)(const __attribute__((address_space(3))) void*)lds;
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(a)
               : "memory");
}
// The wait states a VMEM instruction needs after a VALU write of an SGPR it
// reads (a descriptor built from a readfirstlane value), which the compiler
// does not insert in front of inline asm.
__device__ __forceinline__ void dma_guard() { asm volatile("s_nop 4" ::: "memory"); }

// Block pipeline over S LDS stages for tiles loaded straight from HBM
// (dma16 / dma4).
// issue(blk, stage) issues block blk's loads (exactly LPB vector-memory
// instructions per wave) into LDS stage `stage`; compute(blk, stage) consumes
// it. dtl_prologue issues blocks 0 .. S-2; the caller then loads its register
// operands and waits for all its loads (vmcnt(0)), so that no load the
// compiler tracks is pending inside the loop (its own waits would then also
// wait for the prefetches). In the loop, block ib+S-1 is issued, into the
// stage block ib-1 used, before the MFMAs of block ib: S-1 blocks of loads are
// in flight during the MFMAs. Each iteration waits for this wave's loads of
// block ib, then a barrier makes every wave's loads visible and orders the
// overwrite after all reads of block ib-1.
template <int S, typename Issue>
__device__ __forceinline__ void dtl_prologue(int nblk, Issue issue) {
  static_assert(S >= 2 && S <= 4, "stage count");
#pragma unroll
  for (int i = 0; i < S - 1; ++i)
    if (i < nblk) issue(i, i);
}
template <int S, int LPB, typename Issue, typename Compute>
__device__ __forceinline__ void dtl_loop(int nblk, Issue issue, Compute compute) {
  int stage = 0;
  for (int ib = 0; ib < nblk; ++ib) {
    wait_groups<LPB>(min(S - 2, nblk - 1 - ib));
    lds_barrier();
    if (ib + S - 1 < nblk) issue(ib + S - 1, stage == 0 ? S - 1 : stage - 1);
    compute(ib, stage);
    stage = stage == S - 1 ? 0 : stage + 1;
  }
}

// ---- GeLU (exact erf form, or the tanh approximation) ---------------------------
// erf(x) for x >= 0 from Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26 (rational approximation in t = 1/(1 + p x) times
// exp(-x^2), absolute error at most 1.5e-7), given ex2 = exp(-x^2). Branch
// free, and the exponential is shared with the GeLU derivative.
__device__ __forceinline__ float erf_as7126(float ax, float ex2) {
  const float t = __builtin_amdgcn_rcpf(1.f + 0.3275911f * ax);
  const float poly =
      t * (0.254829592f +
           t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  return 1.f - poly * ex2;
}

// Exact-form GeLU, u * Phi(u) with Phi(u) = (1 + erf(u / sqrt 2)) / 2, and
// its derivative Phi(u) + u phi(u), phi(u) = exp(-u^2 / 2) / sqrt(2 pi).
__device__ __forceinline__ float gelu_f(float u, int tanh_form) {
  if (tanh_form) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    return 0.5f * u * (1.f + tanhf(c * (u + 0.044715f * u * u * u)));
  }
  const float ax = fabsf(u) * 0.7071067811865476f;
  const float ex2 = exp2f(-1.4426950408889634f * ax * ax);  // exp(-u^2/2)
  const float er = copysignf(erf_as7126(ax, ex2), u);
  return 0.5f * u * (1.f + er);
}
// GeLU(u) and GeLU'(u) together (the erf and the exponential shared).
__device__ __forceinline__ void gelu_and_grad(float u, int tanh_form, float* z, float* gp) {
  if (tanh_form) {
    const float c = 0.7978845608028654f;
    const float th = tanhf(c * (u + 0.044715f * u * u * u));
    *z = 0.5f * u * (1.f + th);
    *gp = 0.5f * (1.f + th) + 0.5f * u * (1.f - th * th) * c * (1.f + 0.134145f * u * u);
    return;
  }
  const float ax = fabsf(u) * 0.7071067811865476f;
  const float ex2 = exp2f(-1.4426950408889634f * ax * ax);
  const float cdf = 0.5f * (1.f + copysignf(erf_as7126(ax, ex2), u));  // Phi(u)
  *z = u * cdf;
  *gp = cdf + u * 0.3989422804014327f * ex2;
}
// GeLU'(u) alone: the same arithmetic as gelu_and_grad (bit for bit).
__device__ __forceinline__ float gelu_grad_f(float u, int tanh_form) {
  float z, gp;
  gelu_and_grad(u, tanh_form, &z, &gp);
  return gp;
}

}  // namespace tpl
