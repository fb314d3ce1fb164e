// Internal launch interface of the HIP kernels (host side). Not part of the
// C ABI: tp_layer.cpp is the only caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace tpl {

// Element types. The bf16 layer keeps bf16 at its boundary (inputs, weights,
// output, input gradient) and fp16 for internal activations and gradients;
// the fp32 layer is fp32 throughout.
enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

// ---------------------------------------------------------------------------
// LayerNorm and reductions (norm.hip)
// ---------------------------------------------------------------------------
// y = gamma * (x - mean) * rstd + beta per row of h; saves mean and rstd.
// x is `x_dtype`, gamma/beta are `p_dtype`, y is `y_dtype`. If x_copy != NULL
// the fp32 value of x is also written there (keeps a caller's summed h_mid).
// mean and rstd may be NULL.
hipError_t ln_fwd(int x_dtype, int p_dtype, int y_dtype, const void* x, const void* gamma,
                  const void* beta, void* y, float* mean, float* rstd,
                  float* x_copy, int rows, int h, float eps, hipStream_t s);

// LayerNorm backward plus the residual-gradient add:
//   dx = rstd * (g - mean(g) - xhat * mean(g * xhat)) + dres,  g = dy * gamma
// dy fp32; x is `x_dtype`; dres is `dres_dtype`; gamma is `p_dtype`.
// Writes dx as fp32 (dx_f32, optional) and/or `st_dtype` (dx_st, optional);
// st_scale (optional, device fp32) multiplies the dx_st copy only.
// Column partial sums over row blocks go to part [nblk][3][h]:
//   0: sum dy*xhat (dgamma), 1: sum dy (dbeta), 2: sum dx (if want_dsum).
hipError_t ln_bwd(int p_dtype, const float* dy, int x_dtype, const void* x,
                  const float* mean, const float* rstd, const void* gamma,
                  int dres_dtype, const void* dres, float* dx_f32, int st_dtype, void* dx_st,
                  const float* st_scale, float* part, int rows_per_blk, int rows, int h,
                  int want_dsum, hipStream_t s);
int ln_bwd_blocks(int rows, int h, int* rows_per_blk);

// Column partial sums of a [rows, cols] matrix (leading dim ld) over row
// blocks: part[blk][cols].
hipError_t colsum_partial(int y_dtype, const void* y, int rows, int cols, int ld,
                          float* part, int rows_per_blk, hipStream_t s);
int colsum_blocks(int rows, int cols, int* rows_per_blk);
// colsum_partial of a bf16 matrix that also writes the kAmaxFloats partial
// maxima of |y| to_f16 takes with amax_ready (cols % 8 == 0; at most
// kAmaxFloats workgroups, else hipErrorInvalidValue; rows, cols > 0).
hipError_t colsum_amax_partial(const void* y, int rows, int cols, int ld, float* part,
                               int rows_per_blk, float* amax_part, hipStream_t s);
// out[rows, h] = a (fp32) + bias[h] + r; dtypes DT_F32 / DT_BF16 as listed in
// norm.hip (fp32 bias/r/out, or bf16 bias with bf16 r -> fp32 out, or bf16
// bias with fp32 r -> bf16 out).
hipError_t residual_add(const float* a, int bias_dtype, const void* bias, int r_dtype,
                        const void* r, int out_dtype, void* out, int rows, int h,
                        hipStream_t s);

// out_k[j] (+)= scale * sum_b part[b][k][j] for k < nout (part is
// [nblk][nout][width]; scale: optional device fp32, 1 when null), summed in
// a fixed order (deterministic). reduce_scratch_floats(nblk, nout, width) is
// the size of part in floats.
hipError_t reduce_partials(const float* part, int nblk, int nout, int width,
                           float* out0, float* out1, float* out2, int accumulate,
                           hipStream_t s, const float* scale = nullptr);
size_t reduce_scratch_floats(int nblk, int nout, int width);

// dst[k][i] = fp16(src[k][i]) for bf16 src, i < count[k], k < nseg (1..4).
// With amax_part (kAmaxFloats floats of scratch) and scale_out (2 floats),
// nseg must be 1 and dst = fp16(S * src) with the power of two S that puts
// max|S src| in [1, 2); scale_out receives S and 1/S (device fp32). With
// amax_ready the partial maxima are in amax_part already (colsum_amax_partial).
constexpr int kAmaxFloats = 1024;
hipError_t to_f16(const void* const* src, void* const* dst, const size_t* count, int nseg,
                  hipStream_t s, float* amax_part = nullptr, float* scale_out = nullptr,
                  bool amax_ready = false);

// dst[i] = sum_p parts[p][i]  (fp32 sum in order), written as dst_dtype.
hipError_t exchange_sum(void* dst, int dst_dtype, const float* const* parts,
                        int nparts, size_t count, hipStream_t s);

// ---------------------------------------------------------------------------
// GEMM (gemm.hip): C[M,N] = A[M,K] @ B[K,N] with a fused epilogue.
// ---------------------------------------------------------------------------
enum { EPI_STORE = 0, EPI_BIAS_GELU = 1, EPI_DGELU = 2, EPI_SPLIT16 = 3, EPI_GELU_GRAD = 4 };

struct GemmArgs {
  // Arithmetic: DT_F32 (fp32 FMA, fp32 operands) or DT_F16 (fp16 MFMA,
  // fp32 accumulate, fp16 operands).
  int math;
  int M, N, K;
  // A(m,k) = A[m*lda + k] if a_kmajor else A[k*lda + m]
  const void* A; long lda; int a_kmajor; int a_dtype;
  // B(k,n) = B[n*ldb + k] if b_kmajor else B[k*ldb + n]
  const void* B; long ldb; int b_kmajor; int b_dtype;
  // epilogue, per element: v = acc (+ bias[n]) (+ resid[m,n]);
  //   EPI_BIAS_GELU: C = GeLU'(v) (kept for the backward), C2 = GeLU(v);
  //   EPI_GELU_GRAD: C = GeLU'(v);  EPI_DGELU: C = v * aux[m,n] (aux = GeLU'(u));
  //   EPI_SPLIT16: C = fp16(v), C2 = fp16(v - fp16(v)) (both fp16; v = C + C2
  //   to about 2^-22 relative);
  //   accumulate: C (fp32) += v.
  int epi;
  const void* bias; int bias_dtype;    // [N]
  const void* resid; long ldr; int resid_dtype;
  void* C; long ldc; int c_dtype;
  void* C2; long ldc2; int c2_dtype;
  const void* aux; long ldaux; int aux_dtype;
  int gelu_tanh;
  int accumulate;
  int split;                           // split-K factor (>= 1)
  // fp32 scratch of ws_floats floats: split-K partials (split > 1), or the
  // stream-K pieces of a GEMM the launcher schedules that way (gemm_ws_floats
  // tells how much either needs; without enough the launcher does not use
  // stream-K). Null: neither.
  float* ws;
  size_t ws_floats;
  // optional device fp32 factor applied to the accumulator first (v = scale *
  // acc, before bias and residual): undoes the power-of-two scaling of the
  // backward's fp16 gradient chain in the GEMMs that leave it
  const float* scale;
  // fp32 C written with non-temporal (streaming) stores: for outputs that no
  // later kernel of the step reads (the weight gradients), so the writes do
  // not displace operands from the caches
  int stream_out;
};
hipError_t gemm(const GemmArgs& g, hipStream_t s);
// Split-K factor the launcher would pick for a weight-gradient GEMM g.
int gemm_choose_split(const GemmArgs& g);
// Scratch floats g needs (split-K partials for g.split > 1, stream-K pieces
// when its shape is scheduled that way); 0 for neither.
size_t gemm_ws_floats(const GemmArgs& g);

// ---------------------------------------------------------------------------
// Attention (attn.hip). qkv: [batch*seq, 3*Hl*D] head-interleaved;
// o, dO: [batch*seq, Hl*D]; lse2, delta: [batch, Hl, seq] fp32.
// dtype: DT_F32 (fp32 kernels) or DT_F16 (fp16 operands, MFMA, fp32 accumulate).
// mask: 0 causal, 1 padding (valid_len[batch] keys).
// qkv_lo (DT_F16 only, may be null): the fp16 rounding residuals of qkv, same
// layout; when given, the scores use Q K^T ~ Qh Kh^T + Qh Kl^T + Ql Kh^T.
// ---------------------------------------------------------------------------
hipError_t attn_fwd(int dtype, const void* qkv, const void* qkv_lo, void* o, float* lse2,
                    const int* valid_len, int batch, int seq, int Hl, int D,
                    int mask, hipStream_t s);
hipError_t attn_bwd(int dtype, const void* qkv, const void* qkv_lo, const void* o,
                    const void* dO, const float* lse2, float* delta, void* dqkv,
                    const int* valid_len, int batch, int seq, int Hl, int D,
                    int mask, hipStream_t s);

// ---------------------------------------------------------------------------
// Decode (decode.hip): one new token per sequence, M = decode batch <= 128.
// ---------------------------------------------------------------------------
enum { GEMV_EPI_OUT = 0, GEMV_EPI_GELU = 1 };

// Y[M, N] = X[M, K] @ W[K, N] (row-major, row strides K and N): workgroups
// own `strip`-column strips and kc rows of K staged `chunk` rows at a time,
// the K range split into nsplit pieces (gemv_plan). math DT_F16: X fp16,
// W bf16, fp16 MFMA; DT_F32: X and W fp32 (strip 64). With raw = 1 the
// launch only writes the split partials (also for nsplit = 1) for a consumer
// that sums them itself; otherwise the partials are summed in split order and
// the epilogue writes out.
struct GemvArgs {
  int M, N, K;
  const void* X;
  const void* W;
  int strip, chunk, kc, nsplit;
  int raw;
  float* part;   // [nsplit][M][N] fp32 when nsplit > 1 or raw
  int epi;
  const void* bias; int bias_dt;     // [N] or null
  // GEMV_EPI_OUT: out = v (+ bias) (+ resid); GEMV_EPI_GELU: out = GeLU(v + bias)
  const void* resid; int resid_dt;   // [M, N] or null
  void* out; int out_dt;             // [M, N]
  int gelu_tanh;
};
void gemv_plan(int math, int M, int N, int K, int* strip, int* chunk, int* kc, int* nsplit);
hipError_t gemv(const GemvArgs& g, int math, hipStream_t s);

// Decode attention: waves per launch targeted, maximum cache slices per head.
constexpr int kDecWaves = 4096;
constexpr int kDecMaxSplit = 64;
struct DecAttnArgs {
  // the QKV GEMV's raw split partials [qkv_ns][batch][3*Hl*D] (head-interleaved
  // columns) and its bias: the new token's q, k, v are their sum
  const float* qkv_part; int qkv_ns;
  const void* b_qkv; int bias_dt;
  void* kc; void* vc;              // [batch, Hl, cache_len, D] (fp16 or fp32); row pos written
  _Float16* klo;                   // split scores: fp16 residuals of kc, else null
  const int* pos;                  // [batch]: keys 0..pos attend (clamped to the cache)
  int batch, Hl, cache_len, nsplit, chunk;
  float scale_log2;                // log2(e) / sqrt(D)
  float* part;                     // [batch*Hl][nsplit][D+2] when nsplit > 1
  void* o; int o_dt;               // [batch, Hl*D]
};
// Slices per (sequence, head) for a cache of cache_len rows; *chunk = rows per slice.
int dec_attn_split(int batch, int Hl, int cache_len, int* chunk);
hipError_t dec_attn(int dtype, const DecAttnArgs& g, int D, int split, hipStream_t s);
// h_mid[rows, h] = sum_s part[s] + bias + x (fp32), y = LN(h_mid) (gamma, beta):
// the output projection's split partials [ns][rows][h] finished together with
// the second LayerNorm. dtype DT_F16: bias/x/gamma/beta bf16, y fp16; DT_F32:
// all fp32.
hipError_t dec_resid_ln(int dtype, const float* part, int ns, const void* bias, const void* x,
                        float* h_mid, const void* gamma, const void* beta, void* y, int rows,
                        int h, float eps, hipStream_t s);
// Copies K, V (and K residuals) of a forward's qkv [batch*seq, 3*Hl*D] into caches.
hipError_t kv_fill(int dtype, const void* qkv, const void* qkv_lo, void* kc, void* vc, void* klo,
                   int batch, int seq, int Hl, int D, int cache_len, hipStream_t s);

}  // namespace tpl
