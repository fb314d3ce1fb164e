// C ABI of the tensor-parallel layer shard: argument checks, workspace plan
// and the phase driver that enqueues the HIP kernels in order.
//
// Phase structure: "Megatron-LM: GPU-Cluster Training Parallelism", section
// "Paper 1: The f/g Conjugate Operators" -- two exchanges forward (g after the
// row-parallel output projection and after FC2) and two backward (f before
// the input gradients of the column-parallel QKV and FC1 leave the rank).
// TP_ALL takes every exchange as the identity; the split phases stop at each
// exchange so a caller can sum the ranks' fp32 partials in between.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <initializer_list>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/tp_layer.h"
#include "kernels.hpp"

using namespace tpl;

namespace {

constexpr size_t kAlign = 256;

// TP_SCORES_AUTO keeps the fp16 residuals of Q and K from this hidden size
// on. With N(0, 0.02) weights the scores' spread grows like hidden * 0.02^2,
// and at hidden 25600 (spread about 10) the fp16 rounding of Q and K alone
// moves softmax outputs by several tenths of a percent, visible in the
// gradient of W_qkv; at hidden <= 3072 the spread is about 1.
constexpr int kSplitScoresHidden = 8192;
// opts.overlap = TP_OVERLAP_AUTO overlaps from this width (measured: the 1T
// shard's step about 2 % faster with the two overlaps, the 1.2B and 8.3B
// shards' 0.5 % slower with the backward one).
constexpr int kOverlapHidden = 8192;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Region {
  size_t off = 0, bytes = 0;
};

struct ProfRec {
  int cls;
  hipEvent_t a, b;
  double flops, bytes;
};

struct Prof {
  bool on = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  long launches[TP_K_COUNT] = {};
  double ms[TP_K_COUNT] = {}, flops[TP_K_COUNT] = {}, bytes[TP_K_COUNT] = {};
};

}  // namespace

struct tp_layer {
  int hidden, heads, ffn, seq, batch, t, rank, dtype, mask;
  float eps;
  int gelu_tanh;
  bool dx_f32;  // dx written in fp32 (else in the storage dtype)
  bool split_scores;  // qkv also kept as fp16 residuals; scores from three products
  bool recompute_fc1;  // GeLU'(u) of FC1 recomputed in backward, not kept
  bool sp;             // sequence-parallel layout (phases TP_*_SP_*)
  int nc;              // rows of this rank's token chunk in that layout (n / t)
  // derived
  int n, dh, Hl, hl, fl, esz;
  int sdt;   // storage type at the boundary (x, params, out, dx): DT_BF16 or DT_F32
  int adt;   // internal activations and their gradients: DT_F16 or DT_F32
  // workspace regions
  Region mean1, rstd1, a, qkv, qkv_lo, o, lse2, h_mid, mean2, rstd2, c, u, z;
  Region du, dc, dh_f, dh_s, dO, delta, dqkv, da, part, splitk;
  // stream-K pieces of the GEMMs on the caller's stream (forward, data
  // gradients); splitk holds the weight gradients' split-K partials
  Region skp;
  // column-sum partials of the bias gradients (apart from the LayerNorm
  // backward's, which a bias gradient may follow in the same phase)
  Region part2;
  // fp16 copies of the bf16 weights (made by the forward, read again by the
  // backward) and of the upstream gradient: the MFMA GEMMs read fp16 only
  Region w16_qkv, w16_o, w16_fc1, w16_fc2, dout16;
  // Power-of-two scale S of the backward's fp16 gradient chain (bf16 layers):
  // the partial maxima of |dout| and then S, 1/S. The MLP backward derives S
  // from dout; every fp16 gradient tensor (the dout copy, du, the fp16 copy
  // of dh, dO, dqkv) holds S times its value, and every GEMM or reduction
  // that leaves the chain for fp32 multiplies by 1/S (exact).
  Region gscale;
  size_t ws_bytes;
  int split_w2, split_w1, split_wo, split_wqkv;
  // allowed query-key pairs per forward, for the profile's attention FLOPs:
  // causal from the shape; padding as given to tp_layer_profile (0 = unknown)
  double attn_pairs;
  Prof prof;
  // Side stream of TP_ALL with opts.overlap: in the forward the fp16 copies of
  // the MLP weights (fc1_ev marks the end of W_fc1's), in the backward the
  // output projection's weight gradient, each beside the caller's stream;
  // every call joins it back before returning. Created on the current device
  // by the first call that uses it; null if that failed (then everything
  // runs on the caller's stream).
  hipStream_t side = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr, fc1_ev = nullptr;
  bool side_tried = false;
  bool overlap = false;  // independent pieces of TP_ALL on the side stream (opts)
  // decode (one row per sequence): its own workspace plan
  struct Dec {
    Region a, apart, o, h_mid, c, z, gpart;
    size_t bytes;
    int strip[4], chunk[4], kc[4], ns[4];  // GEMV tiling and K split: qkv, w_o, fc1, fc2
  } dec;
};

namespace {

GemmArgs gemm_base(const tp_layer* L) {
  GemmArgs g = {};
  g.math = L->adt;  // fp16 MFMA for the bf16 layer, fp32 FMA for the fp32 layer
  g.a_dtype = g.b_dtype = g.c_dtype = g.c2_dtype = g.aux_dtype = L->adt;
  g.bias_dtype = g.resid_dtype = L->sdt;
  g.split = 1;
  g.gelu_tanh = L->gelu_tanh;
  return g;
}

// Weight-gradient GEMM: C[M,N] (+)= X^T @ Y with X [n, M], Y [n, N] (both
// token-major, i.e. contiguous along M and N).
GemmArgs wgrad_args(const tp_layer* L, int M, int N, const void* X, const void* Y, float* C,
                    int accumulate) {
  GemmArgs g = gemm_base(L);
  g.M = M;
  g.N = N;
  g.K = L->n;
  g.A = X;
  g.lda = M;
  g.a_kmajor = 0;
  g.B = Y;
  g.ldb = N;
  g.b_kmajor = 0;
  g.C = C;
  g.ldc = N;
  g.c_dtype = DT_F32;
  g.accumulate = accumulate;
  g.stream_out = 1;  // the caller's gradient: no later kernel of the step reads it
  return g;
}

void plan(tp_layer* L) {
  size_t off = 0;
  auto take = [&](Region& r, size_t bytes) {
    r.off = off;
    r.bytes = bytes;
    off += align_up(bytes);
  };
  const size_t n = (size_t)L->n, h = (size_t)L->hidden, e = (size_t)L->esz;
  const size_t stats = (size_t)L->batch * L->Hl * L->seq * 4;
  take(L->mean1, n * 4);
  take(L->rstd1, n * 4);
  take(L->a, n * h * e);
  take(L->qkv, n * 3 * L->hl * e);
  take(L->qkv_lo, L->split_scores ? n * 3 * L->hl * 2 : 0);
  take(L->o, n * L->hl * e);
  take(L->lse2, stats);
  take(L->h_mid, n * h * 4);
  take(L->mean2, n * 4);
  take(L->rstd2, n * 4);
  take(L->c, n * h * e);
  // The "u" region keeps GeLU'(u), the derivative of the FC1 activation at
  // its pre-activation u (all the backward needs of u), from forward unless it
  // is recomputed in backward. du has its own buffer, so a backward leaves the
  // forward's saved tensors intact (it can be run again, e.g. to accumulate);
  // with recompute, du and the recomputed GeLU'(u) share one buffer placed
  // over the attention-backward buffers, which are not yet live while du is.
  take(L->u, L->recompute_fc1 ? 0 : n * L->fl * e);
  take(L->z, n * L->fl * e);
  if (!L->recompute_fc1) take(L->du, n * L->fl * e);
  take(L->dc, n * h * 4);
  take(L->dh_f, n * h * 4);
  take(L->dh_s, n * h * e);
  take(L->dO, n * L->hl * e);
  take(L->delta, stats);
  take(L->dqkv, n * 3 * L->hl * e);
  take(L->da, n * h * 4);
  if (L->recompute_fc1) {
    const size_t need = n * L->fl * e, span = off - L->dh_f.off;
    if (need > span) {
      Region pad;
      take(pad, need - span);
    }
    L->du.off = L->dh_f.off;
    L->du.bytes = need;
  }
  // reduction partials: LayerNorm [nblk][3][h]; column sums [nblk][cols]
  int rpb;
  size_t part = reduce_scratch_floats(ln_bwd_blocks(L->n, L->hidden, &rpb), 3, L->hidden);
  const int cols[3] = {L->hidden, L->fl, 3 * L->hl};
  for (int i = 0; i < 3; ++i) {
    const size_t p = reduce_scratch_floats(colsum_blocks(L->n, cols[i], &rpb), 1, cols[i]);
    if (p > part) part = p;
  }
  take(L->part, part * 4);
  size_t part2 = 0;
  for (int i = 0; i < 3; ++i)
    part2 = std::max(part2, reduce_scratch_floats(colsum_blocks(L->n, cols[i], &rpb), 1, cols[i]));
  take(L->part2, part2 * 4);
  // split-K partials of the weight gradients
  size_t sk = 0;
  struct W {
    int M, N;
    int* split;
  } ws[4] = {{L->fl, L->hidden, &L->split_w2},
             {L->hidden, L->fl, &L->split_w1},
             {L->hl, L->hidden, &L->split_wo},
             {L->hidden, 3 * L->hl, &L->split_wqkv}};
  for (auto& w : ws) {
    GemmArgs g = wgrad_args(L, w.M, w.N, nullptr, nullptr, nullptr, 0);
    *w.split = gemm_choose_split(g);
    g.split = *w.split;
    sk = std::max(sk, gemm_ws_floats(g) * 4);
  }
  take(L->splitk, sk);
  // the other GEMMs (M = n tokens): forward QKV, W_o, FC1, FC2 and the data
  // gradients of FC2, FC1, W_o, QKV
  size_t skp = 0;
  const int MNK[8][2] = {{3 * L->hl, L->hidden}, {L->hidden, L->hl}, {L->fl, L->hidden},
                         {L->hidden, L->fl}, {L->fl, L->hidden}, {L->hidden, L->fl},
                         {L->hl, L->hidden}, {L->hidden, 3 * L->hl}};
  for (auto& d : MNK) {
    GemmArgs g = gemm_base(L);
    g.M = L->n; g.N = d[0]; g.K = d[1];
    skp = std::max(skp, gemm_ws_floats(g) * 4);
  }
  take(L->skp, skp);
  const bool cvt = L->sdt == DT_BF16;
  take(L->w16_qkv, cvt ? h * 3 * L->hl * 2 : 0);
  take(L->w16_o, cvt ? (size_t)L->hl * h * 2 : 0);
  take(L->w16_fc1, cvt ? h * L->fl * 2 : 0);
  take(L->w16_fc2, cvt ? (size_t)L->fl * h * 2 : 0);
  take(L->dout16, cvt ? n * h * 2 : 0);
  take(L->gscale, cvt ? (kAmaxFloats + 2) * 4 : 0);
  L->ws_bytes = off;
}

// Decode workspace: the rows of one token per sequence (B = micro_batch), the
// GEMV split-K partials (one buffer, the GEMVs run one after another) and the
// attention slice partials.
void plan_decode(tp_layer* L) {
  tp_layer::Dec& d = L->dec;
  size_t off = 0;
  auto take = [&](Region& r, size_t bytes) {
    r.off = off;
    r.bytes = bytes;
    off += align_up(bytes);
  };
  const size_t B = (size_t)L->batch, h = (size_t)L->hidden, e = (size_t)L->esz;
  const int MNK[4][2] = {{3 * L->hl, L->hidden}, {L->hidden, L->hl}, {L->fl, L->hidden},
                         {L->hidden, L->fl}};
  size_t gp = 0;
  for (int i = 0; i < 4; ++i) {
    gemv_plan(L->adt, L->batch, MNK[i][0], MNK[i][1], &d.strip[i], &d.chunk[i], &d.kc[i],
              &d.ns[i]);
    gp = std::max(gp, (size_t)d.ns[i] * B * MNK[i][0] * 4);
  }
  const size_t pairs = B * L->Hl;
  take(d.a, B * h * e);
  take(d.apart, ((size_t)kDecWaves + pairs) * (L->dh + 2) * 4);
  take(d.o, B * L->hl * e);
  take(d.h_mid, B * h * 4);
  take(d.c, B * h * e);
  take(d.z, B * L->fl * e);
  take(d.gpart, gp);
  d.bytes = off;
}

template <typename T>
T* at(void* ws, const Region& r) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + r.off);
}

// The fp16 residuals of qkv, or null when scores use qkv alone.
void* qkv_lo(tp_layer* L, void* ws) { return L->split_scores ? at<void>(ws, L->qkv_lo) : nullptr; }

// A weight as the GEMMs read it: the fp16 copy for a bf16 layer, else itself.
const void* wmat(tp_layer* L, void* ws, const Region& copy, const void* w) {
  return L->sdt == DT_BF16 ? at<void>(ws, copy) : w;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    if (!p) return TP_ERR_ARG;
    if (!aligned(p)) return TP_ERR_ALIGN;
  }
  return TP_OK;
}

int check_params(const tp_layer* L, const tp_params* p) {
  if (!p) return TP_ERR_ARG;
  int e = check_ptrs({p->ln1_gamma, p->ln1_beta, p->w_qkv, p->b_qkv, p->w_o, p->b_o,
                      p->ln2_gamma, p->ln2_beta, p->w_fc1, p->b_fc1, p->w_fc2, p->b_fc2});
  if (e) return e;
  if (L->mask == TP_MASK_PADDING) return check_ptrs({p->valid_len});
  return TP_OK;
}

int check_ws(const tp_layer* L, void* ws, size_t bytes) {
  if (!ws || bytes < L->ws_bytes) return TP_ERR_WORKSPACE;
  if (!aligned(ws)) return TP_ERR_ALIGN;
  return TP_OK;
}

#define HIP_TRY(x)                        \
  do {                                    \
    if ((x) != hipSuccess) return TP_ERR_HIP; \
  } while (0)

// Brackets one launch group with a pair of events when profiling is on.
struct Scope {
  tp_layer* L;
  hipStream_t s;
  int cls;
  double fl, by;
  hipEvent_t a = nullptr, b = nullptr;
  static hipEvent_t get(Prof& p) {
    if (!p.pool.empty()) {
      hipEvent_t e = p.pool.back();
      p.pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  Scope(tp_layer* L_, hipStream_t s_, int cls_, double fl_, double by_)
      : L(L_), s(s_), cls(cls_), fl(fl_), by(by_) {
    if (!L->prof.on) return;
    a = get(L->prof);
    b = get(L->prof);
    if (!a || !b || hipEventRecord(a, s) != hipSuccess) {
      if (a) L->prof.pool.push_back(a);
      if (b) L->prof.pool.push_back(b);
      a = b = nullptr;
    }
  }
  ~Scope() {
    if (!a) return;
    (void)hipEventRecord(b, s);
    L->prof.recs.push_back({cls, a, b, fl, by});
  }
};

double gemm_bytes(const tp_layer* L, const GemmArgs& g) {
  const double e = L->esz;
  double b = ((double)g.M * g.K + (double)g.K * g.N) * e;
  b += (double)g.M * g.N * (g.c_dtype == DT_F32 ? 4.0 : e) * (g.accumulate ? 2.0 : 1.0);
  if (g.resid) b += (double)g.M * g.N * (g.resid_dtype == DT_F32 ? 4.0 : e);
  if (g.C2) b += (double)g.M * g.N * e;
  if (g.aux) b += (double)g.M * g.N * e;
  return b;
}

// Runs one GEMM with its scratch: the weight gradients (the backward's side
// stream) use the split-K region, every other GEMM (the caller's stream) the
// stream-K region, so GEMMs running concurrently on the two streams never
// share scratch.
int run_gemm(tp_layer* L, GemmArgs g, hipStream_t s, void* ws, bool wgrad = false) {
  const Region& r = wgrad ? L->splitk : L->skp;
  g.ws = r.bytes ? at<float>(ws, r) : nullptr;
  g.ws_floats = r.bytes / sizeof(float);
  Scope ps(L, s, TP_K_GEMM, 2.0 * g.M * g.N * (double)g.K, gemm_bytes(L, g));
  HIP_TRY(gemm(g, s));
  return TP_OK;
}

// The side stream (created on first use) when the handle overlaps
// (opts.overlap), else the caller's stream; also the caller's
// stream while profiling (each event pair then brackets its launch group
// alone) or if the side stream could not be created.
hipStream_t side_stream(tp_layer* L, hipStream_t s) {
  if (L->prof.on || !L->overlap) return s;
  if (!L->side_tried) {
    L->side_tried = true;
    hipStream_t st = nullptr;
    hipEvent_t a = nullptr, b = nullptr, c = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) == hipSuccess &&
        hipEventCreateWithFlags(&a, hipEventDisableTiming) == hipSuccess &&
        hipEventCreateWithFlags(&b, hipEventDisableTiming) == hipSuccess &&
        hipEventCreateWithFlags(&c, hipEventDisableTiming) == hipSuccess) {
      L->side = st;
      L->fork_ev = a;
      L->join_ev = b;
      L->fc1_ev = c;
    } else {
      if (c) (void)hipEventDestroy(c);
      if (b) (void)hipEventDestroy(b);
      if (a) (void)hipEventDestroy(a);
      if (st) (void)hipStreamDestroy(st);
      (void)hipGetLastError();
    }
  }
  return L->side ? L->side : s;
}

// side waits for everything enqueued on s so far.
int fork_to(tp_layer* L, hipStream_t s, hipStream_t side) {
  if (side == s) return TP_OK;
  HIP_TRY(hipEventRecord(L->fork_ev, s));
  HIP_TRY(hipStreamWaitEvent(side, L->fork_ev, 0));
  return TP_OK;
}

// s waits for everything enqueued on side so far.
int join_from(tp_layer* L, hipStream_t s, hipStream_t side) {
  if (side == s) return TP_OK;
  HIP_TRY(hipEventRecord(L->join_ev, side));
  HIP_TRY(hipStreamWaitEvent(s, L->join_ev, 0));
  return TP_OK;
}

// The gradient chain's S and 1/S (device fp32), or null for an fp32 layer.
const float* chain_scale(tp_layer* L, void* ws) {
  return L->sdt == DT_BF16 ? at<float>(ws, L->gscale) + kAmaxFloats : nullptr;
}
const float* chain_unscale(tp_layer* L, void* ws) {
  return L->sdt == DT_BF16 ? at<float>(ws, L->gscale) + kAmaxFloats + 1 : nullptr;
}

// bf16 -> fp16 copies (nothing to do for an fp32 layer). With scaled, the
// single tensor is the upstream gradient, copied times the chain's S (which
// this call derives from it and stores in the workspace).
int to_f16_copies(tp_layer* L, std::initializer_list<const void*> src,
                  std::initializer_list<const Region*> dst, std::initializer_list<size_t> count,
                  void* ws, hipStream_t s, bool scaled = false, bool amax_ready = false) {
  if (L->sdt != DT_BF16) return TP_OK;
  const void* sp[4];
  void* dp[4];
  size_t np[4];
  int k = 0;
  double bytes = 0;
  auto d = dst.begin();
  auto c = count.begin();
  for (const void* x : src) {
    sp[k] = x;
    dp[k] = at<void>(ws, **d++);
    np[k] = *c++;
    bytes += 4.0 * np[k];
    ++k;
  }
  if (scaled && !amax_ready) bytes += 2.0 * np[0];  // the maximum's pass over the gradient
  Scope ps(L, s, TP_K_CONVERT, 0, bytes);
  float* gs = scaled ? at<float>(ws, L->gscale) : nullptr;
  HIP_TRY(to_f16(sp, dp, np, k, s, gs, scaled ? gs + kAmaxFloats : nullptr, amax_ready));
  return TP_OK;
}

// ---- forward pieces --------------------------------------------------------
// x -> a -> qkv -> o -> (o @ W_o) [+ b_o + x] into `dst` (fp32 [n, h]).
// With a_in (the sequence-parallel layout) LN1 has run per chunk already and
// a_in is the gathered [n, h] LayerNorm output.
int convert_mlp_weights(tp_layer* L, const tp_params* p, void* ws, hipStream_t s);

// With mlp_cvt the MLP weights' copies go to that stream after the QKV GEMM;
// with all_cvt they are made here, in the same launch as W_qkv's and W_o's.
int fwd_attn(tp_layer* L, const tp_params* p, const void* x, float* dst, bool designated,
             void* ws, hipStream_t s, const void* a_in = nullptr, hipStream_t mlp_cvt = nullptr,
             bool all_cvt = false) {
  const int n = L->n, h = L->hidden, hl = L->hl;
  int e;
  const double nh = (double)n * h;
  const size_t hf = (size_t)h * L->fl;
  if (all_cvt) {
    if ((e = to_f16_copies(L, {p->w_qkv, p->w_o, p->w_fc1, p->w_fc2},
                           {&L->w16_qkv, &L->w16_o, &L->w16_fc1, &L->w16_fc2},
                           {(size_t)h * 3 * hl, (size_t)hl * h, hf, hf}, ws, s)))
      return e;
  } else if ((e = to_f16_copies(L, {p->w_qkv, p->w_o}, {&L->w16_qkv, &L->w16_o},
                                {(size_t)h * 3 * hl, (size_t)hl * h}, ws, s))) {
    return e;
  }
  if (!a_in) {
  Scope ps(L, s, TP_K_LN_FWD, 0, nh * 2 * L->esz + 8.0 * n);
  HIP_TRY(ln_fwd(L->sdt, L->sdt, L->adt, x, p->ln1_gamma, p->ln1_beta, at<void>(ws, L->a),
                 at<float>(ws, L->mean1), at<float>(ws, L->rstd1), nullptr, n, h, L->eps, s));
  }
  GemmArgs g = gemm_base(L);
  g.M = n; g.N = 3 * hl; g.K = h;
  g.A = a_in ? a_in : at<void>(ws, L->a); g.lda = h; g.a_kmajor = 1;
  g.B = wmat(L, ws, L->w16_qkv, p->w_qkv); g.ldb = 3 * hl; g.b_kmajor = 0;
  g.bias = p->b_qkv;
  g.C = at<void>(ws, L->qkv); g.ldc = 3 * hl;
  if (L->split_scores) {
    g.epi = EPI_SPLIT16;
    g.C2 = qkv_lo(L, ws); g.ldc2 = 3 * hl; g.c2_dtype = DT_F16;
  }
  if ((e = run_gemm(L, g, s, ws))) return e;
  // the MLP weights' fp16 copies on the side stream while attention runs
  if (mlp_cvt) {
    if ((e = fork_to(L, s, mlp_cvt))) return e;
    if ((e = to_f16_copies(L, {p->w_fc1}, {&L->w16_fc1}, {hf}, ws, mlp_cvt))) return e;
    HIP_TRY(hipEventRecord(L->fc1_ev, mlp_cvt));
    if ((e = to_f16_copies(L, {p->w_fc2}, {&L->w16_fc2}, {hf}, ws, mlp_cvt))) return e;
  }
  {
  Scope ps(L, s, TP_K_ATTN_FWD, 4.0 * L->dh * L->Hl * L->attn_pairs,
           (double)n * 4 * hl * L->esz + 4.0 * n * L->Hl);
  HIP_TRY(attn_fwd(L->adt, at<void>(ws, L->qkv), qkv_lo(L, ws), at<void>(ws, L->o),
                   at<float>(ws, L->lse2), p->valid_len, L->batch, L->seq, L->Hl, L->dh, L->mask,
                   s));
  }
  g = gemm_base(L);
  g.M = n; g.N = h; g.K = hl;
  g.A = at<void>(ws, L->o); g.lda = hl; g.a_kmajor = 1;
  g.B = wmat(L, ws, L->w16_o, p->w_o); g.ldb = h; g.b_kmajor = 0;
  if (designated) {
    g.bias = p->b_o;
    g.resid = x; g.ldr = h; g.resid_dtype = L->sdt;
  }
  g.C = dst; g.ldc = h; g.c_dtype = DT_F32;
  if ((e = run_gemm(L, g, s, ws))) return e;
  return TP_OK;
}

// h_mid (fp32) -> c -> u, z -> (z @ W_fc2) [+ b_fc2 + h_mid] into `out`.
// With c_in (sequence-parallel layout) LN2 has run per chunk already and c_in
// is the gathered [n, h] LayerNorm output.
int convert_mlp_weights(tp_layer* L, const tp_params* p, void* ws, hipStream_t s) {
  const size_t hf = (size_t)L->hidden * L->fl;
  return to_f16_copies(L, {p->w_fc1, p->w_fc2}, {&L->w16_fc1, &L->w16_fc2}, {hf, hf}, ws, s);
}

int fwd_mlp(tp_layer* L, const tp_params* p, const float* h_mid_in, void* out, int out_f32,
            bool designated, void* ws, hipStream_t s, const void* c_in = nullptr,
            hipStream_t side_cvt = nullptr, bool converted_here = false) {
  const bool converted = side_cvt != nullptr || converted_here;
  const int n = L->n, h = L->hidden, fl = L->fl;
  int e;
  float* h_mid = at<float>(ws, L->h_mid);
  if (!converted && (e = convert_mlp_weights(L, p, ws, s))) return e;
  if (!c_in) {
  Scope ps(L, s, TP_K_LN_FWD, 0,
           (double)n * h * (4 + L->esz + (h_mid_in == h_mid ? 0 : 4)) + 8.0 * n);
  HIP_TRY(ln_fwd(DT_F32, L->sdt, L->adt, h_mid_in, p->ln2_gamma, p->ln2_beta, at<void>(ws, L->c),
                 at<float>(ws, L->mean2), at<float>(ws, L->rstd2),
                 h_mid_in == h_mid ? nullptr : h_mid, n, h, L->eps, s));
  }
  GemmArgs g = gemm_base(L);
  g.M = n; g.N = fl; g.K = h;
  g.A = c_in ? c_in : at<void>(ws, L->c); g.lda = h; g.a_kmajor = 1;
  g.B = wmat(L, ws, L->w16_fc1, p->w_fc1); g.ldb = fl; g.b_kmajor = 0;
  g.bias = p->b_fc1;
  g.epi = EPI_BIAS_GELU;
  g.C = L->recompute_fc1 ? nullptr : at<void>(ws, L->u); g.ldc = fl;
  g.C2 = at<void>(ws, L->z); g.ldc2 = fl;
  if ((e = run_gemm(L, g, s, ws))) return e;
  // W_fc2's copy (side stream) may still run beside LN2 and FC1
  if (side_cvt && (e = join_from(L, s, side_cvt))) return e;
  g = gemm_base(L);
  g.M = n; g.N = h; g.K = fl;
  g.A = at<void>(ws, L->z); g.lda = fl; g.a_kmajor = 1;
  g.B = wmat(L, ws, L->w16_fc2, p->w_fc2); g.ldb = h; g.b_kmajor = 0;
  if (designated) {
    g.bias = p->b_fc2;
    g.resid = h_mid; g.ldr = h; g.resid_dtype = DT_F32;
  }
  g.C = out; g.ldc = h; g.c_dtype = out_f32 ? DT_F32 : L->sdt;
  if ((e = run_gemm(L, g, s, ws))) return e;
  return TP_OK;
}

// ---- backward pieces -------------------------------------------------------
// Bias gradient: out (+)= column sums of y [n, cols] (block partials in its
// own scratch, then one deterministic reduction).
int bias_grad(tp_layer* L, const void* y, int y_dtype, int cols, float* out, int accumulate,
              void* ws, hipStream_t s, int rows = -1, const float* scale = nullptr) {
  if (rows < 0) rows = L->n;
  Scope ps(L, s, TP_K_REDUCE, 0, (double)rows * cols * L->esz + 4.0 * cols);
  float* part = at<float>(ws, L->part2);
  int rpb;
  const int nb = colsum_blocks(rows, cols, &rpb);
  HIP_TRY(colsum_partial(y_dtype, y, rows, cols, cols, part, rpb, s));
  HIP_TRY(reduce_partials(part, nb, 1, cols, out, nullptr, nullptr, accumulate, s, scale));
  return TP_OK;
}

// LayerNorm backward + residual-gradient add, then the reduction of its
// column partials into dgamma, dbeta (and the column sums of dx if dsum).
int ln_backward(tp_layer* L, const float* dy, int x_dtype, const void* x, const float* mean,
                const float* rstd, const void* gamma, int dres_dtype, const void* dres,
                float* dx_f32, int st_dtype, void* dx_st, float* dgamma, float* dbeta,
                float* dsum, int accumulate, void* ws, hipStream_t s, int rows = -1,
                const float* st_scale = nullptr) {
  const int n = rows < 0 ? L->n : rows, h = L->hidden;
  float* part = at<float>(ws, L->part);
  int rpb;
  const int nb = ln_bwd_blocks(n, h, &rpb);
  {
    const double x_sz = x_dtype == DT_F32 ? 4 : L->esz, r_sz = dres_dtype == DT_F32 ? 4 : L->esz;
    const double out_sz = (dx_f32 ? 4 : 0) + (dx_st ? L->esz : 0);
    Scope ps(L, s, TP_K_LN_BWD, 0, (double)n * h * (4 + x_sz + r_sz + out_sz) + 8.0 * n);
    HIP_TRY(ln_bwd(L->sdt, dy, x_dtype, x, mean, rstd, gamma, dres_dtype, dres, dx_f32, st_dtype,
                   dx_st, st_scale, part, rpb, n, h, dsum != nullptr, s));
  }
  Scope ps(L, s, TP_K_REDUCE, 0, (double)nb * 3 * h * 4);
  HIP_TRY(reduce_partials(part, nb, 3, h, dgamma, dbeta, dsum, accumulate, s));
  return TP_OK;
}

// dout -> du, dW2, db2, dA, db1, dc (fp32 into `dc_out`).
// Sequence-parallel layout: dout_full is the gathered [n, h] upstream
// gradient, c_in the gathered LN2 output, and io->dout this rank's chunk of
// db2_rows rows (the replicated bias b2 was added per chunk).
int bwd_mlp(tp_layer* L, const tp_params* p, const tp_bwd_io* io, float* dc_out, void* ws,
            hipStream_t s, const void* dout_full = nullptr, const void* c_in = nullptr,
            int db2_rows = -1) {
  const int n = L->n, h = L->hidden, fl = L->fl;
  int e;
  // the upstream gradient as the GEMMs read it (fp16 copy for a bf16 layer)
  const void* dout = dout_full ? dout_full : io->dout;
  // bf16 layer, one [n, h] upstream gradient: a single pass over it gives
  // db2's column partials and the partial maxima of its scaled fp16 copy
  int rpb2 = 0;
  const int nb2 = colsum_blocks(n, h, &rpb2);
  const bool db2_fused = L->sdt == DT_BF16 && !dout_full && n > 0 && h % 8 == 0 &&
                         (long)((h / 8 + 255) / 256) * nb2 <= kAmaxFloats;
  if (db2_fused) {
    Scope ps(L, s, TP_K_REDUCE, 0, (double)n * h * L->esz + 4.0 * h);
    HIP_TRY(colsum_amax_partial(io->dout, n, h, h, at<float>(ws, L->part2), rpb2,
                                at<float>(ws, L->gscale), s));
  }
  if ((e = to_f16_copies(L, {dout}, {&L->dout16}, {(size_t)n * h}, ws, s, true, db2_fused)))
    return e;
  if (L->sdt == DT_BF16) dout = at<void>(ws, L->dout16);
  const float* unscale = chain_unscale(L, ws);
  const void* c_act = c_in ? c_in : at<void>(ws, L->c);
  GemmArgs g;
  if (L->recompute_fc1) {
    // GeLU'(c @ W_fc1,r + b_fc1,r) again, straight into the du buffer
    g = gemm_base(L);
    g.M = n; g.N = fl; g.K = h;
    g.A = c_act; g.lda = h; g.a_kmajor = 1;
    g.B = wmat(L, ws, L->w16_fc1, p->w_fc1); g.ldb = fl; g.b_kmajor = 0;
    g.bias = p->b_fc1;
    g.epi = EPI_GELU_GRAD;
    g.C = at<void>(ws, L->du); g.ldc = fl;
    if ((e = run_gemm(L, g, s, ws))) return e;
  }
  // du = (dout @ W_fc2,r^T) * GeLU'(u), GeLU'(u) kept by the forward (in the
  // u buffer) or recomputed into the du buffer, then overwritten in place
  // (each element is read, then written, by the same thread of the epilogue)
  // db2 and dW2 (need only dout and z)
  if (db2_fused) {
    Scope ps(L, s, TP_K_REDUCE, 0, (double)nb2 * h * 4);
    HIP_TRY(reduce_partials(at<float>(ws, L->part2), nb2, 1, h, io->d_b_fc2, nullptr, nullptr,
                            io->accumulate, s));
  } else if ((e = bias_grad(L, io->dout, L->sdt, h, io->d_b_fc2, io->accumulate, ws, s,
                            db2_rows))) {
    return e;
  }
  g = wgrad_args(L, fl, h, at<void>(ws, L->z), dout, io->d_w_fc2, io->accumulate);
  g.split = L->split_w2; g.scale = unscale;
  if ((e = run_gemm(L, g, s, ws, true))) return e;
  g = gemm_base(L);
  g.M = n; g.N = fl; g.K = h;
  g.A = dout; g.lda = h; g.a_kmajor = 1;
  g.B = wmat(L, ws, L->w16_fc2, p->w_fc2); g.ldb = h; g.b_kmajor = 1;
  g.epi = EPI_DGELU;
  g.aux = at<void>(ws, L->recompute_fc1 ? L->du : L->u); g.ldaux = fl;
  g.C = at<void>(ws, L->du); g.ldc = fl;
  if ((e = run_gemm(L, g, s, ws))) return e;
  // dW1 and db1 (need du)
  g = wgrad_args(L, h, fl, c_act, at<void>(ws, L->du), io->d_w_fc1, io->accumulate);
  g.split = L->split_w1; g.scale = unscale;
  if ((e = run_gemm(L, g, s, ws, true))) return e;
  if ((e = bias_grad(L, at<void>(ws, L->du), L->adt, fl, io->d_b_fc1, io->accumulate, ws, s, -1,
                     unscale)))
    return e;
  g = gemm_base(L);
  g.M = n; g.N = h; g.K = fl;
  g.A = at<void>(ws, L->du); g.lda = fl; g.a_kmajor = 1;
  g.B = wmat(L, ws, L->w16_fc1, p->w_fc1); g.ldb = fl; g.b_kmajor = 1;
  g.C = dc_out; g.ldc = h; g.c_dtype = DT_F32; g.scale = unscale;
  return run_gemm(L, g, s, ws);
}

// dc (summed) -> dh, LN2 grads, db_o -> dW_o, do -> attention -> dqkv ->
// dW_qkv, db_qkv -> da (fp32 into `da_out`).
// Sequence-parallel layout: LN2's backward has run per chunk already; dh_in
// is the gathered [n, h] residual-stream gradient (internal dtype) and a_in
// the gathered LN1 output.
int bwd_attn(tp_layer* L, const tp_params* p, const tp_bwd_io* io, const float* dc,
             float* da_out, void* ws, hipStream_t s, const void* dh_in = nullptr,
             const void* a_in = nullptr) {
  const int n = L->n, h = L->hidden, hl = L->hl;
  int e;
  const float* unscale = chain_unscale(L, ws);
  if (!dh_in &&
      (e = ln_backward(L, dc, DT_F32, at<void>(ws, L->h_mid), at<float>(ws, L->mean2),
                       at<float>(ws, L->rstd2), p->ln2_gamma, L->sdt, io->dout,
                       at<float>(ws, L->dh_f), L->adt, at<void>(ws, L->dh_s), io->d_ln2_gamma,
                       io->d_ln2_beta, io->d_b_o, io->accumulate, ws, s, -1,
                       chain_scale(L, ws))))
    return e;
  const void* dh_s = dh_in ? dh_in : at<void>(ws, L->dh_s);
  const void* a_act = a_in ? a_in : at<void>(ws, L->a);
  // dW_o (needs dh) on the side stream, when the handle overlaps, during dO
  // and the attention backward: the one pairing where the overlap measured
  // faster (the attention kernels leave compute units idle that the GEMM fills)
  hipStream_t sd = side_stream(L, s);
  if ((e = fork_to(L, s, sd))) return e;
  GemmArgs g = wgrad_args(L, hl, h, at<void>(ws, L->o), dh_s, io->d_w_o, io->accumulate);
  g.split = L->split_wo; g.scale = unscale;
  if ((e = run_gemm(L, g, sd, ws, true))) return e;
  g = gemm_base(L);
  g.M = n; g.N = hl; g.K = h;
  g.A = dh_s; g.lda = h; g.a_kmajor = 1;
  g.B = wmat(L, ws, L->w16_o, p->w_o); g.ldb = h; g.b_kmajor = 1;
  g.C = at<void>(ws, L->dO); g.ldc = hl;
  if ((e = run_gemm(L, g, s, ws))) return e;
  {
    Scope ps(L, s, TP_K_ATTN_BWD, 8.0 * L->dh * L->Hl * L->attn_pairs,
             (double)n * 8 * hl * L->esz + 8.0 * n * L->Hl);
    HIP_TRY(attn_bwd(L->adt, at<void>(ws, L->qkv), qkv_lo(L, ws), at<void>(ws, L->o),
                     at<void>(ws, L->dO),
                     at<float>(ws, L->lse2), at<float>(ws, L->delta), at<void>(ws, L->dqkv),
                     p->valid_len, L->batch, L->seq, L->Hl, L->dh, L->mask, s));
  }
  // dW_o is done before dW_qkv, which uses the same weight-gradient scratch
  if ((e = join_from(L, s, sd))) return e;
  // dW_qkv and db_qkv (need dqkv)
  g = wgrad_args(L, h, 3 * hl, a_act, at<void>(ws, L->dqkv), io->d_w_qkv, io->accumulate);
  g.split = L->split_wqkv; g.scale = unscale;
  if ((e = run_gemm(L, g, s, ws, true))) return e;
  if ((e = bias_grad(L, at<void>(ws, L->dqkv), L->adt, 3 * hl, io->d_b_qkv, io->accumulate, ws,
                     s, -1, unscale)))
    return e;
  g = gemm_base(L);
  g.M = n; g.N = h; g.K = 3 * hl;
  g.A = at<void>(ws, L->dqkv); g.lda = 3 * hl; g.a_kmajor = 1;
  g.B = wmat(L, ws, L->w16_qkv, p->w_qkv); g.ldb = 3 * hl; g.b_kmajor = 1;
  g.C = da_out; g.ldc = h; g.c_dtype = DT_F32; g.scale = unscale;
  return run_gemm(L, g, s, ws);
}

// da (summed) -> dx (+ dh), LN1 grads.
int bwd_ln1(tp_layer* L, const tp_params* p, const tp_bwd_io* io, const float* da, void* ws,
            hipStream_t s) {
  float* dx32 = L->dx_f32 ? static_cast<float*>(io->dx) : nullptr;
  void* dxst = L->dx_f32 ? nullptr : io->dx;
  return ln_backward(L, da, L->sdt, io->x, at<float>(ws, L->mean1), at<float>(ws, L->rstd1),
                     p->ln1_gamma, DT_F32, at<void>(ws, L->dh_f), dx32, L->sdt, dxst,
                     io->d_ln1_gamma, io->d_ln1_beta, nullptr, io->accumulate, ws, s);
}

// ---- sequence-parallel phases ------------------------------------------------
// Rank r owns the token rows [r*nc, (r+1)*nc) of the [n, h] token matrix for
// LayerNorm, bias and residual. The all-gather before each column-parallel
// GEMM is this rank writing its rows into the caller's gathered buffer (the
// collective fills the other ranks' rows); the reduce-scatter after each
// row-parallel GEMM hands back this rank's rows of the summed partial.
char* chunk_rows(void* base, const tp_layer* L) {
  return static_cast<char*>(base) + (size_t)L->rank * L->nc * L->hidden * L->esz;
}

int fwd_sp(tp_layer* L, int phase, const tp_params* p, const tp_fwd_io* io, void* ws,
           hipStream_t s) {
  const int nc = L->nc, h = L->hidden;
  int e;
  float* h_mid = at<float>(ws, L->h_mid);  // first nc rows: this rank's chunk
  switch (phase) {
    case TP_FWD_SP_LN1: {
      if ((e = check_ptrs({io->x, io->gathered}))) return e;
      Scope ps(L, s, TP_K_LN_FWD, 0, (double)nc * h * 2 * L->esz + 8.0 * nc);
      HIP_TRY(ln_fwd(L->sdt, L->sdt, L->adt, io->x, p->ln1_gamma, p->ln1_beta,
                     chunk_rows(io->gathered, L), at<float>(ws, L->mean1),
                     at<float>(ws, L->rstd1), nullptr, nc, h, L->eps, s));
      return TP_OK;
    }
    case TP_FWD_SP_ATTN:
      if ((e = check_ptrs({io->gathered, io->out}))) return e;
      return fwd_attn(L, p, nullptr, static_cast<float*>(io->out), false, ws, s, io->gathered);
    case TP_FWD_SP_LN2: {
      if ((e = check_ptrs({io->reduced, io->x, io->gathered}))) return e;
      Scope ps(L, s, TP_K_LN_FWD, 0, (double)nc * h * (4 + L->esz + 4 + 4 + L->esz) + 8.0 * nc);
      HIP_TRY(residual_add(io->reduced, L->sdt, p->b_o, L->sdt, io->x, DT_F32, h_mid, nc, h, s));
      HIP_TRY(ln_fwd(DT_F32, L->sdt, L->adt, h_mid, p->ln2_gamma, p->ln2_beta,
                     chunk_rows(io->gathered, L), at<float>(ws, L->mean2),
                     at<float>(ws, L->rstd2), nullptr, nc, h, L->eps, s));
      return TP_OK;
    }
    case TP_FWD_SP_MLP:
      if ((e = check_ptrs({io->gathered, io->out}))) return e;
      return fwd_mlp(L, p, nullptr, io->out, 1, false, ws, s, io->gathered);
    default: {  // TP_FWD_SP_OUT
      if ((e = check_ptrs({io->reduced, io->out}))) return e;
      Scope ps(L, s, TP_K_LN_FWD, 0, (double)nc * h * (4 + 4 + L->esz));
      HIP_TRY(residual_add(io->reduced, L->sdt, p->b_fc2, DT_F32, h_mid, L->sdt, io->out, nc, h,
                           s));
      return TP_OK;
    }
  }
}

int bwd_sp(tp_layer* L, int phase, const tp_params* p, const tp_bwd_io* io, void* ws,
           hipStream_t s) {
  const int nc = L->nc;
  int e;
  switch (phase) {
    case TP_BWD_SP_MLP:
      if ((e = check_ptrs({io->dout, io->gathered_grad, io->gathered_act, io->partial,
                           io->d_w_fc1, io->d_b_fc1, io->d_w_fc2, io->d_b_fc2})))
        return e;
      return bwd_mlp(L, p, io, io->partial, ws, s, io->gathered_grad, io->gathered_act, nc);
    case TP_BWD_SP_LN2:
      if ((e = check_ptrs({io->dc, io->dout, io->gathered_grad, io->d_ln2_gamma, io->d_ln2_beta,
                           io->d_b_o})))
        return e;
      return ln_backward(L, io->dc, DT_F32, at<void>(ws, L->h_mid), at<float>(ws, L->mean2),
                         at<float>(ws, L->rstd2), p->ln2_gamma, L->sdt, io->dout,
                         at<float>(ws, L->dh_f), L->adt, chunk_rows(io->gathered_grad, L),
                         io->d_ln2_gamma, io->d_ln2_beta, io->d_b_o, io->accumulate, ws, s, nc,
                         chain_scale(L, ws));
    case TP_BWD_SP_ATTN:
      if ((e = check_ptrs({io->gathered_grad, io->gathered_act, io->partial, io->d_w_qkv,
                           io->d_b_qkv, io->d_w_o})))
        return e;
      return bwd_attn(L, p, io, nullptr, io->partial, ws, s, io->gathered_grad, io->gathered_act);
    default: {  // TP_BWD_SP_LN1
      if ((e = check_ptrs({io->x, io->da, io->dx, io->d_ln1_gamma, io->d_ln1_beta}))) return e;
      float* dx32 = L->dx_f32 ? static_cast<float*>(io->dx) : nullptr;
      void* dxst = L->dx_f32 ? nullptr : io->dx;
      return ln_backward(L, io->da, L->sdt, io->x, at<float>(ws, L->mean1), at<float>(ws, L->rstd1),
                         p->ln1_gamma, DT_F32, at<void>(ws, L->dh_f), dx32, L->sdt, dxst,
                         io->d_ln1_gamma, io->d_ln1_beta, nullptr, io->accumulate, ws, s, nc);
    }
  }
}

void prof_fold(Prof& p) {
  for (auto& r : p.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      p.launches[r.cls] += 1;
      p.ms[r.cls] += ms;
      p.flops[r.cls] += r.flops;
      p.bytes[r.cls] += r.bytes;
    }
    p.pool.push_back(r.a);
    p.pool.push_back(r.b);
  }
  p.recs.clear();
}

}  // namespace

// ---- decode ------------------------------------------------------------------
double gemv_bytes(const tp_layer* L, const GemvArgs& g, double out_e) {
  const double e = L->esz;
  double b = (double)g.K * g.N * e + (double)g.M * g.K * e + (double)g.M * g.N * out_e;
  if (g.bias) b += (double)g.N * e;
  if (g.resid) b += (double)g.M * g.N * (g.resid_dt == DT_F32 ? 4.0 : e);
  return b;
}

int run_gemv(tp_layer* L, const GemvArgs& g, double out_e, hipStream_t s) {
  Scope ps(L, s, TP_K_GEMM, 2.0 * g.M * g.N * (double)g.K, gemv_bytes(L, g, out_e));
  HIP_TRY(gemv(g, L->adt, s));
  return TP_OK;
}

GemvArgs gemv_base(tp_layer* L, int which, void* ws) {
  const tp_layer::Dec& d = L->dec;
  GemvArgs g = {};
  g.M = L->batch;
  g.strip = d.strip[which];
  g.chunk = d.chunk[which];
  g.kc = d.kc[which];
  g.nsplit = d.ns[which];
  g.part = at<float>(ws, d.gpart);
  g.bias_dt = g.resid_dt = L->sdt;
  g.gelu_tanh = L->gelu_tanh;
  return g;
}

// x -> a -> qkv partials -> attention (sums them, appends K/V to the cache)
// -> o -> o @ W_o. fused_ln (TP_ALL): the W_o partials are finished together
// with LN2 (h_mid and c in the workspace); else the result [+ b_o + x] goes
// to `dst` (fp32 [B, h]).
int dec_attn_phase(tp_layer* L, const tp_params* p, const tp_decode_io* io, float* dst,
                   bool designated, bool fused_ln, bool* c_done, void* ws, hipStream_t s) {
  const tp_layer::Dec& d = L->dec;
  const int B = L->batch, h = L->hidden, hl = L->hl, D = L->dh;
  int e;
  // one workgroup per row sums the W_o partials in the fused kernel: only
  // worth it while a row's partials are small
  fused_ln = fused_ln && (size_t)d.ns[1] * h * 4 <= 131072;
  *c_done = fused_ln;
  {
  Scope ps(L, s, TP_K_LN_FWD, 0, (double)B * h * 2 * L->esz);
  HIP_TRY(ln_fwd(L->sdt, L->sdt, L->adt, io->x, p->ln1_gamma, p->ln1_beta, at<void>(ws, d.a),
                 nullptr, nullptr, nullptr, B, h, L->eps, s));
  }
  GemvArgs g = gemv_base(L, 0, ws);
  g.N = 3 * hl; g.K = h;
  g.X = at<void>(ws, d.a); g.W = p->w_qkv;
  g.raw = 1;  // the attention kernel sums the partials
  if ((e = run_gemv(L, g, 4.0, s))) return e;
  {
  DecAttnArgs a = {};
  a.qkv_part = at<float>(ws, d.gpart); a.qkv_ns = d.ns[0];
  a.b_qkv = p->b_qkv; a.bias_dt = L->sdt;
  a.kc = io->k_cache; a.vc = io->v_cache;
  a.klo = L->split_scores ? (_Float16*)io->k_cache_lo : nullptr;
  a.pos = io->positions;
  a.batch = B; a.Hl = L->Hl; a.cache_len = io->cache_len;
  a.nsplit = dec_attn_split(B, L->Hl, io->cache_len, &a.chunk);
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  a.part = at<float>(ws, d.apart);
  a.o = at<void>(ws, d.o); a.o_dt = L->adt;
  const double keys = (double)B * L->Hl * io->cache_len;
  Scope ps(L, s, TP_K_ATTN_FWD, 4.0 * D * keys,
           keys * D * L->esz * (L->split_scores ? 3 : 2) + (double)B * hl * L->esz);
  HIP_TRY(dec_attn(L->adt, a, D, L->split_scores, s));
  }
  g = gemv_base(L, 1, ws);
  g.N = h; g.K = hl;
  g.X = at<void>(ws, d.o); g.W = p->w_o;
  if (fused_ln) {
    g.raw = 1;
    if ((e = run_gemv(L, g, 4.0, s))) return e;
    Scope ps(L, s, TP_K_LN_FWD, 0, (double)B * h * (4 + L->esz + 4 + L->esz) + 2.0 * h * L->esz);
    HIP_TRY(dec_resid_ln(L->adt, at<float>(ws, d.gpart), g.nsplit, p->b_o, io->x,
                         at<float>(ws, d.h_mid), p->ln2_gamma, p->ln2_beta, at<void>(ws, d.c), B,
                         h, L->eps, s));
    return TP_OK;
  }
  g.epi = GEMV_EPI_OUT;
  if (designated) {
    g.bias = p->b_o;
    g.resid = io->x;
  }
  g.out = dst; g.out_dt = DT_F32;
  return run_gemv(L, g, 4.0, s);
}

// h_mid (fp32 [B, h]) -> c -> z -> z @ W_fc2 [+ b_fc2 + h_mid] into `out`.
// With have_c, c = LN2(h_mid) is already in the workspace.
int dec_mlp_phase(tp_layer* L, const tp_params* p, const float* h_mid, void* out, int out_dt,
                  bool designated, bool have_c, void* ws, hipStream_t s) {
  const tp_layer::Dec& d = L->dec;
  const int B = L->batch, h = L->hidden, fl = L->fl;
  int e;
  if (!have_c) {
  Scope ps(L, s, TP_K_LN_FWD, 0, (double)B * h * (4 + L->esz));
  HIP_TRY(ln_fwd(DT_F32, L->sdt, L->adt, h_mid, p->ln2_gamma, p->ln2_beta, at<void>(ws, d.c),
                 nullptr, nullptr, nullptr, B, h, L->eps, s));
  }
  GemvArgs g = gemv_base(L, 2, ws);
  g.N = fl; g.K = h;
  g.X = at<void>(ws, d.c); g.W = p->w_fc1;
  g.epi = GEMV_EPI_GELU;
  g.bias = p->b_fc1;
  g.out = at<void>(ws, d.z); g.out_dt = L->adt;
  if ((e = run_gemv(L, g, L->esz, s))) return e;
  g = gemv_base(L, 3, ws);
  g.N = h; g.K = fl;
  g.X = at<void>(ws, d.z); g.W = p->w_fc2;
  g.epi = GEMV_EPI_OUT;
  if (designated) {
    g.bias = p->b_fc2;
    g.resid = h_mid; g.resid_dt = DT_F32;
  }
  g.out = out; g.out_dt = out_dt;
  return run_gemv(L, g, out_dt == DT_F32 ? 4.0 : L->esz, s);
}

extern "C" {

int tp_layer_create(int hidden, int heads, int ffn, int seq, int micro_batch, int t, int rank,
                    int dtype, int mask, const tp_layer_opts* opts, tp_layer** out,
                    size_t* workspace_bytes) {
  if (!out) return TP_ERR_ARG;
  *out = nullptr;
  if (!workspace_bytes) return TP_ERR_ARG;
  if (hidden <= 0 || heads <= 0 || ffn <= 0 || seq <= 0 || micro_batch <= 0 || t <= 0)
    return TP_ERR_ARG;
  if (dtype != TP_DTYPE_F32 && dtype != TP_DTYPE_BF16) return TP_ERR_UNSUPPORTED;
  if (mask != TP_MASK_CAUSAL && mask != TP_MASK_PADDING) return TP_ERR_UNSUPPORTED;
  if (hidden % heads || heads % t || ffn % t || (ffn / t) % 8) return TP_ERR_SHAPE;
  if (rank < 0 || rank >= t) return TP_ERR_SHAPE;
  const int dh = hidden / heads;
  if (dh != 32 && dh != 64 && dh != 96 && dh != 128 && dh != 160) return TP_ERR_UNSUPPORTED;
  if (hidden > 32768) return TP_ERR_UNSUPPORTED;  // LayerNorm keeps a row in registers
  const long n = (long)seq * micro_batch;
  if (n > (1L << 30) / 4) return TP_ERR_UNSUPPORTED;
  float eps = 1e-5f;
  int gelu = TP_GELU_ERF;
  int dx_dtype = TP_DTYPE_F32;
  int scores = TP_SCORES_AUTO;
  int recompute = TP_RECOMPUTE_NONE;
  int seq_par = 0;
  int overlap = TP_OVERLAP_AUTO;
  if (opts) {
    eps = opts->ln_eps;
    gelu = opts->gelu;
    dx_dtype = opts->dx_dtype;
    scores = opts->scores;
    recompute = opts->recompute;
    seq_par = opts->sequence_parallel;
    overlap = opts->overlap;
    if (!(eps > 0.f)) return TP_ERR_ARG;
    if (gelu != TP_GELU_ERF && gelu != TP_GELU_TANH) return TP_ERR_UNSUPPORTED;
    if (dx_dtype != TP_DTYPE_F32 && dx_dtype != dtype) return TP_ERR_UNSUPPORTED;
    if (scores != TP_SCORES_AUTO && scores != TP_SCORES_FP16 && scores != TP_SCORES_SPLIT)
      return TP_ERR_UNSUPPORTED;
    if (scores == TP_SCORES_SPLIT && dtype != TP_DTYPE_BF16) return TP_ERR_UNSUPPORTED;
    if (recompute != TP_RECOMPUTE_NONE && recompute != TP_RECOMPUTE_FC1) return TP_ERR_UNSUPPORTED;
    if (seq_par != 0 && seq_par != 1) return TP_ERR_UNSUPPORTED;
    if (seq_par && n % t) return TP_ERR_SHAPE;
    if (overlap != TP_OVERLAP_AUTO && overlap != TP_OVERLAP_OFF && overlap != TP_OVERLAP_ON)
      return TP_ERR_UNSUPPORTED;
  }
  tp_layer* L = new (std::nothrow) tp_layer();
  if (!L) return TP_ERR_NOMEM;
  L->hidden = hidden; L->heads = heads; L->ffn = ffn; L->seq = seq; L->batch = micro_batch;
  L->t = t; L->rank = rank; L->dtype = dtype; L->mask = mask;
  L->eps = eps; L->gelu_tanh = gelu == TP_GELU_TANH;
  L->dx_f32 = dx_dtype == TP_DTYPE_F32;
  L->recompute_fc1 = recompute == TP_RECOMPUTE_FC1;
  L->sp = seq_par == 1;
  L->overlap = overlap == TP_OVERLAP_ON ||
                     (overlap == TP_OVERLAP_AUTO && hidden >= kOverlapHidden);
  L->nc = (int)(n / t);
  L->split_scores = dtype == TP_DTYPE_BF16 &&
                    (scores == TP_SCORES_SPLIT ||
                     (scores == TP_SCORES_AUTO && hidden >= kSplitScoresHidden));
  L->n = (int)n; L->dh = dh; L->Hl = heads / t; L->hl = L->Hl * dh; L->fl = ffn / t;
  L->esz = dtype == TP_DTYPE_BF16 ? 2 : 4;
  L->sdt = dtype == TP_DTYPE_BF16 ? DT_BF16 : DT_F32;
  L->adt = dtype == TP_DTYPE_BF16 ? DT_F16 : DT_F32;
  L->attn_pairs = mask == TP_MASK_CAUSAL ? (double)micro_batch * seq * (seq + 1) / 2.0 : 0.0;
  plan(L);
  plan_decode(L);
  *out = L;
  *workspace_bytes = L->ws_bytes;
  return TP_OK;
}

int tp_layer_fwd(tp_layer* L, int phase, const tp_fwd_io* io, void* hip_stream) {
  if (!L || !io) return TP_ERR_ARG;
  if (L->sp ? (phase < TP_FWD_SP_LN1 || phase > TP_FWD_SP_OUT)
            : (phase < TP_ALL || phase > TP_FWD_MLP))
    return TP_ERR_PHASE;
  int e = check_params(L, io->params);
  if (e) return e;
  if ((e = check_ws(L, io->workspace, io->workspace_bytes))) return e;
  hipStream_t s = (hipStream_t)hip_stream;
  void* ws = io->workspace;
  const tp_params* p = io->params;
  const bool designated = L->rank == 0;
  switch (phase) {
    case TP_ALL: {
      if ((e = check_ptrs({io->x, io->out}))) return e;
      // bf16: the weights' fp16 copies in one launch, or the MLP's on the side
      // stream (overlap); FC1 then waits for W_fc1's copy only and fwd_mlp
      // joins the rest before FC2
      const bool cvt = L->sdt == DT_BF16;
      hipStream_t sd = cvt ? side_stream(L, s) : s;
      if ((e = fwd_attn(L, p, io->x, at<float>(ws, L->h_mid), true, ws, s, nullptr,
                        sd != s ? sd : nullptr, cvt && sd == s)))
        return e;
      if (sd != s) HIP_TRY(hipStreamWaitEvent(s, L->fc1_ev, 0));
      return fwd_mlp(L, p, at<float>(ws, L->h_mid), io->out, 0, true, ws, s, nullptr,
                     sd != s ? sd : nullptr, cvt && sd == s);
    }
    case TP_FWD_ATTN:
      if ((e = check_ptrs({io->x, io->out}))) return e;
      return fwd_attn(L, p, io->x, (float*)io->out, designated, ws, s);
    case TP_FWD_MLP:
      if ((e = check_ptrs({io->h_mid, io->out}))) return e;
      return fwd_mlp(L, p, io->h_mid, io->out, 1, designated, ws, s);
    default:
      return fwd_sp(L, phase, p, io, ws, s);
  }
}

int tp_layer_bwd(tp_layer* L, int phase, const tp_bwd_io* io, void* hip_stream) {
  if (!L || !io) return TP_ERR_ARG;
  if (L->sp ? (phase < TP_BWD_SP_MLP || phase > TP_BWD_SP_LN1)
            : (phase < TP_ALL || phase > TP_BWD_LN1))
    return TP_ERR_PHASE;
  int e = check_params(L, io->params);
  if (e) return e;
  if ((e = check_ws(L, io->workspace, io->workspace_bytes))) return e;
  hipStream_t s = (hipStream_t)hip_stream;
  void* ws = io->workspace;
  const tp_params* p = io->params;
  switch (phase) {
    case TP_ALL:
      if ((e = check_ptrs({io->x, io->dout, io->dx, io->d_ln1_gamma, io->d_ln1_beta, io->d_w_qkv,
                           io->d_b_qkv, io->d_w_o, io->d_b_o, io->d_ln2_gamma, io->d_ln2_beta,
                           io->d_w_fc1, io->d_b_fc1, io->d_w_fc2, io->d_b_fc2})))
        return e;
      if ((e = bwd_mlp(L, p, io, at<float>(ws, L->dc), ws, s))) return e;
      if ((e = bwd_attn(L, p, io, at<float>(ws, L->dc), at<float>(ws, L->da), ws, s))) return e;
      return bwd_ln1(L, p, io, at<float>(ws, L->da), ws, s);
    case TP_BWD_MLP:
      if ((e = check_ptrs({io->dout, io->partial, io->d_w_fc1, io->d_b_fc1, io->d_w_fc2,
                           io->d_b_fc2})))
        return e;
      return bwd_mlp(L, p, io, io->partial, ws, s);
    case TP_BWD_ATTN:
      if ((e = check_ptrs({io->dout, io->dc, io->partial, io->d_w_qkv, io->d_b_qkv, io->d_w_o,
                           io->d_b_o, io->d_ln2_gamma, io->d_ln2_beta})))
        return e;
      return bwd_attn(L, p, io, io->dc, io->partial, ws, s);
    case TP_BWD_LN1:
      if ((e = check_ptrs({io->x, io->da, io->dx, io->d_ln1_gamma, io->d_ln1_beta}))) return e;
      return bwd_ln1(L, p, io, io->da, ws, s);
    default:
      return bwd_sp(L, phase, p, io, ws, s);
  }
}

int tp_layer_decode_workspace(const tp_layer* L, size_t* bytes) {
  if (!L || !bytes) return TP_ERR_ARG;
  *bytes = L->dec.bytes;
  return TP_OK;
}

// Argument checks shared by both decode entry points (the workspace apart).
static int decode_checks(tp_layer* L, int phase, const tp_decode_io* io) {
  if (!L || !io) return TP_ERR_ARG;
  if (L->mask != TP_MASK_CAUSAL || L->batch > 128) return TP_ERR_UNSUPPORTED;
  if (phase < TP_ALL || phase > TP_FWD_MLP) return TP_ERR_PHASE;
  int e = check_params(L, io->params);
  if (e) return e;
  if (phase != TP_FWD_MLP) {
    if ((e = check_ptrs({io->x, io->out, io->k_cache, io->v_cache, io->positions}))) return e;
    if (L->split_scores && (e = check_ptrs({io->k_cache_lo}))) return e;
    if (io->cache_len < 1) return TP_ERR_ARG;
  } else if ((e = check_ptrs({io->h_mid, io->out}))) {
    return e;
  }
  return TP_OK;
}

// Enqueues one decode phase with `ws` (L->dec.bytes, 16-byte aligned) as its
// workspace.
static int decode_run(tp_layer* L, int phase, const tp_decode_io* io, void* ws, hipStream_t s) {
  int e;
  const tp_params* p = io->params;
  const bool designated = L->rank == 0;
  switch (phase) {
    case TP_ALL: {
      float* hm = at<float>(ws, L->dec.h_mid);
      bool have_c;
      if ((e = dec_attn_phase(L, p, io, hm, true, true, &have_c, ws, s))) return e;
      return dec_mlp_phase(L, p, hm, io->out, L->sdt, true, have_c, ws, s);
    }
    case TP_FWD_ATTN: {
      bool have_c;
      return dec_attn_phase(L, p, io, (float*)io->out, designated, false, &have_c, ws, s);
    }
    default:
      return dec_mlp_phase(L, p, io->h_mid, io->out, DT_F32, designated, false, ws, s);
  }
}

int tp_layer_decode(tp_layer* L, int phase, const tp_decode_io* io, void* hip_stream) {
  int e = decode_checks(L, phase, io);
  if (e) return e;
  if (!io->workspace || io->workspace_bytes < L->dec.bytes) return TP_ERR_WORKSPACE;
  if (!aligned(io->workspace)) return TP_ERR_ALIGN;
  return decode_run(L, phase, io, io->workspace, (hipStream_t)hip_stream);
}

}  // extern "C"

// ---- decode without a caller workspace -----------------------------------------
// The scratch of tp_layer_decode_static: a file-scope device array. Every
// device the library runs on holds its own copy until the process ends. In
// host code `scratch` names a host-side stand-in, not the device memory: its
// device address comes from hipGetSymbolAddress, looked up once per device
// (with that device current) and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[TP_DECODE_STATIC_MAX_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

// This device's scratch address, looked up on the first call on the device.
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TP_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return TP_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return TP_ERR_HIP;
    }
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return TP_OK;
}
}  // namespace

extern "C" {

int tp_layer_decode_static(tp_layer* L, int phase, const tp_decode_io* io, void* hip_stream) {
  int e = decode_checks(L, phase, io);
  if (e) return e;
  if (L->dec.bytes > TP_DECODE_STATIC_MAX_BYTES) return TP_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((e = device_scratch(&ws))) return e;
  // Profiling creates HIP events on first use; this entry point creates
  // nothing, so its launches are not timed.
  const bool prof = L->prof.on;
  L->prof.on = false;
  e = decode_run(L, phase, io, ws, (hipStream_t)hip_stream);
  L->prof.on = prof;
  return e;
}

int tp_layer_kv_fill(const tp_layer* L, const void* workspace, size_t workspace_bytes,
                     void* k_cache, void* v_cache, void* k_cache_lo, int cache_len,
                     void* hip_stream) {
  if (!L) return TP_ERR_ARG;
  if (!workspace || workspace_bytes < L->ws_bytes) return TP_ERR_WORKSPACE;
  if (!aligned(workspace)) return TP_ERR_ALIGN;
  int e = check_ptrs({k_cache, v_cache});
  if (e) return e;
  if (L->split_scores && (e = check_ptrs({k_cache_lo}))) return e;
  if (cache_len < L->seq) return TP_ERR_SHAPE;
  void* ws = const_cast<void*>(workspace);
  if (kv_fill(L->adt, at<void>(ws, L->qkv),
              L->split_scores ? at<void>(ws, L->qkv_lo) : nullptr, k_cache, v_cache,
              L->split_scores ? k_cache_lo : nullptr, L->batch, L->seq, L->Hl, L->dh,
              cache_len, (hipStream_t)hip_stream) != hipSuccess)
    return TP_ERR_HIP;
  return TP_OK;
}

int tp_layer_destroy(tp_layer* L) {
  if (L) {
    prof_fold(L->prof);
    for (hipEvent_t e : L->prof.pool) (void)hipEventDestroy(e);
    if (L->side) {
      (void)hipStreamSynchronize(L->side);
      (void)hipEventDestroy(L->fork_ev);
      (void)hipEventDestroy(L->join_ev);
      (void)hipEventDestroy(L->fc1_ev);
      (void)hipStreamDestroy(L->side);
    }
  }
  delete L;
  return TP_OK;
}

int tp_exchange_sum(void* dst, int dst_dtype, const float* const* parts, int nparts,
                    size_t count, void* hip_stream) {
  if (!dst || !parts || nparts < 1 || nparts > 16) return TP_ERR_ARG;
  if (dst_dtype != TP_DTYPE_F32 && dst_dtype != TP_DTYPE_BF16) return TP_ERR_UNSUPPORTED;
  if (!aligned(dst)) return TP_ERR_ALIGN;
  for (int i = 0; i < nparts; ++i) {
    if (!parts[i]) return TP_ERR_ARG;
    if (!aligned(parts[i])) return TP_ERR_ALIGN;
  }
  if (exchange_sum(dst, dst_dtype, parts, nparts, count, (hipStream_t)hip_stream) != hipSuccess)
    return TP_ERR_HIP;
  return TP_OK;
}

int tp_layer_profile(tp_layer* L, int enable, double attn_pairs) {
  if (!L || !(attn_pairs >= 0.0)) return TP_ERR_ARG;
  if (L->mask == TP_MASK_PADDING) L->attn_pairs = attn_pairs;
  Prof& p = L->prof;
  prof_fold(p);
  for (int k = 0; k < TP_K_COUNT; ++k) {
    p.launches[k] = 0;
    p.ms[k] = p.flops[k] = p.bytes[k] = 0.0;
  }
  p.on = enable != 0;
  return TP_OK;
}

int tp_layer_profile_read(tp_layer* L, int kclass, long* launches, double* ms, double* flops,
                          double* bytes) {
  if (!L || kclass < 0 || kclass >= TP_K_COUNT) return TP_ERR_ARG;
  Prof& p = L->prof;
  prof_fold(p);
  if (launches) *launches = p.launches[kclass];
  if (ms) *ms = p.ms[kclass];
  if (flops) *flops = p.flops[kclass];
  if (bytes) *bytes = p.bytes[kclass];
  return TP_OK;
}

int tp_layer_tap(const tp_layer* L, int tap, size_t* offset, size_t* bytes) {
  if (!L || !offset || !bytes) return TP_ERR_ARG;
  const Region* r = nullptr;
  switch (tap) {
    case TP_TAP_LN1_OUT: r = &L->a; break;
    case TP_TAP_QKV: r = &L->qkv; break;
    case TP_TAP_ATTN_OUT: r = &L->o; break;
    case TP_TAP_LSE: r = &L->lse2; break;
    case TP_TAP_H_MID: r = &L->h_mid; break;
    case TP_TAP_LN2_OUT: r = &L->c; break;
    case TP_TAP_FC1_DGELU:
      if (L->recompute_fc1) return TP_ERR_UNSUPPORTED;  // not kept
      r = &L->u;
      break;
    case TP_TAP_FC1_OUT: r = &L->z; break;
    case TP_TAP_DQKV: r = &L->dqkv; break;
    case TP_TAP_DH: r = &L->dh_f; break;
    case TP_TAP_QKV_LO:
      if (!L->split_scores) return TP_ERR_UNSUPPORTED;
      r = &L->qkv_lo;
      break;
    case TP_TAP_GRAD_SCALE:
      if (L->sdt != DT_BF16) return TP_ERR_UNSUPPORTED;  // no scaling on the fp32 path
      *offset = L->gscale.off + kAmaxFloats * sizeof(float);
      *bytes = 2 * sizeof(float);
      return TP_OK;
    default: return TP_ERR_ARG;
  }
  *offset = r->off;
  *bytes = r->bytes;
  return TP_OK;
}

}  // extern "C"
