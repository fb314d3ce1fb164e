/*
 * tp_layer.h -- one tensor-parallel rank's share of a pre-LayerNorm
 * transformer layer, forward and backward, on an AMD Instinct MI355X (gfx950).
 *
 * What the layer computes is defined in "Megatron-LM: GPU-Cluster Training
 * Parallelism" (blog walkthrough of arXiv 1909.08053 / 2104.04473):
 *   - section "Paper 1: The f/g Conjugate Operators": FC1 is split by columns
 *     (GeLU applied to the local slice), FC2 by rows; the attention block is
 *     split by heads and its output projection by rows. g sums the two
 *     row-parallel outputs in forward (identity in backward); f is the identity
 *     in forward and sums the input gradients of the two column-parallel GEMMs
 *     in backward. Two exchanges per direction per layer.
 *   - section "Paper 1: QKV Column-Parallel Splitting in Detail": the fused QKV
 *     weight has head-interleaved columns [Q_0 K_0 V_0 | Q_1 K_1 V_1 | ...], so
 *     rank r of t owns the contiguous column block [r*3h/t, (r+1)*3h/t), i.e.
 *     whole heads r*H/t .. (r+1)*H/t - 1, and attention needs no exchange.
 *   - section "Paper 1: BERT LayerNorm Rearrangement": pre-LN placement,
 *     y = x + Sublayer(LN(x)).
 *   - section "Fused Transformer Kernels": bias+GeLU after FC1,
 *     bias(+dropout)+residual after the row-parallel GEMMs, scale-mask-softmax
 *     with general or causal masks, attention read in place (no transposes).
 *
 * One rank's forward (TP_ALL), with n = batch*seq tokens, h hidden,
 * H_l = heads/t local heads of dimension dh = hidden/heads, h_l = H_l*dh,
 * f_l = ffn/t:
 *   a     = LN1(x)                               (gamma1, beta1; eps; biased var)
 *   qkv   = a @ W_qkv,r + b_qkv,r                [n, 3*h_l] head-interleaved
 *   o     = softmax_mask(Q K^T / sqrt(dh)) V     per local head, [n, h_l]
 *   h_mid = x + b_o + o @ W_o,r                  (g: sum over ranks)
 *   c     = LN2(h_mid)
 *   z     = GeLU(c @ W_fc1,r + b_fc1,r)          [n, f_l]
 *   out   = h_mid + b_fc2 + z @ W_fc2,r          (g: sum over ranks)
 * Backward is the exact gradient of sum(out * dout).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensors are device pointers, row-major and contiguous, 16-byte
 *    aligned (TP_ERR_ALIGN otherwise). Tokens are [batch, seq, .].
 *  - Weights use the X @ W orientation [in, out]. Shapes of rank r's slices:
 *      ln1_gamma, ln1_beta, ln2_gamma, ln2_beta, b_o, b_fc2 : [h]   (replicated)
 *      w_qkv [h, 3*h_l], b_qkv [3*h_l]  (columns r*3*h_l ... of the full tensor)
 *      w_o   [h_l, h]                   (rows r*h_l ... of the full tensor)
 *      w_fc1 [h, f_l],   b_fc1 [f_l]
 *      w_fc2 [f_l, h]
 *  - Storage dtype (TP_DTYPE_F32 or TP_DTYPE_BF16) applies to x, dout,
 *    out (TP_ALL) and every parameter. Accumulation and statistics are fp32.
 *    dx, the gradient of the residual stream handed to the layer below, is
 *    fp32 by default (tp_layer_opts.dx_dtype selects the storage dtype
 *    instead), as are the other residual-stream tensors crossing phases.
 *    Every gradient of a parameter is written in fp32. With TP_DTYPE_BF16
 *    the activations and gradients kept inside the layer (LayerNorm outputs,
 *    qkv, attention output, FC1 pre/post activation and their gradients) are
 *    IEEE fp16, fed to fp16 MFMA (same rate as bf16 on gfx950). The forward
 *    phases copy the bf16 weights they use into fp16 copies in the workspace
 *    (the backward reads those copies, so the weights must not change in
 *    between), and the MLP backward copies dout to fp16; the conversion is
 *    exact in fp16's normal range. The residual stream h_mid and its
 *    gradient are fp32.
 *  - Exchange partials (the tensors the f/g all-reduce would sum) are fp32
 *    [n, h] buffers owned by the caller.
 *  - The caller owns all memory, including the workspace. The library never
 *    allocates device memory, never synchronises the stream and keeps no
 *    pointer beyond a call. Work is enqueued on `hip_stream` (a hipStream_t;
 *    NULL = the null stream) and the call returns after enqueue. A handle must
 *    not be used on two streams at once. Asynchronous device faults surface at
 *    the caller's synchronisation.
 *  - The backward runs its weight and bias gradients on a second stream of
 *    the handle's own (created, with default priority, on the current device
 *    by the first tp_layer_bwd call) concurrently with the data-gradient
 *    chain: it waits for `hip_stream` through an event before each such
 *    group, and every backward phase makes `hip_stream` wait for it before
 *    returning, so all of a phase's outputs are ordered on `hip_stream` as if
 *    it had run alone (this also holds under stream capture). The handle must
 *    be used on that device afterwards.
 *  - Return value: TP_OK (0) or a negative TP_ERR_* code. No exceptions cross
 *    the ABI, nothing is printed, nothing aborts. After an error the handle
 *    stays valid and nothing has been enqueued (except TP_ERR_HIP, which
 *    reports a failed launch: some kernels of that call may have run).
 */
#ifndef TP_LAYER_H
#define TP_LAYER_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TP_OK = 0,
  TP_ERR_ARG = -1,          /* NULL handle/struct/pointer or a value <= 0 */
  TP_ERR_SHAPE = -2,        /* divisibility or rank range */
  TP_ERR_UNSUPPORTED = -3,  /* dtype, mask, gelu form or head dim not built */
  TP_ERR_ALIGN = -4,        /* a pointer is not 16-byte aligned */
  TP_ERR_WORKSPACE = -5,    /* workspace NULL or smaller than required */
  TP_ERR_HIP = -6,          /* a HIP launch or runtime call failed */
  TP_ERR_PHASE = -7,        /* phase out of range */
  TP_ERR_NOMEM = -8         /* host memory for the handle could not be allocated */
};

enum { TP_DTYPE_F32 = 0, TP_DTYPE_BF16 = 1 };
enum { TP_MASK_CAUSAL = 0, TP_MASK_PADDING = 1 };
enum { TP_GELU_ERF = 0, TP_GELU_TANH = 1 };
/* How the 16-bit path forms the attention scores Q K^T (TP_DTYPE_BF16 only):
 * TP_SCORES_FP16 uses the fp16 Q and K; TP_SCORES_SPLIT also keeps the fp16
 * rounding residuals Ql, Kl of the QKV projection and sums
 * Q K^T as Qh Kh^T + Qh Kl^T + Ql Kh^T (about fp32-accurate
 * scores, three times the score MFMAs); TP_SCORES_AUTO picks SPLIT for
 * hidden >= 8192. */
enum { TP_SCORES_AUTO = 0, TP_SCORES_FP16 = 1, TP_SCORES_SPLIT = 2 };
/* Activation recomputation (selective recomputation, "Megatron-LM:
 * GPU-Cluster Training Parallelism", section "Microbatch and Activation
 * Memory Tradeoff"). TP_RECOMPUTE_NONE keeps GeLU'(u) [n, f_l], the
 * derivative of the FC1 activation at its pre-activation
 * u = c @ W_fc1,r + b_fc1,r (computed in the FC1 epilogue together with
 * GeLU(u)), from forward to backward. TP_RECOMPUTE_FC1 does not keep it: the
 * backward recomputes it (one more FC1 GEMM) and the workspace shrinks by
 * n*f_l elements. The attention probabilities are never
 * kept in either mode (the backward recomputes them from the saved
 * log-sum-exp). */
enum { TP_RECOMPUTE_NONE = 0, TP_RECOMPUTE_FC1 = 1 };

/* Forward phases. TP_ALL runs the whole shard with both g exchanges taken as
 * the identity: the rank's own partial stands in for the sum (exactly the
 * unsharded layer when t = 1). The split phases expose the two g exchanges
 * so a caller can sum the t partials between them. */
enum { TP_ALL = 0, TP_FWD_ATTN = 1, TP_FWD_MLP = 2 };
/* Backward phases (TP_ALL = 0 as above), split at the two f exchanges. */
enum { TP_BWD_MLP = 1, TP_BWD_ATTN = 2, TP_BWD_LN1 = 3 };

/* Sequence-parallel layout (opts->sequence_parallel = 1): the sequence
 * parallelism that the megatron-core package description recommends with
 * tensor parallelism (section "Tensor Parallelism (TP)"), applied to the f
 * and g of "Megatron-LM: GPU-Cluster Training Parallelism", section "Paper 1:
 * The f/g Conjugate Operators". Rank r owns the token rows
 * [r*n/t, (r+1)*n/t) of the [n, h] token matrix ((batch*seq) % t == 0) for
 * everything outside the tensor-parallel GEMMs and attention: both
 * LayerNorms, the residual adds and the replicated biases b_o and b_fc2. In
 * the [batch, seq, h] layout those rows are a contiguous block of tokens; in
 * a [seq, batch, h] layout the same block is a slice of the sequence. Every
 * g all-reduce becomes a reduce-scatter to those rows; every f becomes an
 * all-gather of them. A gathered buffer is a caller-owned [n, h] tensor. A
 * phase that produces rows writes only its own rows [r*n/t, (r+1)*n/t) into
 * it; the all-gather fills the other ranks' rows; on one device the t ranks
 * can share one gathered buffer and need no copy at all. A phase that
 * consumes it reads all n rows. "act" is the internal dtype (fp16 for
 * TP_DTYPE_BF16, fp32 for TP_DTYPE_F32).
 * Forward, in order (reduce-scatters and all-gathers between them):
 *   TP_FWD_SP_LN1 : x = this rank's rows of x            -> gathered rows = LN1 (act)
 *   TP_FWD_SP_ATTN: gathered = all of LN1's output       -> out = fp32 [n, h] partial o @ W_o,r
 *   TP_FWD_SP_LN2 : reduced = this rank's rows of the summed partial (fp32 [n/t, h]),
 *                   x = this rank's rows of x            -> h_mid = reduced + b_o + x (kept),
 *                                                           gathered rows = LN2(h_mid) (act)
 *   TP_FWD_SP_MLP : gathered = all of LN2's output       -> out = fp32 [n, h] partial z @ W_fc2,r
 *   TP_FWD_SP_OUT : reduced = this rank's rows of the summed partial
 *                                                        -> out = reduced + b_fc2 + h_mid
 *                                                           ([n/t, h], storage dtype)
 * Backward, in order:
 *   TP_BWD_SP_MLP : dout = this rank's rows of the output gradient, gathered_grad = all
 *                   of it (storage dtype), gathered_act = the gathered LN2 output of the
 *                   forward            -> partial = fp32 [n, h] du @ W_fc1,r^T; d_w_fc1,
 *                                         d_b_fc1, d_w_fc2 and (this rank's rows) d_b_fc2
 *   TP_BWD_SP_LN2 : dc = this rank's rows of the summed partial, dout as above
 *                                      -> gathered_grad rows = dh (act; dh kept); d_ln2_*,
 *                                         d_b_o over this rank's rows
 *   TP_BWD_SP_ATTN: gathered_grad = all of dh, gathered_act = the gathered LN1 output
 *                                      -> partial = fp32 [n, h] dqkv @ W_qkv,r^T; d_w_o,
 *                                         d_w_qkv, d_b_qkv
 *   TP_BWD_SP_LN1 : da = this rank's rows of the summed partial, x = this rank's rows
 *                                      -> dx rows ([n/t, h]); d_ln1_* over this rank's rows
 * Gradients of the replicated LayerNorm parameters and of b_o, b_fc2 cover
 * this rank's rows only: their sum over the ranks is the full gradient. A
 * handle in this layout accepts only these phases (TP_ERR_PHASE otherwise). */
enum {
  TP_FWD_SP_LN1 = 3, TP_FWD_SP_ATTN = 4, TP_FWD_SP_LN2 = 5, TP_FWD_SP_MLP = 6, TP_FWD_SP_OUT = 7
};
enum { TP_BWD_SP_MLP = 4, TP_BWD_SP_LN2 = 5, TP_BWD_SP_ATTN = 6, TP_BWD_SP_LN1 = 7 };

typedef struct tp_layer tp_layer;

enum { TP_OVERLAP_AUTO = 0, TP_OVERLAP_OFF = 1, TP_OVERLAP_ON = 2 };

typedef struct {
  float ln_eps;     /* LayerNorm epsilon (default 1e-5) */
  int gelu;         /* TP_GELU_ERF (default) or TP_GELU_TANH */
  int dx_dtype;     /* dtype of tp_bwd_io.dx: TP_DTYPE_F32 (default, also the
                       value of a zeroed struct) or the layer's storage dtype */
  int scores;       /* TP_SCORES_AUTO (default), TP_SCORES_FP16 or TP_SCORES_SPLIT */
  int recompute;    /* TP_RECOMPUTE_NONE (default) or TP_RECOMPUTE_FC1 */
  int sequence_parallel;  /* 0 (default) or 1: the TP_*_SP_* phases below */
  int overlap;      /* TP_OVERLAP_AUTO (default, also a zeroed struct),
                       TP_OVERLAP_OFF or TP_OVERLAP_ON: whether TP_ALL runs
                       two independent pieces on a second stream of the
                       handle, joined before its results are used: in the
                       forward (bf16 layers) the fp16 copies of the MLP
                       weights while attention and the output projection run
                       (FC1 waits for W_fc1's copy only, FC2 for W_fc2's);
                       in the backward the gradient of W_o while dO and the
                       attention backward run. Otherwise every kernel runs on
                       the caller's stream. Results are bitwise identical.
                       AUTO overlaps from hidden >= 8192: on one MI355X the
                       two overlaps took the 1T shard's step 13.79 -> 13.67
                       -> 13.30 ms (measured in one box each), while the
                       backward one made the 1.2B and 8.3B shards 0.5 %
                       slower. (Overlapping the other weight gradients with
                       the data-gradient GEMMs measured slower everywhere:
                       the GEMMs compete for the same compute units.) */
} tp_layer_opts;

/* Parameters of rank r (shapes above) and, for TP_MASK_PADDING, the number
 * of valid key positions of each sequence (int32 [batch], values in
 * [1, seq]; keys at positions >= valid_len[b] are excluded, every query row
 * is still computed; values outside [1, seq] give undefined results but no
 * out-of-bounds access). valid_len is ignored for TP_MASK_CAUSAL. */
typedef struct {
  const void *ln1_gamma, *ln1_beta;
  const void *w_qkv, *b_qkv;
  const void *w_o, *b_o;
  const void *ln2_gamma, *ln2_beta;
  const void *w_fc1, *b_fc1;
  const void *w_fc2, *b_fc2;
  const int *valid_len;
} tp_params;

typedef struct {
  const tp_params *params;
  const void *x;         /* [n, h] storage dtype: TP_ALL, TP_FWD_ATTN */
  const float *h_mid;    /* TP_FWD_MLP: the summed fp32 [n, h] from the first g */
  void *out;             /* TP_ALL: [n, h] storage dtype.
                            TP_FWD_ATTN: fp32 [n, h] partial o @ W_o,r
                              (+ x + b_o on rank 0).
                            TP_FWD_MLP: fp32 [n, h] partial z @ W_fc2,r
                              (+ h_mid + b_fc2 on rank 0). */
  void *workspace;       /* tp_layer_create's workspace_bytes, same buffer for
                            the matching backward and untouched in between */
  size_t workspace_bytes;
  const float *reduced;  /* sequence-parallel phases: this rank's rows of a summed
                            fp32 partial, [n/t, h] */
  void *gathered;        /* sequence-parallel phases: [n, h] act buffer (see above) */
} tp_fwd_io;

typedef struct {
  const tp_params *params;
  const void *x;         /* [n, h] storage dtype, the forward input: TP_ALL, TP_BWD_LN1 */
  const void *dout;      /* [n, h] storage dtype: TP_ALL, TP_BWD_MLP, TP_BWD_ATTN */
  const float *dc;       /* TP_BWD_ATTN: summed fp32 [n, h] (first f exchange) */
  const float *da;       /* TP_BWD_LN1: summed fp32 [n, h] (second f exchange) */
  float *partial;        /* TP_BWD_MLP: fp32 [n, h] <- this rank's term of the gradient
                              of LN2's output, du @ W_fc1,r^T (first f exchange input);
                            TP_BWD_ATTN: fp32 [n, h] <- this rank's term of the gradient
                              of LN1's output, dqkv @ W_qkv,r^T (second f exchange input) */
  void *dx;              /* TP_ALL, TP_BWD_LN1: [n, h], fp32 or (opts.dx_dtype)
                            the storage dtype */
  /* fp32 gradients, shapes of the matching parameters. Written by:
   *   TP_BWD_MLP : d_w_fc2, d_b_fc2, d_w_fc1, d_b_fc1
   *   TP_BWD_ATTN: d_ln2_gamma, d_ln2_beta, d_w_o, d_b_o, d_w_qkv, d_b_qkv
   *   TP_BWD_LN1 : d_ln1_gamma, d_ln1_beta
   *   TP_ALL     : all of them */
  float *d_ln1_gamma, *d_ln1_beta;
  float *d_w_qkv, *d_b_qkv;
  float *d_w_o, *d_b_o;
  float *d_ln2_gamma, *d_ln2_beta;
  float *d_w_fc1, *d_b_fc1;
  float *d_w_fc2, *d_b_fc2;
  int accumulate;        /* 0: overwrite the parameter gradients; 1: add to them */
  void *workspace;
  size_t workspace_bytes;
  const void *gathered_act;  /* sequence-parallel phases: gathered LN output [n, h] act */
  void *gathered_grad;       /* sequence-parallel phases: gathered gradient [n, h] */
} tp_bwd_io;

/* Create a handle for rank `rank` of a t-way split of a layer with hidden
 * size `hidden`, `heads` attention heads, FFN size `ffn`, sequence length
 * `seq` and micro-batch `micro_batch`. These are the problem statement of
 * "Megatron-LM: GPU-Cluster Training Parallelism", sections "Paper 1: The f/g
 * Conjugate Operators" (t-way split of both blocks) and "Paper 1: QKV
 * Column-Parallel Splitting in Detail" (whole heads per rank, so heads % t
 * == 0; 3h/t QKV columns per rank).
 *   dtype: TP_DTYPE_F32 or TP_DTYPE_BF16. mask: TP_MASK_CAUSAL/TP_MASK_PADDING.
 *   opts: NULL for the defaults (eps 1e-5, exact-erf GeLU, fp32 dx, automatic
 *     score precision); opts->dx_dtype other than TP_DTYPE_F32 or `dtype`,
 *     an unknown opts->scores or opts->recompute, or TP_SCORES_SPLIT with
 *     TP_DTYPE_F32 are TP_ERR_UNSUPPORTED; opts->sequence_parallel = 1 with
 *     (micro_batch*seq) % t != 0 is TP_ERR_SHAPE.
 * Checks: every size > 0; hidden % heads == 0; heads % t == 0; ffn % t == 0;
 * (ffn/t) % 8 == 0; 0 <= rank < t; head dim in {32, 64, 96, 128, 160}
 * (TP_ERR_UNSUPPORTED otherwise). Allocates no device memory. On success
 * writes the handle to *out and the workspace size the fwd/bwd calls need to
 * *workspace_bytes; on failure sets *out = NULL (TP_ERR_NOMEM if the host
 * allocation of the handle failed). Parameter gradients are always written
 * in fp32 (there is no storage-dtype gradient option): they are what an
 * optimizer accumulates over micro-batches before its step. */
int tp_layer_create(int hidden, int heads, int ffn, int seq, int micro_batch,
                    int t, int rank, int dtype, int mask,
                    const tp_layer_opts *opts, tp_layer **out,
                    size_t *workspace_bytes);

/* Enqueue a forward phase (TP_ALL, TP_FWD_ATTN or TP_FWD_MLP). The layer
 * computed is the pre-LN block of "Megatron-LM: GPU-Cluster Training
 * Parallelism", section "Paper 1: BERT LayerNorm Rearrangement", sharded as
 * in section "Paper 1: The f/g Conjugate Operators", with the fusions of
 * section "Fused Transformer Kernels" (bias + GeLU after FC1, bias + residual
 * after the row-parallel GEMMs, scale-mask-softmax attention read in place).
 * The phases end at the two g exchanges of the forward. */
int tp_layer_fwd(tp_layer *L, int phase, const tp_fwd_io *io, void *hip_stream);

/* Enqueue a backward phase (TP_ALL, TP_BWD_MLP, TP_BWD_ATTN or TP_BWD_LN1):
 * the exact gradient of sum(out * dout) for the forward above; the phases end
 * at the two f exchanges of the backward ("Megatron-LM: GPU-Cluster Training
 * Parallelism", section "Paper 1: The f/g Conjugate Operators": f sums the
 * input gradients of the column-parallel GEMMs, g is the identity).
 * Needs the workspace of the matching forward (TP_ALL after TP_ALL; the split
 * phases after both split forward phases), untouched since, and the backward
 * phases run in order on it: TP_BWD_MLP (or TP_ALL) derives from dout the
 * power of two S (max|S dout| in [1, 2); 1 for TP_DTYPE_F32) by which the
 * fp16 gradient tensors kept inside the layer are scaled, and TP_BWD_ATTN
 * reads it from the workspace. Every output is unscaled: the scaling only
 * keeps bf16 gradients of any magnitude inside fp16's range (scaling dout by
 * 2^k scales every gradient by exactly 2^k). */
int tp_layer_bwd(tp_layer *L, int phase, const tp_bwd_io *io, void *hip_stream);

/* Free the handle (host memory, the backward's side stream and events; no
 * device memory is owned). NULL is allowed. */
int tp_layer_destroy(tp_layer *L);

/* Single-GPU stand-in for the f/g all-reduce: dst[i] = sum_p parts[p][i] for
 * i < count, summed in fp32 in the order p = 0, 1, ... and written as
 * `dst_dtype` (TP_DTYPE_F32 or TP_DTYPE_BF16, round to nearest even).
 * `parts` is a host array of `nparts` (1..16) fp32 device pointers. It is
 * what the sum of the t ranks' partials would produce on t GPUs, used to
 * check the f/g identity with every shard run in sequence on one device. */
int tp_exchange_sum(void *dst, int dst_dtype, const float *const *parts,
                    int nparts, size_t count, void *hip_stream);

/* Decode step with a sharded KV cache ("Megatron-LM: GPU-Cluster Training
 * Parallelism", section "Paper 1: QKV Column-Parallel Splitting in Detail",
 * inference-time behaviour): generation keeps the training split. Each rank
 * appends the K and V of its own heads for the new token to its own shard of
 * the KV cache, which divides the cache memory by t, and the layer's two g
 * sums now cover one row per sequence.
 *
 * One call runs the layer for one new token of each of the handle's
 * micro_batch sequences (the decode batch B, 1 <= B <= 128), handles with
 * TP_MASK_CAUSAL only (TP_ERR_UNSUPPORTED otherwise); the handle's seq is not
 * used and the tensor-parallel phases apply whatever opts.sequence_parallel
 * says. For sequence b with its new token at position pos = positions[b]:
 *   a     = LN1(x[b])
 *   qkv   = a @ W_qkv,r + b_qkv,r
 *   K, V of local head j -> k_cache[b][j][pos], v_cache[b][j][pos]
 *   o_j   = softmax(q_j K_j[0..pos]^T / sqrt(dh)) V_j[0..pos]
 *           (the cache rows 0..pos, the new token included; rows > pos are
 *           never read)
 *   then h_mid, LN2, FC1 + GeLU, FC2 exactly as the forward, with n = B.
 * Phases as tp_layer_fwd: TP_ALL (both g sums the identity; out in the
 * storage dtype), TP_FWD_ATTN (out = fp32 [B, h] partial, + x + b_o on rank
 * 0), TP_FWD_MLP (h_mid = the summed fp32 [B, h]; out = fp32 partial,
 * + h_mid + b_fc2 on rank 0).
 * KV cache: k_cache and v_cache are [B, H_l, cache_len, dh] in the internal
 * activation type (fp16 for TP_DTYPE_BF16, fp32 for TP_DTYPE_F32), owned by
 * the caller; rank r holds heads r*H_l .. (r+1)*H_l - 1. A handle with split
 * scores (see TP_SCORES_*) also needs k_cache_lo, the same shape in fp16: the
 * fp16 rounding residual of each cached K value, the scores then use
 * K = k_cache + k_cache_lo. Positions are int32 device values; a position
 * outside [0, cache_len) gives undefined outputs for that sequence but no
 * access outside the cache (its K and V are not written).
 * Cost: every weight and the cache rows 0..pos are read once per call. */
typedef struct {
  const tp_params *params;
  const void *x;          /* [B, h] storage dtype: TP_ALL, TP_FWD_ATTN */
  const float *h_mid;     /* TP_FWD_MLP: the summed fp32 [B, h] */
  void *out;              /* TP_ALL: [B, h] storage dtype; split phases: fp32 [B, h] */
  void *k_cache, *v_cache;  /* TP_ALL, TP_FWD_ATTN: [B, H_l, cache_len, dh] act */
  void *k_cache_lo;       /* split scores only: [B, H_l, cache_len, dh] fp16 */
  const int *positions;   /* TP_ALL, TP_FWD_ATTN: int32 [B] */
  int cache_len;          /* rows per (sequence, head) of the caches, >= 1 */
  void *workspace;        /* tp_layer_decode_workspace bytes, 16-byte aligned */
  size_t workspace_bytes;
} tp_decode_io;

/* Workspace bytes of tp_layer_decode for this handle (a few MB; it does not
 * depend on cache_len). The contents need no initialisation and may be
 * reused freely between calls. */
int tp_layer_decode_workspace(const tp_layer *L, size_t *bytes);

/* Enqueue one decode phase (TP_ALL, TP_FWD_ATTN or TP_FWD_MLP). */
int tp_layer_decode(tp_layer *L, int phase, const tp_decode_io *io, void *hip_stream);

/* tp_layer_decode without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same phases, arguments, kernels and
 * results as tp_layer_decode, except that io->workspace and
 * io->workspace_bytes are not read: the decode scratch lives in a device
 * array of TP_DECODE_STATIC_MAX_BYTES inside the library, one per device,
 * held until the process ends (its address is looked up on the first call on
 * each device, with that device current; hip_stream must belong to it).
 * Handles whose tp_layer_decode_workspace exceeds that size get
 * TP_ERR_WORKSPACE (32 MB holds every decode batch up to 128 of shards up to
 * hidden 8192, and the 1T shard's up to 8). Nothing is allocated, no
 * allocating library routine is called, and the call is not timed by
 * tp_layer_profile. Every call on a device shares that device's array:
 * calls that overlap on one device (two streams, two threads, two handles)
 * race and must be ordered by the caller. The array keeps the last call's
 * contents; the decode kernels need it in no particular state. */
#define TP_DECODE_STATIC_MAX_BYTES (32u << 20)
int tp_layer_decode_static(tp_layer *L, int phase, const tp_decode_io *io, void *hip_stream);

/* Prefill into a cache: copy the K and V of every token of the last forward
 * on this handle (a TP_ALL, TP_FWD_ATTN or TP_FWD_SP_ATTN phase whose
 * workspace is passed here untouched) into rows 0..seq-1 of the caches of the
 * layout above (cache_len >= seq, else TP_ERR_SHAPE), and with split scores
 * the K residuals into k_cache_lo (required then, ignored otherwise). With a
 * right-padded prompt batch, the rows beyond a sequence's real length hold
 * the padding's K and V; decode steps overwrite them in order and never read
 * a row beyond their own position. */
int tp_layer_kv_fill(const tp_layer *L, const void *workspace, size_t workspace_bytes,
                     void *k_cache, void *v_cache, void *k_cache_lo, int cache_len,
                     void *hip_stream);

/* Test tap: byte offset and size inside the workspace of an intermediate
 * kept between forward and backward (TP_TAP_*). Layout is row-major;
 * "act" is fp16 for TP_DTYPE_BF16 and fp32 for TP_DTYPE_F32:
 *   TP_TAP_LN1_OUT  a      [n, h]      act
 *   TP_TAP_QKV      qkv    [n, 3*h_l]  act
 *   TP_TAP_ATTN_OUT o      [n, h_l]    act
 *   TP_TAP_LSE      log2-domain softmax normaliser [batch, H_l, seq] fp32:
 *                   log2(sum_k exp(S_ik)) with S the scaled scores
 *   TP_TAP_H_MID    h_mid  [n, h]      fp32
 *   TP_TAP_LN2_OUT  c      [n, h]      act
 *   TP_TAP_FC1_DGELU GeLU'(u) [n, f_l] act (derivative of the FC1 activation
 *                                      at the pre-activation u, kept for the
 *                                      backward; TP_ERR_UNSUPPORTED with
 *                                      TP_RECOMPUTE_FC1)
 *   TP_TAP_FC1_OUT  z      [n, f_l]    act
 *   TP_TAP_DQKV     S * dqkv [n, 3*h_l] act (after a backward; S as below)
 *   TP_TAP_DH       dh     [n, h]      fp32 (residual-stream grad, after TP_BWD_ATTN)
 *   TP_TAP_GRAD_SCALE  S, 1/S          2 x fp32 (TP_DTYPE_BF16 only, after a
 *                                      TP_ALL or TP_BWD_MLP backward): the power
 *                                      of two the backward's fp16 gradient chain
 *                                      is scaled by (see tp_layer_bwd);
 *                                      TP_ERR_UNSUPPORTED for TP_DTYPE_F32,
 *                                      where S = 1
 *   TP_TAP_QKV_LO   qkv - fp16(qkv) [n, 3*h_l] fp16: the score residuals kept
 *                                      with split scores (TP_SCORES_*);
 *                                      TP_ERR_UNSUPPORTED when the handle forms
 *                                      scores from qkv alone (this is how a
 *                                      caller learns what TP_SCORES_AUTO chose)
 * Returns TP_ERR_ARG for an unknown id. */
enum {
  TP_TAP_LN1_OUT = 0, TP_TAP_QKV = 1, TP_TAP_ATTN_OUT = 2, TP_TAP_LSE = 3,
  TP_TAP_H_MID = 4, TP_TAP_LN2_OUT = 5, TP_TAP_FC1_DGELU = 6, TP_TAP_FC1_OUT = 7,
  TP_TAP_DQKV = 8, TP_TAP_DH = 9, TP_TAP_GRAD_SCALE = 10, TP_TAP_QKV_LO = 11
};
int tp_layer_tap(const tp_layer *L, int tap, size_t *offset, size_t *bytes);

/* Measurement support (not needed to run the layer). When enabled, every
 * kernel launch group the handle enqueues is bracketed by two hipEvents
 * recorded on the call's stream, tagged with one of the classes below and
 * with its algorithmic work: FLOPs (2*M*N*K per GEMM; 4*dh*H_l per allowed
 * query-key pair for the attention forward, twice that backward) and bytes
 * (each input read once, each output written once). Enabling, disabling or
 * re-enabling clears what was recorded. The events are created on first use
 * and reused; no device memory is allocated. While profiling is on, the
 * backward enqueues everything on the call's stream (no second stream), so
 * each bracket times its launch group alone. */
enum {
  TP_K_GEMM = 0,      /* MFMA / FMA GEMMs incl. their split-K reduction */
  TP_K_ATTN_FWD = 1,  /* attention forward */
  TP_K_ATTN_BWD = 2,  /* attention backward (delta, dK/dV, dQ) */
  TP_K_LN_FWD = 3,    /* LayerNorm forward */
  TP_K_LN_BWD = 4,    /* LayerNorm backward + residual-gradient add */
  TP_K_REDUCE = 5,    /* column sums and partial reductions (bias / gamma / beta grads) */
  TP_K_CONVERT = 6,   /* bf16 -> fp16 copies of the weights and the upstream gradient */
  TP_K_COUNT = 7
};
/* attn_pairs: for a TP_MASK_PADDING handle, the number of allowed query-key
 * pairs per forward of the inputs the profiled calls will see (the sum over
 * sequences of seq * valid_len; the valid lengths are device data the library
 * does not read back), used only for the attention classes' FLOP counts;
 * 0 = unknown (those classes then report 0 FLOPs). Ignored for causal
 * handles, whose pair count follows from seq and micro_batch. */
int tp_layer_profile(tp_layer *L, int enable, double attn_pairs);

/* Totals for one class since profiling was enabled: number of launch groups,
 * summed event time in milliseconds, summed algorithmic FLOPs and bytes.
 * Waits on the host for the recorded events (call after the work is
 * enqueued; it synchronises with the last recorded event). */
int tp_layer_profile_read(tp_layer *L, int kclass, long *launches, double *ms,
                          double *flops, double *bytes);

#ifdef __cplusplus
}
#endif

#endif /* TP_LAYER_H */
