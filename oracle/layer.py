"""fp64 CPU oracle of one tensor-parallel rank's pre-LN transformer layer shard.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
link this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
path.

What it computes, and where the pages fix it
--------------------------------------------
Source: "Megatron-LM: GPU-Cluster Training Parallelism" (blog walkthrough of
arXiv 1909.08053 and 2104.04473).

* Tensor parallelism is an exact re-partitioning of the layer's GEMMs
  (section "Paper 1: The f/g Conjugate Operators"): FC1 ``A = [A_1..A_t]`` is
  split by columns and GeLU is applied to each rank's slice; FC2 is split by
  rows and its outputs are summed by the g all-reduce. The attention block is
  split the same way by heads, and the output projection by rows. f is the
  identity forward and a gradient sum backward; g is a sum forward and the
  identity backward. Hence the oracle is the plain layer definition, run on
  the rank's slices (LOCAL), on the unsharded weights (FULL), or phase by
  phase with explicit sums between phases (PARTIALS).
* The fused QKV projection has head-interleaved columns
  (section "Paper 1: QKV Column-Parallel Splitting in Detail"): local head j
  reads Q from columns ``[3*dh*j, 3*dh*j + dh)``, then K, then V.
* Pre-LN placement (section "Paper 1: BERT LayerNorm Rearrangement"): each
  sublayer reads LN of the residual stream and adds its output to the
  un-normalised stream: ``y = x + Sublayer(LN(x))``.
* Bias + GeLU after FC1, bias + residual after the row-parallel GEMMs, and a
  scaled, masked softmax (general or causal mask) inside attention
  (section "Fused Transformer Kernels").

Readings where the pages are silent (each is listed in the design notes):
LayerNorm uses eps = 1e-5 and the biased (1/h) variance; GeLU is the exact
erf form ``u/2 * (1 + erf(u/sqrt(2)))`` (tanh form optional); the softmax scale
is ``1/sqrt(dh)``; masked entries are excluded exactly (P = 0); a padding
mask hides keys at positions >= the sequence's valid length, while every query
row is still computed; there is no dropout; the row-parallel biases b_o and
b_fc2 are added once, after the sum over ranks (LOCAL: by the calling rank;
PARTIALS: by rank 0). Backward is the exact gradient of
``loss = sum(out * dout)``.

All arrays are float64. Inputs may be any real arrays (the harness passes the
same bf16- or fp32-grid values the GPU receives).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

SQRT2 = np.sqrt(2.0)
INV_SQRT_2PI = 1.0 / np.sqrt(2.0 * np.pi)


# ----------------------------------------------------------------------------
# Elementary pieces
# ----------------------------------------------------------------------------
def layernorm_fwd(x, gamma, beta, eps):
    """LayerNorm over the last axis: mean, biased variance, rstd = (v+eps)^-1/2.
    Returns (y, xhat, rstd)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu) * rstd
    return gamma * xhat + beta, xhat, rstd


def layernorm_bwd(dy, xhat, rstd, gamma):
    """Exact gradient of LayerNorm. Returns (dx, dgamma, dbeta)."""
    g = dy * gamma
    dx = rstd * (g - g.mean(axis=-1, keepdims=True)
                 - xhat * (g * xhat).mean(axis=-1, keepdims=True))
    red = tuple(range(dy.ndim - 1))
    return dx, (dy * xhat).sum(axis=red), dy.sum(axis=red)


def gelu(u, form="erf"):
    if form == "erf":
        return 0.5 * u * (1.0 + erf(u / SQRT2))
    c = np.sqrt(2.0 / np.pi)
    return 0.5 * u * (1.0 + np.tanh(c * (u + 0.044715 * u ** 3)))


def gelu_grad(u, form="erf"):
    """d GeLU / du: Phi(u) + u * phi(u) for the erf form."""
    if form == "erf":
        return 0.5 * (1.0 + erf(u / SQRT2)) + u * INV_SQRT_2PI * np.exp(-0.5 * u * u)
    c = np.sqrt(2.0 / np.pi)
    inner = c * (u + 0.044715 * u ** 3)
    th = np.tanh(inner)
    return 0.5 * (1.0 + th) + 0.5 * u * (1.0 - th * th) * c * (1.0 + 3 * 0.044715 * u * u)


def key_mask(seq, mask, valid_len):
    """Boolean [b, s_q, s_k]: True where query i may attend to key k.
    causal: k <= i. padding: k < valid_len[b]."""
    b = len(valid_len)
    i = np.arange(seq)[:, None]
    k = np.arange(seq)[None, :]
    if mask == "causal":
        m = np.broadcast_to(k <= i, (b, seq, seq))
    else:
        m = np.stack([np.broadcast_to(k < int(L), (seq, seq)) for L in valid_len])
    return m


def attention_fwd(q, k, v, allowed):
    """q, k, v: [b, H, s, dh]; allowed: [b, s, s]. Scaled masked softmax
    attention. Returns (o [b, H, s, dh], p [b, H, s, s], lse [b, H, s]) where
    lse is the natural log of the softmax normaliser of the scaled scores."""
    dh = q.shape[-1]
    s = np.matmul(q, np.swapaxes(k, -1, -2)) / np.sqrt(dh)
    allowed = allowed[:, None, :, :]
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.where(allowed, np.exp(s - m), 0.0)
    tot = e.sum(axis=-1, keepdims=True)
    p = e / tot
    return np.matmul(p, v), p, (m + np.log(tot))[..., 0]


def attention_bwd(q, k, v, p, do):
    """Gradients of o = softmax_masked(q k^T / sqrt(dh)) v given p (masked
    entries exactly 0)."""
    dh = q.shape[-1]
    dv = np.matmul(np.swapaxes(p, -1, -2), do)
    dp = np.matmul(do, np.swapaxes(v, -1, -2))
    ds = p * (dp - (dp * p).sum(axis=-1, keepdims=True))
    dq = np.matmul(ds, k) / np.sqrt(dh)
    dk = np.matmul(np.swapaxes(ds, -1, -2), q) / np.sqrt(dh)
    return dq, dk, dv


def split_heads(qkv, b, s, heads, dh):
    """Head-interleaved [n, 3*heads*dh] -> q, k, v each [b, heads, s, dh]."""
    t = qkv.reshape(b, s, heads, 3, dh)
    q = np.ascontiguousarray(t[:, :, :, 0, :].transpose(0, 2, 1, 3))
    k = np.ascontiguousarray(t[:, :, :, 1, :].transpose(0, 2, 1, 3))
    v = np.ascontiguousarray(t[:, :, :, 2, :].transpose(0, 2, 1, 3))
    return q, k, v


def merge_heads(q, k, v):
    """Inverse of split_heads: [b, heads, s, dh] x3 -> [b*s, 3*heads*dh]."""
    b, H, s, dh = q.shape
    t = np.stack([q, k, v], axis=3)            # [b, H, s, 3, dh]
    return t.transpose(0, 2, 1, 3, 4).reshape(b * s, H * 3 * dh)


def heads_to_rows(o):
    """[b, H, s, dh] -> [b*s, H*dh] with head-major columns (j*dh + e)."""
    b, H, s, dh = o.shape
    return o.transpose(0, 2, 1, 3).reshape(b * s, H * dh)


def rows_to_heads(x, b, s, H, dh):
    return x.reshape(b, s, H, dh).transpose(0, 2, 1, 3)


def _f64(p):
    return {k: np.asarray(v, dtype=np.float64) for k, v in p.items()}


# ----------------------------------------------------------------------------
# The layer on one set of weights (LOCAL on a rank's slices, FULL on all)
# ----------------------------------------------------------------------------
def layer(params, x, dout, heads, mask="causal", valid_len=None, eps=1e-5,
          gelu_form="erf", want_p=False, progress=None):
    """Forward and backward of the pre-LN layer on the given weights.

    params: dict of ln1_gamma, ln1_beta, w_qkv [h, 3*hl], b_qkv, w_o [hl, h],
    b_o, ln2_gamma, ln2_beta, w_fc1 [h, fl], b_fc1, w_fc2 [fl, h], b_fc2.
    heads: number of heads those weights hold (hl = heads * dh).
    x, dout: [b, s, h]. Returns a dict of outputs, gradients and the
    intermediates (rows are tokens, n = b*s). ``progress(step)`` is called
    after each step when given (long runs report as they go)."""
    say = progress or (lambda step: None)
    P = _f64(params)
    x = np.asarray(x, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    b, s, h = x.shape
    n = b * s
    hl = P["w_o"].shape[0]
    dh = hl // heads
    if valid_len is None:
        valid_len = np.full(b, s)
    allowed = key_mask(s, mask, valid_len)
    X = x.reshape(n, h)
    D = dout.reshape(n, h)

    # forward
    a, xhat1, rstd1 = layernorm_fwd(X, P["ln1_gamma"], P["ln1_beta"], eps)
    qkv = a @ P["w_qkv"] + P["b_qkv"]
    q, k, v = split_heads(qkv, b, s, heads, dh)
    say("qkv")
    oh, p, lse = attention_fwd(q, k, v, allowed)
    o = heads_to_rows(oh)
    say("attention")
    h_mid = X + P["b_o"] + o @ P["w_o"]
    c, xhat2, rstd2 = layernorm_fwd(h_mid, P["ln2_gamma"], P["ln2_beta"], eps)
    u = c @ P["w_fc1"] + P["b_fc1"]
    z = gelu(u, gelu_form)
    out = h_mid + P["b_fc2"] + z @ P["w_fc2"]
    say("forward")

    # backward of loss = sum(out * dout)
    g = {}
    g["b_fc2"] = D.sum(axis=0)
    g["w_fc2"] = z.T @ D
    dz = D @ P["w_fc2"].T
    du = dz * gelu_grad(u, gelu_form)
    g["b_fc1"] = du.sum(axis=0)
    g["w_fc1"] = c.T @ du
    dc = du @ P["w_fc1"].T
    say("mlp backward")
    dh2, g["ln2_gamma"], g["ln2_beta"] = layernorm_bwd(dc, xhat2, rstd2, P["ln2_gamma"])
    dhm = dh2 + D
    g["b_o"] = dhm.sum(axis=0)
    g["w_o"] = o.T @ dhm
    do = dhm @ P["w_o"].T
    dq, dk, dv = attention_bwd(q, k, v, p, rows_to_heads(do, b, s, heads, dh))
    dqkv = merge_heads(dq, dk, dv)
    say("attention backward")
    g["b_qkv"] = dqkv.sum(axis=0)
    g["w_qkv"] = a.T @ dqkv
    da = dqkv @ P["w_qkv"].T
    dx1, g["ln1_gamma"], g["ln1_beta"] = layernorm_bwd(da, xhat1, rstd1, P["ln1_gamma"])
    dx = dx1 + dhm
    say("backward")

    res = {
        "out": out.reshape(b, s, h), "dx": dx.reshape(b, s, h), "grads": g,
        "a": a, "mean1": X.mean(axis=1), "rstd1": rstd1[:, 0], "qkv": qkv, "o": o,
        "h_mid": h_mid, "rstd2": rstd2[:, 0], "c": c, "u": u, "z": z,
        "du": du, "dc": dc, "dh": dhm, "do": do, "dqkv": dqkv, "da": da,
        "lse": lse,
    }
    if want_p:
        res["p"] = p
    return res


def layer_local(rank_params, x, dout, dims, valid_len=None, **kw):
    """LOCAL(r): the rank's slices with identity exchanges (the measured
    function; the whole layer when t = 1)."""
    return layer(rank_params, x, dout, dims.heads_local, dims.mask, valid_len, **kw)


def layer_full(full_params, x, dout, dims, valid_len=None, **kw):
    """FULL: the unsharded layer."""
    return layer(full_params, x, dout, dims.heads, dims.mask, valid_len, **kw)


# ----------------------------------------------------------------------------
# PARTIALS: each rank's phase outputs with explicit sums for f and g
# ----------------------------------------------------------------------------
def layer_partials(per_rank, x, dout, dims, valid_len=None, eps=1e-5, gelu_form="erf"):
    """Runs all t ranks phase by phase. g sums the row-parallel partials in
    forward; f sums the column-parallel input gradients in backward. Rank 0
    adds the row-parallel biases and the residuals (once).

    Returns dict with per-rank partials ("pa", "po", "dc_part", "da_part"),
    the summed tensors ("h_mid", "out", "dc", "da", "dx") and per-rank grads."""
    t = len(per_rank)
    P = [_f64(p) for p in per_rank]
    x = np.asarray(x, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    b, s, h = x.shape
    n = b * s
    Hl = dims.heads_local
    dh = dims.head_dim
    if valid_len is None:
        valid_len = np.full(b, s)
    allowed = key_mask(s, dims.mask, valid_len)
    X = x.reshape(n, h)
    D = dout.reshape(n, h)
    R0 = P[0]  # replicated parameters are identical on every rank

    a, xhat1, rstd1 = layernorm_fwd(X, R0["ln1_gamma"], R0["ln1_beta"], eps)
    attn = []
    pa = []
    for r in range(t):
        qkv = a @ P[r]["w_qkv"] + P[r]["b_qkv"]
        q, k, v = split_heads(qkv, b, s, Hl, dh)
        oh, p, _ = attention_fwd(q, k, v, allowed)
        o = heads_to_rows(oh)
        part = o @ P[r]["w_o"]
        if r == 0:
            part = part + X + R0["b_o"]
        pa.append(part)
        attn.append((q, k, v, p, o))
    h_mid = sum(pa)                                      # g (forward sum)
    c, xhat2, rstd2 = layernorm_fwd(h_mid, R0["ln2_gamma"], R0["ln2_beta"], eps)
    po, us, zs = [], [], []
    for r in range(t):
        u = c @ P[r]["w_fc1"] + P[r]["b_fc1"]
        z = gelu(u, gelu_form)
        part = z @ P[r]["w_fc2"]
        if r == 0:
            part = part + h_mid + R0["b_fc2"]
        po.append(part)
        us.append(u)
        zs.append(z)
    out = sum(po)                                        # g (forward sum)

    grads = [dict() for _ in range(t)]
    dc_part = []
    for r in range(t):                                   # g backward = identity
        g = grads[r]
        g["b_fc2"] = D.sum(axis=0)
        g["w_fc2"] = zs[r].T @ D
        du = (D @ P[r]["w_fc2"].T) * gelu_grad(us[r], gelu_form)
        g["b_fc1"] = du.sum(axis=0)
        g["w_fc1"] = c.T @ du
        dc_part.append(du @ P[r]["w_fc1"].T)
    dc = sum(dc_part)                                    # f (backward sum)
    dh2, dg2, db2 = layernorm_bwd(dc, xhat2, rstd2, R0["ln2_gamma"])
    dhm = dh2 + D
    da_part = []
    for r in range(t):
        g = grads[r]
        g["ln2_gamma"], g["ln2_beta"] = dg2, db2
        g["b_o"] = dhm.sum(axis=0)
        q, k, v, p, o = attn[r]
        g["w_o"] = o.T @ dhm
        do = dhm @ P[r]["w_o"].T
        dq, dk, dv = attention_bwd(q, k, v, p, rows_to_heads(do, b, s, Hl, dh))
        dqkv = merge_heads(dq, dk, dv)
        g["b_qkv"] = dqkv.sum(axis=0)
        g["w_qkv"] = a.T @ dqkv
        da_part.append(dqkv @ P[r]["w_qkv"].T)
    da = sum(da_part)                                    # f (backward sum)
    dx1, dg1, db1 = layernorm_bwd(da, xhat1, rstd1, R0["ln1_gamma"])
    for g in grads:
        g["ln1_gamma"], g["ln1_beta"] = dg1, db1
    dx = dx1 + dhm
    return {
        "pa": pa, "po": po, "dc_part": dc_part, "da_part": da_part,
        "h_mid": h_mid, "out": out.reshape(b, s, h), "dc": dc, "dh": dhm, "da": da,
        "dx": dx.reshape(b, s, h), "grads": grads,
    }


def assemble_full_grads(grads_per_rank, t):
    """Concatenate per-rank gradients of sharded tensors into unsharded layout
    (columns for QKV/FC1, rows for W_o/FC2); replicated grads from rank 0."""
    out = {}
    for name in grads_per_rank[0]:
        if name in ("w_qkv", "w_fc1"):
            out[name] = np.concatenate([g[name] for g in grads_per_rank], axis=1)
        elif name in ("b_qkv", "b_fc1", "w_o", "w_fc2"):
            out[name] = np.concatenate([g[name] for g in grads_per_rank], axis=0)
        else:
            out[name] = grads_per_rank[0][name]
    return out


# ----------------------------------------------------------------------------
# Algorithmic FLOP count (what the method must compute; no recompute, no
# masked work, no LayerNorm/elementwise work)
# ----------------------------------------------------------------------------
def flops_fwd_bwd(dims, valid_len=None):
    n = dims.tokens
    h, hl, fl = dims.hidden, dims.hidden_local, dims.ffn_local
    gemm = 2 * n * (h * 3 * hl + hl * h + h * fl + fl * h)
    if dims.mask == "causal":
        pairs = dims.batch * dims.seq * (dims.seq + 1) // 2
    else:
        pairs = dims.seq * int(np.sum(valid_len))
    attn = 4 * dims.head_dim * dims.heads_local * pairs
    return 3 * (gemm + attn)
