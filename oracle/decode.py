"""fp64 CPU oracle of one tensor-parallel rank's decode step with a sharded KV cache.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
link this module; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
path.

What it computes, and where the pages fix it
--------------------------------------------
Source: "Megatron-LM: GPU-Cluster Training Parallelism", section "Paper 1: QKV
Column-Parallel Splitting in Detail", its inference-time paragraph and table:
in generation the column split is the same as in training; each rank appends
the K and V of its own heads for the new token to its local share of the KV
cache (so the cache memory is divided by t), and the layer still needs the two
g sums per token, now over a single row per sequence. The layer itself is the
pre-LN layer of ``oracle.layer`` (sections "Paper 1: The f/g Conjugate
Operators", "Paper 1: BERT LayerNorm Rearrangement", "Fused Transformer
Kernels") restricted to one query row per sequence:

  a = LN1(x)                 qkv = a W_qkv + b_qkv (head-interleaved columns)
  cache[b, j, pos_b] <- (K_j, V_j) of the new token, for every local head j
  o_j = softmax(q_j K_j[0..pos_b]^T / sqrt(dh)) V_j[0..pos_b]   (causal: keys up
                                                            to and including the
                                                            new token's position)
  h_mid = x + b_o + o W_o    c = LN2(h_mid)    z = GeLU(c W_fc1 + b_fc1)
  out = h_mid + b_fc2 + z W_fc2

Readings where the pages are silent (listed in the design notes): the cache of
sequence b holds positions 0..cache_len-1 of that sequence, the new token of
sequence b sits at position pos_b (the number of tokens already cached), and
cache rows beyond pos_b are never read. Decode is causal generation; the
padding-mask layer has no decode step.

Pinned (tests/test_oracle_decode.py) against the batched causal forward of
``oracle.layer``, which has its own pins: a decode step equals the forward's
row at that position when the cache holds the forward's K and V of the earlier
rows, for every position, chained over several steps; plus closed forms
(position 0 copies the new V; equal keys average the cached V) and the sum over
ranks against the unsharded step.
"""
from __future__ import annotations

import numpy as np

from .layer import gelu, layernorm_fwd, _f64


def _qkv_heads(qkv, heads, dh):
    """Head-interleaved [B, 3*heads*dh] -> q, k, v each [B, heads, dh]."""
    t = qkv.reshape(qkv.shape[0], heads, 3, dh)
    return t[:, :, 0, :], t[:, :, 1, :], t[:, :, 2, :]


def decode_attention(q, kc, vc, pos):
    """One sequence: q [H, dh]; caches [H, L, dh] already holding the new
    token at ``pos``. Scaled softmax over keys 0..pos, then the weighted sum
    of the values. Returns o [H, dh]."""
    dh = q.shape[-1]
    k = kc[:, :pos + 1, :]
    v = vc[:, :pos + 1, :]
    s = np.einsum("hd,hkd->hk", q, k) / np.sqrt(dh)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=-1, keepdims=True)
    return np.einsum("hk,hkd->hd", p, v)


def _append_and_attend(qkv, k_cache, v_cache, positions, heads, dh):
    q, k, v = _qkv_heads(qkv, heads, dh)
    B = qkv.shape[0]
    o = np.zeros((B, heads, dh))
    for b in range(B):
        p = int(positions[b])
        k_cache[b, :, p, :] = k[b]
        v_cache[b, :, p, :] = v[b]
        o[b] = decode_attention(q[b], k_cache[b], v_cache[b], p)
    return o.reshape(B, heads * dh)


def decode_step(params, x, k_cache, v_cache, positions, heads, eps=1e-5, gelu_form="erf"):
    """The decode step on the given weights (a rank's slices with the g sums
    taken as the identity, or the unsharded weights).

    x [B, h]: the new token of each sequence; k_cache, v_cache
    [B, heads, L, dh]; positions int [B] in [0, L). The caches are not
    modified: updated copies are returned. Returns a dict with out, h_mid,
    a, qkv, o, c, z and the updated caches."""
    P = _f64(params)
    X = np.asarray(x, dtype=np.float64)
    kc = np.array(k_cache, dtype=np.float64)
    vc = np.array(v_cache, dtype=np.float64)
    dh = kc.shape[-1]
    a, _, _ = layernorm_fwd(X, P["ln1_gamma"], P["ln1_beta"], eps)
    qkv = a @ P["w_qkv"] + P["b_qkv"]
    o = _append_and_attend(qkv, kc, vc, positions, heads, dh)
    h_mid = X + P["b_o"] + o @ P["w_o"]
    c, _, _ = layernorm_fwd(h_mid, P["ln2_gamma"], P["ln2_beta"], eps)
    z = gelu(c @ P["w_fc1"] + P["b_fc1"], gelu_form)
    out = h_mid + P["b_fc2"] + z @ P["w_fc2"]
    return {"out": out, "h_mid": h_mid, "a": a, "qkv": qkv, "o": o, "c": c, "z": z,
            "k_cache": kc, "v_cache": vc}


def decode_partials(per_rank, x, caches, positions, dims, eps=1e-5, gelu_form="erf"):
    """All t ranks phase by phase, with the two g sums explicit: each rank
    attends over its own heads and its own cache shard; rank 0 adds the
    residuals and the row-parallel biases once.

    per_rank: the t parameter dicts; caches: t pairs (k, v) of
    [B, H_l, L, dh]. Returns the per-rank partials ("pa", "po"), the sums
    ("h_mid", "out") and the updated caches."""
    t = len(per_rank)
    P = [_f64(p) for p in per_rank]
    R0 = P[0]
    X = np.asarray(x, dtype=np.float64)
    Hl, dh = dims.heads_local, dims.head_dim
    a, _, _ = layernorm_fwd(X, R0["ln1_gamma"], R0["ln1_beta"], eps)
    pa, new_caches = [], []
    for r in range(t):
        kc = np.array(caches[r][0], dtype=np.float64)
        vc = np.array(caches[r][1], dtype=np.float64)
        qkv = a @ P[r]["w_qkv"] + P[r]["b_qkv"]
        o = _append_and_attend(qkv, kc, vc, positions, Hl, dh)
        part = o @ P[r]["w_o"]
        if r == 0:
            part = part + X + R0["b_o"]
        pa.append(part)
        new_caches.append((kc, vc))
    h_mid = sum(pa)                                    # g (forward sum)
    c, _, _ = layernorm_fwd(h_mid, R0["ln2_gamma"], R0["ln2_beta"], eps)
    po = []
    for r in range(t):
        z = gelu(c @ P[r]["w_fc1"] + P[r]["b_fc1"], gelu_form)
        part = z @ P[r]["w_fc2"]
        if r == 0:
            part = part + h_mid + R0["b_fc2"]
        po.append(part)
    return {"pa": pa, "po": po, "h_mid": h_mid, "out": sum(po), "caches": new_caches}

