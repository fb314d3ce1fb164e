"""Pure-Python loop forward of the pre-LN layer shard (no NumPy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). It is written
independently of ``oracle.layer``: every sum is an explicit loop over scalars,
so it pins the vectorised oracle's indexing (head interleave, transposes,
masks, residual placement) on small shapes. Definitions follow
"Megatron-LM: GPU-Cluster Training Parallelism", sections
"Paper 1: The f/g Conjugate Operators", "Paper 1: QKV Column-Parallel
Splitting in Detail", "Paper 1: BERT LayerNorm Rearrangement" and
"Fused Transformer Kernels", with the same readings as ``oracle.layer``
(eps 1e-5, biased variance, exact-erf GeLU, scale 1/sqrt(dh), masked keys
excluded).
"""
from __future__ import annotations

import math


def _tolist(a):
    return a.tolist() if hasattr(a, "tolist") else a


def _layernorm_row(row, gamma, beta, eps):
    h = len(row)
    mu = 0.0
    for v in row:
        mu += v
    mu /= h
    var = 0.0
    for v in row:
        var += (v - mu) * (v - mu)
    var /= h
    rstd = 1.0 / math.sqrt(var + eps)
    return [gamma[j] * (row[j] - mu) * rstd + beta[j] for j in range(h)]


def _vecmat(row, w, bias):
    """row [K] times w [K][N] plus bias [N]."""
    n_out = len(w[0])
    out = list(bias)
    for kk, rv in enumerate(row):
        wr = w[kk]
        for c in range(n_out):
            out[c] += rv * wr[c]
    return out


def forward(params, x, heads, mask="causal", valid_len=None, eps=1e-5, want_lse=False):
    """params: dict of arrays/lists (rank slice or unsharded); x [b][s][h].
    Returns out as nested lists [b][s][h]; with want_lse also the natural-log
    softmax normaliser of every attention row, lse[b][head][i] =
    log(sum over allowed keys of exp(scaled score)), from the same loop."""
    p = {k: _tolist(v) for k, v in params.items()}
    x = _tolist(x)
    b = len(x)
    s = len(x[0])
    hl = len(p["w_o"])
    dh = hl // heads
    if valid_len is None:
        valid_len = [s] * b
    valid_len = [int(v) for v in _tolist(valid_len)]
    scale = 1.0 / math.sqrt(dh)
    out = []
    lse = []
    for bi in range(b):
        rows = x[bi]
        lse_b = [[0.0] * s for _ in range(heads)]
        a = [_layernorm_row(r, p["ln1_gamma"], p["ln1_beta"], eps) for r in rows]
        qkv = [_vecmat(ar, p["w_qkv"], p["b_qkv"]) for ar in a]
        o = [[0.0] * hl for _ in range(s)]
        for j in range(heads):
            q0, k0, v0 = 3 * dh * j, 3 * dh * j + dh, 3 * dh * j + 2 * dh
            for i in range(s):
                keys = [kk for kk in range(s)
                        if (kk <= i if mask == "causal" else kk < valid_len[bi])]
                sc = []
                for kk in keys:
                    acc = 0.0
                    for e in range(dh):
                        acc += qkv[i][q0 + e] * qkv[kk][k0 + e]
                    sc.append(acc * scale)
                m = max(sc)
                ex = [math.exp(v - m) for v in sc]
                tot = 0.0
                for v in ex:
                    tot += v
                lse_b[j][i] = m + math.log(tot)
                for e in range(dh):
                    acc = 0.0
                    for w_, kk in zip(ex, keys):
                        acc += w_ * qkv[kk][v0 + e]
                    o[i][j * dh + e] = acc / tot
        h_mid = []
        for i in range(s):
            proj = _vecmat(o[i], p["w_o"], p["b_o"])
            h_mid.append([rows[i][c] + proj[c] for c in range(len(proj))])
        seq_out = []
        for i in range(s):
            cn = _layernorm_row(h_mid[i], p["ln2_gamma"], p["ln2_beta"], eps)
            u = _vecmat(cn, p["w_fc1"], p["b_fc1"])
            z = [0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in u]
            y = _vecmat(z, p["w_fc2"], p["b_fc2"])
            seq_out.append([h_mid[i][c] + y[c] for c in range(len(y))])
        out.append(seq_out)
        lse.append(lse_b)
    return (out, lse) if want_lse else out
