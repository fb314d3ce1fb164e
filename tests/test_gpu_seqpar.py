"""Sequence-parallel layout: all t ranks run in sequence on one GPU.

The all-gathers are the ranks writing their own token rows into one shared
gathered buffer. The reduce-scatters are an on-device sum of the t fp32
partials, of which each rank reads only its own rows. The assembled result is
compared with the unsharded fp64 oracle: out and dx row by row, the
tensor-parallel parameter gradients slice by slice, and the replicated ones
(LayerNorm gamma/beta, b_o, b_fc2) summed over the ranks, each of which
covers only its own rows.
"""
import numpy as np
import pytest

from harness import TAU, err_ratio, fmt, to_np
from oracle import layer as OL
from tensor_model_transformer_amd.synth import (LayerDims, Workload, WORKLOADS, full_params,
                                                layer_inputs, rank_params)

pytestmark = pytest.mark.gpu

REPLICATED = ("ln1_gamma", "ln1_beta", "ln2_gamma", "ln2_beta", "b_o", "b_fc2")


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_sp(w):
    import torch
    from tensor_model_transformer_amd import binding as B
    from tensor_model_transformer_amd.shard import Shard, _check, exchange_sum

    d = w.dims
    t, n, h = d.t, d.tokens, d.hidden
    assert n % t == 0
    nc = n // t
    x, dout, vl = layer_inputs(w)
    shards = [Shard(d, r, sequence_parallel=True) for r in range(t)]
    params = [s.upload_params(rank_params(w, r), vl if d.mask == "padding" else None)
              for r, s in enumerate(shards)]
    s0 = shards[0]
    stream = s0.stream()
    act = torch.float16 if d.dtype == "bf16" else torch.float32
    xd, doutd = s0.act(x), s0.act(dout)
    rows = [slice(r * nc, (r + 1) * nc) for r in range(t)]
    g_a = torch.empty(n, h, dtype=act, device=s0.device)    # gathered LN1 output
    g_c = torch.empty(n, h, dtype=act, device=s0.device)    # gathered LN2 output
    g_dh = torch.empty(n, h, dtype=act, device=s0.device)   # gathered residual gradient
    parts = [s0.empty_act(fp32=True) for _ in range(t)]
    red = s0.empty_act(fp32=True)
    out = s0.empty_act()
    dx = s0.empty_dx()

    # forward
    for r, s in enumerate(shards):
        _check("sp ln1", s.fwd(params[r], None, x=xd[rows[r]], gathered=g_a, phase=B.TP_FWD_SP_LN1))
    for r, s in enumerate(shards):
        _check("sp attn", s.fwd(params[r], parts[r], gathered=g_a, phase=B.TP_FWD_SP_ATTN))
    exchange_sum(red, parts, stream)  # every rank then reads only its rows
    for r, s in enumerate(shards):
        _check("sp ln2", s.fwd(params[r], None, x=xd[rows[r]], reduced=red[rows[r]], gathered=g_c,
                               phase=B.TP_FWD_SP_LN2))
    for r, s in enumerate(shards):
        _check("sp mlp", s.fwd(params[r], parts[r], gathered=g_c, phase=B.TP_FWD_SP_MLP))
    exchange_sum(red, parts, stream)
    for r, s in enumerate(shards):
        _check("sp out", s.fwd(params[r], out[rows[r]], reduced=red[rows[r]], phase=B.TP_FWD_SP_OUT))

    # backward
    grads = [s.zero_grads() for s in shards]
    for r, s in enumerate(shards):
        _check("sp bwd mlp", s.bwd(params[r], grads[r], dout=doutd[rows[r]], gathered_grad=doutd,
                                   gathered_act=g_c, partial=parts[r], phase=B.TP_BWD_SP_MLP))
    exchange_sum(red, parts, stream)
    for r, s in enumerate(shards):
        _check("sp bwd ln2", s.bwd(params[r], grads[r], dc=red[rows[r]], dout=doutd[rows[r]],
                                   gathered_grad=g_dh, phase=B.TP_BWD_SP_LN2))
    for r, s in enumerate(shards):
        _check("sp bwd attn", s.bwd(params[r], grads[r], gathered_grad=g_dh, gathered_act=g_a,
                                    partial=parts[r], phase=B.TP_BWD_SP_ATTN))
    exchange_sum(red, parts, stream)
    for r, s in enumerate(shards):
        _check("sp bwd ln1", s.bwd(params[r], grads[r], da=red[rows[r]], x=xd[rows[r]],
                                   dx=dx[rows[r]], phase=B.TP_BWD_SP_LN1))
    torch.cuda.synchronize()
    res = {"out": to_np(out).reshape(d.batch, d.seq, h), "dx": to_np(dx).reshape(d.batch, d.seq, h),
           "grads": [{k: to_np(v) for k, v in g.items()} for g in grads]}
    for s in shards:
        s.close()
    return res


def sp_report(w, gpu, full):
    d = w.dims
    hl, fl = d.hidden_local, d.ffn_local
    G = full["grads"]
    rep = {"out": err_ratio(gpu["out"], full["out"]), "dx": err_ratio(gpu["dx"], full["dx"])}
    for k in REPLICATED:
        rep["d_" + k] = err_ratio(sum(g[k] for g in gpu["grads"]), G[k])
    for r in range(d.t):
        want = {
            "w_qkv": G["w_qkv"][:, 3 * hl * r:3 * hl * (r + 1)],
            "b_qkv": G["b_qkv"][3 * hl * r:3 * hl * (r + 1)],
            "w_o": G["w_o"][hl * r:hl * (r + 1)],
            "w_fc1": G["w_fc1"][:, fl * r:fl * (r + 1)],
            "b_fc1": G["b_fc1"][fl * r:fl * (r + 1)],
            "w_fc2": G["w_fc2"][fl * r:fl * (r + 1)],
        }
        for k, v in want.items():
            rep[f"d_{k}_r{r}"] = err_ratio(gpu["grads"][r][k], v)
    return rep


SEQPAR = [
    WORKLOADS["tiny_gpt_fp32"].with_(affine="perturbed"),
    Workload("sp_t4_bf16_padding", LayerDims(2, 72, 512, 8, 1024, t=4, dtype="bf16", mask="padding"),
             seed=41, affine="perturbed", len_range=(10, 72)),
    Workload("sp_t2_bf16_ragged", LayerDims(3, 130, 384, 6, 768, t=2, dtype="bf16", mask="causal"),
             seed=42, affine="perturbed"),
]


@pytest.mark.parametrize("w", SEQPAR, ids=lambda w: w.name)
def test_sequence_parallel_equals_unsharded(w):
    _need_gpu()
    d = w.dims
    print(f"\n[seqpar] {w.name} dims={d}", flush=True)
    gpu = run_sp(w)
    x, dout, vl = layer_inputs(w)
    full = OL.layer_full(full_params(w), x, dout, d, vl)
    rep = sp_report(w, gpu, full)
    print(f"[seqpar] {w.name}: {fmt(rep)}", flush=True)
    assert all(v <= TAU[d.dtype] for v in rep.values()), fmt(rep)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_sequence_parallel_8p3b_all_ranks():
    # the 8.3B shard's eight ranks in the sequence-parallel layout at full size
    _need_gpu()
    w = WORKLOADS["gpt_8p3b_t8"]
    d = w.dims
    print(f"\n[seqpar-full] {w.name} {d}", flush=True)
    gpu = run_sp(w)
    print("[seqpar-full] GPU done", flush=True)
    x, dout, vl = layer_inputs(w)
    full = OL.layer_full(full_params(w), x, dout, d, vl,
                         progress=lambda step: print(f"[seqpar-full] oracle {step}", flush=True))
    rep = sp_report(w, gpu, full)
    print(f"[seqpar-full] {fmt(rep)}", flush=True)
    assert all(v <= TAU["bf16"] for v in rep.values()), fmt(rep)
