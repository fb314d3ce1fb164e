"""Decode step with a sharded KV cache on the GPU, against the fp64 decode oracle.

The HIP decode path (tp_layer_decode, tp_layer_kv_fill) is called through the
C ABI on seeded inputs; the oracle (oracle/decode.py, pinned to the batched
causal forward) gets the same inputs. Compared per tensor with
max|err| <= tau * RMS(reference): the layer output, the K and V rows the step
appends to the cache; every other cache row must come back bit-identical.
"""
import numpy as np
import pytest

from harness import TAU, err_ratio, fmt, to_np
from oracle import decode as OD
from oracle import layer as OL
from tensor_model_transformer_amd.synth import (LayerDims, Workload, WORKLOADS, decode_inputs,
                                                full_caches, full_params, layer_inputs,
                                                rank_caches, rank_params)

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _wl(name, batch, hidden, heads, ffn, t=1, dtype="bf16", seed=60, rank=0, seq=16):
    return Workload(name, LayerDims(batch, seq, hidden, heads, ffn, t=t, dtype=dtype,
                                    mask="causal"), rank=rank, seed=seed, affine="perturbed")


def run_decode(w, cache_len, positions="ragged", scores=0, rank=None, gelu="erf", eps=1e-5,
               params=None):
    """One TP_ALL decode step of one rank on the GPU. Returns numpy results
    and the inputs it used. `params` replaces the rank's generated
    parameters (values on the storage grid)."""
    import torch
    from tensor_model_transformer_amd.shard import Shard, _check

    d = w.dims
    r = w.rank if rank is None else rank
    x, pos = decode_inputs(w, cache_len, positions)
    kc, vc = rank_caches(w, r, cache_len)
    from tensor_model_transformer_amd import binding as B
    sh = Shard(d, r, scores=scores, eps=eps,
               gelu=B.TP_GELU_TANH if gelu == "tanh" else B.TP_GELU_ERF)
    p = sh.upload_params(rank_params(w, r) if params is None else params)
    xd = torch.from_numpy(x).to(sh.device).to(sh.dtype)
    kd, vd = sh.upload_cache(kc), sh.upload_cache(vc)
    klo = torch.zeros_like(kd) if sh.split_scores else None
    posd = torch.from_numpy(pos).to(sh.device)
    out = torch.empty(d.batch, d.hidden, dtype=sh.dtype, device=sh.device)
    print(f"[decode] {w.name} B={d.batch} h={d.hidden} dh={d.head_dim} L={cache_len} "
          f"pos={positions} scores={scores}", flush=True)
    _check("decode", sh.decode(p, out, x=xd, k_cache=kd, v_cache=vd, k_cache_lo=klo,
                               positions=posd))
    torch.cuda.synchronize()
    res = {"out": to_np(out), "k": to_np(kd), "v": to_np(vd),
           "klo": to_np(klo) if klo is not None else None}
    sh.close()
    return res, (x, pos, kc, vc)


def compare_decode(w, gpu, inputs, tau, gelu="erf", eps=1e-5):
    d = w.dims
    x, pos, kc, vc = inputs
    ref = OD.decode_step(rank_params(w, w.rank), x, kc, vc, pos, d.heads_local, eps=eps,
                         gelu_form=gelu)
    rep = {"out": err_ratio(gpu["out"], ref["out"])}
    B_, Hl = d.batch, d.heads_local
    newk = np.stack([ref["k_cache"][b, :, pos[b]] for b in range(B_)])
    newv = np.stack([ref["v_cache"][b, :, pos[b]] for b in range(B_)])
    gk = np.stack([gpu["k"][b, :, pos[b]] for b in range(B_)])
    if gpu["klo"] is not None:
        gk = gk + np.stack([gpu["klo"][b, :, pos[b]] for b in range(B_)])
    gv = np.stack([gpu["v"][b, :, pos[b]] for b in range(B_)])
    rep["k_new"] = err_ratio(gk, newk)
    rep["v_new"] = err_ratio(gv, newv)
    keep = np.ones(kc.shape[:3], bool)
    for b in range(B_):
        keep[b, :, pos[b]] = False
    assert np.array_equal(gpu["k"][keep], kc[keep]), "cache rows other than pos changed (K)"
    assert np.array_equal(gpu["v"][keep], vc[keep]), "cache rows other than pos changed (V)"
    return rep


CASES = [
    (WORKLOADS["tiny_gpt_fp32"], 64, "ragged", 0),
    (WORKLOADS["tiny_gpt_fp32"].with_(rank=1, affine="perturbed"), 200, "ragged", 0),
    (_wl("dec_f32_dh160", 3, 640, 4, 512, dtype="f32"), 130, "ragged", 0),
    (_wl("dec_bf16_dh32", 4, 128, 4, 512), 100, "ragged", 0),
    (_wl("dec_bf16_dh64_t2", 3, 512, 8, 1024, t=2, rank=1), 200, "ragged", 0),
    (_wl("dec_bf16_dh96", 5, 384, 4, 768), 333, "ragged", 0),
    (_wl("dec_bf16_dh128", 2, 512, 4, 1024), 64, "full", 0),
    (_wl("dec_bf16_dh160", 3, 640, 4, 1280), 150, "ragged", 0),
    (_wl("dec_bf16_dh160_split", 3, 640, 4, 1280), 150, "ragged", 2),
    (_wl("dec_bf16_dh64_split", 2, 256, 4, 512), 97, "ragged", 2),
    (_wl("dec_bf16_b1_empty", 1, 256, 4, 512), 32, "empty", 0),
    (_wl("dec_bf16_b20", 20, 256, 4, 520), 70, "ragged", 0),
    (_wl("dec_bf16_b70", 70, 256, 4, 512), 40, "ragged", 0),
    (_wl("dec_bf16_long", 2, 256, 2, 512), 5000, "ragged", 0),
]


@pytest.mark.parametrize("w,cache_len,positions,scores", CASES,
                         ids=[f"{c[0].name}-L{c[1]}-{c[2]}" for c in CASES])
def test_decode_matches_oracle(w, cache_len, positions, scores):
    _need_gpu()
    gpu, inputs = run_decode(w, cache_len, positions, scores)
    rep = compare_decode(w, gpu, inputs, TAU[w.dims.dtype])
    print(f"[decode] {w.name}: {fmt(rep)}", flush=True)
    assert all(v <= TAU[w.dims.dtype] for v in rep.values()), fmt(rep)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_gelu_tanh_and_eps(dtype):
    # opts.gelu = TP_GELU_TANH in the FC1 GEMV epilogue, opts.ln_eps in both
    # LayerNorms (the decode-only fused residual + LN2 kernel included)
    _need_gpu()
    w = _wl(f"dec_tanh_eps_{dtype}", 3, 384, 4, 768, dtype=dtype, seed=61)
    gpu, inputs = run_decode(w, 90, "ragged", gelu="tanh", eps=1e-3)
    rep = compare_decode(w, gpu, inputs, TAU[dtype], gelu="tanh", eps=1e-3)
    print(f"[decode] {w.name}: {fmt(rep)}", flush=True)
    assert all(v <= TAU[dtype] for v in rep.values()), fmt(rep)


def test_decode_weights_beyond_fp16_are_not_silent():
    # The GEMVs read the bf16 weights as fp16 operands. A weight beyond fp16's
    # largest finite value (65504) must come out as a non-finite result, as in
    # the training path, not as a finite value saturated at 65504.
    _need_gpu()
    w = _wl("dec_range_bf16", 3, 384, 4, 768, dtype="bf16", seed=62)
    p = dict(rank_params(w, w.rank))
    m = np.array(p["w_o"], copy=True)
    m[:, 5] = np.float32(99840.0)  # 1e5 on the bf16 grid
    p["w_o"] = m
    gpu, _ = run_decode(w, 40, "ragged", params=p)
    assert not np.all(np.isfinite(gpu["out"]))


def test_decode_is_deterministic():
    # split-K partials and cache slices are merged in a fixed order
    _need_gpu()
    w = _wl("dec_det", 8, 512, 4, 2048)
    a, _ = run_decode(w, 300)
    b, _ = run_decode(w, 300)
    assert np.array_equal(a["out"], b["out"])
    assert np.array_equal(a["k"], b["k"]) and np.array_equal(a["v"], b["v"])


@pytest.mark.parametrize("scores", [0, 2])
def test_prefill_then_decode_equals_forward(scores):
    """GPU forward over a prompt, kv_fill, then decode steps one position at
    a time: each output row equals the oracle's causal forward over the whole
    sequence at that row."""
    _need_gpu()
    import torch
    from tensor_model_transformer_amd.shard import Shard, _check

    S, extra = 40, 4
    w = Workload("prefill_decode", LayerDims(3, S + extra, 512, 4, 1024, t=2, dtype="bf16",
                                             mask="causal"), rank=1, seed=71, affine="perturbed")
    d = w.dims
    params = rank_params(w, 1)
    x, dout, _ = layer_inputs(w)                    # [B, S+extra, h]
    ref = OL.layer(params, x, dout, d.heads_local, "causal")["out"]
    pd = LayerDims(d.batch, S, d.hidden, d.heads, d.ffn, t=d.t, dtype="bf16", mask="causal")
    sh = Shard(pd, 1, scores=scores)
    p = sh.upload_params(params)
    prompt = np.ascontiguousarray(x[:, :S])
    xd = sh.act(prompt)
    out = sh.empty_act()
    _check("prefill", sh.fwd(p, out, x=xd))
    L = S + extra + 3
    kd, vd = sh.empty_cache(L), sh.empty_cache(L)
    klo = sh.empty_cache(L) if scores == 2 else None
    _check("kv_fill", sh.kv_fill(kd, vd, klo))
    rep = {"prefill": err_ratio(to_np(out).reshape(d.batch, S, -1), ref[:, :S])}
    dout_t = torch.empty(d.batch, d.hidden, dtype=sh.dtype, device=sh.device)
    for s in range(S, S + extra):
        posd = torch.full((d.batch,), s, dtype=torch.int32, device=sh.device)
        xs = torch.from_numpy(np.ascontiguousarray(x[:, s])).to(sh.device).to(sh.dtype)
        _check("decode", sh.decode(p, dout_t, x=xs, k_cache=kd, v_cache=vd, k_cache_lo=klo,
                                   positions=posd))
        torch.cuda.synchronize()
        rep[f"pos{s}"] = err_ratio(to_np(dout_t), ref[:, s])
    sh.close()
    print(f"[prefill+decode] scores={scores}: {fmt(rep)}", flush=True)
    assert all(v <= TAU["bf16"] for v in rep.values()), fmt(rep)


def run_decode_phased(w, cache_len):
    """All t ranks, phase by phase, with on-device sums between the phases."""
    import torch
    from tensor_model_transformer_amd import binding as B
    from tensor_model_transformer_amd.shard import Shard, _check, exchange_sum

    d = w.dims
    t = d.t
    x, pos = decode_inputs(w, cache_len, "ragged")
    shards = [Shard(d, r) for r in range(t)]
    params = [s.upload_params(rank_params(w, r)) for r, s in enumerate(shards)]
    s0 = shards[0]
    stream = s0.stream()
    caches = [tuple(s.upload_cache(c) for c in rank_caches(w, r, cache_len))
              for r, s in enumerate(shards)]
    xd = torch.from_numpy(x).to(s0.device).to(s0.dtype)
    posd = torch.from_numpy(pos).to(s0.device)
    parts = [torch.empty(d.batch, d.hidden, dtype=torch.float32, device=s0.device)
             for _ in range(t)]
    h_mid = torch.empty_like(parts[0])
    out = torch.empty_like(parts[0])
    for r, s in enumerate(shards):
        _check("decode attn", s.decode(params[r], parts[r], x=xd, k_cache=caches[r][0],
                                       v_cache=caches[r][1], positions=posd,
                                       phase=B.TP_FWD_ATTN))
    exchange_sum(h_mid, parts, stream)
    for r, s in enumerate(shards):
        _check("decode mlp", s.decode(params[r], parts[r], h_mid=h_mid, phase=B.TP_FWD_MLP))
    exchange_sum(out, parts, stream)
    torch.cuda.synchronize()
    res = {"out": to_np(out), "h_mid": to_np(h_mid),
           "k": np.concatenate([to_np(c[0]) for c in caches], axis=1),
           "v": np.concatenate([to_np(c[1]) for c in caches], axis=1)}
    for s in shards:
        s.close()
    return res, x, pos


@pytest.mark.parametrize("w,cache_len", [
    (_wl("dec_phased_t4", 4, 512, 8, 1024, t=4, seed=81), 180),
    (WORKLOADS["tiny_gpt_fp32"].with_(affine="perturbed"), 64),
], ids=["bf16_t4", "fp32_t2"])
def test_decode_all_ranks_phased_equals_unsharded(w, cache_len):
    _need_gpu()
    d = w.dims
    gpu, x, pos = run_decode_phased(w, cache_len)
    kf, vf = full_caches(w, cache_len)
    ref = OD.decode_step(full_params(w), x, kf, vf, pos, d.heads)
    rep = {"out": err_ratio(gpu["out"], ref["out"]), "h_mid": err_ratio(gpu["h_mid"], ref["h_mid"])}
    for name, key in (("k", "k_cache"), ("v", "v_cache")):
        g = np.stack([gpu[name][b, :, pos[b]] for b in range(d.batch)])
        o = np.stack([ref[key][b, :, pos[b]] for b in range(d.batch)])
        rep[name + "_new"] = err_ratio(g, o)
    print(f"[decode-phased] {w.name}: {fmt(rep)}", flush=True)
    assert all(v <= TAU[d.dtype] for v in rep.values()), fmt(rep)


def test_decode_graph_replay_matches_eager():
    """The decode step captured in a HIP graph (no memset nodes, no
    allocation) replays bit-identically, with eager work in between."""
    _need_gpu()
    import torch
    from tensor_model_transformer_amd.shard import Shard, _check

    w = _wl("dec_graph", 8, 512, 4, 2048, seed=90)
    d = w.dims
    L = 256
    x, pos = decode_inputs(w, L, "ragged")
    kc, vc = rank_caches(w, 0, L)
    sh = Shard(d, 0)
    p = sh.upload_params(rank_params(w, 0))
    xd = torch.from_numpy(x).to(sh.device).to(sh.dtype)
    kd, vd = sh.upload_cache(kc), sh.upload_cache(vc)
    posd = torch.from_numpy(pos).to(sh.device)
    out = torch.empty(d.batch, d.hidden, dtype=sh.dtype, device=sh.device)
    sh.decode_workspace()
    stream = torch.cuda.Stream(device=sh.device)
    with torch.cuda.stream(stream):
        _check("eager decode", sh.decode(p, out, x=xd, k_cache=kd, v_cache=vd, positions=posd))
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        rc = sh.decode(p, out, x=xd, k_cache=kd, v_cache=vd, positions=posd)
    _check("captured decode", rc)
    for i in range(3):
        out.zero_()
        junk = torch.randn(1 << 20, device=sh.device).sum()  # eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs"
        del junk
    del graph
    sh.close()


# ---------------------------------------------------------------------------
# full-size shards (the bench's decode shapes): every output row is checked
# ---------------------------------------------------------------------------
@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,cache_len,positions", [
    ("gpt_1p2b_t1", 1024, "full"),
    ("gpt_1p2b_t1", 2048, "ragged"),
    ("gpt_1t_t8", 2048, "full"),
])
def test_decode_full_size(name, cache_len, positions):
    _need_gpu()
    w = WORKLOADS[name]
    gpu, inputs = run_decode(w, cache_len, positions)
    print(f"[decode-full] {name} GPU done", flush=True)
    rep = compare_decode(w, gpu, inputs, TAU["bf16"])
    print(f"[decode-full] {name}: {fmt(rep)}", flush=True)
    assert all(v <= TAU["bf16"] for v in rep.values()), fmt(rep)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_decode_8p3b_all_ranks_phased():
    _need_gpu()
    w = WORKLOADS["gpt_8p3b_t8"]
    d = w.dims
    gpu, x, pos = run_decode_phased(w, 1024)
    kf, vf = full_caches(w, 1024)
    ref = OD.decode_step(full_params(w), x, kf, vf, pos, d.heads)
    rep = {"out": err_ratio(gpu["out"], ref["out"]), "h_mid": err_ratio(gpu["h_mid"], ref["h_mid"])}
    print(f"[decode-full] 8.3B all ranks: {fmt(rep)}", flush=True)
    assert all(v <= TAU["bf16"] for v in rep.values()), fmt(rep)
