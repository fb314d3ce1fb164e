"""GPU parity of the HIP layer shard against the fp64 oracle (through the C ABI).

Tolerance: max|err| <= 1e-4 * RMS on the fp32 path and <= 2e-2 * RMS on the
bf16 / fp32-accumulate path, for out, dx and every parameter gradient (and
the workspace intermediates where tapped).
"""
import numpy as np
import pytest

from harness import TAU, compare_local, fmt, oracle_local, run_gpu_local, to_np
from oracle import layer as OL
from tensor_model_transformer_amd.synth import (LayerDims, Workload, WORKLOADS, full_params,
                                                layer_inputs, rank_params)

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(w, rank=None, taps=False, scores=0, gelu="erf", eps=1e-5):
    _need_gpu()
    print(f"\n[parity] {w.name} dims={w.dims} rank={w.rank if rank is None else rank} "
          f"scores={scores} gelu={gelu} eps={eps}", flush=True)
    gpu = run_gpu_local(w, rank, taps=taps, scores=scores, gelu=gelu, eps=eps)
    ref = oracle_local(w, rank, gelu=gelu, eps=eps)
    ok, rep = compare_local(gpu, ref, TAU[w.dims.dtype], taps=taps)
    print(f"[parity] {w.name}: {fmt(rep)}", flush=True)
    assert ok, f"{w.name}: {fmt(rep)}"


# ---------------------------------------------------------------------------
# the tiny fp32 GPT workload (both ranks), with the intermediates tapped
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rank", [0, 1])
def test_tiny_gpt_fp32_local(rank):
    _run(WORKLOADS["tiny_gpt_fp32"], rank, taps=True)


def test_tiny_gpt_fp32_perturbed_affine():
    _run(WORKLOADS["tiny_gpt_fp32"].with_(affine="perturbed", name="tiny_gpt_fp32_aff"), 1,
         taps=True)


# ---------------------------------------------------------------------------
# small bf16 shapes: every head dim, both masks, ragged token/column counts
# that span several GEMM and attention tiles
# ---------------------------------------------------------------------------
SMALL_BF16 = [
    Workload("d32_causal", LayerDims(2, 200, 256, 8, 1040, t=2, dtype="bf16", mask="causal"),
             rank=1, seed=21, affine="perturbed"),
    Workload("d64_padding", LayerDims(3, 130, 384, 6, 768, t=2, dtype="bf16", mask="padding"),
             rank=0, seed=22, affine="perturbed", len_range=(1, 130)),
    Workload("d96_causal_t1", LayerDims(2, 150, 384, 4, 1536, t=1, dtype="bf16", mask="causal"),
             rank=0, seed=23, affine="perturbed"),
    Workload("d128_causal", LayerDims(1, 257, 512, 4, 2048, t=2, dtype="bf16", mask="causal"),
             rank=1, seed=24, affine="perturbed"),
    Workload("d160_padding", LayerDims(2, 96, 640, 4, 1280, t=2, dtype="bf16", mask="padding"),
             rank=0, seed=25, affine="perturbed", len_range=(33, 96)),
]


@pytest.mark.parametrize("w", SMALL_BF16, ids=lambda w: w.name)
def test_small_bf16_local(w):
    _run(w, taps=True)


# Attention job lists over the 8 XCDs: 6 (sequence, head) pairs x 4 query
# blocks (the pairs do not divide by 8: each pair is cut into 4 parts by block
# rank modulo 4 and every XCD takes 3 parts) and 16 pairs x 3 blocks (whole
# pairs per XCD, three ranks of blocks); the backward's grid holds both roles.
PLACEMENT = [
    Workload("pairs6_blocks4", LayerDims(2, 400, 384, 6, 768, t=2, dtype="bf16", mask="causal"),
             rank=1, seed=27, affine="perturbed"),
    Workload("pairs16_blocks3", LayerDims(4, 300, 256, 4, 512, t=1, dtype="bf16", mask="causal"),
             rank=0, seed=28, affine="perturbed"),
]


@pytest.mark.parametrize("w", PLACEMENT, ids=lambda w: w.name)
def test_attention_placement(w):
    _run(w, taps=True)


@pytest.mark.parametrize("w", [SMALL_BF16[i] for i in (1, 3, 4)], ids=lambda w: w.name)
def test_small_bf16_split_scores(w):
    # scores from the fp16 Q, K plus their rounding residuals
    from tensor_model_transformer_amd import binding as B
    _run(w, taps=True, scores=B.TP_SCORES_SPLIT)


def test_small_fp32_d160_padding():
    w = SMALL_BF16[4].with_(name="d160_padding_f32",
                            dims=LayerDims(2, 40, 320, 2, 640, t=1, dtype="f32", mask="padding"),
                            len_range=(7, 40))
    _run(w, taps=True)


def test_dx_in_storage_dtype():
    # opts.dx_dtype = bf16: the residual-stream gradient rounded to bf16 on output
    _need_gpu()
    w = SMALL_BF16[3]
    gpu = run_gpu_local(w, dx_fp32=False)
    ref = oracle_local(w)
    ok, rep = compare_local(gpu, ref, TAU["bf16"])
    print(f"[parity] {w.name} dx bf16: {fmt(rep)}", flush=True)
    assert ok, fmt(rep)
    assert gpu["dx_dtype"] == "bfloat16"


@pytest.mark.parametrize("w", [SMALL_BF16[0], SMALL_BF16[4]], ids=lambda w: w.name)
def test_recompute_fc1_is_bitwise_equal(w):
    # TP_RECOMPUTE_FC1 recomputes u = c @ W_fc1 + b_fc1 in backward with the same
    # kernel and inputs as the forward, so every result is bitwise unchanged
    _need_gpu()
    from tensor_model_transformer_amd import binding as B
    a = run_gpu_local(w)
    b = run_gpu_local(w, recompute=B.TP_RECOMPUTE_FC1)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["dx"], b["dx"])
    for k in a["grads"]:
        assert np.array_equal(a["grads"][k], b["grads"][k]), k


@pytest.mark.parametrize("w", [SMALL_BF16[0], SMALL_BF16[4]], ids=lambda w: w.name)
def test_overlap_is_bitwise_equal(w):
    # opts.overlap = TP_OVERLAP_ON runs the weight and bias gradients
    # on the handle's second stream: the same kernels on the same inputs, so
    # every result is bitwise unchanged, also when the gradients accumulate
    _need_gpu()
    from tensor_model_transformer_amd import binding as B
    for twice in (False, True):
        a = run_gpu_local(w, accumulate_twice=twice, overlap=B.TP_OVERLAP_OFF)
        b = run_gpu_local(w, accumulate_twice=twice, overlap=B.TP_OVERLAP_ON)
        assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["dx"], b["dx"])
        for k in a["grads"]:
            assert np.array_equal(a["grads"][k], b["grads"][k]), (k, twice)


def test_recompute_fc1_fp32_parity():
    _need_gpu()
    from tensor_model_transformer_amd import binding as B
    w = WORKLOADS["tiny_gpt_fp32"]
    gpu = run_gpu_local(w, 1, taps=True, recompute=B.TP_RECOMPUTE_FC1)
    ref = oracle_local(w, 1)
    ok, rep = compare_local(gpu, ref, TAU["f32"], taps=True)
    print(f"[parity] tiny fp32 recompute: {fmt(rep)}", flush=True)
    assert ok, fmt(rep)


def test_single_token_sequence():
    # degenerate: seq = 1 (attention is the identity on V), batch 3
    _run(Workload("seq1", LayerDims(3, 1, 128, 4, 256, t=1, dtype="bf16", mask="causal"),
                  seed=26, affine="perturbed"))


# ---------------------------------------------------------------------------
# determinism and gradient accumulation
# ---------------------------------------------------------------------------
def test_bitwise_deterministic():
    _need_gpu()
    w = SMALL_BF16[0]
    a = run_gpu_local(w)
    b = run_gpu_local(w)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["dx"], b["dx"])
    for k in a["grads"]:
        assert np.array_equal(a["grads"][k], b["grads"][k]), k


def test_accumulate_adds_gradients():
    _need_gpu()
    w = SMALL_BF16[2]
    gpu = run_gpu_local(w, accumulate_twice=True)
    ref = oracle_local(w)
    from harness import err_ratio
    for k, g in gpu["grads"].items():
        assert err_ratio(g, 2.0 * ref["grads"][k]) <= TAU["bf16"], k


@pytest.mark.parametrize("overlap", [1, 2], ids=["serial", "overlap"])
def test_graph_replay_matches_eager(overlap):
    """Forward + backward (TP_ALL) captured in a HIP graph on a side stream;
    with TP_OVERLAP_ON the backward's second stream joins the capture
    through its fork/join events. Every replay, with eager work in between,
    reproduces the eager outputs and gradients bit for bit."""
    _need_gpu()
    import torch
    from tensor_model_transformer_amd.shard import Shard, _check
    w = SMALL_BF16[0]
    d = w.dims
    print(f"\n[graph] {w.name} dims={d} overlap={overlap}", flush=True)
    x, dout, vl = layer_inputs(w)
    sh = Shard(d, 0, overlap=overlap)
    p = sh.upload_params(rank_params(w, 0), vl if d.mask == "padding" else None)
    xd, doutd = sh.act(x), sh.act(dout)
    out, dx = sh.empty_act(), sh.empty_dx()
    grads = sh.zero_grads()
    stream = torch.cuda.Stream(device=sh.device)

    def step():
        _check("tp_layer_fwd", sh.fwd(p, out, x=xd))
        _check("tp_layer_bwd", sh.bwd(p, grads, x=xd, dout=doutd, dx=dx))

    with torch.cuda.stream(stream):
        step()
    torch.cuda.synchronize()
    eager = {"out": out.clone(), "dx": dx.clone(), **{k: v.clone() for k, v in grads.items()}}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    for i in range(3):
        out.zero_()
        dx.zero_()
        for v in grads.values():
            v.zero_()
        junk = torch.randn(1 << 20, device=sh.device).sum()  # eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {"out": out, "dx": dx, **grads}
        for k, v in eager.items():
            assert torch.equal(got[k], v), f"replay {i}: {k} differs"
        del junk
    del graph
    sh.close()


# ---------------------------------------------------------------------------
# f/g identity: all t shards in sequence on one GPU, partials summed on-device
# ---------------------------------------------------------------------------
def run_phased(w):
    import torch
    from tensor_model_transformer_amd import binding as B
    from tensor_model_transformer_amd.shard import Shard, _check, exchange_sum

    d = w.dims
    x, dout, vl = layer_inputs(w)
    shards = [Shard(d, r) for r in range(d.t)]
    params = [s.upload_params(rank_params(w, r), vl if d.mask == "padding" else None)
              for r, s in enumerate(shards)]
    s0 = shards[0]
    xd, doutd = s0.act(x), s0.act(dout)
    stream = s0.stream()
    parts = [s0.empty_act(fp32=True) for _ in range(d.t)]
    h_mid = s0.empty_act(fp32=True)
    out = s0.empty_act()
    for r, s in enumerate(shards):
        _check("fwd attn", s.fwd(params[r], parts[r], x=xd, phase=B.TP_FWD_ATTN))
    exchange_sum(h_mid, parts, stream)
    for r, s in enumerate(shards):
        _check("fwd mlp", s.fwd(params[r], parts[r], h_mid=h_mid, phase=B.TP_FWD_MLP))
    exchange_sum(out, parts, stream)
    grads = [s.zero_grads() for s in shards]
    dc = s0.empty_act(fp32=True)
    da = s0.empty_act(fp32=True)
    for r, s in enumerate(shards):
        _check("bwd mlp", s.bwd(params[r], grads[r], dout=doutd, partial=parts[r],
                                phase=B.TP_BWD_MLP))
    exchange_sum(dc, parts, stream)
    for r, s in enumerate(shards):
        _check("bwd attn", s.bwd(params[r], grads[r], dout=doutd, dc=dc, partial=parts[r],
                                 phase=B.TP_BWD_ATTN))
    exchange_sum(da, parts, stream)
    dxs = []
    for r, s in enumerate(shards):
        dx = s0.empty_dx()
        _check("bwd ln1", s.bwd(params[r], grads[r], x=xd, da=da, dx=dx, phase=B.TP_BWD_LN1))
        dxs.append(dx)
    torch.cuda.synchronize()
    res = {"out": to_np(out).reshape(d.batch, d.seq, d.hidden),
           "dx": [to_np(t).reshape(d.batch, d.seq, d.hidden) for t in dxs],
           "h_mid": to_np(h_mid), "grads": [{k: to_np(v) for k, v in g.items()} for g in grads]}
    for s in shards:
        s.close()
    return res


PHASED = [
    WORKLOADS["tiny_gpt_fp32"].with_(affine="perturbed"),
    Workload("t4_bf16_padding", LayerDims(2, 72, 512, 8, 1024, t=4, dtype="bf16", mask="padding"),
             seed=31, affine="perturbed", len_range=(10, 72)),
    Workload("t8_32heads_bf16", LayerDims(2, 64, 1024, 32, 2048, t=8, dtype="bf16",
                                          mask="causal"), seed=32, affine="perturbed"),
]


@pytest.mark.parametrize("w", PHASED, ids=lambda w: w.name)
def test_phased_sum_over_shards_equals_unsharded(w):
    _need_gpu()
    d = w.dims
    print(f"\n[phased] {w.name} dims={d}", flush=True)
    gpu = run_phased(w)
    x, dout, vl = layer_inputs(w)
    full = OL.layer_full(full_params(w), x, dout, d, vl)
    tau = TAU[d.dtype]
    from harness import err_ratio
    rep = {"out": err_ratio(gpu["out"], full["out"]), "h_mid": err_ratio(gpu["h_mid"], full["h_mid"])}
    for r in range(d.t):
        rep[f"dx_r{r}"] = err_ratio(gpu["dx"][r], full["dx"])
    per = [rank_params(w, r) for r in range(d.t)]
    part = OL.layer_partials(per, x, dout, d, vl)
    for r in range(d.t):
        for k, g in gpu["grads"][r].items():
            rep[f"d_{k}_r{r}"] = err_ratio(g, part["grads"][r][k])
    print(f"[phased] {w.name}: {fmt(rep)}", flush=True)
    assert all(v <= tau for v in rep.values()), fmt(rep)


# ---------------------------------------------------------------------------
# the ABI's other GeLU form and LayerNorm epsilons (opts.gelu, opts.ln_eps)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("w", [SMALL_BF16[2], WORKLOADS["tiny_gpt_fp32"].with_(affine="perturbed")],
                         ids=lambda w: w.name)
def test_gelu_tanh_form(w):
    # TP_GELU_TANH: the tanh approximation in the FC1 epilogue (GeLU and the
    # kept derivative), against the oracle's tanh form
    _run(w, taps=True, gelu="tanh")


@pytest.mark.parametrize("eps", [1e-6, 1e-3])
@pytest.mark.parametrize("w", [SMALL_BF16[0], WORKLOADS["tiny_gpt_fp32"].with_(affine="perturbed")],
                         ids=lambda w: w.name)
def test_layernorm_eps(w, eps):
    _run(w, taps=True, eps=eps)


# ---------------------------------------------------------------------------
# GEMMs long in K (8192 = 128 K steps) and short in M: the launcher schedules
# them stream-K (the K steps of a column of tiles spread over slots of
# workgroups, split columns summed by the fix-up kernel), as it does for the
# 1T shard's M = 2048 GEMMs. One row tile (M = 200: 256 slots, some of them
# empty) and two (M = 320, the second partial: 128 slots). hidden 8192 also
# turns split scores on.
# ---------------------------------------------------------------------------
STREAM_K = [
    Workload("sk_h8192_causal", LayerDims(1, 200, 8192, 64, 16384, t=8, dtype="bf16",
                                          mask="causal"), rank=3, seed=41, affine="perturbed"),
    Workload("sk_h8192_padding", LayerDims(2, 160, 8192, 64, 16384, t=8, dtype="bf16",
                                           mask="padding"), rank=5, seed=42, affine="perturbed",
             len_range=(40, 160)),
    # M within 8 row tiles and K of 2048..6144: stream-K below 128 K steps
    Workload("sk_h4096_t2_causal", LayerDims(1, 136, 4096, 32, 8192, t=2, dtype="bf16",
                                             mask="causal"), rank=1, seed=43, affine="perturbed"),
]


@pytest.mark.parametrize("w", STREAM_K, ids=lambda w: w.name)
def test_stream_k_shapes(w):
    _run(w, taps=True)
