"""Full-size parity: the five measured workloads, in the launch configuration
bench.py times (TP_ALL forward + backward, one rank), against the complete
fp64 oracle. Also the 8.3B shard with all 8 ranks run in sequence and their
partials summed on-device, against the unsharded oracle.

These are the slowest GPU tests (the oracle runs on the host in fp64); each
prints a line per oracle step so a long run reports progress.
"""
import time

import numpy as np
import pytest

from harness import TAU, compare_local, err_ratio, fmt, run_gpu_local
from oracle import layer as OL
from tensor_model_transformer_amd.synth import WORKLOADS, full_params, layer_inputs, rank_params

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _progress(tag):
    t0 = time.time()

    def say(step):
        print(f"[{tag}] oracle {step} ({time.time() - t0:.1f} s)", flush=True)
    return say


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_gpt_fp32", "gpt_1p2b_t1", "gpt_8p3b_t8",
                                  "bert_3p9b_t4", "gpt_1t_t8"])
def test_workload_local_parity(name):
    _need_gpu()
    w = WORKLOADS[name]
    d = w.dims
    print(f"\n[full] {name} {d} rank={w.rank}", flush=True)
    t0 = time.time()
    gpu = run_gpu_local(w)
    print(f"[full] {name}: GPU done ({time.time() - t0:.1f} s)", flush=True)
    x, dout, vl = layer_inputs(w)
    ref = OL.layer_local(rank_params(w), x, dout, d, vl, progress=_progress(name))
    ok, rep = compare_local(gpu, ref, TAU[d.dtype])
    print(f"[full] {name}: {fmt(rep)}", flush=True)
    assert ok, f"{name}: {fmt(rep)}"


@pytest.mark.timeout(900)
def test_8p3b_all_ranks_phased_equals_unsharded():
    _need_gpu()
    from test_gpu_parity import run_phased
    w = WORKLOADS["gpt_8p3b_t8"]
    d = w.dims
    print(f"\n[phased-full] {w.name} {d}", flush=True)
    gpu = run_phased(w)
    print("[phased-full] GPU done", flush=True)
    x, dout, vl = layer_inputs(w)
    full = OL.layer_full(full_params(w), x, dout, d, vl, progress=_progress("phased-full"))
    rep = {"out": err_ratio(gpu["out"], full["out"]),
           "h_mid": err_ratio(gpu["h_mid"], full["h_mid"])}
    for r in range(d.t):
        rep[f"dx_r{r}"] = err_ratio(gpu["dx"][r], full["dx"])
    # rank r's gradient slices of the unsharded gradients (sharded tensors by
    # column/row block; replicated tensors whole)
    hl, fl = d.hidden_local, d.ffn_local
    G = full["grads"]
    for r in range(d.t):
        want = {
            "w_qkv": G["w_qkv"][:, 3 * hl * r:3 * hl * (r + 1)],
            "b_qkv": G["b_qkv"][3 * hl * r:3 * hl * (r + 1)],
            "w_o": G["w_o"][hl * r:hl * (r + 1)],
            "w_fc1": G["w_fc1"][:, fl * r:fl * (r + 1)],
            "b_fc1": G["b_fc1"][fl * r:fl * (r + 1)],
            "w_fc2": G["w_fc2"][fl * r:fl * (r + 1)],
        }
        for k, g in gpu["grads"][r].items():
            rep[f"d_{k}_r{r}"] = err_ratio(g, want.get(k, G[k]))
    print(f"[phased-full] {fmt(rep)}", flush=True)
    assert all(v <= TAU["bf16"] for v in rep.values()), fmt(rep)
