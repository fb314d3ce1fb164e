"""Magnitude range of the bf16 layer's fp16 internals, against the fp64 oracle.

bf16 has fp32's exponent range; the fp16 tensors the layer keeps inside
(activations, and in the backward the upstream gradient's copy, du, dh's
copy, dO and dqkv) span only about 2^-24 .. 65504. The backward therefore
multiplies its fp16 gradient chain by a power of two S, chosen on the device
from max|dout| so that max|S dout| lies in [1, 2), and every GEMM or column sum
that leaves the chain multiplies by 1/S. Both factors are powers of two, so an
upstream gradient scaled by 2^k gives gradients scaled by exactly 2^k: bit for
bit, not only within the tolerance. The cases here are the scales bf16
training produces without loss scaling (2^-20, 2^-30), one that would
overflow fp16 (2^16), a layer input of magnitude ~1e5 (LayerNorm takes it out
of the internal tensors) and row-parallel weights 2^14 times larger (their
outputs and the gradients they feed reach ~1e4). Weights or activations
beyond fp16's largest value (65504) are outside the handled range; the test
of that limit checks that the result is then non-finite rather than wrong.

Each result is also compared with the oracle on the same inputs:
max|err| <= 2e-2 * RMS(reference) per tensor.
"""
import numpy as np
import pytest

from harness import TAU, compare_local, fmt, local_inputs, oracle_local, run_gpu_local
from tensor_model_transformer_amd.synth import LayerDims, PARAM_NAMES, Workload

pytestmark = pytest.mark.gpu

CASES = [
    Workload("range_d96_causal", LayerDims(2, 150, 384, 4, 1536, t=1, dtype="bf16",
                                           mask="causal"), rank=0, seed=31, affine="perturbed"),
    Workload("range_d64_padding", LayerDims(3, 130, 384, 6, 768, t=2, dtype="bf16",
                                            mask="padding"), rank=1, seed=32, affine="perturbed",
             len_range=(1, 130)),
]


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _parity(w, inputs, what, out_rounding=False):
    """Every tensor within 2e-2 * RMS of the oracle. With out_rounding, `out`
    (bf16 at the boundary) is held to 2e-2 * RMS(out) plus its own bf16
    rounding, 2^-8 |out| per element: a 2^14-times larger output projection
    makes h_mid, hence out, follow the attention output, whose first causal
    rows (a single value row, no averaging) stand far above RMS(out), so the
    bf16 rounding of those rows alone exceeds 2e-2 * RMS(out). Every other
    tensor (fp32 or graded against its own RMS) keeps the plain bound."""
    gpu = run_gpu_local(w, inputs=inputs, taps=True)
    ref = oracle_local(w, inputs=inputs)
    if out_rounding:
        g, r = gpu["out"], ref["out"]
        bound = TAU["bf16"] * float(np.sqrt(np.mean(np.square(r)))) + 2.0 ** -8 * np.abs(r)
        excess = float((np.abs(g - r) - bound).max())
        print(f"[range] {w.name} {what}: out, max excess over the rounding-aware bound "
              f"{excess:.3e}", flush=True)
        assert excess <= 0.0, f"{w.name} {what}: out"
        gpu = dict(gpu, out=ref["out"])  # graded above
    ok, rep = compare_local(gpu, ref, TAU["bf16"], taps=True)
    print(f"[range] {w.name} {what}: {fmt(rep)}", flush=True)
    assert ok, f"{w.name} {what}: {fmt(rep)}"
    return gpu


@pytest.mark.parametrize("k", [-30, -20, 16])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_upstream_gradient_scale(w, k):
    _need_gpu()
    print(f"\n[range] {w.name} dout * 2^{k}", flush=True)
    params, x, dout, vl = local_inputs(w)
    base = run_gpu_local(w, inputs=(params, x, dout, vl), taps=True)
    scaled = _parity(w, (params, x, dout * np.float32(2.0 ** k), vl), f"dout*2^{k}")
    f = 2.0 ** k
    assert np.array_equal(scaled["out"], base["out"])
    assert np.array_equal(scaled["dx"], base["dx"] * f), "dx does not scale exactly"
    for name in PARAM_NAMES:
        assert np.array_equal(scaled["grads"][name], base["grads"][name] * f), name
    # the chain's S follows the gradient: S(2^k dout) = 2^-k S(dout)
    assert scaled["grad_scale"] * f == base["grad_scale"]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_zero_upstream_gradient(w):
    _need_gpu()
    params, x, dout, vl = local_inputs(w)
    r = run_gpu_local(w, inputs=(params, x, np.zeros_like(dout), vl))
    assert not np.any(r["dx"])
    for name in PARAM_NAMES:
        assert not np.any(r["grads"][name]), name


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_large_layer_input(w):
    # |x| up to ~2.6e5 (N(0,1) * 2^16): LayerNorm's statistics are fp32 and
    # its output is O(1); the residual stream (h_mid, out, dx) is fp32 / bf16
    _need_gpu()
    print(f"\n[range] {w.name} x * 2^16", flush=True)
    params, x, dout, vl = local_inputs(w)
    _parity(w, (params, x * np.float32(2.0 ** 16), dout, vl), "x*2^16")


@pytest.mark.parametrize("which", ["w_fc2", "w_o"])
@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_large_weights(w, which):
    # a row-parallel weight 2^14 times larger (sigma ~330, max |w| ~1.5e3):
    # its output (out or h_mid) grows to ~1e4 and so do the gradients it feeds
    # in the backward (du or dO, then the rest of the fp16 chain); all of it
    # stays inside fp16's range, which the power-of-two scaling of the chain
    # (from max|dout|, not from these) leaves room for
    _need_gpu()
    print(f"\n[range] {w.name} {which} * 2^14", flush=True)
    params, x, dout, vl = local_inputs(w)
    p = dict(params)
    p[which] = params[which] * np.float32(2.0 ** 14)
    _parity(w, (p, x, dout, vl), f"{which}*2^14", out_rounding=True)


@pytest.mark.parametrize("w", CASES[:1], ids=lambda w: w.name)
def test_weights_beyond_fp16_are_not_silent(w):
    # The documented limit: weights (or activations) at or beyond fp16's
    # largest finite value overflow the fp16 copies and tensors inside the
    # layer. The result is then visibly non-finite, not a finite wrong value.
    _need_gpu()
    params, x, dout, vl = local_inputs(w)
    p = dict(params)
    m = np.array(params["w_o"], copy=True)
    m[:, 5] = np.float32(99840.0)  # 1e5 rounded to the bf16 grid
    p["w_o"] = m
    r = run_gpu_local(w, inputs=(p, x, dout, vl))
    assert not np.all(np.isfinite(r["out"]))
