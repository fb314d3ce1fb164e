"""Seeded synthetic inputs for one tensor-parallel rank's layer shard.

This module draws numbers and nothing else: it holds none of the layer's
arithmetic. Both the fp64 CPU oracle (through the tests and the bench) and the
HIP path consume exactly what it returns, so input quantisation is never
counted as error.

Parameter layout follows "Megatron-LM: GPU-Cluster Training Parallelism"
(blog walkthrough), sections "Paper 1: The f/g Conjugate Operators" and
"Paper 1: QKV Column-Parallel Splitting in Detail":

* weights are stored in the ``X @ W`` orientation ``[in, out]``;
* the fused QKV weight has head-interleaved columns ``[Q_0 K_0 V_0 | Q_1 ...]``
  so that rank ``r`` of ``t`` owns the contiguous column block
  ``[r*3h/t, (r+1)*3h/t)`` (whole heads ``r*H/t ... (r+1)*H/t - 1``);
* FC1 (``A``) is split by columns, the output projection ``W_o`` and FC2 by rows.

Determinism: every tensor is drawn per (tensor id, rank) from
``SeedSequence([seed, tensor_id, rank_slot])`` -> PCG64, in float32, scaled by
its standard deviation and (bf16 storage) rounded to the nearest bf16 with ties
to even. The unsharded tensor is *defined* as the concatenation of the rank
slices, so a single rank's slice never needs the whole tensor and the
all-ranks check sees the same values. Replicated tensors (LayerNorm affine,
row-parallel biases, the input and the upstream gradient) use rank slot
``REPLICATED``.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

REPLICATED = 0xFFFF

# Stable ids; never renumber (they are part of the seed).
TENSOR_IDS = {
    "x": 1, "dout": 2, "valid_len": 3,
    "x_new": 4, "k_cache": 5, "v_cache": 6, "positions": 7,
    "ln1_gamma": 10, "ln1_beta": 11, "ln2_gamma": 12, "ln2_beta": 13,
    "w_qkv": 20, "b_qkv": 21, "w_o": 22, "b_o": 23,
    "w_fc1": 24, "b_fc1": 25, "w_fc2": 26, "b_fc2": 27,
}

SHARDED = ("w_qkv", "b_qkv", "w_o", "w_fc1", "b_fc1", "w_fc2")
REPLICATED_PARAMS = ("ln1_gamma", "ln1_beta", "ln2_gamma", "ln2_beta", "b_o", "b_fc2")
PARAM_NAMES = ("ln1_gamma", "ln1_beta", "w_qkv", "b_qkv", "w_o", "b_o",
               "ln2_gamma", "ln2_beta", "w_fc1", "b_fc1", "w_fc2", "b_fc2")


@dataclass(frozen=True)
class LayerDims:
    """Problem statement of one layer shard: hidden size, heads, FFN size,
    sequence, micro-batch, split factor t, storage dtype and mask kind."""
    batch: int
    seq: int
    hidden: int
    heads: int
    ffn: int
    t: int = 1
    dtype: str = "bf16"          # "f32" or "bf16" (storage); accumulation is fp32
    mask: str = "causal"         # "causal" or "padding"

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    @property
    def heads_local(self) -> int:
        return self.heads // self.t

    @property
    def hidden_local(self) -> int:
        return self.heads_local * self.head_dim

    @property
    def ffn_local(self) -> int:
        return self.ffn // self.t

    def shapes(self, full: bool = False) -> Dict[str, tuple]:
        """Shapes of the parameters: the rank slice, or the unsharded tensors."""
        h = self.hidden
        hl = self.hidden if full else self.hidden_local
        fl = self.ffn if full else self.ffn_local
        return {
            "ln1_gamma": (h,), "ln1_beta": (h,), "ln2_gamma": (h,), "ln2_beta": (h,),
            "w_qkv": (h, 3 * hl), "b_qkv": (3 * hl,),
            "w_o": (hl, h), "b_o": (h,),
            "w_fc1": (h, fl), "b_fc1": (fl,),
            "w_fc2": (fl, h), "b_fc2": (h,),
        }


@dataclass(frozen=True)
class Workload:
    """A named, seeded workload: dims, rank under test, and the init recipe."""
    name: str
    dims: LayerDims
    rank: int = 0
    seed: int = 1000
    weight_std: float = 0.02
    out_proj_std: float = 0.02      # W_o and FC2 (the output projections)
    affine: str = "plain"           # "plain": biases 0, gamma 1, beta 0; "perturbed": all random
    len_range: Optional[tuple] = None  # padding mask: valid length ~ U{lo..hi} (inclusive)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the measurement plan (names say what they are).
WORKLOADS = {
    "tiny_gpt_fp32": Workload(
        "tiny_gpt_fp32", LayerDims(2, 64, 128, 4, 512, t=2, dtype="f32", mask="causal"),
        rank=0, seed=1000),
    "gpt_1p2b_t1": Workload(
        "gpt_1p2b_t1", LayerDims(8, 1024, 1536, 16, 6144, t=1, dtype="bf16", mask="causal"),
        rank=0, seed=1001),
    "gpt_8p3b_t8": Workload(
        "gpt_8p3b_t8", LayerDims(8, 1024, 3072, 32, 12288, t=8, dtype="bf16", mask="causal"),
        rank=0, seed=1002),
    "bert_3p9b_t4": Workload(
        "bert_3p9b_t4", LayerDims(16, 512, 2560, 40, 10240, t=4, dtype="bf16", mask="padding"),
        rank=0, seed=1003, len_range=(128, 512)),
    "gpt_1t_t8": Workload(
        "gpt_1t_t8", LayerDims(1, 2048, 25600, 160, 102400, t=8, dtype="bf16", mask="causal"),
        rank=0, seed=1004, out_proj_std=0.02 / np.sqrt(2.0 * 128.0)),
}
WORKLOAD_ORDER = ("tiny_gpt_fp32", "gpt_1p2b_t1", "gpt_8p3b_t8", "bert_3p9b_t4", "gpt_1t_t8")


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round a float32 array in place to the nearest bfloat16 value (ties to
    even) and return it, still as float32. Inputs are finite."""
    assert a.dtype == np.float32
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    u += bias
    u &= np.uint32(0xFFFF0000)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of a float32 array whose values are already bf16 values."""
    assert a.dtype == np.float32
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _rng(seed: int, name: str, slot: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, TENSOR_IDS[name], slot])))


def _normal(seed, name, slot, shape, std, mean, dtype) -> np.ndarray:
    g = _rng(seed, name, slot)
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    if dtype == "bf16":
        round_to_bf16(a)
    return a


def _param_recipe(w: Workload, name: str):
    """(std, mean) of a parameter under the workload's init recipe."""
    if name in ("w_qkv", "w_fc1"):
        return w.weight_std, 0.0
    if name in ("w_o", "w_fc2"):
        return w.out_proj_std, 0.0
    if w.affine == "plain":
        if name in ("ln1_gamma", "ln2_gamma"):
            return None, 1.0
        return None, 0.0
    # perturbed: exercises the bias and affine paths
    if name in ("ln1_gamma", "ln2_gamma"):
        return 0.1, 1.0
    if name in ("ln1_beta", "ln2_beta"):
        return 0.1, 0.0
    return 0.02, 0.0


def rank_params(w: Workload, rank: Optional[int] = None) -> Dict[str, np.ndarray]:
    """The parameters rank ``rank`` holds (float32 arrays on the storage grid)."""
    d = w.dims
    r = w.rank if rank is None else rank
    assert 0 <= r < d.t
    shapes = d.shapes(full=False)
    out = {}
    for name in PARAM_NAMES:
        std, mean = _param_recipe(w, name)
        slot = r if name in SHARDED else REPLICATED
        if std is None:
            out[name] = np.full(shapes[name], mean, dtype=np.float32)
        else:
            out[name] = _normal(w.seed, name, slot, shapes[name], std, mean, d.dtype)
    return out


def full_params(w: Workload) -> Dict[str, np.ndarray]:
    """Unsharded parameters: the concatenation of all t rank slices
    (columns for QKV and FC1, rows for W_o and FC2)."""
    d = w.dims
    per = [rank_params(w, r) for r in range(d.t)]
    out = {}
    for name in PARAM_NAMES:
        if name in ("w_qkv", "w_fc1"):
            out[name] = np.concatenate([p[name] for p in per], axis=1)
        elif name in ("b_qkv", "b_fc1", "w_o", "w_fc2"):
            out[name] = np.concatenate([p[name] for p in per], axis=0)
        else:
            out[name] = per[0][name]
    return out


def layer_inputs(w: Workload):
    """x [b, s, h], upstream gradient dout [b, s, h] (both N(0,1)), and the
    per-sequence valid key length [b] (int32; all ``seq`` for a causal mask)."""
    d = w.dims
    x = _normal(w.seed, "x", REPLICATED, (d.batch, d.seq, d.hidden), 1.0, 0.0, d.dtype)
    dout = _normal(w.seed, "dout", REPLICATED, (d.batch, d.seq, d.hidden), 1.0, 0.0, d.dtype)
    if d.mask == "padding":
        lo, hi = w.len_range if w.len_range is not None else (1, d.seq)
        lens = _rng(w.seed, "valid_len", REPLICATED).integers(lo, hi + 1, size=d.batch)
        valid = lens.astype(np.int32)
    else:
        valid = np.full(d.batch, d.seq, dtype=np.int32)
    return x, dout, valid


# ----------------------------------------------------------------------------
# Decode-step inputs: one new token per sequence against a KV cache
# ----------------------------------------------------------------------------
def round_to_fp16(a: np.ndarray) -> np.ndarray:
    """Nearest IEEE half value (ties to even), returned as float32."""
    return a.astype(np.float16).astype(np.float32)


def kv_std(w: Workload) -> float:
    """Spread of the cached K and V values: a unit-variance LayerNorm output
    times a weight column of ``hidden`` N(0, weight_std^2) entries."""
    return float(w.weight_std * np.sqrt(w.dims.hidden))


def rank_caches(w: Workload, rank: int, cache_len: int):
    """K and V caches of rank ``rank``: [batch, H_l, cache_len, dh] each, float32 on
    the grid of the layer's internal activation type (fp16 for bf16 storage).
    The unsharded cache is the concatenation of the rank caches over heads."""
    d = w.dims
    shape = (d.batch, d.heads_local, cache_len, d.head_dim)
    out = []
    for name in ("k_cache", "v_cache"):
        a = _rng(w.seed, name, rank).standard_normal(shape, dtype=np.float32)
        a *= np.float32(kv_std(w))
        out.append(round_to_fp16(a) if d.dtype == "bf16" else a)
    return out[0], out[1]


def full_caches(w: Workload, cache_len: int):
    per = [rank_caches(w, r, cache_len) for r in range(w.dims.t)]
    return (np.concatenate([k for k, _ in per], axis=1),
            np.concatenate([v for _, v in per], axis=1))


def decode_inputs(w: Workload, cache_len: int, positions: str = "ragged"):
    """x_new [batch, h] (N(0,1) on the storage grid) and the position of each
    sequence's new token (int32 [batch]): "full" puts every token at
    cache_len - 1, "empty" at 0, "ragged" draws U{0..cache_len-1} with the
    first sequence at 0 and the last at cache_len - 1."""
    d = w.dims
    x = _normal(w.seed, "x_new", REPLICATED, (d.batch, d.hidden), 1.0, 0.0, d.dtype)
    if positions == "full":
        pos = np.full(d.batch, cache_len - 1)
    elif positions == "empty":
        pos = np.zeros(d.batch)
    else:
        pos = _rng(w.seed, "positions", REPLICATED).integers(0, cache_len, size=d.batch)
        pos[0] = 0
        if d.batch > 1:
            pos[-1] = cache_len - 1
    return x, pos.astype(np.int32)
