"""tp_layer_decode_static: the decode step with the library's own per-device
scratch instead of a caller workspace (for callers that cannot allocate).

Its kernels are tp_layer_decode's, so on the same inputs its outputs (the
layer output and the K and V rows it appends) must equal tp_layer_decode's
bit for bit, and both must match the fp64 decode oracle within
max|err| <= tau * RMS. Two calls in a row, the second on a smaller input
(fewer sequences, a shorter cache, another head dim), so the second runs on
what the first left in the shared scratch.
"""
import ctypes

import numpy as np
import pytest

from harness import TAU, err_ratio, to_np
from oracle import decode as OD
from tensor_model_transformer_amd import binding as B
from tensor_model_transformer_amd.synth import (LayerDims, Workload, decode_inputs, rank_caches,
                                                rank_params)


def _wl(name, batch, hidden, heads, ffn, t=1, dtype="bf16", seed=70, rank=0):
    return Workload(name, LayerDims(batch, 16, hidden, heads, ffn, t=t, dtype=dtype,
                                    mask="causal"), rank=rank, seed=seed, affine="perturbed")


def _decode_both(w, cache_len):
    """Runs one TP_ALL decode step through tp_layer_decode (own workspace)
    and through tp_layer_decode_static on copies of the same caches."""
    import torch
    from tensor_model_transformer_amd.shard import Shard, _check

    d = w.dims
    x, pos = decode_inputs(w, cache_len, "ragged")
    kc, vc = rank_caches(w, w.rank, cache_len)
    sh = Shard(d, w.rank)
    p = sh.upload_params(rank_params(w))
    xd = torch.from_numpy(x).to(sh.device).to(sh.dtype)
    posd = torch.from_numpy(pos).to(sh.device)
    res = {}
    for name in ("workspace", "static"):
        kd, vd = sh.upload_cache(kc), sh.upload_cache(vc)
        klo = torch.zeros_like(kd) if sh.split_scores else None
        out = torch.empty(d.batch, d.hidden, dtype=sh.dtype, device=sh.device)
        print(f"[no-alloc] {w.name} B={d.batch} h={d.hidden} dh={d.head_dim} L={cache_len} "
              f"via {name}", flush=True)
        if name == "workspace":
            rc = sh.decode(p, out, x=xd, k_cache=kd, v_cache=vd, k_cache_lo=klo, positions=posd)
        else:
            io = B.tp_decode_io()
            io.params = p.ptr()
            io.x, io.h_mid, io.out = xd.data_ptr(), None, out.data_ptr()
            io.k_cache, io.v_cache = kd.data_ptr(), vd.data_ptr()
            io.k_cache_lo = klo.data_ptr() if klo is not None else None
            io.positions = posd.data_ptr()
            io.cache_len = cache_len
            io.workspace, io.workspace_bytes = None, 0
            rc = B.tp_layer_decode_static(sh.handle, B.TP_ALL, io, sh.stream())
        _check(f"decode ({name})", rc)
        torch.cuda.synchronize()
        res[name] = {"out": to_np(out), "k": to_np(kd), "v": to_np(vd)}
    sh.close()
    return res, (x, pos, kc, vc)


@pytest.mark.gpu
def test_static_scratch_matches_workspace_twice():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cases = [(_wl("noalloc_first", 6, 640, 4, 1280), 333),    # head dim 160
             (_wl("noalloc_second", 2, 256, 4, 512, seed=71), 64)]  # smaller: head dim 64
    for w, cache_len in cases:
        res, (x, pos, kc, vc) = _decode_both(w, cache_len)
        a, b = res["workspace"], res["static"]
        for k in ("out", "k", "v"):
            assert np.array_equal(a[k], b[k]), f"{w.name}: {k} differs from tp_layer_decode"
        d = w.dims
        ref = OD.decode_step(rank_params(w, w.rank), x, kc, vc, pos, d.heads_local)
        e = err_ratio(b["out"], ref["out"])
        newk = np.stack([ref["k_cache"][i, :, pos[i]] for i in range(d.batch)])
        gk = np.stack([b["k"][i, :, pos[i]] for i in range(d.batch)])
        ek = err_ratio(gk, newk)
        print(f"[no-alloc] {w.name}: out {e:.2e}, k_new {ek:.2e}", flush=True)
        assert e <= TAU[d.dtype] and ek <= TAU[d.dtype]


def test_static_scratch_size_limit():
    # a handle whose decode scratch exceeds the library's array is refused
    # before anything is enqueued (no GPU needed: the checks come first)
    rc, h, _ = B.tp_layer_create(25600, 160, 102400, 2048, 32, 8, 0, B.TP_DTYPE_BF16,
                                 B.TP_MASK_CAUSAL, None)
    assert rc == B.TP_OK
    rc, need = B.tp_layer_decode_workspace(h)
    assert rc == B.TP_OK and need > B.TP_DECODE_STATIC_MAX_BYTES
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced
    prm = B.tp_params(*([fake.value] * 12), None)
    io = B.tp_decode_io()
    io.params = ctypes.pointer(prm)
    io.x = io.out = io.k_cache = io.v_cache = io.k_cache_lo = io.positions = fake.value
    io.cache_len = 16
    assert B.tp_layer_decode_static(h, B.TP_ALL, io, None) == B.TP_ERR_WORKSPACE
    assert B.tp_layer_decode_static(h, 9, io, None) == B.TP_ERR_PHASE
    B.tp_layer_destroy(h)
