"""Device-memory plumbing around the C ABI for one rank's layer shard.

PyTorch only provides device buffers and the stream here; every step of the
layer runs in ``libtplayer.so`` through ``binding``. Used by the tests, the
bench and the smoke entry point.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import binding as B
from .synth import LayerDims, PARAM_NAMES


class TpError(RuntimeError):
    def __init__(self, what, rc):
        super().__init__(f"{what} failed: {B.ERROR_NAMES.get(rc, rc)} ({rc})")
        self.rc = rc


def _check(what, rc):
    if rc != B.TP_OK:
        raise TpError(what, rc)


def torch_dtype(dims: LayerDims):
    return torch.bfloat16 if dims.dtype == "bf16" else torch.float32


def to_device(a: np.ndarray, dtype, device) -> torch.Tensor:
    """Upload a float32 array (already on the storage grid) as `dtype`."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device).to(dtype).contiguous()


class Shard:
    """One handle of the library plus its workspace."""

    def __init__(self, dims: LayerDims, rank: int, device="cuda:0", gelu: int = B.TP_GELU_ERF,
                 eps: float = 1e-5, dx_fp32: bool = True, scores: int = B.TP_SCORES_AUTO,
                 recompute: int = B.TP_RECOMPUTE_NONE, sequence_parallel: bool = False,
                 overlap: int = B.TP_OVERLAP_AUTO):
        self.dims = dims
        self.rank = rank
        self.device = torch.device(device)
        self.dtype = torch_dtype(dims)
        rc, self.handle, self.ws_bytes = B.tp_layer_create(
            dims.hidden, dims.heads, dims.ffn, dims.seq, dims.batch, dims.t, rank,
            B.TP_DTYPE_BF16 if dims.dtype == "bf16" else B.TP_DTYPE_F32,
            B.TP_MASK_PADDING if dims.mask == "padding" else B.TP_MASK_CAUSAL,
            {"ln_eps": eps, "gelu": gelu,
             "dx_dtype": B.TP_DTYPE_F32 if dx_fp32 or dims.dtype == "f32" else B.TP_DTYPE_BF16,
             "scores": scores, "recompute": recompute,
             "sequence_parallel": int(sequence_parallel),
             "overlap": overlap})
        self.dx_fp32 = dx_fp32
        _check("tp_layer_create", rc)
        # whether the handle keeps the score residuals (what TP_SCORES_AUTO chose)
        self.split_scores = B.tp_layer_tap(self.handle, "qkv_lo")[0] == B.TP_OK
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)
        self.dws = None
        self.dws_bytes = 0

    def close(self):
        if self.handle:
            B.tp_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- tensors ---------------------------------------------------------
    def upload_params(self, params: Dict[str, np.ndarray], valid_len=None):
        dev = {k: to_device(params[k], self.dtype, self.device) for k in PARAM_NAMES}
        vl = None
        if valid_len is not None:
            vl = torch.from_numpy(np.asarray(valid_len, dtype=np.int32)).to(self.device)
        return DeviceParams(dev, vl)

    def act(self, a: np.ndarray) -> torch.Tensor:
        return to_device(a.reshape(self.dims.tokens, self.dims.hidden), self.dtype, self.device)

    def empty_act(self, fp32=False) -> torch.Tensor:
        return torch.empty(self.dims.tokens, self.dims.hidden,
                           dtype=torch.float32 if fp32 else self.dtype, device=self.device)

    def empty_dx(self) -> torch.Tensor:
        return self.empty_act(fp32=self.dx_fp32)

    def zero_grads(self) -> Dict[str, torch.Tensor]:
        shapes = self.dims.shapes()
        return {k: torch.zeros(shapes[k], dtype=torch.float32, device=self.device)
                for k in PARAM_NAMES}

    def tap(self, name: str) -> torch.Tensor:
        rc, off, nbytes = B.tp_layer_tap(self.handle, name)
        _check("tp_layer_tap", rc)
        return self.ws[off:off + nbytes]

    def act_dtype(self):
        """Internal activation type: fp16 for the bf16 layer (also the KV cache)."""
        return torch.float16 if self.dims.dtype == "bf16" else torch.float32

    def upload_cache(self, a: np.ndarray) -> torch.Tensor:
        """A [B, H_l, L, dh] cache array (already on the act grid) on the device."""
        return to_device(a, self.act_dtype(), self.device)

    def empty_cache(self, cache_len: int) -> torch.Tensor:
        d = self.dims
        return torch.zeros(d.batch, d.heads_local, cache_len, d.head_dim, dtype=self.act_dtype(),
                           device=self.device)

    def decode_workspace(self) -> torch.Tensor:
        if self.dws is None:
            rc, self.dws_bytes = B.tp_layer_decode_workspace(self.handle)
            _check("tp_layer_decode_workspace", rc)
            self.dws = torch.empty(max(self.dws_bytes, 256), dtype=torch.uint8, device=self.device)
        return self.dws

    # -- calls -----------------------------------------------------------
    def stream(self) -> int:
        return torch.cuda.current_stream(self.device).cuda_stream

    def fwd(self, p: "DeviceParams", out: Optional[torch.Tensor], x: Optional[torch.Tensor] = None,
            h_mid: Optional[torch.Tensor] = None, phase: int = B.TP_ALL,
            reduced: Optional[torch.Tensor] = None, gathered: Optional[torch.Tensor] = None) -> int:
        io = B.tp_fwd_io()
        io.params = p.ptr()
        io.x = x.data_ptr() if x is not None else None
        io.h_mid = h_mid.data_ptr() if h_mid is not None else None
        io.out = out.data_ptr() if out is not None else None
        io.reduced = reduced.data_ptr() if reduced is not None else None
        io.gathered = gathered.data_ptr() if gathered is not None else None
        io.workspace = self.ws.data_ptr()
        io.workspace_bytes = self.ws_bytes
        return B.tp_layer_fwd(self.handle, phase, io, self.stream())

    def bwd(self, p: "DeviceParams", grads: Dict[str, torch.Tensor], x=None, dout=None, dx=None,
            dc=None, da=None, partial=None, accumulate=0, phase: int = B.TP_ALL,
            gathered_act=None, gathered_grad=None) -> int:
        io = B.tp_bwd_io()
        io.params = p.ptr()
        for name, t in (("x", x), ("dout", dout), ("dx", dx), ("dc", dc), ("da", da),
                        ("partial", partial), ("gathered_act", gathered_act),
                        ("gathered_grad", gathered_grad)):
            setattr(io, name, t.data_ptr() if t is not None else None)
        for k in PARAM_NAMES:
            g = grads.get(k) if grads is not None else None
            setattr(io, "d_" + k, g.data_ptr() if g is not None else None)
        io.accumulate = accumulate
        io.workspace = self.ws.data_ptr()
        io.workspace_bytes = self.ws_bytes
        return B.tp_layer_bwd(self.handle, phase, io, self.stream())


    def decode(self, p: "DeviceParams", out: Optional[torch.Tensor], x=None, h_mid=None,
               k_cache=None, v_cache=None, k_cache_lo=None, positions=None,
               phase: int = B.TP_ALL) -> int:
        ws = self.decode_workspace()
        io = B.tp_decode_io()
        io.params = p.ptr()
        for name, t in (("x", x), ("h_mid", h_mid), ("out", out), ("k_cache", k_cache),
                        ("v_cache", v_cache), ("k_cache_lo", k_cache_lo),
                        ("positions", positions)):
            setattr(io, name, t.data_ptr() if t is not None else None)
        io.cache_len = int(k_cache.shape[2]) if k_cache is not None else 0
        io.workspace = ws.data_ptr()
        io.workspace_bytes = self.dws_bytes
        return B.tp_layer_decode(self.handle, phase, io, self.stream())

    def kv_fill(self, k_cache, v_cache, k_cache_lo=None) -> int:
        return B.tp_layer_kv_fill(self.handle, self.ws.data_ptr(), self.ws_bytes,
                                  k_cache.data_ptr(), v_cache.data_ptr(),
                                  k_cache_lo.data_ptr() if k_cache_lo is not None else None,
                                  int(k_cache.shape[2]), self.stream())


class DeviceParams:
    def __init__(self, tensors: Dict[str, torch.Tensor], valid_len: Optional[torch.Tensor]):
        self.t = tensors
        self.valid_len = valid_len
        self._s = B.tp_params()
        for k in PARAM_NAMES:
            setattr(self._s, k, tensors[k].data_ptr())
        self._s.valid_len = valid_len.data_ptr() if valid_len is not None else None

    def ptr(self):
        import ctypes
        return ctypes.pointer(self._s)


def exchange_sum(dst: torch.Tensor, parts, stream: int) -> None:
    """On-device sum of fp32 partial buffers (the single-GPU exchange)."""
    dt = B.TP_DTYPE_BF16 if dst.dtype == torch.bfloat16 else B.TP_DTYPE_F32
    _check("tp_exchange_sum",
           B.tp_exchange_sum(dst.data_ptr(), dt, [p.data_ptr() for p in parts], dst.numel(), stream))
