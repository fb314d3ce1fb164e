"""ctypes binding of ``libtplayer.so`` (the C ABI in ``include/tp_layer.h``).

Argument marshalling only: every computation runs in the HIP library. The
functions keep the C names and return the C status code (0 = TP_OK); pointer
arguments are integers (device addresses, e.g. ``tensor.data_ptr()``) and a
stream is a ``hipStream_t`` as an integer (``torch.cuda.current_stream().cuda_stream``).
If the library is missing this module raises on import of the library --
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_float, c_int, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtplayer.so")

TP_OK = 0
TP_ERR_ARG = -1
TP_ERR_SHAPE = -2
TP_ERR_UNSUPPORTED = -3
TP_ERR_ALIGN = -4
TP_ERR_WORKSPACE = -5
TP_ERR_HIP = -6
TP_ERR_PHASE = -7
TP_ERR_NOMEM = -8
ERROR_NAMES = {0: "TP_OK", -1: "TP_ERR_ARG", -2: "TP_ERR_SHAPE", -3: "TP_ERR_UNSUPPORTED",
               -4: "TP_ERR_ALIGN", -5: "TP_ERR_WORKSPACE", -6: "TP_ERR_HIP", -7: "TP_ERR_PHASE",
               -8: "TP_ERR_NOMEM"}

TP_DTYPE_F32, TP_DTYPE_BF16 = 0, 1
TP_SCORES_AUTO, TP_SCORES_FP16, TP_SCORES_SPLIT = 0, 1, 2
TP_RECOMPUTE_NONE, TP_RECOMPUTE_FC1 = 0, 1
TP_OVERLAP_AUTO, TP_OVERLAP_OFF, TP_OVERLAP_ON = 0, 1, 2
TP_FWD_SP_LN1, TP_FWD_SP_ATTN, TP_FWD_SP_LN2, TP_FWD_SP_MLP, TP_FWD_SP_OUT = 3, 4, 5, 6, 7
TP_BWD_SP_MLP, TP_BWD_SP_LN2, TP_BWD_SP_ATTN, TP_BWD_SP_LN1 = 4, 5, 6, 7
TP_MASK_CAUSAL, TP_MASK_PADDING = 0, 1
TP_GELU_ERF, TP_GELU_TANH = 0, 1
TP_ALL, TP_FWD_ATTN, TP_FWD_MLP = 0, 1, 2
TP_BWD_MLP, TP_BWD_ATTN, TP_BWD_LN1 = 1, 2, 3
TAPS = {"a": 0, "qkv": 1, "o": 2, "lse2": 3, "h_mid": 4, "c": 5, "dgelu": 6, "z": 7,
        "dqkv": 8, "dh": 9, "grad_scale": 10, "qkv_lo": 11}

PARAM_FIELDS = ("ln1_gamma", "ln1_beta", "w_qkv", "b_qkv", "w_o", "b_o",
                "ln2_gamma", "ln2_beta", "w_fc1", "b_fc1", "w_fc2", "b_fc2")
GRAD_FIELDS = tuple("d_" + f for f in PARAM_FIELDS)

# Every symbol the header declares (checked by the CPU test of the library).
EXPORTS = ("tp_layer_create", "tp_layer_fwd", "tp_layer_bwd", "tp_layer_destroy",
           "tp_exchange_sum", "tp_layer_tap", "tp_layer_profile", "tp_layer_profile_read",
           "tp_layer_decode_workspace", "tp_layer_decode", "tp_layer_kv_fill",
           "tp_layer_decode_static")
TP_DECODE_STATIC_MAX_BYTES = 32 << 20
KCLASSES = ("gemm", "attn_fwd", "attn_bwd", "ln_fwd", "ln_bwd", "reduce", "convert")


class tp_layer_opts(Structure):
    _fields_ = [("ln_eps", c_float), ("gelu", c_int), ("dx_dtype", c_int), ("scores", c_int),
                ("recompute", c_int), ("sequence_parallel", c_int), ("overlap", c_int)]


class tp_params(Structure):
    _fields_ = [(f, c_void_p) for f in PARAM_FIELDS] + [("valid_len", c_void_p)]


class tp_fwd_io(Structure):
    _fields_ = [("params", POINTER(tp_params)), ("x", c_void_p), ("h_mid", c_void_p),
                ("out", c_void_p), ("workspace", c_void_p), ("workspace_bytes", c_size_t),
                ("reduced", c_void_p), ("gathered", c_void_p)]


class tp_bwd_io(Structure):
    _fields_ = ([("params", POINTER(tp_params)), ("x", c_void_p), ("dout", c_void_p),
                 ("dc", c_void_p), ("da", c_void_p), ("partial", c_void_p), ("dx", c_void_p)]
                + [(f, c_void_p) for f in GRAD_FIELDS]
                + [("accumulate", c_int), ("workspace", c_void_p), ("workspace_bytes", c_size_t),
                   ("gathered_act", c_void_p), ("gathered_grad", c_void_p)])


class tp_decode_io(Structure):
    _fields_ = [("params", POINTER(tp_params)), ("x", c_void_p), ("h_mid", c_void_p),
                ("out", c_void_p), ("k_cache", c_void_p), ("v_cache", c_void_p),
                ("k_cache_lo", c_void_p), ("positions", c_void_p), ("cache_len", c_int),
                ("workspace", c_void_p), ("workspace_bytes", c_size_t)]


_lib = None


def lib():
    """The loaded library (loaded once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m tensor_model_transformer_amd.build`"
                " (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        L.tp_layer_create.argtypes = [c_int] * 9 + [POINTER(tp_layer_opts), POINTER(c_void_p),
                                                    POINTER(c_size_t)]
        L.tp_layer_create.restype = c_int
        L.tp_layer_fwd.argtypes = [c_void_p, c_int, POINTER(tp_fwd_io), c_void_p]
        L.tp_layer_fwd.restype = c_int
        L.tp_layer_bwd.argtypes = [c_void_p, c_int, POINTER(tp_bwd_io), c_void_p]
        L.tp_layer_bwd.restype = c_int
        L.tp_layer_destroy.argtypes = [c_void_p]
        L.tp_layer_destroy.restype = c_int
        L.tp_exchange_sum.argtypes = [c_void_p, c_int, POINTER(c_void_p), c_int, c_size_t,
                                      c_void_p]
        L.tp_exchange_sum.restype = c_int
        L.tp_layer_tap.argtypes = [c_void_p, c_int, POINTER(c_size_t), POINTER(c_size_t)]
        L.tp_layer_tap.restype = c_int
        L.tp_layer_profile.argtypes = [c_void_p, c_int, ctypes.c_double]
        L.tp_layer_profile.restype = c_int
        L.tp_layer_profile_read.argtypes = [c_void_p, c_int, POINTER(ctypes.c_long),
                                            POINTER(ctypes.c_double), POINTER(ctypes.c_double),
                                            POINTER(ctypes.c_double)]
        L.tp_layer_profile_read.restype = c_int
        L.tp_layer_decode_workspace.argtypes = [c_void_p, POINTER(c_size_t)]
        L.tp_layer_decode_workspace.restype = c_int
        L.tp_layer_decode.argtypes = [c_void_p, c_int, POINTER(tp_decode_io), c_void_p]
        L.tp_layer_decode.restype = c_int
        L.tp_layer_kv_fill.argtypes = [c_void_p, c_void_p, c_size_t, c_void_p, c_void_p, c_void_p,
                                       c_int, c_void_p]
        L.tp_layer_kv_fill.restype = c_int
        L.tp_layer_decode_static.argtypes = [c_void_p, c_int, POINTER(tp_decode_io), c_void_p]
        L.tp_layer_decode_static.restype = c_int
        _lib = L
    return _lib


def tp_layer_create(hidden, heads, ffn, seq, micro_batch, t, rank, dtype, mask, opts=None):
    """Returns (status, handle, workspace_bytes)."""
    h = c_void_p()
    ws = c_size_t()
    o = None
    if opts is not None:
        o = ctypes.byref(tp_layer_opts(float(opts.get("ln_eps", 1e-5)), int(opts.get("gelu", 0)),
                                       int(opts.get("dx_dtype", TP_DTYPE_F32)),
                                       int(opts.get("scores", TP_SCORES_AUTO)),
                                       int(opts.get("recompute", TP_RECOMPUTE_NONE)),
                                       int(opts.get("sequence_parallel", 0)),
                                       int(opts.get("overlap", TP_OVERLAP_AUTO))))
    rc = lib().tp_layer_create(hidden, heads, ffn, seq, micro_batch, t, rank, dtype, mask, o,
                               ctypes.byref(h), ctypes.byref(ws))
    return rc, h.value, ws.value


def tp_layer_fwd(handle, phase, io: tp_fwd_io, stream=0):
    return lib().tp_layer_fwd(handle, phase, ctypes.byref(io), stream)


def tp_layer_bwd(handle, phase, io: tp_bwd_io, stream=0):
    return lib().tp_layer_bwd(handle, phase, ctypes.byref(io), stream)


def tp_layer_destroy(handle):
    return lib().tp_layer_destroy(handle)


def tp_exchange_sum(dst, dst_dtype, parts, count, stream=0):
    arr = (c_void_p * len(parts))(*parts)
    return lib().tp_exchange_sum(dst, dst_dtype, arr, len(parts), count, stream)


def tp_layer_tap(handle, tap):
    """Returns (status, offset, bytes) of a workspace intermediate."""
    off = c_size_t()
    nb = c_size_t()
    rc = lib().tp_layer_tap(handle, TAPS[tap] if isinstance(tap, str) else tap,
                            ctypes.byref(off), ctypes.byref(nb))
    return rc, off.value, nb.value


def tp_layer_profile(handle, enable, attn_pairs=0.0):
    return lib().tp_layer_profile(handle, int(enable), float(attn_pairs))


def tp_layer_profile_read(handle, kclass):
    """Returns (status, launches, ms, flops, bytes) for a kernel class."""
    n = ctypes.c_long()
    ms, fl, by = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    k = KCLASSES.index(kclass) if isinstance(kclass, str) else kclass
    rc = lib().tp_layer_profile_read(handle, k, ctypes.byref(n), ctypes.byref(ms),
                                     ctypes.byref(fl), ctypes.byref(by))
    return rc, n.value, ms.value, fl.value, by.value


def tp_layer_decode_workspace(handle):
    """Returns (status, bytes)."""
    nb = c_size_t()
    rc = lib().tp_layer_decode_workspace(handle, ctypes.byref(nb))
    return rc, nb.value


def tp_layer_decode(handle, phase, io: tp_decode_io, stream=0):
    return lib().tp_layer_decode(handle, phase, ctypes.byref(io), stream)


def tp_layer_decode_static(handle, phase, io: tp_decode_io, stream=0):
    """tp_layer_decode with the library's own per-device scratch (io.workspace unused)."""
    return lib().tp_layer_decode_static(handle, phase, ctypes.byref(io), stream)


def tp_layer_kv_fill(handle, workspace, workspace_bytes, k_cache, v_cache, k_cache_lo,
                     cache_len, stream=0):
    return lib().tp_layer_kv_fill(handle, workspace, workspace_bytes, k_cache, v_cache,
                                  k_cache_lo, cache_len, stream)
