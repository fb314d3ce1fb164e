"""Host-side tests of the C ABI library (no GPU, no kernel launch).

The library loads, exports every function ``include/tp_layer.h`` declares,
and its argument checks return the documented codes before anything is
enqueued.
"""
import ctypes
import os
import re

import pytest

from tensor_model_transformer_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_layer.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*int\s+(tp_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libtplayer.so is not built: run `python -m tensor_model_transformer_amd.build`")
    return B.lib()


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert set(declared) == set(B.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_enum_values_match_header():
    src = open(HEADER).read()
    for name in ("TP_OK", "TP_ERR_ARG", "TP_ERR_SHAPE", "TP_ERR_UNSUPPORTED", "TP_ERR_ALIGN",
                 "TP_ERR_WORKSPACE", "TP_ERR_HIP", "TP_ERR_PHASE", "TP_ERR_NOMEM", "TP_DTYPE_F32",
                 "TP_DTYPE_BF16", "TP_MASK_CAUSAL", "TP_MASK_PADDING", "TP_FWD_ATTN",
                 "TP_FWD_MLP", "TP_BWD_MLP", "TP_BWD_ATTN", "TP_BWD_LN1"):
        m = re.search(rf"\b{name}\s*=\s*(-?\d+)", src)
        assert m, name
        assert int(m.group(1)) == getattr(B, name), name


def create(**kw):
    a = dict(hidden=128, heads=4, ffn=512, seq=64, micro_batch=2, t=2, rank=0,
             dtype=B.TP_DTYPE_BF16, mask=B.TP_MASK_CAUSAL)
    a.update(kw)
    return B.tp_layer_create(a["hidden"], a["heads"], a["ffn"], a["seq"], a["micro_batch"],
                             a["t"], a["rank"], a["dtype"], a["mask"], a.get("opts"))


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=0), B.TP_ERR_ARG),
    (dict(seq=-1), B.TP_ERR_ARG),
    (dict(t=0), B.TP_ERR_ARG),
    (dict(hidden=130), B.TP_ERR_SHAPE),           # hidden % heads
    (dict(heads=6, hidden=192, t=4), B.TP_ERR_SHAPE),  # heads % t
    (dict(ffn=510), B.TP_ERR_SHAPE),              # ffn % t
    (dict(ffn=12, t=2), B.TP_ERR_SHAPE),          # (ffn/t) % 8
    (dict(rank=2), B.TP_ERR_SHAPE),
    (dict(rank=-1), B.TP_ERR_SHAPE),
    (dict(hidden=192, heads=4, t=1), B.TP_ERR_UNSUPPORTED),   # head dim 48
    (dict(dtype=7), B.TP_ERR_UNSUPPORTED),
    (dict(mask=3), B.TP_ERR_UNSUPPORTED),
    (dict(opts={"ln_eps": 1e-5, "gelu": 5}), B.TP_ERR_UNSUPPORTED),
    (dict(opts={"ln_eps": 0.0, "gelu": 0}), B.TP_ERR_ARG),
    (dict(opts={"dx_dtype": 7}), B.TP_ERR_UNSUPPORTED),
    (dict(dtype=B.TP_DTYPE_F32, opts={"dx_dtype": B.TP_DTYPE_BF16}), B.TP_ERR_UNSUPPORTED),
    (dict(opts={"scores": 3}), B.TP_ERR_UNSUPPORTED),
    (dict(opts={"recompute": 2}), B.TP_ERR_UNSUPPORTED),
    (dict(opts={"sequence_parallel": 2}), B.TP_ERR_UNSUPPORTED),
    (dict(opts={"overlap": 3}), B.TP_ERR_UNSUPPORTED),
    (dict(seq=63, micro_batch=1, opts={"sequence_parallel": 1}), B.TP_ERR_SHAPE),  # n % t
    (dict(dtype=B.TP_DTYPE_F32, opts={"scores": B.TP_SCORES_SPLIT}), B.TP_ERR_UNSUPPORTED),
])
def test_create_validation(lib, kw, code):
    rc, h, ws = create(**kw)
    assert rc == code
    assert h is None


def test_create_ok_and_workspace_plan(lib):
    rc, h, ws = create()
    assert rc == B.TP_OK and h
    assert ws > 0
    seen = []
    for name in B.TAPS:
        rc, off, nb = B.tp_layer_tap(h, name)
        if name == "qkv_lo":  # kept only with split scores (not chosen at hidden 128)
            assert rc == B.TP_ERR_UNSUPPORTED
            continue
        assert rc == B.TP_OK
        assert off % 256 == 0 and off + nb <= ws
        seen.append((off, off + nb))
    seen.sort()
    for (a0, a1), (b0, b1) in zip(seen, seen[1:]):
        assert a1 <= b0  # intermediates do not overlap
    assert B.tp_layer_tap(h, 99)[0] == B.TP_ERR_ARG
    assert B.tp_layer_destroy(h) == B.TP_OK
    assert B.tp_layer_destroy(None) == B.TP_OK


def test_scale_and_residual_taps(lib):
    # the gradient-chain scale exists on the 16-bit path only; the score
    # residuals exactly when split scores are on (AUTO: from hidden 8192)
    rc, h, _ = create(dtype=B.TP_DTYPE_F32)
    assert rc == B.TP_OK
    assert B.tp_layer_tap(h, "grad_scale")[0] == B.TP_ERR_UNSUPPORTED
    assert B.tp_layer_tap(h, "qkv_lo")[0] == B.TP_ERR_UNSUPPORTED
    B.tp_layer_destroy(h)
    rc, h, _ = create()
    rc2, off, nb = B.tp_layer_tap(h, "grad_scale")
    assert rc2 == B.TP_OK and nb == 8
    B.tp_layer_destroy(h)
    for opts, hidden, split in (({"scores": B.TP_SCORES_SPLIT}, 128, True),
                                ({"scores": B.TP_SCORES_FP16}, 8192, False),
                                (None, 8192, True), (None, 4096, False)):
        rc, h, _ = create(hidden=hidden, heads=hidden // 64, ffn=4 * hidden, opts=opts)
        assert rc == B.TP_OK
        rc2, _, nb = B.tp_layer_tap(h, "qkv_lo")
        assert (rc2 == B.TP_OK) == split, (opts, hidden)
        if split:  # fp16 [n, 3*h_l], n = 2*64 tokens, t = 2
            assert nb == 2 * 64 * 3 * (hidden // 2) * 2
        B.tp_layer_destroy(h)


def test_profile_arguments(lib):
    rc, h, _ = create()
    assert B.tp_layer_profile(h, 1, -1.0) == B.TP_ERR_ARG
    assert B.tp_layer_profile(h, 1, 0.0) == B.TP_OK
    assert B.tp_layer_profile(h, 0) == B.TP_OK
    assert B.tp_layer_profile(None, 0) == B.TP_ERR_ARG
    B.tp_layer_destroy(h)


def test_split_scores_workspace(lib):
    # the score residuals take one more fp16 [n, 3*h_l] region; AUTO keeps
    # them only from hidden 8192 on
    n, hl = 2 * 64, 64
    sizes = {}
    for mode in (B.TP_SCORES_AUTO, B.TP_SCORES_FP16, B.TP_SCORES_SPLIT):
        rc, h, ws = create(opts={"scores": mode})
        assert rc == B.TP_OK
        sizes[mode] = ws
        B.tp_layer_destroy(h)
    assert sizes[B.TP_SCORES_AUTO] == sizes[B.TP_SCORES_FP16]
    assert sizes[B.TP_SCORES_SPLIT] - sizes[B.TP_SCORES_FP16] >= n * 3 * hl * 2
    big = dict(hidden=8192, heads=64, ffn=512, seq=8, micro_batch=1, t=8)
    rc, h, ws_auto = create(**big)
    B.tp_layer_destroy(h)
    rc, h, ws_fp16 = create(opts={"scores": B.TP_SCORES_FP16}, **big)
    B.tp_layer_destroy(h)
    assert ws_auto - ws_fp16 >= 8 * 3 * 1024 * 2


def test_recompute_fc1_workspace(lib):
    # without the kept FC1 pre-activation the workspace shrinks by n*f_l
    # 16-bit elements; du then lives in the attention-backward buffers
    kw = dict(hidden=256, heads=4, ffn=1024, seq=64, micro_batch=2, t=1)
    n, fl = 128, 1024
    rc, h0, ws0 = create(**kw)
    assert rc == B.TP_OK
    rc, h1, ws1 = create(opts={"recompute": B.TP_RECOMPUTE_FC1}, **kw)
    assert rc == B.TP_OK
    assert ws0 - ws1 >= n * fl * 2
    assert B.tp_layer_tap(h1, B.TAPS["dgelu"])[0] == B.TP_ERR_UNSUPPORTED
    assert B.tp_layer_tap(h0, B.TAPS["dgelu"])[0] == B.TP_OK
    B.tp_layer_destroy(h0)
    B.tp_layer_destroy(h1)


def test_sequence_parallel_phases_are_separate(lib):
    # a handle in the sequence-parallel layout takes only the TP_*_SP_* phases,
    # and the ordinary handle none of them; the phase is checked before
    # anything touches a device
    rc, hs, ws = create(opts={"sequence_parallel": 1})
    assert rc == B.TP_OK
    rc, hn, _ = create()
    assert rc == B.TP_OK
    fio, bio = B.tp_fwd_io(), B.tp_bwd_io()
    for ph in (B.TP_ALL, 1, 2):
        assert B.tp_layer_fwd(hs, ph, fio) == B.TP_ERR_PHASE
    for ph in (B.TP_FWD_SP_LN1, B.TP_FWD_SP_OUT, 8):
        assert B.tp_layer_fwd(hn, ph, fio) == B.TP_ERR_PHASE
    for ph in (B.TP_ALL, 1, 2, 3):
        assert B.tp_layer_bwd(hs, ph, bio) == B.TP_ERR_PHASE
    for ph in (B.TP_BWD_SP_MLP, B.TP_BWD_SP_LN1):
        assert B.tp_layer_bwd(hn, ph, bio) == B.TP_ERR_PHASE
    B.tp_layer_destroy(hs)
    B.tp_layer_destroy(hn)


def test_call_argument_errors_need_no_device(lib):
    rc, h, ws = create()
    assert rc == B.TP_OK
    io = B.tp_fwd_io()
    assert B.tp_layer_fwd(None, B.TP_ALL, io, 0) == B.TP_ERR_ARG
    assert B.tp_layer_fwd(h, 9, io, 0) == B.TP_ERR_PHASE
    assert B.tp_layer_fwd(h, B.TP_ALL, io, 0) == B.TP_ERR_ARG  # no params
    p = B.tp_params()
    fake = 1 << 20  # never dereferenced: validation stops before any launch
    for f in B.PARAM_FIELDS:
        setattr(p, f, fake)
    io.params = ctypes.pointer(p)
    assert B.tp_layer_fwd(h, B.TP_ALL, io, 0) == B.TP_ERR_WORKSPACE
    io.workspace = fake
    io.workspace_bytes = ws - 1
    assert B.tp_layer_fwd(h, B.TP_ALL, io, 0) == B.TP_ERR_WORKSPACE
    io.workspace_bytes = ws
    io.workspace = fake + 8
    assert B.tp_layer_fwd(h, B.TP_ALL, io, 0) == B.TP_ERR_ALIGN
    io.workspace = fake
    assert B.tp_layer_fwd(h, B.TP_ALL, io, 0) == B.TP_ERR_ARG  # x/out missing
    setattr(p, "w_o", fake + 4)
    assert B.tp_layer_fwd(h, B.TP_ALL, io, 0) == B.TP_ERR_ALIGN
    bio = B.tp_bwd_io()
    assert B.tp_layer_bwd(h, 4, bio, 0) == B.TP_ERR_PHASE
    assert B.tp_layer_bwd(h, B.TP_ALL, bio, 0) == B.TP_ERR_ARG
    assert B.tp_exchange_sum(fake, B.TP_DTYPE_F32, [], 16, 0) == B.TP_ERR_ARG
    assert B.tp_exchange_sum(fake, B.TP_DTYPE_F32, [fake] * 17, 16, 0) == B.TP_ERR_ARG
    assert B.tp_exchange_sum(fake + 2, B.TP_DTYPE_F32, [fake], 16, 0) == B.TP_ERR_ALIGN
    B.tp_layer_destroy(h)


def test_padding_mask_requires_valid_len(lib):
    rc, h, ws = create(mask=B.TP_MASK_PADDING)
    assert rc == B.TP_OK
    p = B.tp_params()
    for f in B.PARAM_FIELDS:
        setattr(p, f, 1 << 20)
    io = B.tp_fwd_io()
    io.params = ctypes.pointer(p)
    io.workspace = 1 << 20
    io.workspace_bytes = ws
    assert B.tp_layer_fwd(h, B.TP_ALL, io, 0) == B.TP_ERR_ARG
    B.tp_layer_destroy(h)


def _decode_io(ws_bytes, fake=1 << 20):
    p = B.tp_params()
    for f in B.PARAM_FIELDS:
        setattr(p, f, fake)
    io = B.tp_decode_io()
    io.params = ctypes.pointer(p)
    io.workspace = fake
    io.workspace_bytes = ws_bytes
    for f in ("x", "out", "k_cache", "v_cache", "positions"):
        setattr(io, f, fake)
    io.cache_len = 16
    return io, p


def test_decode_workspace_is_small_and_independent_of_seq(lib):
    sizes = []
    for seq in (64, 4096):
        rc, h, ws = create(seq=seq, micro_batch=8)
        assert rc == B.TP_OK
        rc, dws = B.tp_layer_decode_workspace(h)
        assert rc == B.TP_OK and 0 < dws < ws
        sizes.append(dws)
        B.tp_layer_destroy(h)
    assert sizes[0] == sizes[1]
    assert B.tp_layer_decode_workspace(None)[0] == B.TP_ERR_ARG


def test_decode_argument_errors_need_no_device(lib):
    rc, h, _ = create(micro_batch=4)
    assert rc == B.TP_OK
    _, dws = B.tp_layer_decode_workspace(h)
    io, p = _decode_io(dws)
    assert B.tp_layer_decode(None, B.TP_ALL, io, 0) == B.TP_ERR_ARG
    assert B.tp_layer_decode(h, 3, io, 0) == B.TP_ERR_PHASE
    io.workspace_bytes = dws - 1
    assert B.tp_layer_decode(h, B.TP_ALL, io, 0) == B.TP_ERR_WORKSPACE
    io.workspace_bytes = dws
    io.workspace = (1 << 20) + 8
    assert B.tp_layer_decode(h, B.TP_ALL, io, 0) == B.TP_ERR_ALIGN
    io.workspace = 1 << 20
    io.positions = None
    assert B.tp_layer_decode(h, B.TP_FWD_ATTN, io, 0) == B.TP_ERR_ARG
    io.positions = 1 << 20
    io.cache_len = 0
    assert B.tp_layer_decode(h, B.TP_ALL, io, 0) == B.TP_ERR_ARG
    # the MLP phase needs neither the caches nor the token rows, only h_mid and out
    io2, _ = _decode_io(dws)
    io2.x = io2.k_cache = io2.v_cache = io2.positions = None
    io2.h_mid = None
    assert B.tp_layer_decode(h, B.TP_FWD_MLP, io2, 0) == B.TP_ERR_ARG
    # kv_fill: training workspace, cache at least seq rows
    rc, h2, ws2 = create(seq=64)
    assert B.tp_layer_kv_fill(h2, 1 << 20, ws2 - 1, 1 << 20, 1 << 20, None, 64, 0) == \
        B.TP_ERR_WORKSPACE
    assert B.tp_layer_kv_fill(h2, 1 << 20, ws2, 1 << 20, 1 << 20, None, 63, 0) == B.TP_ERR_SHAPE
    assert B.tp_layer_kv_fill(h2, 1 << 20, ws2, None, 1 << 20, None, 64, 0) == B.TP_ERR_ARG
    B.tp_layer_destroy(h2)
    B.tp_layer_destroy(h)


def test_decode_needs_causal_mask_batch_limit_and_split_residuals(lib):
    rc, h, _ = create(mask=B.TP_MASK_PADDING)
    _, dws = B.tp_layer_decode_workspace(h)
    io, p = _decode_io(dws)
    p.valid_len = 1 << 20
    assert B.tp_layer_decode(h, B.TP_ALL, io, 0) == B.TP_ERR_UNSUPPORTED
    B.tp_layer_destroy(h)
    rc, h, _ = create(micro_batch=129)
    _, dws = B.tp_layer_decode_workspace(h)
    io, _ = _decode_io(dws)
    assert B.tp_layer_decode(h, B.TP_ALL, io, 0) == B.TP_ERR_UNSUPPORTED
    B.tp_layer_destroy(h)
    opts = {"scores": B.TP_SCORES_SPLIT}
    rc, h, _ = create(opts=opts)
    _, dws = B.tp_layer_decode_workspace(h)
    io, _ = _decode_io(dws)
    assert B.tp_layer_decode(h, B.TP_ALL, io, 0) == B.TP_ERR_ARG  # k_cache_lo missing
    B.tp_layer_destroy(h)
