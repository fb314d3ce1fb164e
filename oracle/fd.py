"""Central finite differences of loss = sum(out * dout) for the oracle layer.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``). Used on tiny shapes
to pin the analytic backward of ``oracle.layer`` (the chain rule through
LayerNorm, GeLU, masked softmax attention and the head-interleaved QKV).
"""
from __future__ import annotations

import numpy as np

from . import layer as L


def loss(params, x, dout, heads, mask, valid_len, eps=1e-5, gelu_form="erf"):
    r = L.layer(params, x, dout, heads, mask, valid_len, eps=eps, gelu_form=gelu_form)
    return float(np.sum(r["out"] * np.asarray(dout, dtype=np.float64)))


def directional(params, x, dout, heads, mask, valid_len, name, direction, step=1e-6, **kw):
    """(loss(theta + step*v) - loss(theta - step*v)) / (2*step) for a
    direction v in parameter ``name`` (or ``"x"`` for the input)."""
    def shifted(sign):
        p = {k: np.array(v, dtype=np.float64) for k, v in params.items()}
        xx = np.array(x, dtype=np.float64)
        if name == "x":
            xx = xx + sign * step * direction
        else:
            p[name] = p[name] + sign * step * direction
        return loss(p, xx, dout, heads, mask, valid_len, **kw)
    return (shifted(+1.0) - shifted(-1.0)) / (2.0 * step)


def elementwise(params, x, dout, heads, mask, valid_len, name, step=1e-6, **kw):
    """Full finite-difference gradient of one (small) tensor."""
    base = np.asarray(x if name == "x" else params[name], dtype=np.float64)
    g = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        e = np.zeros_like(base)
        e[idx] = 1.0
        g[idx] = directional(params, x, dout, heads, mask, valid_len, name, e, step, **kw)
    return g
