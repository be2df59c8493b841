"""ctypes wrapper around oracle/moe_ref.c and the per-token MoE layer driver.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The layer output is the definition (FreeToken write-up, "Bandwidth-adaptive
execution": exact merge of partial sums, no approximation):
    out[t] = sum_j w[t,j] * f_{e[t,j]}(x_t)
with routing from oracle/route.py. Expert weights come in as logical matrices
(gate [I,H], up [I,H], down [H,I]) through a callback, so the oracle never
sees the packed expert-bank layout.

Pins (tests/test_oracle_moe.py): dense torch fp64 silu/matmul on tiny inputs
(a library special case), x = 0 and W_gate = 0 give exactly 0, k = 1 reduces
to one expert, scaling W_down by 2 doubles the output exactly, the E2M1 value
table of the OCP MX specification (tests/golden/), exact bf16 widening.
"""
import ctypes
import os
import subprocess

import numpy as np

from . import route as _route

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libmoeref.so")
_lib = None

F32, BF16, MXFP4 = 0, 1, 2


def build(force=True):
    """Compile oracle/moe_ref.c (gcc -O2, OpenMP, no fast-math)."""
    src = os.path.join(_HERE, "moe_ref.c")
    if not force and os.path.exists(_SO) and os.path.getmtime(_SO) >= os.path.getmtime(src):
        return _SO
    tmp = _SO + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-shared", "-fPIC", "-o", tmp,
                           src, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        L.oracle_expert.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_decode_weights.argtypes = [i32, vp, vp, i32, i32, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _split(wfmt, m):
    if wfmt == MXFP4:
        codes, scales = m
        return np.ascontiguousarray(codes, np.uint8), np.ascontiguousarray(scales, np.uint8)
    dt = np.float32 if wfmt == F32 else np.uint16
    return np.ascontiguousarray(m, dt), None


def decode_weights(wfmt, m):
    """Logical matrix (f32 / bf16 bits / (codes, scales)) -> float64 values."""
    w, s = _split(wfmt, m)
    rows, cols = w.shape
    out = np.empty((rows, cols), np.float64)
    lib().oracle_decode_weights(wfmt, _p(w), _p(s), rows, cols, _p(out))
    return out


def expert(wfmt, mats, x, want_act=False):
    """f_e(x) in fp64 for one token: mats = dict(gate, up, down) logical matrices."""
    g, sg = _split(wfmt, mats["gate"])
    u, su = _split(wfmt, mats["up"])
    d, sd = _split(wfmt, mats["down"])
    I, H = g.shape
    x = np.ascontiguousarray(x, np.float64)
    y = np.empty(H, np.float64)
    act = np.empty(I, np.float64)
    lib().oracle_expert(wfmt, H, I, _p(g), _p(sg), _p(u), _p(su), _p(d), _p(sd), _p(x), _p(y), _p(act))
    return (y, act) if want_act else y


def moe_tokens(wfmt, x, logits, k, get_expert, tokens=None):
    """out[t] (fp64) for the given token rows of one layer.

    x [T,H] float (already widened), logits [T,E] float32, get_expert(e) ->
    logical matrices of expert e of this layer. Returns (out [n,H], ids, w).
    """
    rows = range(len(x)) if tokens is None else tokens
    sel_logits = [logits[t] for t in rows]
    ids, ws = _route.route(sel_logits, k)
    cache = {}
    out = np.zeros((len(sel_logits), x.shape[1]), np.float64)
    for n, t in enumerate(rows):
        acc = np.zeros(x.shape[1], np.float64)
        for e, w in zip(ids[n], ws[n]):
            if e not in cache:
                cache[e] = get_expert(e)
            acc += w * expert(wfmt, cache[e], x[t])
        out[n] = acc
    return out, ids, ws
