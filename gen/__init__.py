"""Seeded synthetic inputs shared by the GPU path's tests and the CPU oracle.

Only input generation lives here (numbers drawn from splitmix64 and packed into
the expert-bank byte layout); none of the MoE layer's arithmetic does. The C
source is gen/ecgen.c, built to gen/libecgen.so.
"""
import ctypes
import os
import subprocess

import numpy as np

from .configs import F32, BF16, MXFP4, Workload  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libecgen.so")
_lib = None

TAG_GATE, TAG_UP, TAG_DOWN = 0, 1, 2
TAG_X, TAG_PLOGIT, TAG_PX, TAG_VEC, TAG_ROUTER = 11, 12, 13, 14, 15


def build(force=True):
    """Compile gen/ecgen.c with gcc (OpenMP) into gen/libecgen.so."""
    src = os.path.join(_HERE, "ecgen.c")
    if not force and os.path.exists(_SO) and os.path.getmtime(_SO) >= os.path.getmtime(src):
        return _SO
    tmp = _SO + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O3", "-mavx2", "-mfma", "-fopenmp", "-shared", "-fPIC", "-o", tmp, src, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, i32, i64, dbl, vp = (ctypes.c_uint64, ctypes.c_int, ctypes.c_int64, ctypes.c_double,
                                  ctypes.c_void_p)
        L.ecg_key.restype = u64
        L.ecg_key.argtypes = [u64] * 5
        L.ecg_normals_f64.argtypes = [u64, u64, u64, u64, u64, u64, i64, dbl, vp]
        L.ecg_normals_f32.argtypes = [u64, u64, u64, u64, u64, i64, dbl, vp]
        L.ecg_normals_bf16.argtypes = [u64, u64, u64, u64, u64, i64, dbl, vp]
        L.ecg_expert_matrix.argtypes = [u64, i32, i32, i32, i32, i32, i32, dbl, vp]
        L.ecg_expert_matrix_mxfp4.argtypes = [u64, i32, i32, i32, i32, i32, dbl, vp, vp]
        L.ecg_expert_bytes.restype = u64
        L.ecg_expert_bytes.argtypes = [i32, i32, i32]
        L.ecg_fill_pool.argtypes = [u64, i32, i32, i32, i32, dbl, i32, i32, i32, vp]
        L.ecg_decode_logits.argtypes = [u64, i32, i32, i32, i32, i32, dbl, vp]
        _lib = L
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def expert_bytes(wdtype, H, I):
    return int(lib().ecg_expert_bytes(wdtype, H, I))


def expert_logical(cfg: Workload, layer: int, expert: int):
    """Logical matrices of one expert: gate [I,H], up [I,H], down [H,I].

    f32 -> float32 arrays; bf16 -> uint16 bit patterns; MXFP4 -> (codes uint8
    one per element, scales uint8 [rows, cols/32]) pairs.
    """
    H, I = cfg.H, cfg.I
    out = {}
    for tag, name in ((TAG_GATE, "gate"), (TAG_UP, "up"), (TAG_DOWN, "down")):
        rows, cols = (H, I) if tag == TAG_DOWN else (I, H)
        if cfg.wdtype == MXFP4:
            codes = np.empty((rows, cols), np.uint8)
            scales = np.empty((rows, cols // 32), np.uint8)
            lib().ecg_expert_matrix_mxfp4(cfg.seed, layer, expert, tag, H, I, cfg.sigma,
                                          _ptr(codes), _ptr(scales))
            out[name] = (codes, scales)
        else:
            a = np.empty((rows, cols), np.float32 if cfg.wdtype == F32 else np.uint16)
            lib().ecg_expert_matrix(cfg.seed, cfg.wdtype, layer, expert, tag, H, I, cfg.sigma, _ptr(a))
            out[name] = a
    return out


def fill_pool_ptr(cfg: Workload, dst_ptr: int, l0=0, l1=None, layer_period=0):
    """Pack layers [l0, l1) of the expert bank into memory at dst_ptr (layer l0)."""
    l1 = cfg.L if l1 is None else l1
    lib().ecg_fill_pool(cfg.seed, cfg.wdtype, cfg.E, cfg.H, cfg.I, cfg.sigma, l0, l1, layer_period,
                        ctypes.c_void_p(dst_ptr))


def pool_array(cfg: Workload, l0=0, l1=None):
    """The packed expert bank of layers [l0, l1) as a uint8 numpy array."""
    l1 = cfg.L if l1 is None else l1
    a = np.empty((l1 - l0) * cfg.E * cfg.expert_bytes, np.uint8)
    fill_pool_ptr(cfg, a.ctypes.data, l0, l1)
    return a


def decode_logits(cfg: Workload, steps=None, p=None, T=None, L=None):
    """Router logits [steps, L, T, E] float32 with step-to-step overlap p."""
    steps = cfg.steps if steps is None else steps
    p = cfg.p if p is None else p
    T = cfg.T if T is None else T
    L = cfg.L if L is None else L
    out = np.empty((steps, L, T, cfg.E), np.float32)
    lib().ecg_decode_logits(cfg.seed, steps, L, T, cfg.E, cfg.k, float(p), _ptr(out))
    return out


def normals(cfg: Workload, tag, a, b, c, n, sigma=1.0, bf16=False):
    """n draws N(0, sigma) of stream (tag, a, b, c): float32, or bf16 bit patterns."""
    if bf16:
        out = np.empty(n, np.uint16)
        lib().ecg_normals_bf16(cfg.seed, tag, a, b, c, n, sigma, _ptr(out))
    else:
        out = np.empty(n, np.float32)
        lib().ecg_normals_f32(cfg.seed, tag, a, b, c, n, sigma, _ptr(out))
    return out


def decode_x(cfg: Workload, step, layer, T=None):
    """Layer input x [T, H] ~ N(0,1): float32 for f32 workloads, else bf16 bits."""
    T = cfg.T if T is None else T
    return normals(cfg, TAG_X, step, layer, 0, T * cfg.H, bf16=cfg.act_bf16).reshape(T, cfg.H)


def prefill_logits(cfg: Workload, layer, T=None):
    """Prefill router logits [T, E] i.i.d. N(0,1) float32."""
    T = cfg.T if T is None else T
    return normals(cfg, TAG_PLOGIT, layer, 0, 0, T * cfg.E).reshape(T, cfg.E)


def prefill_x(cfg: Workload, layer, T=None):
    """Prefill hidden states [T, H] ~ N(0,1) in bf16 bits."""
    T = cfg.T if T is None else T
    return normals(cfg, TAG_PX, layer, 0, 0, T * cfg.H, bf16=True).reshape(T, cfg.H)


def router_weights(cfg: Workload, layer):
    """Router matrix W_r [E, H] of one layer ~ N(0, 1/sqrt(H)) (logits of N(0,1) inputs are then
    about N(0,1)): float32 for f32 workloads, else bf16 bits."""
    n = cfg.E * cfg.H
    return normals(cfg, TAG_ROUTER, layer, 0, 0, n, sigma=1.0 / np.sqrt(cfg.H),
                   bf16=cfg.act_bf16).reshape(cfg.E, cfg.H)


def bf16_to_f32(a):
    """Widen bf16 bit patterns (uint16) to float32 (exact)."""
    return (a.astype(np.uint32) << 16).view(np.float32)
