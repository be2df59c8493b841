"""Pins for the fp64 MoE reference (oracle/moe_ref.c, oracle/moe.py)."""
import os

import numpy as np
import pytest
import torch

import gen
from gen.configs import F32, BF16, MXFP4, TINY
from oracle import moe

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def e2m1_table():
    tab = {}
    for line in open(os.path.join(GOLD, "e2m1_values.txt")):
        if line.strip() and not line.startswith("#"):
            c, v = line.split()
            tab[int(c)] = float(v)
    return tab


def golden_mx_decode(codes, scales):
    tab = e2m1_table()
    vals = np.vectorize(lambda c: tab[int(c)])(codes).astype(np.float64)
    exps = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    return vals * np.exp2(exps.astype(np.float64))


def torch_expert(Wg, Wu, Wd, x):
    """Library special case: dense torch fp64 silu + matmul."""
    Wg, Wu, Wd, x = (torch.as_tensor(a, dtype=torch.float64) for a in (Wg, Wu, Wd, x))
    return (Wd @ (torch.nn.functional.silu(Wg @ x) * (Wu @ x))).numpy()


def test_mxfp4_decode_matches_ocp_table():
    codes = np.tile(np.arange(16, dtype=np.uint8), 6).reshape(3, 32)
    scales = np.array([[120], [127], [131]], np.uint8)
    got = moe.decode_weights(MXFP4, (codes, scales))
    np.testing.assert_array_equal(got, golden_mx_decode(codes, scales))


def test_bf16_widening_matches_torch():
    bits = np.random.default_rng(0).integers(0, 65536, size=(8, 64)).astype(np.uint16)
    bits[(bits & 0x7f80) == 0x7f80] = 0x3f80  # no inf/nan
    got = moe.decode_weights(BF16, bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(got, ref)


def _tiny_mats(wfmt, layer=0, expert=3, H=64, I=32):
    cfg = TINY.with_(H=H, I=I, wdtype=wfmt)
    return cfg, gen.expert_logical(cfg, layer, expert)


def _dense(wfmt, mats):
    if wfmt == MXFP4:
        return [golden_mx_decode(*mats[n]) for n in ("gate", "up", "down")]
    if wfmt == BF16:
        return [torch.from_numpy(mats[n].view(np.int16)).view(torch.bfloat16).double().numpy()
                for n in ("gate", "up", "down")]
    return [mats[n].astype(np.float64) for n in ("gate", "up", "down")]


@pytest.mark.parametrize("wfmt", [F32, BF16, MXFP4])
def test_expert_matches_torch_dense(wfmt):
    cfg, mats = _tiny_mats(wfmt)
    x = np.random.default_rng(1).normal(size=cfg.H)
    y, act = moe.expert(wfmt, mats, x, want_act=True)
    Wg, Wu, Wd = _dense(wfmt, mats)
    ref = torch_expert(Wg, Wu, Wd, x)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-15 * np.abs(ref).max())
    g = Wg @ x
    np.testing.assert_allclose(act, g / (1 + np.exp(-g)) * (Wu @ x), rtol=1e-12, atol=1e-18)


def test_special_cases_exact():
    cfg, mats = _tiny_mats(F32)
    zero = np.zeros(cfg.H)
    assert np.all(moe.expert(F32, mats, zero) == 0.0)
    x = np.random.default_rng(2).normal(size=cfg.H)
    m0 = dict(mats, gate=np.zeros_like(mats["gate"]))
    assert np.all(moe.expert(F32, m0, x) == 0.0)
    m2 = dict(mats, down=mats["down"] * np.float32(2.0))
    np.testing.assert_array_equal(moe.expert(F32, m2, x), 2.0 * moe.expert(F32, mats, x))


def test_layer_k1_is_one_expert_and_weights_combine():
    cfg = TINY.with_(H=64, I=32)
    rng = np.random.default_rng(3)
    x = rng.normal(size=(4, cfg.H))
    logits = rng.normal(size=(4, cfg.E)).astype(np.float32)
    get = lambda e: gen.expert_logical(cfg, 0, e)
    out1, ids1, w1 = moe.moe_tokens(F32, x, logits, 1, get)
    for t in range(4):
        assert w1[t] == [1.0]
        np.testing.assert_array_equal(out1[t], moe.expert(F32, get(ids1[t][0]), x[t]))
    out2, ids2, w2 = moe.moe_tokens(F32, x, logits, 2, get)
    for t in range(4):
        ref = sum(w * torch_expert(*_dense(F32, get(e)), x[t]) for e, w in zip(ids2[t], w2[t]))
        np.testing.assert_allclose(out2[t], ref, rtol=1e-12, atol=1e-16)
