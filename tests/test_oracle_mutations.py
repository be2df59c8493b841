"""Planted mistakes in the oracle must fail its pins.

Each case copies an oracle source file, plants one plausible mistake (a
swapped operand, a wrong sign or bias, a dropped term, a reversed order),
builds or loads the copy on the CPU and checks that at least one pin rejects
it. The oracle itself is never modified.
"""
import ctypes
import json
import os
import subprocess
import types

import numpy as np
import pytest
import torch

import gen
from gen.configs import F32, MXFP4, TINY

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = os.path.join(ROOT, "tests", "golden")

C_MUTANTS = {
    "swap_gate_up": ("act[i] = silu(g) * u;", "act[i] = silu(u) * g;"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "down_index": ("s += rg[i] * act[i];", "s += rg[I - 1 - i] * act[i];"),
    "mx_bias": ("sc[r * (cols / 32) + c0 / 32] - 127", "sc[r * (cols / 32) + c0 / 32] - 128"),
    "e2m1_subnormal": ("0.5 * man", "1.0 * man"),
    "dropped_term": ("g += rg[h] * x[h];", "g += (h ? rg[h] * x[h] : 0.0);"),
    "mx_block_row": ("sc[r * (cols / 32) + c0 / 32]", "sc[(r / 2) * (cols / 32) + c0 / 32]"),
    "mx_code_sign": ("val[code] = e2m1_value(code);", "val[code] = e2m1_value(code & 7u);"),
}


def _build_mutant(tmp_path, name, old, new):
    src = open(os.path.join(ROOT, "oracle", "moe_ref.c")).read()
    assert old in src, name
    path = tmp_path / (name + ".c")
    path.write_text(src.replace(old, new))
    so = tmp_path / (name + ".so")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", str(so), str(path), "-lm"])
    lib = ctypes.CDLL(str(so))
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.oracle_expert.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    return lib


def _pins_pass(lib):
    """The numeric pins of tests/test_oracle_moe.py, against a given build."""
    tab = {}
    for line in open(os.path.join(GOLD, "e2m1_values.txt")):
        if line.strip() and not line.startswith("#"):
            c, v = line.split()
            tab[int(c)] = float(v)
    ok = True
    for wfmt in (F32, MXFP4):
        cfg = TINY.with_(H=64, I=32, wdtype=wfmt)
        mats = gen.expert_logical(cfg, 0, 5)
        x = np.random.default_rng(7).normal(size=cfg.H)
        dense, ptrs = [], []
        for n in ("gate", "up", "down"):
            if wfmt == MXFP4:
                codes, scales = mats[n]
                v = np.vectorize(lambda c: tab[int(c)])(codes) * np.exp2(
                    np.repeat(scales.astype(np.int64) - 127, 32, axis=1).astype(np.float64))
                dense.append(v)
                ptrs += [codes.ctypes.data, scales.ctypes.data]
            else:
                dense.append(mats[n].astype(np.float64))
                ptrs += [mats[n].ctypes.data, None]
        y = np.empty(cfg.H)
        act = np.empty(cfg.I)
        lib.oracle_expert(wfmt, cfg.H, cfg.I, *ptrs, x.ctypes.data, y.ctypes.data, act.ctypes.data)
        Wg, Wu, Wd = (torch.from_numpy(d) for d in dense)
        xt = torch.from_numpy(x)
        ref = (Wd @ (torch.nn.functional.silu(Wg @ xt) * (Wu @ xt))).numpy()
        ok &= bool(np.allclose(y, ref, rtol=1e-12, atol=1e-15 * np.abs(ref).max()))
    return ok


def test_unmutated_c_oracle_passes(tmp_path):
    assert _pins_pass(_build_mutant(tmp_path, "none", "return z", "return z"))


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_mutant_is_caught(tmp_path, name):
    old, new = C_MUTANTS[name]
    assert not _pins_pass(_build_mutant(tmp_path, name, old, new))


PY_MUTANTS = {
    "lru_mru_end": ("lru_sim.py", "walk = iter(list(self.recency.keys()))",
                    "walk = iter(list(reversed(self.recency.keys())))"),
    "recency_desc": ("lru_sim.py", "for u, hit in zip(U, is_hit):\n            if hit or u in fills:",
                     "for u, hit in reversed(list(zip(U, is_hit))):\n            if hit or u in fills:"),
    "q_ceil": ("lru_sim.py", "(m * bp) // bh", "-((-m * bp) // bh)"),
    "free_desc": ("lru_sim.py", "v = self.free.pop(0)", "v = self.free.pop()"),
    "fill_last_misses": ("lru_sim.py", "F = M[:q]\n        Hs = M[q:]", "F = M[m - q:]\n        Hs = M[:m - q]"),
    "hit_not_excluded": ("lru_sim.py", "if s not in hit_slots and s not in victims",
                         "if s not in victims"),
    "route_ties_high": ("route.py", "key=lambda i: (-vals[i], i)", "key=lambda i: (-vals[i], -i)"),
    "route_no_shift": ("route.py", "ex = [math.exp(vals[i] - top) for i in order]",
                       "ex = [math.exp(vals[i] - top) for i in order[:1]] + [math.exp(vals[i]) for i in order[1:]]"),
}


def _load_mutant(fname, old, new):
    src = open(os.path.join(ROOT, "oracle", fname)).read()
    assert old in src, (fname, old)
    mod = types.ModuleType("mutant_" + fname.replace(".", "_"))
    mod.__dict__["__package__"] = "oracle"  # relative imports of the oracle package resolve
    exec(compile(src.replace(old, new), fname, "exec"), mod.__dict__)
    return mod


CHAIN_MUTANTS = {
    "bf16_truncate": ("up = (rem > half) | ((rem == half) & ((keep & np.uint64(1)) == np.uint64(1)))",
                      "up = rem > rem"),
    "bf16_ties_away": ("up = (rem > half) | ((rem == half) & ((keep & np.uint64(1)) == np.uint64(1)))",
                       "up = rem >= half"),
    "no_residual": ("nxt = xv + out", "nxt = out"),
    "logits_transposed": ("return x @ w.T", "return x @ w"),
    "margin_shifted": ("margin = srt[:, k - 1] - srt[:, k]", "margin = srt[:, k] - srt[:, k + 1]"),
    "widen_low_half": ("b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)",
                       "b = np.asarray(bits, np.uint16).astype(np.uint32)"),
}


def _chain_pins_pass(mod, tmp_path):
    """The pins of tests/test_oracle_chain.py against a given copy of oracle/chain.py."""
    import tests.test_oracle_chain as T
    saved = T.chain
    T.chain = mod
    try:
        for f in (T.test_bf16_rounding_matches_hand_derived_values, T.test_bf16_round_trip_of_representable_values,
                  T.test_rounding_is_to_the_nearest_bf16, T.test_gate_logits_exact_on_integers_and_brute_force_dot,
                  T.test_gate_logits_linear_in_x, T.test_block_with_zero_down_weights_returns_its_input,
                  T.test_block_routes_on_the_data_and_adds_the_residual):
            f()
        return True
    except Exception:  # a failed pin or a crash both reject the copy
        return False
    finally:
        T.chain = saved


def test_unmutated_chain_oracle_passes(tmp_path):
    assert _chain_pins_pass(_load_mutant("chain.py", "import numpy as np", "import numpy as np"), tmp_path)


@pytest.mark.parametrize("name", sorted(CHAIN_MUTANTS))
def test_chain_mutant_is_caught(name, tmp_path):
    old, new = CHAIN_MUTANTS[name]
    assert not _chain_pins_pass(_load_mutant("chain.py", old, new), tmp_path)


def _lru_pins_pass(mod):
    from oracle.brute_lru import BruteLRU
    g = json.load(open(os.path.join(GOLD, "lru_trace_tiny.json")))
    sim = mod.LRUSim(g["L"], g["E"], g["C"], g["K"], 1000, 1000)
    for s in g["steps"]:
        sim.set_bandwidth(s["bp"], s["bh"])
        r = sim.step(s["layer"], s["ids"])
        for f in ("uniq", "h", "m", "q", "fills", "victims", "host_list", "rewritten"):
            if r[f] != s[f]:
                return False
    try:
        for seed in range(12):
            rng = np.random.default_rng(100 + seed)
            C, K = int(rng.integers(0, 7)), int(rng.integers(1, 5))
            bp, bh = [(1000, 1000), (500, 1000), (300, 1000), (2000, 1000)][seed % 4]
            a, b = mod.LRUSim(2, 8, C, K, bp, bh), BruteLRU(C, K, bp, bh)
            for _ in range(60):
                l = int(rng.integers(0, 2))
                ids = [[int(e) for e in rng.choice(8, size=2, replace=False)]]
                ra, rb = a.step(l, ids), b.step(l, ids)
                if any(ra[f] != rb[f] for f in ("h", "m", "q", "victims", "evicted")):
                    return False
    except StopIteration:
        return False
    return True



def _route_pins_pass(mod):
    for c in json.load(open(os.path.join(GOLD, "route_cases.json")))["cases"]:
        ids, w = mod.route_row(c["logits"], c["k"])
        if ids != c["ids"] or (c["w"] is not None and not np.allclose(w, c["w"], rtol=0, atol=1e-15)):
            return False
    return True


def test_unmutated_py_oracle_passes():
    assert _lru_pins_pass(_load_mutant("lru_sim.py", "HIT", "HIT"))
    assert _route_pins_pass(_load_mutant("route.py", "import math", "import math"))


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_py_mutant_is_caught(name):
    fname, old, new = PY_MUTANTS[name]
    mod = _load_mutant(fname, old, new)
    check = _route_pins_pass if fname == "route.py" else _lru_pins_pass
    try:
        passed = check(mod)
    except Exception:  # a crash is a caught mistake too
        passed = False
    assert not passed
