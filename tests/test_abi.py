"""The C-ABI library loads on the CPU, exports every declared entry point, and
its host-only calls (layout, workspace sizing, argument checks) behave as the
header states. No device compute runs here."""
import ctypes
import os
import re

import pytest

import gen
from gen.configs import ALL, MXFP4

import expert_cached_decode_amd as E
from expert_cached_decode_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "ec_api.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "moe_decode_layer" in names and "cache_rebuild" in names and len(names) >= 16
    lib = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(B.EXPORTS)


@pytest.mark.parametrize("cfg", ALL, ids=lambda c: c.name)
def test_layout_matches_expert_bank(cfg):
    lay = E.layout(E.make_shape(cfg.L, cfg.E, cfg.k, cfg.H, cfg.I, cfg.wdtype))
    assert lay.expert_bytes == cfg.expert_bytes == gen.expert_bytes(cfg.wdtype, cfg.H, cfg.I)
    assert lay.layer_bytes == cfg.E * cfg.expert_bytes
    n = cfg.H * cfg.I
    if cfg.wdtype == MXFP4:
        assert (lay.up_off, lay.down_off, lay.gate_scale_off) == (n // 2, n, 3 * n // 2)
        assert (lay.up_scale_off, lay.down_scale_off) == (3 * n // 2 + n // 32, 3 * n // 2 + n // 16)


def test_layout_bytes_of_the_pages_workloads():
    # expert bytes: bf16 3*2048*512*2; MXFP4 codes + E8M0 scales for 4096 x 2048
    assert E.layout(E.make_shape(40, 256, 8, 2048, 512, 1)).layer_bytes * 40 == 64424509440
    assert E.layout(E.make_shape(43, 256, 6, 4096, 2048, 2)).expert_bytes == 13369344


def _cfg(**kw):
    d = dict(L=2, E=16, k=2, H=256, I=128, wd=0, T=1, C=8, K=0, bp=1000, bh=1000, thr=0, pre=0)
    d.update(kw)
    return B.ec_config(B.make_shape(d["L"], d["E"], d["k"], d["H"], d["I"], d["wd"]), d["T"], d["C"], d["K"],
                       d["bp"], d["bh"], d["thr"], d["pre"])


def test_workspace_size_and_argument_errors():
    dev, pin = E.workspace_size(_cfg())
    assert dev > 0 and pin > 0
    dev2, _ = E.workspace_size(_cfg(pre=512, wd=1))
    assert dev2 > dev
    bad = [dict(bh=0), dict(C=33), dict(K=65), dict(T=0), dict(T=65), dict(k=17, E=16), dict(H=100),
           dict(E=5000), dict(wd=3), dict(pre=16), dict(T=64, k=32, E=64)]
    codes = []
    for kw in bad:
        with pytest.raises(E.ECError) as ei:
            E.workspace_size(_cfg(**kw))
        codes.append(ei.value.status)
    assert set(codes) <= {-1, -2, -6}
    assert B.lib().ec_strerror(-3) == b"caller buffer too small"


def test_route_argument_checks_enqueue_nothing():
    lib = B.lib()
    assert lib.moe_route(None, 0, 16, 2, None, None, None) == 0   # T = 0: nothing to do
    assert lib.moe_route(None, 1, 16, 17, None, None, None) == -1 # k > E
    assert lib.moe_route(None, 1, 16, 2, None, None, None) == -1  # NULL pointers
    assert lib.ec_destroy(None) == -1
    assert lib.ec_epoch(None) == 0


def test_calibration_rejects_a_null_context():
    lib = E.lib()
    assert lib.ec_calibrate_bandwidth(None, 8, 1, None, None) == -1


def test_last_step_rejects_null_arguments():
    lib = E.lib()
    v = B.ec_step_view()
    assert lib.ec_last_step(None, ctypes.byref(v)) == -1
    assert lib.ec_last_step(None, None) == -1


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: any other --gpus (or a multi-rank launch) exits with a message
    before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py")], capture_output=True, text=True,
                       timeout=120, env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr
