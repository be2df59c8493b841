"""The decode host branch (host_pool_run: SwiGLU experts on host cores) on the CPU, against the
oracle, through the test driver tests/host_branch/harness.cpp built with g++ (no GPU).

FreeToken edge-MoE write-up, "Bandwidth-adaptive execution" (decode): misses that are not filled
run on the CPU; their partial sums enter the same exact merge as the GPU's. Each partial sum
y[t, :, j] (host-side pair j of token t, before its routing weight) must equal the oracle's
f_e(x_t) within 1e-2 relative error per row, on both instruction paths of the host code:
the AVX-512 BF16 dot unit (bf16 and MXFP4 rows; activations rounded to bf16 as on the GPU) and
the AVX2 path (f32 activations; forced with -DEC_HOST_NO_BF16_DOT), including MXFP4 rows whose
scales fall outside the range the bf16 path handles exactly (those rows take the AVX2 path on a
BF16 host). The same jobs run under ThreadSanitizer and under AddressSanitizer +
UndefinedBehaviorSanitizer: every job is run several times back to back on one worker pool
(spinning workers, as in decode), and every run must give bit-identical sums and leave the
GPU-side pairs' entries untouched (harness.cpp checks both).
"""
import os
import subprocess

import numpy as np
import pytest

import gen
from gen.configs import DSV4_DECODE, F32, QWEN_DECODE, TINY
from oracle import moe as oracle_moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "expert_cached_decode_amd", "csrc")
HARNESS = os.path.join(ROOT, "tests", "host_branch", "harness.cpp")
BASE = ["g++", "-std=c++17", "-mavx2", "-mfma", "-mf16c", "-pthread", "-I", CSRC]
VARIANTS = {
    "native": ["-O2"],
    "avx2": ["-O2", "-DEC_HOST_NO_BF16_DOT"],
    "tsan": ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=thread"],
    "asan_ubsan": ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                   "-fno-sanitize-recover=all"],
}


def host_has_bf16_dot():
    try:
        flags = open("/proc/cpuinfo").read()
    except OSError:
        return False
    return all(f in flags for f in ("avx512f", "avx512bw", "avx512_bf16"))


@pytest.fixture(scope="module")
def drivers(tmp_path_factory):
    d = tmp_path_factory.mktemp("host_branch")
    out = {}
    for name, flags in VARIANTS.items():
        exe = str(d / ("harness_" + name))
        r = subprocess.run(BASE + flags + [HARNESS, os.path.join(CSRC, "host_experts.cpp"), "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        out[name] = exe
    return out


def make_case(cfg, E_bank, T, host_of, rng, bad_scale_expert=None):
    """One layer step: a bank of E_bank experts (layer 0), tokens x, and rewritten ids where
    host_of[t][j] is the bank expert of a host-side pair or None for a GPU-side pair (slot id)."""
    c = cfg.with_(E=E_bank)
    bank = gen.pool_array(c, 0, 1)
    eb = c.expert_bytes
    mats = {e: gen.expert_logical(c, 0, e) for e in range(E_bank)}
    if bad_scale_expert is not None:
        # scales outside [2, 252] in gate row 0 (block 1) and down row 0 (block 0), in the bank and
        # in the logical matrices alike: those rows cannot use the exact bf16 exponent shift
        e = bad_scale_expert
        H, I = c.H, c.I
        base = e * eb + 3 * I * H // 2
        bank[base + 1] = 1
        mats[e]["gate"][1][0, 1] = 1
        bank[base + 2 * I * (H // 32)] = 1
        mats[e]["down"][1][0, 0] = 1
    k = len(host_of[0])
    x = gen.decode_x(c, 7, 0, T=T)
    hosts = []
    rw = np.empty((T, k), np.int32)
    for t in range(T):
        for j in range(k):
            e = host_of[t][j]
            if e is None:
                rw[t, j] = int(rng.integers(0, 100))
            else:
                if e not in hosts:
                    hosts.append(e)
                rw[t, j] = -(1 + hosts.index(e))
    return dict(cfg=c, bank=bank, x=x, rw=rw, hosts=hosts, mats=mats, T=T, k=k)


def write_input(case, path, reps):
    c = case["cfg"]
    hdr = np.array([case["T"], case["k"], c.H, c.I, c.wdtype, len(case["hosts"]), c.E, c.expert_bytes, reps],
                   np.int64)
    with open(path, "wb") as f:
        f.write(hdr.tobytes())
        f.write(np.array(case["hosts"], np.int32).tobytes())
        f.write(case["rw"].tobytes())
        f.write(np.ascontiguousarray(case["x"]).tobytes())
        f.write(case["bank"].tobytes())


def run_driver(exe, case, tmp_path, threads, reps):
    inp, outp = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    write_input(case, inp, reps)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1", ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe, inp, outp, str(threads)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.returncode, r.stderr[-3000:])
    assert "WARNING: ThreadSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
    c = case["cfg"]
    return np.fromfile(outp, np.float32).reshape(case["T"], c.H, case["k"])


def check_against_oracle(case, y, tol=1e-2):
    c = case["cfg"]
    xs = case["x"].astype(np.float64) if c.wdtype == F32 else gen.bf16_to_f32(case["x"]).astype(np.float64)
    ref = {}
    worst = 0.0
    for t in range(case["T"]):
        for j in range(case["k"]):
            r = int(case["rw"][t, j])
            if r >= 0:
                continue
            e = case["hosts"][-r - 1]
            if (e, t) not in ref:
                ref[(e, t)] = oracle_moe.expert(c.wdtype, case["mats"][e], xs[t])
            want = ref[(e, t)]
            got = y[t, :, j].astype(np.float64)
            err = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
            # and element by element against the row's largest magnitude, so that a mistake
            # confined to a few elements of a row (one scale block, one row of a matrix) shows
            el = np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-30)
            worst = max(worst, err, el)
            assert err <= tol and el <= tol, (t, j, e, err, el)
    return worst


def cases():
    rng = np.random.default_rng(2026)
    N = None
    qwen = make_case(QWEN_DECODE, 6, 5, [[0, 1, N, 2, N, 3, 4, N], [1, N, 5, N, 0, N, N, 2],
                                         [N, N, N, N, N, N, N, 3], [N] * 8, [5, 4, 3, 2, 1, 0, N, N]], rng)
    mx = make_case(DSV4_DECODE, 4, 2, [[0, N, 1, 2, N, 3], [N, 2, N, N, 0, N]], rng, bad_scale_expert=2)
    f32 = make_case(TINY.with_(H=256, I=128, k=3), 5, 3, [[0, 1, N], [N, 4, 0], [2, N, 3]], rng)
    return {"bf16_qwen_shapes": qwen, "mxfp4_dsv4_shapes": mx, "f32_tiny": f32}


@pytest.fixture(scope="module")
def all_cases():
    return cases()


@pytest.mark.parametrize("variant", ["native", "avx2"])
def test_host_branch_matches_oracle(drivers, all_cases, tmp_path, variant):
    if variant == "native" and not host_has_bf16_dot():
        pytest.skip("this host has no AVX-512 BF16 unit: the native build takes the AVX2 path")
    for name, case in all_cases.items():
        y = run_driver(drivers[variant], case, tmp_path, threads=6, reps=3)
        check_against_oracle(case, y)


def test_paths_differ_where_they_should(drivers, all_cases, tmp_path):
    """On a BF16 host the bf16-dot build rounds the SwiGLU activations to bf16 and the AVX2 build
    does not: bf16 results differ in the last bits (both within tolerance of the oracle), f32
    weights take one path in both builds and agree bit for bit."""
    if not host_has_bf16_dot():
        pytest.skip("needs an AVX-512 BF16 host")
    c = all_cases["bf16_qwen_shapes"]
    a = run_driver(drivers["native"], c, tmp_path, threads=3, reps=1)
    b = run_driver(drivers["avx2"], c, tmp_path, threads=3, reps=1)
    host = c["rw"] < 0
    assert not np.array_equal(a.transpose(0, 2, 1)[host], b.transpose(0, 2, 1)[host])
    f = all_cases["f32_tiny"]
    a = run_driver(drivers["native"], f, tmp_path, threads=2, reps=1)
    b = run_driver(drivers["avx2"], f, tmp_path, threads=2, reps=1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("variant", ["tsan", "asan_ubsan"])
def test_host_branch_under_sanitizers(drivers, all_cases, tmp_path, variant):
    for name in ("bf16_qwen_shapes", "mxfp4_dsv4_shapes", "f32_tiny"):
        case = all_cases[name]
        y = run_driver(drivers[variant], case, tmp_path, threads=8, reps=4)
        check_against_oracle(case, y)
