"""Expert-bank files: write, parallel (direct) read, validation. Host only, no GPU."""
import numpy as np
import pytest

import gen
from gen.configs import BF16, TINY

import expert_cached_decode_amd as E


def _aligned(nbytes, offset=0):
    raw = np.empty(nbytes + 8192, np.uint8)
    start = (-raw.ctypes.data) % 4096 + offset
    return raw[start:start + nbytes]


def _shape(cfg):
    return E.make_shape(cfg.L, cfg.E, cfg.k, cfg.H, cfg.I, cfg.wdtype)


@pytest.mark.parametrize("offset", [0, 64], ids=["aligned", "unaligned"])
def test_round_trip_several_chunks_and_a_tail(tmp_path, offset):
    # 16 bf16 experts of 1024 x 512: 50 MB, more than one 32 MiB read chunk plus a tail
    cfg = TINY.with_(L=2, E=16, k=2, H=1024, I=512, wdtype=BF16)
    bank = gen.pool_array(cfg, 0, 1)
    path = str(tmp_path / "bank.ecb")
    E.bank_write(path, _shape(cfg), 1, bank.ctypes.data, bank.nbytes)
    dst = _aligned(bank.nbytes, offset)
    sec, direct = E.bank_read(path, _shape(cfg), 1, dst.ctypes.data, dst.nbytes, threads=4)
    assert np.array_equal(dst, bank)
    if offset:
        assert direct != 1
    assert sec > 0


def test_every_pool_layer_lands_in_place(tmp_path):
    cfg = TINY.with_(L=3)
    bank = gen.pool_array(cfg, 0, 3)
    path = str(tmp_path / "b.ecb")
    E.bank_write(path, _shape(cfg), 3, bank.ctypes.data, bank.nbytes)
    dst = _aligned(bank.nbytes)
    E.bank_read(path, _shape(cfg), 3, dst.ctypes.data, dst.nbytes, threads=3)
    assert np.array_equal(dst, bank)


def test_shape_size_and_format_checks(tmp_path):
    cfg = TINY.with_(L=2)
    bank = gen.pool_array(cfg, 0, 2)
    path = str(tmp_path / "b.ecb")
    E.bank_write(path, _shape(cfg), 2, bank.ctypes.data, bank.nbytes)
    dst = _aligned(bank.nbytes)
    with pytest.raises(E.ECError) as ei:  # another shape
        E.bank_read(path, _shape(cfg.with_(I=64)), 2, dst.ctypes.data, dst.nbytes)
    assert ei.value.status == -2
    with pytest.raises(E.ECError) as ei:  # another layer count
        E.bank_read(path, _shape(cfg), 1, dst.ctypes.data, dst.nbytes)
    assert ei.value.status == -2
    with pytest.raises(E.ECError) as ei:  # destination too small
        E.bank_read(path, _shape(cfg), 2, dst.ctypes.data, dst.nbytes - 1)
    assert ei.value.status == -3
    raw = open(path, "rb").read()
    bad = str(tmp_path / "bad.ecb")
    open(bad, "wb").write(b"NOTABANK" + raw[8:])
    with pytest.raises(E.ECError) as ei:
        E.bank_read(path.replace("b.ecb", "bad.ecb"), _shape(cfg), 2, dst.ctypes.data, dst.nbytes)
    assert ei.value.status == -2
    trunc = str(tmp_path / "trunc.ecb")
    open(trunc, "wb").write(raw[:4096 + bank.nbytes // 2])
    with pytest.raises(E.ECError) as ei:
        E.bank_read(trunc, _shape(cfg), 2, dst.ctypes.data, dst.nbytes)
    assert ei.value.status == -1
    with pytest.raises(E.ECError):
        E.bank_write(path, _shape(cfg), 3, bank.ctypes.data, bank.nbytes)  # P > layers
