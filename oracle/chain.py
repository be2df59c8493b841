"""Chained MoE decode block: router logits computed from the data, and the residual.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Definition. A token's router scores every expert of the layer (FreeToken
write-up, "Why personal MoE is hard": k of E experts are routed per token), the
decode layer is the exact MoE of "Bandwidth-adaptive execution", and the block
adds its output to its input, so the sum is the next layer's input:
    logits = W_r x                         (fp64; the top-k decision is then taken
                                            on the fp64 value rounded to fp32, the
                                            precision the kernel decides in)
    x_next = round(x + moe(x; logits))     (one rounding, to bf16 RNE or to f32)

Pins (tests/test_oracle_chain.py): integer-valued W_r and x give exact logits;
doubling x doubles the logits exactly; a brute-force Python dot on a tiny case;
bf16 rounding against values derived by hand from the IEEE round-to-nearest-even
rule (tests/golden/bf16_rne.txt); zero down-projection weights leave x unchanged
bit for bit.
"""
import numpy as np

from . import moe as _moe


def gate_logits(w_router, x):
    """fp64 logits [T, E] = x [T, H] . W_r[E, H]^T (both already widened to fp64)."""
    w = np.asarray(w_router, np.float64)
    x = np.asarray(x, np.float64)
    return x @ w.T


def round_bf16(v):
    """fp64 values -> bf16 bit patterns (uint16), round to nearest, ties to even, in one step
    from the fp64 value. Finite normal bf16 results only (asserted); zeros keep their sign."""
    v = np.asarray(v, np.float64)
    bits = v.view(np.uint64)
    sign = (bits >> np.uint64(63)).astype(np.uint64)
    exp = ((bits >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    mant = bits & np.uint64((1 << 52) - 1)
    zero = (exp == 0) & (mant == 0)
    e_b = exp - 1023 + 127
    assert np.all(zero | ((e_b >= 1) & (e_b <= 254))), "value outside the bf16 normal range"
    keep = mant >> np.uint64(45)                    # 7 stored mantissa bits
    rem = mant & np.uint64((1 << 45) - 1)
    half = np.uint64(1 << 44)
    up = (rem > half) | ((rem == half) & ((keep & np.uint64(1)) == np.uint64(1)))
    mag = (e_b.astype(np.uint64) << np.uint64(7)) + keep + up.astype(np.uint64)  # carry into the exponent
    out = np.where(zero, np.uint64(0), mag) | (sign << np.uint64(15))
    return out.astype(np.uint16)


def widen_bf16(bits):
    """bf16 bit patterns -> exact fp64 values."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def block(wfmt, x, w_router, k, get_expert):
    """One chained block for the token rows of x.

    wfmt: expert weight format (moe.F32, BF16 or MXFP4); the token stream x and W_r are f32
    when wfmt is F32 (x given as float32) and bf16 bit patterns otherwise.
    Returns (x_next in the stream's representation, ids, w, margin) where margin[t] is the gap
    between the k-th and (k+1)-th largest fp32 logit (how far the top-k set is from a tie)."""
    f32 = wfmt == _moe.F32
    xv = np.asarray(x, np.float64) if f32 else widen_bf16(x)
    wv = np.asarray(w_router, np.float64) if f32 else widen_bf16(w_router)
    l64 = gate_logits(wv, xv)
    l32 = l64.astype(np.float32)
    out, ids, ws = _moe.moe_tokens(wfmt, xv, l32, k, get_expert)
    nxt = xv + out
    x_next = nxt.astype(np.float32) if f32 else round_bf16(nxt)
    srt = -np.sort(-l32.astype(np.float64), axis=1)
    margin = srt[:, k - 1] - srt[:, k] if l32.shape[1] > k else np.full(len(l32), np.inf)
    return x_next, ids, ws, margin
