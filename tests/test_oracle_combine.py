"""Pins for the combine oracle: identity at k=1, a hand-worked exact sum,
and agreement with an fp64 sum rounded to fp16 within one fp16 ulp."""
import numpy as np

from oracle import combine as CB


def test_k1_identity():
    rng = np.random.default_rng(0)
    out = rng.standard_normal((40, 16)).astype(np.float16)
    prow = rng.permutation(40)[:10]
    y = CB.combine(out, prow, 10, 1)
    assert np.array_equal(y.view(np.uint16), out[prow].view(np.uint16))


def test_handworked_sum():
    # 1 + 2^-11 + 2^-11: each addend is an fp16; the fp32 sum is exactly
    # 1 + 2^-10, which fp16 represents; adding in fp16 instead would round
    # 1 + 2^-11 back to 1 twice (ties to even) and give 1.
    out = np.array([[1.0], [2.0 ** -11], [2.0 ** -11], [0.0]], np.float16)
    y = CB.combine(out, [0, 1, 2], 1, 3)
    assert float(y[0, 0]) == 1.0 + 2.0 ** -10
    y0 = CB.combine(out, [3, 3, 3], 1, 3)
    assert float(y0[0, 0]) == 0.0


def test_close_to_fp64():
    rng = np.random.default_rng(1)
    T, k, H = 50, 6, 64
    out = rng.standard_normal((T * k + 7, H)).astype(np.float16)
    prow = rng.permutation(T * k + 7)[:T * k]
    y = CB.combine(out, prow, T, k).astype(np.float64)
    ref = out[prow].astype(np.float64).reshape(T, k, H).sum(axis=1)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -14))) - 10)
    assert np.all(np.abs(y - ref) <= ulp + 1e-6)
