"""Pins the oracle's hand-written binary16 conversions to numpy's IEEE
conversions (a library routine): exhaustive over binary16, and over the
rounding boundaries of fp32 -> fp16 (ties to even, subnormals, overflow)."""
import ctypes

import numpy as np


def _to_f32_all(L):
    out = np.empty(65536, np.float32)
    for b in range(65536):
        out[b] = L.oracle_f16_to_f32(ctypes.c_uint16(b))
    return out


def test_f16_to_f32_exhaustive(oracle_lib):
    got = _to_f32_all(oracle_lib)
    want = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def _round(L, vals):
    return np.array([L.oracle_f32_to_f16(ctypes.c_float(float(v))) for v in vals], np.uint16)


def _check(L, vals):
    vals = np.asarray(vals, np.float32)
    got = _round(L, vals)
    want = vals.astype(np.float16).view(np.uint16)
    nan = np.isnan(vals)
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)
    bad = np.nonzero(got[~nan] != want[~nan])[0]
    assert bad.size == 0, (vals[~nan][bad[:5]], got[~nan][bad[:5]], want[~nan][bad[:5]])


def test_f32_to_f16_exact_values(oracle_lib):
    every = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    _check(oracle_lib, every)


def test_f32_to_f16_ties_and_neighbours(oracle_lib):
    # midpoints between consecutive finite positive binary16 values, and the
    # fp32 values one ulp either side of each midpoint
    pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)    # exact in fp32
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    vals = np.concatenate([mids, up, dn])
    _check(oracle_lib, vals)
    _check(oracle_lib, -vals)


def test_f32_to_f16_specials_and_random(oracle_lib):
    specials = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 65504.0, 65519.99, 65520.0,
                         1e9, -1e9, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26,
                         2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -11), 1e-45, 3e-38, 1.0, -1.0,
                         np.float32(2.0) ** -149], np.float32)
    _check(oracle_lib, specials)
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=40000, dtype=np.uint64).astype(np.uint32)
    _check(oracle_lib, bits.view(np.float32))
    # dense sampling of the exponent range fp16 cares about
    v = (rng.standard_normal(40000) * np.exp2(rng.uniform(-27, 17, 40000))).astype(np.float32)
    _check(oracle_lib, v)
