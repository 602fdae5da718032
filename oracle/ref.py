"""ctypes front end of the C oracle (``moe_ref.c``).

TEST INFRASTRUCTURE ONLY.  Arrays are numpy; fp16 tensors travel as their
uint16 bit patterns.  The computation itself lives in the C file (see its
header for what it follows on the pages); this module only marshals.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f32p = ctypes.POINTER(ctypes.c_float)
        i32p = ctypes.POINTER(ctypes.c_int32)
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_moe_row.argtypes = [u16p, u16p, u16p, u16p, ctypes.c_float, ctypes.c_int64,
                                     ctypes.c_int64, u16p, u16p, f32p]
        L.oracle_moe_row.restype = None
        L.oracle_moe_forward.argtypes = [u16p, u16p, u16p, u16p, f32p, i32p, i32p, i32p, i32p,
                                         ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, u16p,
                                         u16p, f32p, ctypes.c_int32]
        L.oracle_moe_forward.restype = ctypes.c_int64
        pp = ctypes.POINTER(ctypes.c_void_p)
        L.oracle_moe_rows.argtypes = [ctypes.c_int64, pp, pp, pp, pp, f32p, ctypes.c_int64,
                                      ctypes.c_int64, u16p, u16p, f32p, ctypes.c_int32]
        L.oracle_moe_rows.restype = None
        _lib = L
    return _lib


def _threads(n_threads):
    if n_threads is None:
        n_threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    return max(1, int(n_threads))


def _p(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return a


def f32_to_f16_bits(v: float) -> int:
    return int(lib().oracle_f32_to_f16(ctypes.c_float(v)))


def f16_bits_to_f32(b: int) -> float:
    return float(lib().oracle_f16_to_f32(ctypes.c_uint16(b)))


def moe_forward(x_stacked, wg, wu, wd, w_compact, group_sizes, group_offsets,
                group_padded_offsets, group_idx_for_bx, hid, out, n_threads=None) -> int:
    """Oracle forward over the padded layout.  ``hid`` [Tp, I] and ``out``
    [Tp, H] are fp16 (or uint16) numpy arrays updated in place; rows that no
    block computes keep whatever they held.  Returns rows computed."""
    x = _u16(x_stacked)
    wg, wu, wd = _u16(wg), _u16(wu), _u16(wd)
    E, I, H = wg.shape
    assert wu.shape == (E, I, H) and wd.shape == (E, H, I) and x.shape[1] == H
    hv, ov = hid.view(np.uint16), out.view(np.uint16)
    assert hv.flags.c_contiguous and ov.flags.c_contiguous
    assert hv.shape == (x.shape[0], I) and ov.shape == (x.shape[0], H)
    wc = np.ascontiguousarray(w_compact, dtype=np.float32)
    gs = np.ascontiguousarray(group_sizes, dtype=np.int32)
    go = np.ascontiguousarray(group_offsets, dtype=np.int32)
    gpo = np.ascontiguousarray(group_padded_offsets, dtype=np.int32)
    gidx = np.ascontiguousarray(group_idx_for_bx, dtype=np.int32)
    M = gidx.shape[0]
    assert M * 128 <= x.shape[0]
    nt = _threads(n_threads)
    scratch = np.empty(nt * max(I, 1), dtype=np.float32)
    return int(lib().oracle_moe_forward(
        _p(x, ctypes.c_uint16), _p(wg, ctypes.c_uint16), _p(wu, ctypes.c_uint16),
        _p(wd, ctypes.c_uint16), _p(wc, ctypes.c_float), _p(gs, ctypes.c_int32),
        _p(go, ctypes.c_int32), _p(gpo, ctypes.c_int32), _p(gidx, ctypes.c_int32), M, H, I,
        _p(hv, ctypes.c_uint16), _p(ov, ctypes.c_uint16), _p(scratch, ctypes.c_float), nt))


def moe_rows(x_rows, wg_list, wu_list, wd_list, weights, n_threads=None):
    """Oracle for a list of rows with their own expert slices.  Each x_rows[j]
    is [H] fp16, wg_list[j]/wu_list[j] [I, H], wd_list[j] [H, I].  Returns
    (hid [n, I] fp16, out [n, H] fp16)."""
    n = len(x_rows)
    keep = []
    xs = [_u16(a) for a in x_rows]
    gs = [_u16(a) for a in wg_list]
    us = [_u16(a) for a in wu_list]
    ds = [_u16(a) for a in wd_list]
    keep += xs + gs + us + ds
    if n == 0:
        return np.zeros((0, 0), np.float16), np.zeros((0, 0), np.float16)
    I, H = gs[0].shape
    for j in range(n):
        assert xs[j].shape == (H,) and gs[j].shape == (I, H) and us[j].shape == (I, H)
        assert ds[j].shape == (H, I)

    def ptrs(lst):
        arr = (ctypes.c_void_p * n)(*[a.ctypes.data for a in lst])
        return ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p)), arr

    px, kx = ptrs(xs)
    pg, kg = ptrs(gs)
    pu, ku = ptrs(us)
    pd, kd = ptrs(ds)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    hid = np.zeros((n, I), np.uint16)
    out = np.zeros((n, H), np.uint16)
    nt = _threads(n_threads)
    scratch = np.empty(nt * I, dtype=np.float32)
    lib().oracle_moe_rows(n, px, pg, pu, pd, _p(w, ctypes.c_float), H, I,
                          _p(hid, ctypes.c_uint16), _p(out, ctypes.c_uint16),
                          _p(scratch, ctypes.c_float), nt)
    del keep, kx, kg, ku, kd
    return hid.view(np.float16), out.view(np.float16)
