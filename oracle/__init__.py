"""CPU oracle for the k-quant prefill MMQ -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or executes anything here, and this
package imports nothing from the product.

The arithmetic lives in ``qig_oracle.c`` (plain C, fp64 accumulation, built
with gcc -O2 -fopenmp, no fast-math); this module only marshals numpy arrays.
Each wrapped function documents the passage of the minfer optimisation pages
it follows; see the C file for the definitions.  The q4_K block byte layout
is not on those pages (GGUF q4_K restated): parity unpinned against real model
files, pinned only to hand-derived fixtures.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qig_oracle.c")
_LIB = os.path.join(_HERE, "libqig_oracle.so")
_lib = None

_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_i8p = np.ctypeslib.ndpointer(dtype=np.int8, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64


def build() -> str:
    """Compile ``qig_oracle.c`` into ``libqig_oracle.so`` (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-Wall", "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_float_to_half_rne.argtypes = [ctypes.c_float]
    lib.oracle_float_to_half_rne.restype = ctypes.c_uint16
    lib.oracle_quantize_q8_pad40.argtypes = [_f32p, _i64, _i64, _i64, _u8p]
    lib.oracle_quantize_q8_pad40.restype = None
    lib.oracle_q6k_decode.argtypes = [_u8p, _i8p, _i8p, ctypes.POINTER(ctypes.c_double)]
    lib.oracle_q6k_decode.restype = None
    lib.oracle_q4k_decode.argtypes = [_u8p, _u8p, _u8p, _u8p,
                                      ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_double)]
    lib.oracle_q4k_decode.restype = None
    lib.oracle_expand_q6k_dense.argtypes = [_u8p, _i64, _i64, _i64, _i8p]
    lib.oracle_expand_q6k_dense.restype = None
    lib.oracle_q6k_partials.argtypes = [_u8p, _i64, _i64, _i64, _u8p, _i64,
                                        _i64, _i64, _i64, _i64, _i32p]
    lib.oracle_q6k_partials.restype = ctypes.c_int
    lib.oracle_q4k_partials.argtypes = [_u8p, _i64, _i64, _u8p, _i64,
                                        _i64, _i64, _i64, _i64, _i32p]
    lib.oracle_q4k_partials.restype = ctypes.c_int
    lib.oracle_mmq_q6k.argtypes = [_u8p, _i64, _i64, _i64, _u8p, _i64, _f64p]
    lib.oracle_mmq_q6k.restype = None
    lib.oracle_mmq_q4k.argtypes = [_u8p, _i64, _i64, _u8p, _i64, _f64p]
    lib.oracle_mmq_q4k.restype = None
    lib.oracle_mmq_q6k_points.argtypes = [_u8p, _i64, _i64, _i64, _u8p, _i64,
                                          _i64p, _i64p, _i64, _f64p]
    lib.oracle_mmq_q6k_points.restype = None
    lib.oracle_mmq_q4k_points.argtypes = [_u8p, _i64, _i64, _u8p, _i64,
                                          _i64p, _i64p, _i64, _f64p]
    lib.oracle_mmq_q4k_points.restype = None
    lib.oracle_mmq_q6k_from_plane.argtypes = [_i8p, _i64, _i64, _i64, _u8p, _i64, _i64, _i64,
                                              _u8p, _i64, _f64p]
    lib.oracle_mmq_q6k_from_plane.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    _lib = lib
    return lib


def _u8(a):
    return np.ascontiguousarray(a, dtype=np.uint8).reshape(-1)


# --------------------------------------------------------------------------
# fp16
# --------------------------------------------------------------------------
def half_to_double(bits: int) -> float:
    """binary16 bit pattern -> exact double (subnormals kept)."""
    return _load().oracle_half_to_double(int(bits) & 0xFFFF)


def float_to_half_rne(f: float) -> int:
    """float32 -> binary16 bits, round to nearest even (subnormals kept)."""
    return int(_load().oracle_float_to_half_rne(float(np.float32(f))))


# --------------------------------------------------------------------------
# activation quantisation (pad40 blocks; layout from the r20/r21 pages)
# --------------------------------------------------------------------------
def q8_pad40_bytes(nt: int, id_: int) -> int:
    return nt * (id_ // 32) * 40


def quantize_q8_pad40(x: np.ndarray, id_: int | None = None) -> np.ndarray:
    """fp32 x[nt][ldx] -> pad40 plane as uint8[nt * id/32 * 40]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    nt, ldx = x.shape
    id_ = ldx if id_ is None else id_
    out = np.zeros(q8_pad40_bytes(nt, id_), dtype=np.uint8)
    if nt:
        _load().oracle_quantize_q8_pad40(x.reshape(-1), nt, id_, ldx, out)
    return out


def q8_fields(q8: np.ndarray, nt: int, id_: int):
    """Split a pad40 plane into (d_bits u16 [nt,nb32], qs i8 [nt,id], ssum f32
    [nt,nb32], pad u8 [nt,nb32,2]) by the byte offsets of the pad40 block."""
    nb32 = id_ // 32
    b = _u8(q8).reshape(nt, nb32, 40)
    d_bits = b[:, :, 0].astype(np.uint16) | (b[:, :, 1].astype(np.uint16) << 8)
    qs = b[:, :, 4:36].view(np.int8).reshape(nt, id_)
    ssum = np.ascontiguousarray(b[:, :, 36:40]).view(np.float32).reshape(nt, nb32)
    return d_bits, qs, ssum, b[:, :, 2:4]


# --------------------------------------------------------------------------
# weight decoding
# --------------------------------------------------------------------------
def q6k_decode_block(blk: np.ndarray):
    """One block_q6_K -> (c6 int8[256], sc int8[16], d float)."""
    c6 = np.zeros(256, dtype=np.int8)
    sc = np.zeros(16, dtype=np.int8)
    d = ctypes.c_double()
    _load().oracle_q6k_decode(_u8(blk)[:210].copy(), c6, sc, ctypes.byref(d))
    return c6, sc, d.value


def q4k_decode_block(blk: np.ndarray):
    """One block_q4_K -> (q uint8[256], sc uint8[8], m uint8[8], d, dmin)."""
    q = np.zeros(256, dtype=np.uint8)
    sc = np.zeros(8, dtype=np.uint8)
    m = np.zeros(8, dtype=np.uint8)
    d = ctypes.c_double()
    dmin = ctypes.c_double()
    _load().oracle_q4k_decode(_u8(blk)[:144].copy(), q, sc, m, ctypes.byref(d),
                              ctypes.byref(dmin))
    return q, sc, m, d.value, dmin.value


def expand_q6k_dense(W: np.ndarray, bstride: int, od: int, id_: int) -> np.ndarray:
    """Padded raw q6_K plane -> dense centred int8 plane W_exp[od][id]."""
    out = np.zeros((od, id_), dtype=np.int8)
    if od:
        _load().oracle_expand_q6k_dense(_u8(W), bstride, od, id_, out.reshape(-1))
    return out


# --------------------------------------------------------------------------
# partials and GEMM
# --------------------------------------------------------------------------
def q6k_partials(W, bstride, od, id_, q8, nt, t0, t1, j0, j1) -> np.ndarray:
    """int32 P6[t1-t0][j1-j0][16*nsb] (sub-blocks of 16)."""
    P = np.zeros((t1 - t0, j1 - j0, 16 * (id_ // 256)), dtype=np.int32)
    rc = _load().oracle_q6k_partials(_u8(W), bstride, od, id_, _u8(q8), nt,
                                     t0, t1, j0, j1, P.reshape(-1))
    assert rc == 0, "q6_K partial overflowed int32"
    return P


def q4k_partials(W, od, id_, q8, nt, t0, t1, j0, j1) -> np.ndarray:
    """int32 P4[t1-t0][j1-j0][8*nsb] (sub-blocks of 32)."""
    P = np.zeros((t1 - t0, j1 - j0, 8 * (id_ // 256)), dtype=np.int32)
    rc = _load().oracle_q4k_partials(_u8(W), od, id_, _u8(q8), nt,
                                     t0, t1, j0, j1, P.reshape(-1))
    assert rc == 0, "q4_K partial overflowed int32"
    return P


def mmq_q6k(W, bstride, od, id_, q8, nt) -> np.ndarray:
    """fp64 y[nt][od] of q6_K weights times the pad40 plane."""
    y = np.zeros((nt, od), dtype=np.float64)
    if nt and od:
        _load().oracle_mmq_q6k(_u8(W), bstride, od, id_, _u8(q8), nt, y.reshape(-1))
    return y


def mmq_q4k(W, od, id_, q8, nt) -> np.ndarray:
    """fp64 y[nt][od] of q4_K weights times the pad40 plane."""
    y = np.zeros((nt, od), dtype=np.float64)
    if nt and od:
        _load().oracle_mmq_q4k(_u8(W), od, id_, _u8(q8), nt, y.reshape(-1))
    return y


def mmq_q6k_points(W, bstride, od, id_, q8, nt, tt, jj) -> np.ndarray:
    tt = np.ascontiguousarray(tt, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    out = np.zeros(len(tt), dtype=np.float64)
    _load().oracle_mmq_q6k_points(_u8(W), bstride, od, id_, _u8(q8), nt, tt, jj,
                                  len(tt), out)
    return out


def mmq_q4k_points(W, od, id_, q8, nt, tt, jj) -> np.ndarray:
    tt = np.ascontiguousarray(tt, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    out = np.zeros(len(tt), dtype=np.float64)
    _load().oracle_mmq_q4k_points(_u8(W), od, id_, _u8(q8), nt, tt, jj, len(tt), out)
    return out


def mmq_q6k_from_plane(plane, row_stride, sb_stride, W, bstride, od, id_, q8, nt) -> np.ndarray:
    """q6_K GEMM reading the quants from a dense plane at the given strides
    (scales and d from W); see the C function for the mutant it models."""
    plane = np.ascontiguousarray(plane, dtype=np.int8).reshape(-1)
    y = np.zeros((nt, od), dtype=np.float64)
    _load().oracle_mmq_q6k_from_plane(plane, plane.size, row_stride, sb_stride, _u8(W), bstride,
                                      od, id_, _u8(q8), nt, y.reshape(-1))
    return y


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count of later oracle calls (0 restores the default)."""
    _load().oracle_set_num_threads(int(n))


def within_tolerance(y: np.ndarray, y_ref: np.ndarray, rms: float | None = None,
                     rel: float = 1e-4, floor: float = 1e-3):
    """Per-element check |y - y_ref| <= max(rel*|y_ref|, floor*rms(y_ref)).

    Returns (ok, worst_ratio) where worst_ratio is the largest error divided by
    its allowance (<= 1 passes)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if rms is None:
        rms = float(np.sqrt(np.mean(y_ref * y_ref))) if y_ref.size else 0.0
    allow = np.maximum(rel * np.abs(y_ref), floor * rms)
    err = np.abs(y - y_ref)
    if err.size == 0:
        return True, 0.0
    ratio = np.where(allow > 0, err / np.where(allow > 0, allow, 1.0),
                     np.where(err > 0, np.inf, 0.0))
    worst = float(np.max(ratio))
    return worst <= 1.0, worst
