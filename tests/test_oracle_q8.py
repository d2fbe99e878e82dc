"""Pins for the oracle's fp16 codec and pad40 activation quantizer (CPU only).

The pad40 block layout follows the r21 page ('Coalesced block-linear A
staging', s2.1) and the r20 page ('Split-phase A staging', s3.2 addressing);
the fill rule is the reading recorded with the oracle.  Pins: numpy's IEEE
binary16 conversion (a library routine), hand-derived blocks, and invariants
that any correct quantizer must satisfy.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_half_to_double_all_patterns(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_mod.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros and subnormals keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_float_to_half_rne_matches_numpy(oracle_mod):
    g = np.random.Generator(np.random.PCG64(7))
    vals = np.concatenate([
        g.standard_normal(4000).astype(np.float32) * np.float32(10.0) ** g.integers(-9, 6, 4000).astype(np.float32),
        # values on and around rounding ties of the fp16 grid, incl. subnormal range
        (np.arange(-3000, 3000, dtype=np.float32) * np.float32(2.0 ** -25)),
        (np.arange(1, 4000, dtype=np.float32) * np.float32(0.5) + np.float32(2048.0)),
        np.array([65504.0, 65519.996, 65520.0, 65536.0, 1e30, -65520.0, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -26, 0.0, -0.0], dtype=np.float32),
    ])
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle_mod.float_to_half_rne(v) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def _load_cases():
    with open(os.path.join(GOLDEN, "q8_pad40_handbuilt.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_cases(), ids=lambda c: c["name"])
def test_quantize_handbuilt_blocks(oracle_mod, case):
    x = np.zeros((1, 32), dtype=np.float32)
    for k, v in case["x"].items():
        x[0, int(k)] = np.float32(v)
    blk = oracle_mod.quantize_q8_pad40(x)
    assert blk.size == 40
    d_bits = int(blk[0]) | (int(blk[1]) << 8)
    assert d_bits == int(case["d_bits"], 16)
    assert blk[2] == 0 and blk[3] == 0
    qs = blk[4:36].view(np.int8)
    want = np.zeros(32, dtype=np.int8)
    for k, v in case["qs"].items():
        want[int(k)] = v
    assert np.array_equal(qs, want), (qs, want)
    ssum_bits = int(blk[36:40].view(np.uint32)[0])
    assert ssum_bits == int(case["ssum_bits"], 16)


def _random_planes():
    g = np.random.Generator(np.random.PCG64(11))
    nt, id_ = 9, 96
    planes = [
        g.standard_normal((nt, id_), dtype=np.float32),
        (g.standard_t(2.0, size=(nt, id_))).astype(np.float32) * np.float32(3.0),
        g.standard_normal((nt, id_), dtype=np.float32) * np.float32(1e-6),   # fp16-subnormal d
        np.round(g.standard_normal((nt, id_)) * 40).astype(np.float32),     # integer inputs, many ties
    ]
    z = g.standard_normal((nt, id_), dtype=np.float32)
    z[::2, :32] = 0.0                                                        # whole chunks of zeros
    planes.append(z)
    return planes


@pytest.mark.parametrize("pi", range(5))
def test_quantize_invariants(oracle_mod, pi):
    x = _random_planes()[pi]
    nt, id_ = x.shape
    nb32 = id_ // 32
    q8 = oracle_mod.quantize_q8_pad40(x)
    d_bits, qs, ssum, pad = oracle_mod.q8_fields(q8, nt, id_)
    assert np.all(pad == 0)
    xc = x.reshape(nt, nb32, 32)
    qc = qs.reshape(nt, nb32, 32).astype(np.int64)
    amax = np.max(np.abs(xc), axis=2)
    d32 = amax / np.float32(127.0)                       # IEEE fp32 division (numpy)
    # stored d is fp16(d32), round to nearest even (numpy's IEEE conversion)
    assert np.array_equal(d_bits, d32.astype(np.float16).view(np.uint16))
    assert np.all(np.abs(qc) <= 127)
    nz = d32 > 0
    # the largest magnitude always maps to +-127
    assert np.all(np.max(np.abs(qc), axis=2)[nz] == 127)
    assert np.all(qc[~nz] == 0)
    # reconstruction error at most half a step plus the rounding of x/d
    # (|x/d| < 128, so one fp32 ulp is at most 2^-16)
    err = np.abs(xc.astype(np.float64) - d32[..., None].astype(np.float64) * qc)
    lim = d32[..., None].astype(np.float64) * (0.5 + 2.0 ** -16)
    assert np.all(err[nz] <= lim[nz] + 0.0)
    # ssum carries sum(q) exactly: ssum / d_fp16 == sum(q)
    dh = d_bits.view(np.float16).astype(np.float64)
    s = qc.sum(axis=2)
    assert np.array_equal(ssum.astype(np.float64), dh * s)


def test_quantize_matches_ieee_recomputation(oracle_mod):
    # Independent re-derivation with numpy's IEEE fp32 division and exact
    # float64 round-half-away; catches offset and indexing mistakes.
    for x in _random_planes():
        nt, id_ = x.shape
        nb32 = id_ // 32
        q8 = oracle_mod.quantize_q8_pad40(x)
        _, qs, _, _ = oracle_mod.q8_fields(q8, nt, id_)
        xc = x.reshape(nt, nb32, 32)
        d32 = np.max(np.abs(xc), axis=2) / np.float32(127.0)
        with np.errstate(divide="ignore", invalid="ignore"):
            v = (xc / d32[..., None]).astype(np.float64)
        r = np.where(v >= 0, np.floor(v + 0.5), np.ceil(v - 0.5))
        r = np.clip(np.nan_to_num(r), -127, 127)
        r[d32 == 0] = 0
        assert np.array_equal(qs.reshape(nt, nb32, 32), r.astype(np.int8))


def test_quantize_exact_and_near_ties(oracle_mod):
    # Exact halves: x / d32 = k + 1/2 exactly, so round-half-away gives k + 1
    # for k >= 0 and k for k < 0 (closed form).  Near ties: the numpy IEEE
    # re-derivation decides each one from the correctly rounded quotient.
    import xkinds
    g = np.random.Generator(np.random.PCG64(77))
    nt, id_ = 6, 512
    nb32 = id_ // 32
    x = xkinds.x_variant(g, nt, id_, "halves")
    _, qs, _, _ = oracle_mod.q8_fields(oracle_mod.quantize_q8_pad40(x), nt, id_)
    xc = x.reshape(nt, nb32, 32).astype(np.float64)
    d = np.max(np.abs(xc), axis=2, keepdims=True) / 127.0     # a power of two
    v = xc / d
    want = np.where(np.abs(v) == 127.0, v, np.where(v >= 0, v + 0.5, v - 0.5))
    assert np.all((np.abs(v - np.trunc(v)) == 0.5) | (np.abs(v) == 127.0))
    assert np.array_equal(qs.reshape(nt, nb32, 32), want.astype(np.int8))
    x = xkinds.x_variant(g, nt, id_, "neartie")
    _, qs, _, _ = oracle_mod.q8_fields(oracle_mod.quantize_q8_pad40(x), nt, id_)
    xc = x.reshape(nt, nb32, 32)
    d32 = np.max(np.abs(xc), axis=2) / np.float32(127.0)
    v = (xc / d32[..., None]).astype(np.float64)
    r = np.where(v >= 0, np.floor(v + 0.5), np.ceil(v - 0.5))
    assert np.count_nonzero(np.abs(np.abs(v - np.trunc(v)) - 0.5) < 1e-5) > nt * id_ // 2
    assert np.array_equal(qs.reshape(nt, nb32, 32), r.astype(np.int8))


def test_quantize_row_stride(oracle_mod):
    g = np.random.Generator(np.random.PCG64(3))
    x = g.standard_normal((5, 160), dtype=np.float32)
    a = oracle_mod.quantize_q8_pad40(x, id_=128)         # ldx=160 > id
    b = oracle_mod.quantize_q8_pad40(np.ascontiguousarray(x[:, :128]))
    assert np.array_equal(a, b)
