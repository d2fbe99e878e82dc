"""Pins for the oracle's sub-block partials and fp64 GEMM (CPU only).

* Special cases that reduce to a textbook integer matmul (numpy int64): unit
  weight scales and activations whose chunks have max |x| = 127 (so the
  stored fp16 d is exactly 1 and the quants are x itself).
* The q4_K min term alone (all nibbles 0): y = -dmin * m * sum of ssum.
* Brute force on tiny shapes: every weight and activation dequantised to fp64
  and a plain triple loop, against the sub-block formulation.
* Partials against brute-force integer dot products.
The single-term scaling per sub-block follows the r44 page ('W_exp stride
mismatch root cause', s1.1 sixteen sub-blocks of 16; s2.1 one d*sc per
sub-block).
"""
import numpy as np
import pytest

from quant_integer_gemm_amd import inputs


def _int_activations(g, nt, id_):
    """Integer x in [-127, 127] with max |x| = 127 in every 32-chunk."""
    x = g.integers(-127, 128, size=(nt, id_)).astype(np.float32)
    x[:, ::32] = np.where(g.integers(0, 2, size=(nt, id_ // 32)) == 1, 127.0, -127.0)
    return x


def _set_q6_scales(W, od, id_, sc_val, d_val, bstride=224):
    W = W.copy().reshape(od, id_ // 256, bstride)
    W[:, :, 192:208] = np.int8(sc_val).view(np.uint8)
    W[:, :, 208:210] = np.array([d_val], dtype=np.float16).view(np.uint8)
    return W.reshape(od, -1)


def test_q6k_reduces_to_integer_matmul(oracle_mod):
    g = inputs.rng(21)
    nt, od, id_ = 5, 6, 512
    W = _set_q6_scales(inputs.q6k_weights(g, od, id_), od, id_, 1, 1.0)
    x = _int_activations(g, nt, id_)
    q8 = oracle_mod.quantize_q8_pad40(x)
    d_bits, qs, _, _ = oracle_mod.q8_fields(q8, nt, id_)
    assert np.all(d_bits == 0x3C00) and np.array_equal(qs.astype(np.float32), x)
    c6 = oracle_mod.expand_q6k_dense(W, 224, od, id_)
    want = x.astype(np.int64) @ c6.astype(np.int64).T
    y = oracle_mod.mmq_q6k(W, 224, od, id_, q8, nt)
    assert np.array_equal(y, want.astype(np.float64))


def test_q6k_one_hot_scale_selects_subblock_and_chunk(oracle_mod):
    """sc = 1 on sub-block s only, d = 1: y = da(chunk of s) * P6(s).  With a
    different activation scale per chunk this pins the sub-block -> chunk map
    (two sub-blocks of 16 per pad40 chunk)."""
    g = inputs.rng(22)
    nt, od, id_ = 3, 4, 256
    x = g.standard_normal((nt, id_), dtype=np.float32) * np.repeat(
        np.float32(2.0) ** np.arange(8, dtype=np.float32), 32)[None, :]
    q8 = oracle_mod.quantize_q8_pad40(x)
    d_bits, qs, _, _ = oracle_mod.q8_fields(q8, nt, id_)
    da = d_bits.view(np.float16).astype(np.float64)
    W0 = inputs.q6k_weights(g, od, id_)
    c6 = oracle_mod.expand_q6k_dense(W0, 224, od, id_).astype(np.int64)
    for s in range(16):
        sc = np.zeros(16, dtype=np.int8)
        sc[s] = 1
        W = _set_q6_scales(W0, od, id_, sc, 1.0)
        y = oracle_mod.mmq_q6k(W, 224, od, id_, q8, nt)
        P = qs[:, 16 * s:16 * s + 16].astype(np.int64) @ c6[:, 16 * s:16 * s + 16].T
        assert np.array_equal(y, da[:, s // 2][:, None] * P.astype(np.float64))


def _set_q4(W, od, id_, d, dmin, S=None, qbyte=None):
    W = W.copy().reshape(od, id_ // 256, 144)
    W[:, :, 0:2] = np.array([d], dtype=np.float16).view(np.uint8)
    W[:, :, 2:4] = np.array([dmin], dtype=np.float16).view(np.uint8)
    if S is not None:
        W[:, :, 4:16] = S
    if qbyte is not None:
        W[:, :, 16:144] = qbyte
    return W.reshape(od, -1)


def test_q4k_reduces_to_integer_matmul(oracle_mod):
    g = inputs.rng(23)
    nt, od, id_ = 4, 5, 512
    # every sc = 1 and m = 0: S[0..3] = 1, S[4..7] = 0, S[8..11] = 0x01
    S = np.array([1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1], dtype=np.uint8)
    W = _set_q4(inputs.q4k_weights(g, od, id_), od, id_, 1.0, 0.0, S=S)
    for blk in W.reshape(-1, 144)[:3]:
        _, sc, m, _, _ = oracle_mod.q4k_decode_block(blk)
        assert np.all(sc == 1) and np.all(m == 0)
    x = _int_activations(g, nt, id_)
    q8 = oracle_mod.quantize_q8_pad40(x)
    q4 = np.zeros((od, id_), dtype=np.int64)
    for j in range(od):
        for sb in range(id_ // 256):
            q, _, _, _, _ = oracle_mod.q4k_decode_block(W[j, sb * 144:(sb + 1) * 144])
            q4[j, 256 * sb:256 * (sb + 1)] = q
    want = x.astype(np.int64) @ q4.T
    y = oracle_mod.mmq_q4k(W, od, id_, q8, nt)
    assert np.array_equal(y, want.astype(np.float64))


def test_q4k_min_term_alone(oracle_mod):
    """All nibbles 0 so the scaled term vanishes; sc arbitrary; every m = 1,
    dmin = 1: y(t, j) = -sum_c ssum(t, c), and ssum = d_fp16 * sum(q)."""
    g = inputs.rng(24)
    nt, od, id_ = 6, 3, 768
    S = np.array([0x45, 0x45, 0x45, 0x45, 1, 1, 1, 1, 0x11, 0x11, 0x11, 0x11], dtype=np.uint8)
    W = _set_q4(inputs.q4k_weights(g, od, id_), od, id_, 0.5, 1.0, S=S, qbyte=0)
    _, sc, m, _, _ = oracle_mod.q4k_decode_block(W[0, :144])
    assert np.all(m == 1)
    x = g.standard_normal((nt, id_), dtype=np.float32)
    q8 = oracle_mod.quantize_q8_pad40(x)
    d_bits, qs, ssum, _ = oracle_mod.q8_fields(q8, nt, id_)
    dh = d_bits.view(np.float16).astype(np.float64)
    s = qs.reshape(nt, id_ // 32, 32).astype(np.int64).sum(axis=2)
    assert np.array_equal(ssum.astype(np.float64), dh * s)       # min-term invariant
    y = oracle_mod.mmq_q4k(W, od, id_, q8, nt)
    want = -ssum.astype(np.float64).sum(axis=1)
    assert np.allclose(y, np.repeat(want[:, None], od, axis=1), rtol=1e-13, atol=0)


def _brute_q6(oracle_mod, W, od, id_, q8, nt):
    nsb = id_ // 256
    wf = np.zeros((od, id_))
    for j in range(od):
        for sb in range(nsb):
            c6, sc, d = oracle_mod.q6k_decode_block(W[j, sb * 224:(sb + 1) * 224])
            for e in range(256):
                wf[j, 256 * sb + e] = d * float(sc[e // 16]) * float(c6[e])
    return wf


def _brute_q4(oracle_mod, W, od, id_):
    nsb = id_ // 256
    wf = np.zeros((od, id_))
    for j in range(od):
        for sb in range(nsb):
            q, sc, m, d, dmin = oracle_mod.q4k_decode_block(W[j, sb * 144:(sb + 1) * 144])
            for e in range(256):
                wf[j, 256 * sb + e] = d * float(sc[e // 32]) * float(q[e]) - dmin * float(m[e // 32])
    return wf


def _dequant_acts(oracle_mod, q8, nt, id_):
    d_bits, qs, _, _ = oracle_mod.q8_fields(q8, nt, id_)
    da = d_bits.view(np.float16).astype(np.float64)
    a = np.zeros((nt, id_))
    for t in range(nt):
        for k in range(id_):
            a[t, k] = da[t, k // 32] * float(qs[t, k])
    return a


@pytest.mark.parametrize("qtype", ["q6_K", "q4_K"])
def test_brute_force_tiny(oracle_mod, qtype):
    g = inputs.rng(25)
    nt, od, id_ = 3, 5, 512
    x = g.standard_normal((nt, id_), dtype=np.float32)
    q8 = oracle_mod.quantize_q8_pad40(x)
    a = _dequant_acts(oracle_mod, q8, nt, id_)
    if qtype == "q6_K":
        W = inputs.q6k_weights(g, od, id_)
        wf = _brute_q6(oracle_mod, W, od, id_, q8, nt)
        y = oracle_mod.mmq_q6k(W, 224, od, id_, q8, nt)
    else:
        W = inputs.q4k_weights(g, od, id_)
        wf = _brute_q4(oracle_mod, W, od, id_)
        y = oracle_mod.mmq_q4k(W, od, id_, q8, nt)
    want = np.zeros((nt, od))
    for t in range(nt):
        for j in range(od):
            s = 0.0
            for k in range(id_):
                s += a[t, k] * wf[j, k]
            want[t, j] = s
    scale = np.max(np.abs(want))
    assert np.max(np.abs(y - want)) <= 1e-12 * scale


def test_partials_brute_force(oracle_mod):
    g = inputs.rng(26)
    nt, od, id_ = 4, 3, 512
    x = g.standard_normal((nt, id_), dtype=np.float32)
    q8 = oracle_mod.quantize_q8_pad40(x)
    _, qs, _, _ = oracle_mod.q8_fields(q8, nt, id_)
    W6 = inputs.q6k_weights(g, od, id_)
    c6 = oracle_mod.expand_q6k_dense(W6, 224, od, id_)
    P6 = oracle_mod.q6k_partials(W6, 224, od, id_, q8, nt, 1, 4, 1, 3)
    for t in range(1, 4):
        for j in range(1, 3):
            for s in range(2 * 16):
                want = sum(int(qs[t, 16 * s + i]) * int(c6[j, 16 * s + i]) for i in range(16))
                assert P6[t - 1, j - 1, s] == want
    W4 = inputs.q4k_weights(g, od, id_)
    P4 = oracle_mod.q4k_partials(W4, od, id_, q8, nt, 0, 2, 0, 3)
    for j in range(3):
        q4 = []
        for sb in range(2):
            q, _, _, _, _ = oracle_mod.q4k_decode_block(W4[j, sb * 144:(sb + 1) * 144])
            q4.extend(int(v) for v in q)
        for t in range(2):
            for b in range(16):
                want = sum(int(qs[t, 32 * b + i]) * q4[32 * b + i] for i in range(32))
                assert P4[t, j, b] == want


def test_points_match_full(oracle_mod):
    g = inputs.rng(27)
    nt, od, id_ = 7, 9, 512
    x = g.standard_normal((nt, id_), dtype=np.float32)
    q8 = oracle_mod.quantize_q8_pad40(x)
    W6 = inputs.q6k_weights(g, od, id_)
    W4 = inputs.q4k_weights(g, od, id_)
    tt = g.integers(0, nt, 20)
    jj = g.integers(0, od, 20)
    y6 = oracle_mod.mmq_q6k(W6, 224, od, id_, q8, nt)
    y4 = oracle_mod.mmq_q4k(W4, od, id_, q8, nt)
    assert np.array_equal(oracle_mod.mmq_q6k_points(W6, 224, od, id_, q8, nt, tt, jj), y6[tt, jj])
    assert np.array_equal(oracle_mod.mmq_q4k_points(W4, od, id_, q8, nt, tt, jj), y4[tt, jj])


def test_tolerance_helper():
    import oracle
    ok, w = oracle.within_tolerance(np.array([1.0, 2.0]), np.array([1.0, 2.0]))
    assert ok and w == 0.0
    ok, _ = oracle.within_tolerance(np.array([1.01, 2.0]), np.array([1.0, 2.0]))
    assert not ok


def test_dense_plane_consumer_and_stride_mutant(oracle_mod):
    """Consumer gate on the CPU (r44 page 'W_exp stride mismatch root cause',
    s2.3-2.5): the dense plane read at its own strides (id, 256) gives the
    raw-block result exactly; read at the padded raw-W strides (nsb*224, 224)
    it gives a wrong result that the parity tolerance rejects, although every
    byte of the plane is correct."""
    g = inputs.rng(28)
    nt, od, id_ = 6, 9, 768
    W = inputs.q6k_weights(g, od, id_)
    x = g.standard_normal((nt, id_), dtype=np.float32)
    q8 = oracle_mod.quantize_q8_pad40(x)
    plane = oracle_mod.expand_q6k_dense(W, 224, od, id_)
    y_raw = oracle_mod.mmq_q6k(W, 224, od, id_, q8, nt)
    y_ok = oracle_mod.mmq_q6k_from_plane(plane, id_, 256, W, 224, od, id_, q8, nt)
    assert np.array_equal(y_ok, y_raw)
    nsb = id_ // 256
    y_bad = oracle_mod.mmq_q6k_from_plane(plane, nsb * 224, 224, W, 224, od, id_, q8, nt)
    ok, worst = oracle_mod.within_tolerance(y_bad, y_raw)
    assert not ok and worst > 10
