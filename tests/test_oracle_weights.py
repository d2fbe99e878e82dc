"""Pins for the oracle's weight decoders and the dense W_exp expansion (CPU).

q6_K: hand-built blocks (r44 page 'W_exp stride mismatch root cause', s2.2
field order and s3.2 expander doc-comment), a bit-probe bijection (the 1536
quant bits of ql/qh feed exactly one element each, at a fixed weight), the
agreement of the element decoder with the byte-scatter expander (the two
listings of the r44 page), and the r44 page's worked stride-mismatch example.
q4_K: hand-derived fixture for the GGUF reading (layout not on the pages).
"""
import json
import os

import numpy as np
import pytest

from quant_integer_gemm_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _q6_block(spec):
    blk = np.zeros(224, dtype=np.uint8)
    if "ql_all" in spec:
        blk[0:128] = int(spec["ql_all"], 16)
    if "qh_all" in spec:
        blk[128:192] = int(spec["qh_all"], 16)
    for k, v in spec.get("ql", {}).items():
        blk[int(k)] = int(v, 16)
    for k, v in spec.get("qh", {}).items():
        blk[128 + int(k)] = int(v, 16)
    for k, v in spec.get("sc", {}).items():
        blk[192 + int(k)] = np.int8(v).view(np.uint8)
    db = int(spec["d_bits"], 16)
    blk[208] = db & 0xFF
    blk[209] = db >> 8
    return blk


def _q6_cases():
    with open(os.path.join(GOLDEN, "q6k_handbuilt.json")) as f:
        return json.load(f)["blocks"]


@pytest.mark.parametrize("spec", _q6_cases(), ids=lambda s: s["name"])
def test_q6k_handbuilt(oracle_mod, spec):
    blk = _q6_block(spec)
    c6, sc, d = oracle_mod.q6k_decode_block(blk)
    want = np.full(256, spec["expect_default"], dtype=np.int8)
    for k, v in spec["expect"].items():
        want[int(k)] = v
    assert np.array_equal(c6, want), np.nonzero(c6 != want)
    want_sc = np.zeros(16, dtype=np.int8)
    for k, v in spec["expect_sc"].items():
        want_sc[int(k)] = v
    assert np.array_equal(sc, want_sc)
    assert d == spec["expect_d"]
    # the dense expander agrees on the same block
    dense = oracle_mod.expand_q6k_dense(blk, 224, 1, 256)
    assert np.array_equal(dense[0], want)


def test_q6k_bit_probe_bijection(oracle_mod):
    """Every one of the 1536 bits of ql/qh feeds exactly one element; ql bits
    carry weights 1,2,4,8 (either nibble), qh bits weights 16,32; and every
    (element, bit-of-6) pair is reached exactly once."""
    base = np.zeros(224, dtype=np.uint8)
    c0, _, _ = oracle_mod.q6k_decode_block(base)
    assert np.all(c0 == -32)
    seen = set()
    for byte in range(192):
        for bit in range(8):
            blk = base.copy()
            blk[byte] = 1 << bit
            c, _, _ = oracle_mod.q6k_decode_block(blk)
            delta = c.astype(np.int32) - c0
            nz = np.nonzero(delta)[0]
            assert nz.size == 1, (byte, bit, nz)
            e = int(nz[0])
            w = int(delta[e])
            if byte < 128:
                assert w == 1 << (bit % 4)
            else:
                assert w == 16 << (bit % 2)
            assert (e, w) not in seen
            seen.add((e, w))
    assert len(seen) == 256 * 6


def test_q6k_page_byte_pair_statements(oracle_mod):
    """The r44 page (s3.2, doc-comment of the host expander): for it in {0,1}
    and r < 64, elements it*128+r and it*128+r+64 use the low and high nibble
    of ql[it*64+r], and the top bits of qh[it*32 + r%32] at fields 2*(r//32)
    and 2*(r//32)+4."""
    base = np.zeros(224, dtype=np.uint8)
    for it in range(2):
        for r in range(64):
            e0 = it * 128 + r
            blk = base.copy()
            blk[it * 64 + r] = 0x01          # low nibble bit 0
            c, _, _ = oracle_mod.q6k_decode_block(blk)
            assert c[e0] == -31 and np.sum(c != -32) == 1
            blk = base.copy()
            blk[it * 64 + r] = 0x10          # high nibble bit 0
            c, _, _ = oracle_mod.q6k_decode_block(blk)
            assert c[e0 + 64] == -31 and np.sum(c != -32) == 1
            s0 = 2 * (r // 32)
            blk = base.copy()
            blk[128 + it * 32 + r % 32] = 1 << s0
            c, _, _ = oracle_mod.q6k_decode_block(blk)
            assert c[e0] == -16 and np.sum(c != -32) == 1
            blk = base.copy()
            blk[128 + it * 32 + r % 32] = 1 << (s0 + 4)
            c, _, _ = oracle_mod.q6k_decode_block(blk)
            assert c[e0 + 64] == -16 and np.sum(c != -32) == 1


def test_q6k_decoder_equals_scatter_expander(oracle_mod):
    g = inputs.rng(101)
    od, id_ = 7, 768
    W = inputs.q6k_weights(g, od, id_)
    dense = oracle_mod.expand_q6k_dense(W, 224, od, id_)
    nsb = id_ // 256
    for j in range(od):
        for sb in range(nsb):
            blk = W[j, sb * 224:(sb + 1) * 224]
            c6, sc, d = oracle_mod.q6k_decode_block(blk)
            assert np.array_equal(dense[j, 256 * sb:256 * (sb + 1)], c6)
            assert np.array_equal(sc, blk[192:208].view(np.int8))
            assert d == float(blk[208:210].view(np.float16)[0])
    assert dense.min() >= -32 and dense.max() <= 31


def test_expand_respects_bstride(oracle_mod):
    g = inputs.rng(5)
    W224 = inputs.q6k_weights(g, 3, 512, bstride=224)
    nsb = 2
    W240 = np.zeros((3, nsb * 240), dtype=np.uint8)
    for sb in range(nsb):
        W240[:, sb * 240:sb * 240 + 224] = W224[:, sb * 224:(sb + 1) * 224]
    a = oracle_mod.expand_q6k_dense(W224, 224, 3, 512)
    b = oracle_mod.expand_q6k_dense(W240, 240, 3, 512)
    assert np.array_equal(a, b)


def test_r44_worked_stride_mismatch(oracle_mod):
    """r44 page s2.3 worked example: reading the dense plane with the padded
    raw-W strides (row pitch nsb*224) at id=256 makes the kernel's row 2 the
    tail 64 elements of dense row 1 followed by the first 192 of dense row 2;
    at id=3584 the drift is 448 bytes per row."""
    g = inputs.rng(9)
    od, id_ = 4, 256
    W = inputs.q6k_weights(g, od, id_)
    dense = oracle_mod.expand_q6k_dense(W, 224, od, id_).reshape(-1)
    wrong_row2 = dense[2 * 224:2 * 224 + 256]
    rows = dense.reshape(od, id_)
    assert np.array_equal(wrong_row2[:64], rows[1, 192:256])
    assert np.array_equal(wrong_row2[64:], rows[2, 0:192])
    nsb = 3584 // 256
    assert 3584 - nsb * 224 == 448


def _q4_cases():
    with open(os.path.join(GOLDEN, "q4k_handbuilt.json")) as f:
        return json.load(f)["blocks"]


@pytest.mark.parametrize("spec", _q4_cases(), ids=lambda s: s["name"])
def test_q4k_handbuilt(oracle_mod, spec):
    blk = np.zeros(144, dtype=np.uint8)
    blk[4:16] = [int(s, 16) for s in spec["S"]]
    for k, v in spec["qs"].items():
        blk[16 + int(k)] = int(v, 16)
    db, mb = int(spec["d_bits"], 16), int(spec["dmin_bits"], 16)
    blk[0], blk[1], blk[2], blk[3] = db & 0xFF, db >> 8, mb & 0xFF, mb >> 8
    q, sc, m, d, dmin = oracle_mod.q4k_decode_block(blk)
    assert list(sc) == spec["expect_sc"]
    assert list(m) == spec["expect_m"]
    want = np.full(256, spec["expect_q_default"], dtype=np.uint8)
    for k, v in spec["expect_q"].items():
        want[int(k)] = v
    assert np.array_equal(q, want)
    assert d == spec["expect_d"] and dmin == spec["expect_dmin"]


def test_q4k_bit_probe_bijection(oracle_mod):
    """Each of the 96 scale bits feeds exactly one 6-bit sc or m value, each
    (value, bit) pair once; each of the 1024 nibble bits feeds one element."""
    base = np.zeros(144, dtype=np.uint8)
    q0, sc0, m0, _, _ = oracle_mod.q4k_decode_block(base)
    seen = set()
    for byte in range(4, 16):
        for bit in range(8):
            blk = base.copy()
            blk[byte] = 1 << bit
            q, sc, m, _, _ = oracle_mod.q4k_decode_block(blk)
            assert np.array_equal(q, q0)
            ds = np.nonzero(sc != sc0)[0]
            dm = np.nonzero(m != m0)[0]
            assert ds.size + dm.size == 1
            if ds.size:
                key = ("sc", int(ds[0]), int(sc[ds[0]]))
            else:
                key = ("m", int(dm[0]), int(m[dm[0]]))
            assert key[2] in (1, 2, 4, 8, 16, 32)
            assert key not in seen
            seen.add(key)
    assert len(seen) == 96
    seen = set()
    for byte in range(16, 144):
        for bit in range(8):
            blk = base.copy()
            blk[byte] = 1 << bit
            q, _, _, _, _ = oracle_mod.q4k_decode_block(blk)
            nz = np.nonzero(q)[0]
            assert nz.size == 1 and q[nz[0]] == 1 << (bit % 4)
            key = (int(nz[0]), int(q[nz[0]]))
            assert key not in seen
            seen.add(key)
    assert len(seen) == 1024
