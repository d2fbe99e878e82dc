"""GPU parity of the HIP path against the CPU oracle (run on an MI355X).

Bars: pad40 bytes, W_exp bytes and int32 sub-block partials bit-exact; fp32 y
within |y - y_ref| <= max(1e-4 |y_ref|, 1e-3 rms(y_ref)) per element, y_ref
being the oracle's fp64 result.  Shapes span several tiles (64 tokens x 64
rows per workgroup) with ragged tails, the five workloads at full size (every
output of every GEMM, the nt=2630 layer included, through the pad40 calls and
through the tiled-plane calls bench.py times), and the degenerate cases
(empty inputs, one token, one row).
"""
import numpy as np
import pytest

import oracle
import xkinds
from quant_integer_gemm_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def qig():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quant_integer_gemm_amd as q
    q.load()
    return q


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _x_variant(g, nt, id_, kind):
    return xkinds.x_variant(g, nt, id_, kind)


# ---------------------------------------------------------------------------
# quantize
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("nt,id_,kind", [
    (16, 512, "normal"), (1, 32, "normal"), (3, 96, "ties"), (37, 4096, "tiny"),
    (70, 1024, "zeros"), (9, 2048, "heavy"), (512, 3584, "normal"), (512, 18944, "scaled2"),
    (2630, 18944, "normal"), (64, 1024, "halves"), (130, 2048, "neartie"),
])
def test_quantize_bit_exact(qig, nt, id_, kind):
    g = inputs.rng(1000 + nt + id_)
    x = _x_variant(g, nt, id_, kind)
    want = oracle.quantize_q8_pad40(x)
    got = host(qig.quantize_q8_pad40(dev(x)))
    assert got.shape == want.shape
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


def test_quantize_row_stride(qig):
    g = inputs.rng(3)
    x = g.standard_normal((5, 160), dtype=np.float32)
    want = oracle.quantize_q8_pad40(x, id_=128)
    got = host(qig.quantize_q8_pad40(dev(x), id_=128))
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# GEMM helpers
# ---------------------------------------------------------------------------
def _weights(qtype, g, od, id_, bstride=224):
    if qtype == "q4_K":
        return inputs.q4k_weights(g, od, id_)
    return inputs.q6k_weights(g, od, id_, bstride=bstride)


def _gpu_gemm(qig, qtype, Wd, od, id_, q8d, nt, bstride=224, Wexp=None, y=None, ldy=None):
    if qtype == "q4_K":
        return qig.mmq_q4k(Wd, od, id_, q8d, nt, y=y, ldy=ldy)
    return qig.mmq_q6k(Wd, bstride, od, id_, q8d, nt, W_exp=Wexp, y=y, ldy=ldy)


def _oracle_gemm(qtype, W, od, id_, q8, nt, bstride=224):
    if qtype == "q4_K":
        return oracle.mmq_q4k(W, od, id_, q8, nt)
    return oracle.mmq_q6k(W, bstride, od, id_, q8, nt)


def _assert_close(y, y_ref, what=""):
    ok, worst = oracle.within_tolerance(y, y_ref)
    assert ok, f"{what}: worst error/allowance = {worst:.3g}"


SMALL = [(16, 256, 512), (1, 1, 256), (70, 130, 768), (129, 257, 512), (64, 128, 256),
         (200, 300, 1024), (3, 1000, 256), (65, 129, 2304)]


@pytest.mark.parametrize("qtype", ["q4_K", "q6_K"])
@pytest.mark.parametrize("nt,od,id_", SMALL)
def test_gemm_small(qig, qtype, nt, od, id_):
    g = inputs.rng(nt * 7 + od * 13 + id_)
    W = _weights(qtype, g, od, id_)
    x = g.standard_normal((nt, id_), dtype=np.float32)
    q8 = oracle.quantize_q8_pad40(x)
    y = host(_gpu_gemm(qig, qtype, dev(W), od, id_, dev(q8), nt))
    _assert_close(y, _oracle_gemm(qtype, W, od, id_, q8, nt), f"{qtype} {nt}x{od}x{id_}")


@pytest.mark.parametrize("qtype", ["q4_K", "q6_K"])
def test_gemm_integer_special_case_exact(qig, qtype):
    """Unit scales and integer activations with max |x| = 127 per chunk: the
    fp32 output must equal the integer matmul exactly."""
    g = inputs.rng(31)
    nt, od, id_ = 70, 150, 512
    x = g.integers(-127, 128, size=(nt, id_)).astype(np.float32)
    x[:, ::32] = 127.0
    if qtype == "q4_K":
        W = inputs.q4k_weights(g, od, id_).reshape(od, -1, 144)
        W[:, :, 0:2] = np.array([1.0], dtype=np.float16).view(np.uint8)
        W[:, :, 2:4] = 0
        W[:, :, 4:16] = np.array([1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1], dtype=np.uint8)
        W = W.reshape(od, -1)
        wq = np.zeros((od, id_), dtype=np.int64)
        for j in range(od):
            for sb in range(id_ // 256):
                q, _, _, _, _ = oracle.q4k_decode_block(W[j, sb * 144:(sb + 1) * 144])
                wq[j, 256 * sb:256 * sb + 256] = q
    else:
        W = inputs.q6k_weights(g, od, id_).reshape(od, -1, 224)
        W[:, :, 192:208] = 1
        W[:, :, 208:210] = np.array([1.0], dtype=np.float16).view(np.uint8)
        W = W.reshape(od, -1)
        wq = oracle.expand_q6k_dense(W, 224, od, id_).astype(np.int64)
    want = (x.astype(np.int64) @ wq.T).astype(np.float64)
    assert np.max(np.abs(want)) < 2 ** 24
    q8 = oracle.quantize_q8_pad40(x)
    y = host(_gpu_gemm(qig, qtype, dev(W), od, id_, dev(q8), nt))
    assert np.array_equal(y.astype(np.float64), want)


def test_q4k_subnormal_scales(qig):
    g = inputs.rng(32)
    nt, od, id_ = 40, 140, 512
    W = inputs.q4k_weights(g, od, id_).reshape(od, -1, 144)
    W[:, :, 0:2] = np.array([3e-6], dtype=np.float16).view(np.uint8)    # subnormal d
    W[:, :, 2:4] = np.array([5e-7], dtype=np.float16).view(np.uint8)    # subnormal dmin
    W = W.reshape(od, -1)
    x = g.standard_normal((nt, id_), dtype=np.float32) * np.float32(1e-6)   # subnormal da
    q8 = oracle.quantize_q8_pad40(x)
    y = host(qig.mmq_q4k(dev(W), od, id_, dev(q8), nt))
    _assert_close(y, oracle.mmq_q4k(W, od, id_, q8, nt), "subnormal")


@pytest.mark.parametrize("qtype", ["q4_K", "q6_K"])
@pytest.mark.parametrize("od", [1, 17, 256, 512, 3584])
@pytest.mark.parametrize("nt", [1, 15, 16, 70, 128, 256, 512, 2630])
def test_shape_sweep(qig, qtype, nt, od):
    """Token and row counts from one element to several tiles with ragged
    tails, where single shapes hide tail bugs: y within tolerance of the
    oracle, and the tiled-plane GEMM bit-identical to the pad40 one."""
    id_ = 512
    gm = inputs.Gemm("sweep", qtype, od, id_, nt)
    W, x = inputs.make_gemm_inputs(gm, inputs.SEED_BASE + 500 + 7 * nt + od)
    q8 = oracle.quantize_q8_pad40(x)
    Wd, xd = dev(W), dev(x)
    q8d = qig.quantize_q8_pad40(xd)
    q8td = qig.quantize_q8_tiled(xd)
    if qtype == "q4_K":
        y = qig.mmq_q4k(Wd, od, id_, q8d, nt)
        yt = qig.mmq_q4k_q8t(Wd, od, id_, q8td, nt)
    else:
        y = qig.mmq_q6k(Wd, 224, od, id_, q8d, nt)
        yt = qig.mmq_q6k_q8t(Wd, 224, od, id_, q8td, nt)
    y, yt = host(y), host(yt)
    _assert_close(y, _oracle_gemm(qtype, W, od, id_, q8, nt), f"{qtype} {nt}x{od}x{id_}")
    assert np.array_equal(yt.view(np.uint32), y.view(np.uint32))


def _extreme_inputs(qtype, g, nt, od, id_):
    """Quants at their extremes, activations +-127 (so d_a = 1 and qs = x) and
    extreme sub-block scales: the first half of the tokens is all +127 and
    reaches the largest |P| the formats allow."""
    x = np.where(g.random((nt, id_)) < 0.5, -127.0, 127.0).astype(np.float32)
    x[: nt // 2] = 127.0
    if qtype == "q6_K":
        W = inputs.q6k_weights(g, od, id_).reshape(od, -1, 224)
        W[: od // 2, :, 0:192] = 0x00                    # every quant -32
        W[od // 2:, :, 0:192] = 0xFF                     # every quant +31
        W[:, :, 192:208] = np.where(np.arange(16) % 2 == 0, -128, 127).astype(np.int8).view(np.uint8)
        W[:, :, 208:210] = np.array([0.5], dtype=np.float16).view(np.uint8)
    else:
        W = inputs.q4k_weights(g, od, id_).reshape(od, -1, 144)
        W[:, :, 16:144] = 0xFF                           # every quant 15
        W[:, :, 4:16] = 0xFF                             # sc = m = 63 in all 8 sub-blocks
        W[:, :, 0:2] = np.array([0.5], dtype=np.float16).view(np.uint8)
        W[:, :, 2:4] = np.array([0.25], dtype=np.float16).view(np.uint8)
    return W.reshape(od, -1), x


@pytest.mark.parametrize("qtype", ["q4_K", "q6_K"])
def test_extreme_magnitudes(qig, qtype):
    """|P| at its bound (16*127*32 = 65024 for q6_K, 32*127*15 = 60960 for
    q4_K): partials bit-exact, and y of every arm within tolerance."""
    g = inputs.rng(61)
    nt, od, id_ = 70, 130, 512
    W, x = _extreme_inputs(qtype, g, nt, od, id_)
    q8 = oracle.quantize_q8_pad40(x)
    Wd, q8d = dev(W), dev(q8)
    if qtype == "q4_K":
        want_p = oracle.q4k_partials(W, od, id_, q8, nt, 0, nt, 0, od)
        got_p = host(qig.mmq_q4k_partials(Wd, od, id_, q8d, nt, 0, nt, 0, od))
        bound = 32 * 127 * 15
    else:
        want_p = oracle.q6k_partials(W, 224, od, id_, q8, nt, 0, nt, 0, od)
        got_p = host(qig.mmq_q6k_partials(Wd, 224, od, id_, q8d, nt, 0, nt, 0, od))
        bound = 16 * 127 * 32
    assert int(np.max(np.abs(want_p))) == bound
    assert np.array_equal(got_p, want_p), f"{np.sum(got_p != want_p)} partials differ"
    y_ref = _oracle_gemm(qtype, W, od, id_, q8, nt)
    q8td = qig.quantize_q8_tiled(dev(x))
    if qtype == "q4_K":
        Wp = qig.prepare_q4k(Wd, od, id_)
        ys = {"raw": qig.mmq_q4k(Wd, od, id_, q8d, nt),
              "prepared": qig.mmq_q4k_prepared(Wp, od, id_, q8d, nt),
              "tiled": qig.mmq_q4k_q8t(Wd, od, id_, q8td, nt),
              "prepared tiled": qig.mmq_q4k_prepared_q8t(Wp, od, id_, q8td, nt)}
    else:
        We = qig.expand_q6k_dense(Wd, 224, od, id_)
        Wp = qig.prepare_q6k(Wd, 224, od, id_)
        ys = {"raw": qig.mmq_q6k(Wd, 224, od, id_, q8d, nt),
              "W_exp": qig.mmq_q6k(Wd, 224, od, id_, q8d, nt, W_exp=We),
              "prepared": qig.mmq_q6k_prepared(Wp, od, id_, q8d, nt),
              "tiled": qig.mmq_q6k_q8t(Wd, 224, od, id_, q8td, nt),
              "W_exp tiled": qig.mmq_q6k_q8t(Wd, 224, od, id_, q8td, nt, W_exp=We)}
    for k, y in ys.items():
        _assert_close(host(y), y_ref, f"{qtype} extreme {k}")


# ---------------------------------------------------------------------------
# partials
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("qtype", ["q4_K", "q6_K"])
@pytest.mark.parametrize("nt,od,id_,win", [
    (16, 256, 512, None), (70, 130, 768, None), (129, 257, 512, (60, 129, 100, 257)),
    (512, 3584, 3584, (40, 90, 3450, 3584)),
])
def test_partials_bit_exact(qig, qtype, nt, od, id_, win):
    g = inputs.rng(41 + nt + od)
    W = _weights(qtype, g, od, id_)
    x = g.standard_normal((nt, id_), dtype=np.float32)
    q8 = oracle.quantize_q8_pad40(x)
    t0, t1, j0, j1 = win if win else (0, nt, 0, od)
    if qtype == "q4_K":
        want = oracle.q4k_partials(W, od, id_, q8, nt, t0, t1, j0, j1)
        got = host(qig.mmq_q4k_partials(dev(W), od, id_, dev(q8), nt, t0, t1, j0, j1))
    else:
        want = oracle.q6k_partials(W, 224, od, id_, q8, nt, t0, t1, j0, j1)
        got = host(qig.mmq_q6k_partials(dev(W), 224, od, id_, dev(q8), nt, t0, t1, j0, j1))
    assert got.shape == want.shape
    assert np.array_equal(got, want), f"{np.sum(got != want)} partials differ"


# ---------------------------------------------------------------------------
# W_exp arm: content gate, then consumer gate
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("nt,od,id_,bstride", [(16, 256, 512, 224), (70, 130, 768, 240),
                                               (512, 3584, 3584, 224)])
def test_wexp_content_and_consumer(qig, nt, od, id_, bstride):
    g = inputs.rng(51 + od)
    W = inputs.q6k_weights(g, od, id_, bstride=bstride)
    x = g.standard_normal((nt, id_), dtype=np.float32)
    q8 = oracle.quantize_q8_pad40(x)
    Wd, q8d = dev(W), dev(q8)
    wexp = qig.expand_q6k_dense(Wd, bstride, od, id_)
    want_plane = oracle.expand_q6k_dense(W, bstride, od, id_)
    assert np.array_equal(host(wexp), want_plane)                        # content
    y_raw = host(qig.mmq_q6k(Wd, bstride, od, id_, q8d, nt))
    y_exp = host(qig.mmq_q6k(Wd, bstride, od, id_, q8d, nt, W_exp=wexp))
    assert np.array_equal(y_raw.view(np.uint32), y_exp.view(np.uint32))  # consumer: identical
    _assert_close(y_exp, oracle.mmq_q6k(W, bstride, od, id_, q8, nt), "W_exp arm")
    t1, j1 = min(nt, 40), min(od, 140)
    p_raw = host(qig.mmq_q6k_partials(Wd, bstride, od, id_, q8d, nt, 0, t1, 0, j1))
    p_exp = host(qig.mmq_q6k_partials(Wd, bstride, od, id_, q8d, nt, 0, t1, 0, j1, W_exp=wexp))
    assert np.array_equal(p_raw, p_exp)


# ---------------------------------------------------------------------------
# full-size workloads
# ---------------------------------------------------------------------------
def _run_workload_gemm(qig, gm, seed):
    """Every output of one workload GEMM against the oracle (the tolerance's
    rms floor taken from the oracle's y), through the plain pad40 call and
    through the launch configuration bench.py times: the tiled activation
    plane with a stream-K workspace."""
    W, x = inputs.make_gemm_inputs(gm, seed)
    nt, od, id_ = gm.nt, gm.od, gm.id
    xd, Wd = dev(x), dev(W)
    q8d = qig.quantize_q8_pad40(xd)
    q8 = oracle.quantize_q8_pad40(x)
    assert np.array_equal(host(q8d), q8)
    y_ref = _oracle_gemm(gm.qtype, W, od, id_, q8, nt)
    y = host(_gpu_gemm(qig, gm.qtype, Wd, od, id_, q8d, nt))
    assert np.isfinite(y).all(), f"{gm.name}: non-finite outputs"
    _assert_close(y, y_ref, gm.name)
    q8td = qig.quantize_q8_tiled(xd)
    ws = qig.new_workspace("cuda")
    if gm.qtype == "q4_K":
        yt = qig.mmq_q4k_q8t(Wd, od, id_, q8td, nt, ws=ws)
    else:
        yt = qig.mmq_q6k_q8t(Wd, 224, od, id_, q8td, nt, ws=ws)
    yt = host(yt)
    assert np.isfinite(yt).all(), f"{gm.name} tiled: non-finite outputs"
    _assert_close(yt, y_ref, gm.name + " tiled plane, stream-K workspace")
    assert int(torch.count_nonzero(ws[-16384:]).item()) == 0
    if gm.qtype == "q4_K":
        # the q4_K arm the FFN and layer steps of bench.py run: the staged buffer
        Wst = qig.prepare_q4k_staged(Wd, od, id_)
        ys = host(qig.mmq_q4k_staged_q8t(Wst, od, id_, q8td, nt, ws=ws))
        assert np.array_equal(ys.view(np.uint32), yt.view(np.uint32)), f"{gm.name}: staged differs from raw"
        assert int(torch.count_nonzero(ws[-16384:]).item()) == 0
    if gm.qtype == "q6_K":
        # the q6_K arm the FFN and layer steps of bench.py run: the limb buffer
        Wl = qig.prepare_q6k_limbs(Wd, 224, od, id_)
        yl = host(qig.mmq_q6k_limbs_q8t(Wl, od, id_, q8td, nt, ws=ws))
        assert np.isfinite(yl).all(), f"{gm.name} limbs: non-finite outputs"
        _assert_close(yl, y_ref, gm.name + " limb buffer, tiled plane, stream-K workspace")
        assert int(torch.count_nonzero(ws[-16384:]).item()) == 0


# ---------------------------------------------------------------------------
# prepared weights (registration-time quant + scale planes)
# ---------------------------------------------------------------------------
def _prepared_expected(qtype, W, od, id_):
    """Quant plane and fp32 scale plane from the oracle's block decoders
    (q4_K quant plane: the raw blocks' packed quant bytes, 128 per block)."""
    nsb = id_ // 256
    Q = np.zeros((od, id_ // 2 if qtype == "q4_K" else id_), dtype=np.int8)
    S = np.zeros((od, nsb, 16), dtype=np.float32)
    if qtype == "q6_K":
        Q[:] = oracle.expand_q6k_dense(W, 224, od, id_)
        Wb = W.reshape(od, nsb, 224)
        for j in range(od):
            for sb in range(nsb):
                _, sc, d = oracle.q6k_decode_block(Wb[j, sb])
                S[j, sb] = (d * sc.astype(np.float64)).astype(np.float32)   # exact products
    else:
        Wb = W.reshape(od, nsb, 144)
        for j in range(od):
            for sb in range(nsb):
                q, sc, m, d, dmin = oracle.q4k_decode_block(Wb[j, sb])
                qs = Wb[j, sb, 16:144]
                # the packed bytes decode to the oracle's elements (low nibble
                # of byte 32g+i = element 64g+i, high nibble = 64g+32+i)
                g_, i_ = np.divmod(np.arange(128), 32)
                assert np.array_equal(qs & 15, q[64 * g_ + i_]) and np.array_equal(qs >> 4, q[64 * g_ + 32 + i_])
                Q[j, 128 * sb:128 * sb + 128] = qs.view(np.int8)
                S[j, sb, 0::2] = (d * sc.astype(np.float64)).astype(np.float32)
                S[j, sb, 1::2] = (dmin * m.astype(np.float64)).astype(np.float32)
    return Q, S


@pytest.mark.parametrize("qtype", ["q4_K", "q6_K"])
@pytest.mark.parametrize("od,id_", [(130, 768), (64, 256)])
def test_prepared_planes_content(qig, qtype, od, id_):
    gm = inputs.Gemm("prep", qtype, od, id_, 1)
    W, _ = inputs.make_gemm_inputs(gm, inputs.SEED_BASE + 300 + od)
    if qtype == "q6_K":
        Wp = host(qig.prepare_q6k(dev(W), 224, od, id_))
    else:
        Wp = host(qig.prepare_q4k(dev(W), od, id_))
    assert Wp.size == qig.prepared_bytes(qtype, od, id_)
    Q, S = _prepared_expected(qtype, W, od, id_)
    assert np.array_equal(Wp[:Q.size].view(np.int8).reshape(Q.shape), Q)
    got = Wp[Q.size:].view(np.float32).reshape(S.shape)
    assert np.array_equal(got.view(np.uint32), S.view(np.uint32))


@pytest.mark.parametrize("qtype", ["q4_K", "q6_K"])
@pytest.mark.parametrize("nt,od,id_", [(16, 256, 512), (70, 130, 768), (129, 257, 512), (1, 1, 256),
                                       (512, 3584, 3584)])
def test_prepared_gemm_matches_raw_bitwise(qig, qtype, nt, od, id_):
    gm = inputs.Gemm("prep", qtype, od, id_, nt)
    W, x = inputs.make_gemm_inputs(gm, inputs.SEED_BASE + 400 + nt)
    q8d = qig.quantize_q8_pad40(dev(x))
    Wd = dev(W)
    if qtype == "q6_K":
        y_raw = qig.mmq_q6k(Wd, 224, od, id_, q8d, nt)
        y_prep = qig.mmq_q6k_prepared(qig.prepare_q6k(Wd, 224, od, id_), od, id_, q8d, nt)
    else:
        y_raw = qig.mmq_q4k(Wd, od, id_, q8d, nt)
        y_prep = qig.mmq_q4k_prepared(qig.prepare_q4k(Wd, od, id_), od, id_, q8d, nt)
    y_raw, y_prep = host(y_raw), host(y_prep)
    assert np.array_equal(y_prep.view(np.uint32), y_raw.view(np.uint32))
    if nt * od <= 70 * 130:
        q8 = oracle.quantize_q8_pad40(x)
        _assert_close(y_prep, _oracle_gemm(qtype, W, od, id_, q8, nt), f"prepared {qtype} {nt}x{od}x{id_}")


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_workload_full(qig, cfg):
    for i, gm in enumerate(inputs.WORKLOADS[cfg]):
        _run_workload_gemm(qig, gm, inputs.SEED_BASE + cfg + 10 * i)


@pytest.mark.parametrize("i", range(len(inputs.WORKLOADS[4])))
def test_workload_layer_full(qig, i):
    """The nt=2630 layer: every output of each of its seven GEMMs."""
    gm = inputs.WORKLOADS[4][i]
    _run_workload_gemm(qig, gm, inputs.SEED_BASE + 4 + 10 * i)


def test_workload_layer_q6k_attn_v(qig):
    """The layer's v projection stored as q6_K (as the pages' model keeps it,
    r44 s2.4): 512 x 3584 at nt = 2630, every output."""
    _run_workload_gemm(qig, inputs.LAYER_Q6K_ATTN_V, inputs.SEED_BASE + 4 + 10 * 7)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("qtype", ["q4_K", "q6_K"])
def test_empty_and_strided_output(qig, qtype):
    g = inputs.rng(61)
    nt, od, id_ = 33, 70, 512
    W = _weights(qtype, g, od, id_)
    x = g.standard_normal((nt, id_), dtype=np.float32)
    q8 = oracle.quantize_q8_pad40(x)
    Wd, q8d = dev(W), dev(q8)
    # empty: nothing written
    y0 = torch.full((4, od), 7.0, device="cuda")
    _gpu_gemm(qig, qtype, Wd, od, id_, q8d, 0, y=y0, ldy=od)
    assert np.all(host(y0) == 7.0)
    # ldy > od: padding columns untouched, NaN-filled outputs overwritten
    ybig = torch.full((nt, od + 13), float("nan"), device="cuda")
    _gpu_gemm(qig, qtype, Wd, od, id_, q8d, nt, y=ybig, ldy=od + 13)
    yb = host(ybig)
    assert np.all(np.isnan(yb[:, od:]))
    _assert_close(yb[:, :od], _oracle_gemm(qtype, W, od, id_, q8, nt), "ldy")


@pytest.mark.parametrize("qtype", ["q4_K", "q6_K"])
def test_deterministic(qig, qtype):
    g = inputs.rng(71)
    nt, od, id_ = 300, 520, 1024
    W = _weights(qtype, g, od, id_)
    x = g.standard_normal((nt, id_), dtype=np.float32)
    Wd, q8d = dev(W), qig.quantize_q8_pad40(dev(x))
    a = host(_gpu_gemm(qig, qtype, Wd, od, id_, q8d, nt))
    b = host(_gpu_gemm(qig, qtype, Wd, od, id_, q8d, nt))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
