"""GPU parity of the tiled activation plane (quantization in the GEMM's
staging layout) and of the GEMMs that read it.

Bars: the tiled plane bit-exact against the oracle's pad40 quantization laid
out as the C header documents (quants with swizzled halves, fp32 d in
register order, -ssum split into bf16 hi + lo); every GEMM on the tiled plane
bit-identical to the same GEMM on the pad40 plane (whole tiles and stream-K),
and within the output tolerance of the oracle on small shapes.
"""
import numpy as np
import pytest

import layouts
import oracle
import xkinds
from quant_integer_gemm_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

REC = layouts.Q8T_RECORD


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


_tiled_expected = layouts.tiled_plane


@pytest.mark.parametrize("nt,id_,kind", [(16, 512, "normal"), (70, 768, "zeros"), (1, 256, "normal"),
                                         (129, 2304, "tiny"), (512, 3584, "normal"), (300, 18944, "heavy"),
                                         (64, 1024, "halves"), (130, 2048, "neartie"),
                                         (1000, 16384, "neartie")])   # 1024 records: two tokens per lane group
def test_tiled_plane_bit_exact(qig, nt, id_, kind):
    g = inputs.rng(4000 + nt + id_)
    x = xkinds.x_variant(g, nt, id_, kind)
    want = _tiled_expected(oracle.quantize_q8_pad40(x), nt, id_)
    got = host(qig.quantize_q8_tiled(dev(x)))
    assert got.size == qig.q8_tiled_bytes(nt, id_) == want.size
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]} (record offsets {bad[:8] % REC})"


def test_tiled_plane_row_stride(qig):
    g = inputs.rng(4100)
    x = g.standard_normal((37, 800), dtype=np.float32)
    want = _tiled_expected(oracle.quantize_q8_pad40(x, id_=768), 37, 768)
    got = host(qig.quantize_q8_tiled(dev(x), id_=768))
    assert np.array_equal(got, want)


ARMS = ["q4_K", "q4_K_prepared", "q6_K", "q6_K_wexp", "q6_K_prepared"]


def _gemm_pair(qig, arm, W, od, id_, q8d, q8td, nt, ws=None):
    """(y on pad40, y on the tiled plane) for one arm; ws: None or a stream-K workspace."""
    Wd = dev(W)
    if arm == "q4_K":
        a = qig.mmq_q4k_streamk(Wd, od, id_, q8d, nt, ws=ws) if ws is not None else qig.mmq_q4k(Wd, od, id_, q8d, nt)
        b = qig.mmq_q4k_q8t(Wd, od, id_, q8td, nt, ws=ws)
    elif arm in ("q6_K", "q6_K_wexp"):
        We = qig.expand_q6k_dense(Wd, 224, od, id_) if arm == "q6_K_wexp" else None
        a = (qig.mmq_q6k_streamk(Wd, 224, od, id_, q8d, nt, W_exp=We, ws=ws) if ws is not None
             else qig.mmq_q6k(Wd, 224, od, id_, q8d, nt, W_exp=We))
        b = qig.mmq_q6k_q8t(Wd, 224, od, id_, q8td, nt, W_exp=We, ws=ws)
    elif arm == "q4_K_prepared":
        Wp = qig.prepare_q4k(Wd, od, id_)
        a = (qig.mmq_q4k_prepared_streamk(Wp, od, id_, q8d, nt, ws=ws) if ws is not None
             else qig.mmq_q4k_prepared(Wp, od, id_, q8d, nt))
        b = qig.mmq_q4k_prepared_q8t(Wp, od, id_, q8td, nt, ws=ws)
    else:
        Wp = qig.prepare_q6k(Wd, 224, od, id_)
        a = (qig.mmq_q6k_prepared_streamk(Wp, od, id_, q8d, nt, ws=ws) if ws is not None
             else qig.mmq_q6k_prepared(Wp, od, id_, q8d, nt))
        b = qig.mmq_q6k_prepared_q8t(Wp, od, id_, q8td, nt, ws=ws)
    return host(a), host(b)


@pytest.mark.parametrize("arm", ARMS)
@pytest.mark.parametrize("nt,od,id_", [(16, 256, 512), (70, 130, 768), (129, 257, 512), (1, 1, 256),
                                       (512, 3584, 3584)])
def test_tiled_gemm_matches_pad40_bitwise(qig, arm, nt, od, id_):
    gm = inputs.Gemm("t", arm[:4], od, id_, nt)
    W, x = inputs.make_gemm_inputs(gm, inputs.SEED_BASE + 1100 + nt + od)
    xd = dev(x)
    y_pad, y_til = _gemm_pair(qig, arm, W, od, id_, qig.quantize_q8_pad40(xd), qig.quantize_q8_tiled(xd), nt)
    assert np.array_equal(y_til.view(np.uint32), y_pad.view(np.uint32))
    if nt * od <= 129 * 257:
        q8 = oracle.quantize_q8_pad40(x)
        ref = oracle.mmq_q4k(W, od, id_, q8, nt) if arm.startswith("q4") else oracle.mmq_q6k(W, 224, od, id_, q8, nt)
        ok, worst = oracle.within_tolerance(y_til, ref)
        assert ok, f"{arm} {nt}x{od}x{id_}: worst error/allowance = {worst:.3g}"


@pytest.mark.parametrize("arm", ARMS)
@pytest.mark.parametrize("nt,od,id_", [(100, 200, 2048), (64, 64, 10240), (2630, 512, 3584)])
def test_tiled_gemm_streamk_matches_pad40_bitwise(qig, arm, nt, od, id_):
    """Split tiles: the same decomposition and fix-up order on both planes."""
    gm = inputs.Gemm("t", arm[:4], od, id_, nt)
    W, x = inputs.make_gemm_inputs(gm, inputs.SEED_BASE + 1200 + nt + od)
    xd = dev(x)
    ws = qig.new_workspace("cuda")
    y_pad, y_til = _gemm_pair(qig, arm, W, od, id_, qig.quantize_q8_pad40(xd), qig.quantize_q8_tiled(xd), nt,
                              ws=ws)
    assert np.array_equal(y_til.view(np.uint32), y_pad.view(np.uint32))
    assert int(torch.count_nonzero(ws[-16384:]).item()) == 0


@pytest.mark.parametrize("nt,od,id_", [(2630, 3584, 18944), (512, 18944, 3584)])
def test_tiled_gemm_large_matches_pad40_bitwise(qig, nt, od, id_):
    """The layer's largest GEMMs (74 super-blocks per row; 296 row tiles) on
    both planes: bit-identical y."""
    qt = "q6_K" if id_ == 18944 else "q4_K"
    gm = inputs.Gemm("t", qt, od, id_, nt)
    W, x = inputs.make_gemm_inputs(gm, inputs.SEED_BASE + 1300 + nt)
    xd = dev(x)
    y_pad, y_til = _gemm_pair(qig, qt, W, od, id_, qig.quantize_q8_pad40(xd), qig.quantize_q8_tiled(xd), nt)
    assert np.array_equal(y_til.view(np.uint32), y_pad.view(np.uint32))


@pytest.mark.parametrize("arm", ["q4_K", "q6_K", "q6_K_wexp"])
def test_bench_path_full_oracle(qig, arm):
    """The step bench.py times, on its own inputs (its seeds, 512 x 3584 x
    3584): quantize_q8_tiled, then mmq_q4k_q8t or mmq_q6k_q8t on raw blocks or
    on the dense plane, whole tiles.  The tiled plane bit-exact against the
    oracle's quantization and every output within tolerance of the oracle."""
    import bench
    qt = arm[:4]
    gm = inputs.WORKLOADS[1][0] if qt == "q4_K" else inputs.WORKLOADS[2][0]
    assert (gm.nt, gm.od, gm.id) == (bench.NT, bench.OD, bench.ID)
    W, x = inputs.make_gemm_inputs(gm, bench.SEED4 if qt == "q4_K" else bench.SEED6)
    q8 = oracle.quantize_q8_pad40(x)
    q8td = qig.quantize_q8_tiled(dev(x))
    assert np.array_equal(host(q8td), _tiled_expected(q8, gm.nt, gm.id))
    Wd = dev(W)
    if qt == "q4_K":
        y = qig.mmq_q4k_q8t(Wd, gm.od, gm.id, q8td, gm.nt)
        ref = oracle.mmq_q4k(W, gm.od, gm.id, q8, gm.nt)
    else:
        We = qig.expand_q6k_dense(Wd, 224, gm.od, gm.id) if arm == "q6_K_wexp" else None
        y = qig.mmq_q6k_q8t(Wd, 224, gm.od, gm.id, q8td, gm.nt, W_exp=We)
        ref = oracle.mmq_q6k(W, 224, gm.od, gm.id, q8, gm.nt)
    y = host(y)
    assert np.isfinite(y).all()
    ok, worst = oracle.within_tolerance(y, ref)
    assert ok, f"bench {arm}: worst error/allowance = {worst:.3g}"
