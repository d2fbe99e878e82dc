"""GPU parity of the q4_K GEMM that quantizes its own activations
(mmq_q4k_xf32): y bit-identical to the tiled prepass followed by the tiled
GEMM (whole tiles and stream-K), on ragged shapes, the layer's k/v projection
and the q-projection shape, with a row stride, and within the output
tolerance of the oracle."""
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


def _pair(qig, W, od, id_, x, ws=None):
    Wd, xd = dev(W), dev(x)
    a = qig.mmq_q4k_xf32(Wd, od, id_, xd, ws=ws)
    b = qig.mmq_q4k_q8t(Wd, od, id_, qig.quantize_q8_tiled(xd), x.shape[0], ws=ws)
    return host(a), host(b)


@pytest.mark.parametrize("nt,od,id_", [(16, 256, 512), (70, 130, 768), (129, 257, 512), (1, 1, 256),
                                       (512, 3584, 3584), (2630, 512, 3584)])
def test_xf32_matches_prepass_bitwise(qig, nt, od, id_):
    gm = inputs.Gemm("t", "q4_K", od, id_, nt)
    W, x = inputs.make_gemm_inputs(gm, inputs.SEED_BASE + 1400 + nt + od)
    y_f, y_p = _pair(qig, W, od, id_, x)
    assert np.isfinite(y_f).all()
    assert np.array_equal(y_f.view(np.uint32), y_p.view(np.uint32))
    if nt * od <= 129 * 257:
        ref = oracle.mmq_q4k(W, od, id_, oracle.quantize_q8_pad40(x), nt)
        ok, worst = oracle.within_tolerance(y_f, ref)
        assert ok, f"{nt}x{od}x{id_}: worst error/allowance = {worst:.3g}"


@pytest.mark.parametrize("nt,od,id_", [(100, 200, 2048), (64, 64, 10240), (2630, 512, 3584)])
def test_xf32_streamk_matches_prepass_bitwise(qig, nt, od, id_):
    gm = inputs.Gemm("t", "q4_K", od, id_, nt)
    W, x = inputs.make_gemm_inputs(gm, inputs.SEED_BASE + 1500 + nt + od)
    ws = qig.new_workspace("cuda")
    y_f, y_p = _pair(qig, W, od, id_, x, ws=ws)
    assert np.array_equal(y_f.view(np.uint32), y_p.view(np.uint32))
    assert int(torch.count_nonzero(ws[-16384:]).item()) == 0


@pytest.mark.parametrize("kind", ["zeros", "tiny", "heavy", "neartie", "halves"])
def test_xf32_activation_kinds(qig, kind):
    """The in-kernel quantization takes the same rounding decisions as the
    prepass on exact and near ties, zero chunks, tiny and heavy-tailed values."""
    nt, od, id_ = 70, 96, 1024
    g = inputs.rng(4600 + len(kind))
    W, _ = inputs.make_gemm_inputs(inputs.Gemm("t", "q4_K", od, id_, nt), inputs.SEED_BASE + 1600)
    x = xkinds.x_variant(g, nt, id_, kind)
    y_f, y_p = _pair(qig, W, od, id_, x)
    assert np.array_equal(y_f.view(np.uint32), y_p.view(np.uint32))
    ref = oracle.mmq_q4k(W, od, id_, oracle.quantize_q8_pad40(x), nt)
    ok, worst = oracle.within_tolerance(y_f, ref)
    assert ok, f"{kind}: worst error/allowance = {worst:.3g}"


def test_xf32_row_stride_and_empty(qig):
    nt, od, id_ = 37, 80, 768
    W, _ = inputs.make_gemm_inputs(inputs.Gemm("t", "q4_K", od, id_, nt), inputs.SEED_BASE + 1700)
    xw = inputs.rng(4700).standard_normal((nt, 800), dtype=np.float32)
    Wd = dev(W)
    y_f = host(qig.mmq_q4k_xf32(Wd, od, id_, dev(xw)))
    y_p = host(qig.mmq_q4k_q8t(Wd, od, id_, qig.quantize_q8_tiled(dev(xw), id_=id_), nt))
    assert np.array_equal(y_f.view(np.uint32), y_p.view(np.uint32))
    e = qig.mmq_q4k_xf32(Wd, od, id_, dev(np.zeros((0, id_), dtype=np.float32)))
    assert tuple(e.shape) == (0, od)
