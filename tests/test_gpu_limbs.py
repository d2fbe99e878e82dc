"""GPU parity of the q6_K limb arm (sub-block scales folded into two int8
limbs per element, v = sc * c6 = 128 H + L) against the CPU oracle.

Bars: the limb buffer's H, L and d planes bit-exact against limbs computed
from the oracle's block decoder (and 128 H + L == sc * c6 everywhere); y within
the output tolerance of the oracle's fp64 result on ragged shapes, at the
largest |Q| the format allows, through stream-K splits and at the bench shape;
exact on the integer special case.
"""
import numpy as np
import pytest

import layouts
import oracle
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


_expected_planes = layouts.limb_planes


@pytest.mark.parametrize("od,id_,bstride", [(130, 768, 224), (64, 256, 240), (17, 512, 224)])
def test_limb_planes_content(qig, od, id_, bstride):
    g = inputs.rng(7000 + od)
    W = inputs.q6k_weights(g, od, id_, bstride=bstride, sc_range=(-128, 127))
    buf = host(qig.prepare_q6k_limbs(dev(W), bstride, od, id_))
    assert buf.size == qig.q6k_limbs_bytes(od, id_) == 2 * od * id_ + od * (id_ // 256) * 4
    H, L, d = _expected_planes(W, bstride, od, id_)
    assert np.array_equal(buf[:od * id_].view(np.int8).reshape(od, id_), H)
    assert np.array_equal(buf[od * id_:2 * od * id_].view(np.int8).reshape(od, id_), L)
    assert np.array_equal(buf[2 * od * id_:].view(np.float32).reshape(od, -1), d)


def _limbs_y(qig, W, x, od, id_, nt, ws=None, y=None, ldy=None):
    Wd = dev(W)
    Wl = qig.prepare_q6k_limbs(Wd, 224, od, id_)
    q8t = qig.quantize_q8_tiled(dev(x))
    return host(qig.mmq_q6k_limbs_q8t(Wl, od, id_, q8t, nt, ws=ws, y=y, ldy=ldy))


# (2000, 1100, 512): 32 x 18 = 576 whole tiles, more than one round of two
# per CU, so the launch takes the three-per-CU build of the kernel
SHAPES = [(16, 256, 512), (1, 1, 256), (70, 130, 768), (129, 257, 512), (64, 128, 256), (200, 300, 1024),
          (3, 1000, 256), (65, 129, 2304), (512, 3584, 3584), (2000, 1100, 512)]


@pytest.mark.parametrize("nt,od,id_", SHAPES)
def test_limbs_gemm_matches_oracle(qig, nt, od, id_):
    gm = inputs.Gemm("limbs", "q6_K", od, id_, nt)
    W, x = inputs.make_gemm_inputs(gm, inputs.SEED_BASE + 7100 + nt + od)
    y = _limbs_y(qig, W, x, od, id_, nt)
    assert np.isfinite(y).all()
    ok, worst = oracle.within_tolerance(y, oracle.mmq_q6k(W, 224, od, id_, oracle.quantize_q8_pad40(x), nt))
    assert ok, f"{nt}x{od}x{id_}: worst error/allowance = {worst:.3g}"


def test_limbs_bench_inputs(qig):
    """The bench's q6_K inputs (its seed, 512 x 3584 x 3584), every output."""
    import bench
    gm = inputs.WORKLOADS[2][0]
    W, x = inputs.make_gemm_inputs(gm, bench.SEED6)
    y = _limbs_y(qig, W, x, gm.od, gm.id, gm.nt)
    ok, worst = oracle.within_tolerance(y, oracle.mmq_q6k(W, 224, gm.od, gm.id, oracle.quantize_q8_pad40(x), gm.nt))
    assert ok, f"worst error/allowance = {worst:.3g}"


def test_limbs_extreme_magnitudes(qig):
    """Scales -128 / 127, every quant -32 or +31 and activations +-127: the
    chunk sums reach |Q| = 32 * 127 * 4096 (near 2^24), where the limb
    combination must stay exact."""
    g = inputs.rng(7200)
    nt, od, id_ = 70, 130, 512
    x = np.where(g.random((nt, id_)) < 0.5, -127.0, 127.0).astype(np.float32)
    x[: nt // 2] = 127.0
    W = inputs.q6k_weights(g, od, id_).reshape(od, -1, 224)
    W[: od // 2, :, 0:192] = 0x00          # every quant -32
    W[od // 2:, :, 0:192] = 0xFF           # every quant +31
    W[:, :, 192:208] = np.where(np.arange(16) % 2 == 0, -128, 127).astype(np.int8).view(np.uint8)
    W[: od // 4, :, 192:208] = np.array([-128], dtype=np.int8).view(np.uint8)   # sc * c6 = 4096 throughout
    W[:, :, 208:210] = np.array([0.5], dtype=np.float16).view(np.uint8)
    W = W.reshape(od, -1)
    q8 = oracle.quantize_q8_pad40(x)
    y = _limbs_y(qig, W, x, od, id_, nt)
    y_ref = oracle.mmq_q6k(W, 224, od, id_, q8, nt)
    assert np.max(np.abs(y_ref)) >= 32 * 127 * 4096 * 0.5 * 16     # all 16 chunks at the bound, d = 0.5
    ok, worst = oracle.within_tolerance(y, y_ref)
    assert ok, f"worst error/allowance = {worst:.3g}"


def test_limbs_integer_special_case_exact(qig):
    """d = 1, unit scales and integer activations with max |x| = 127 per chunk:
    y equals the integer matmul exactly."""
    g = inputs.rng(7300)
    nt, od, id_ = 70, 150, 512
    x = g.integers(-127, 128, size=(nt, id_)).astype(np.float32)
    x[:, ::32] = 127.0
    W = inputs.q6k_weights(g, od, id_).reshape(od, -1, 224)
    W[:, :, 192:208] = 1
    W[:, :, 208:210] = np.array([1.0], dtype=np.float16).view(np.uint8)
    W = W.reshape(od, -1)
    wq = oracle.expand_q6k_dense(W, 224, od, id_).astype(np.int64)
    want = (x.astype(np.int64) @ wq.T).astype(np.float64)
    y = _limbs_y(qig, W, x, od, id_, nt)
    assert np.array_equal(y.astype(np.float64), want)


# (2000, 1100, 512): 576 tiles, more than two per CU but at most 3/4 of three
# per CU, so the split runs on the three-per-CU build over all its slots
@pytest.mark.parametrize("nt,od,id_", [(64, 64, 10240), (100, 200, 2048), (33, 700, 4096), (2630, 512, 3584),
                                       (2000, 1100, 512)])
def test_limbs_streamk_matches_oracle(qig, nt, od, id_):
    """Tiles split between workgroups (stream-K workspace): within tolerance,
    counters back to zero, and y bit-identical from call to call."""
    gm = inputs.Gemm("limbs", "q6_K", od, id_, nt)
    W, x = inputs.make_gemm_inputs(gm, inputs.SEED_BASE + 7400 + nt + od)
    ws = qig.new_workspace("cuda")
    y = _limbs_y(qig, W, x, od, id_, nt, ws=ws)
    y2 = _limbs_y(qig, W, x, od, id_, nt, ws=ws)
    assert int(torch.count_nonzero(ws[-16384:]).item()) == 0
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    ok, worst = oracle.within_tolerance(y, oracle.mmq_q6k(W, 224, od, id_, oracle.quantize_q8_pad40(x), nt))
    assert ok, f"{nt}x{od}x{id_}: worst error/allowance = {worst:.3g}"


def test_limbs_strided_output_and_empty(qig):
    nt, od, id_ = 70, 130, 768
    gm = inputs.Gemm("limbs", "q6_K", od, id_, nt)
    W, x = inputs.make_gemm_inputs(gm, inputs.SEED_BASE + 7500)
    Wl = qig.prepare_q6k_limbs(dev(W), 224, od, id_)
    q8t = qig.quantize_q8_tiled(dev(x))
    y0 = torch.full((4, od), 7.0, device="cuda")
    qig.mmq_q6k_limbs_q8t(Wl, od, id_, q8t, 0, y=y0, ldy=od)
    assert np.all(host(y0) == 7.0)
    ybig = torch.full((nt, od + 13), float("nan"), device="cuda")
    qig.mmq_q6k_limbs_q8t(Wl, od, id_, q8t, nt, y=ybig, ldy=od + 13)
    yb = host(ybig)
    assert np.all(np.isnan(yb[:, od:]))
    ok, worst = oracle.within_tolerance(yb[:, :od], oracle.mmq_q6k(W, 224, od, id_, oracle.quantize_q8_pad40(x), nt))
    assert ok, f"worst error/allowance = {worst:.3g}"
