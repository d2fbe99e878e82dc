"""GPU parity of the staged q4_K buffer (records that are the bytes of the
GEMM's LDS weight stage) and of the GEMM that reads it.

Bars: the records bit-exact against values built here from the oracle's
block decoder, per the layout the C header states (nibble units swizzled
per row, d*sc and -M*d*sc as fp32, dmin*m split into bf16 hi + lo, zero rows
past od); the GEMM's y bit-identical to mmq_q4k_q8t on the raw blocks (whole
tiles and stream-K) and within the output tolerance of the oracle."""
import numpy as np
import pytest

import layouts
import oracle
from quant_integer_gemm_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

REC = layouts.Q4S_RECORD


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


_expected_records = layouts.staged_records


@pytest.mark.parametrize("od,id_", [(130, 512), (64, 256), (1, 768)])
def test_staged_records_bit_exact(qig, od, id_):
    g = inputs.rng(7600 + od)
    W = inputs.q4k_weights(g, od, id_)
    got = host(qig.prepare_q4k_staged(dev(W), od, id_))
    assert got.size == qig.q4k_staged_bytes(od, id_) == (od + 63) // 64 * (id_ // 256) * REC
    want = _expected_records(W, od, id_)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]} (record offsets {bad[:8] % REC})"


def _pair(qig, W, x, od, id_, nt, ws=None):
    Wd = dev(W)
    q8t = qig.quantize_q8_tiled(dev(x))
    Ws = qig.prepare_q4k_staged(Wd, od, id_)
    a = host(qig.mmq_q4k_staged_q8t(Ws, od, id_, q8t, nt, ws=ws))
    b = host(qig.mmq_q4k_q8t(Wd, od, id_, q8t, nt, ws=ws))
    return a, b


@pytest.mark.parametrize("nt,od,id_", [(16, 256, 512), (70, 130, 768), (129, 257, 512), (1, 1, 256),
                                       (512, 3584, 3584), (2000, 1100, 512)])
def test_staged_gemm_matches_raw_bitwise(qig, nt, od, id_):
    gm = inputs.Gemm("s", "q4_K", od, id_, nt)
    W, x = inputs.make_gemm_inputs(gm, inputs.SEED_BASE + 7700 + nt + od)
    y_s, y_r = _pair(qig, W, x, od, id_, nt)
    assert np.isfinite(y_s).all()
    assert np.array_equal(y_s.view(np.uint32), y_r.view(np.uint32))
    if nt * od <= 129 * 257:
        ref = oracle.mmq_q4k(W, od, id_, oracle.quantize_q8_pad40(x), nt)
        ok, worst = oracle.within_tolerance(y_s, ref)
        assert ok, f"{nt}x{od}x{id_}: worst error/allowance = {worst:.3g}"


@pytest.mark.parametrize("nt,od,id_", [(100, 200, 2048), (64, 64, 10240), (2630, 512, 3584)])
def test_staged_gemm_streamk_matches_raw_bitwise(qig, nt, od, id_):
    gm = inputs.Gemm("s", "q4_K", od, id_, nt)
    W, x = inputs.make_gemm_inputs(gm, inputs.SEED_BASE + 7800 + nt + od)
    ws = qig.new_workspace("cuda")
    y_s, y_r = _pair(qig, W, x, od, id_, nt, ws=ws)
    assert np.array_equal(y_s.view(np.uint32), y_r.view(np.uint32))
    assert int(torch.count_nonzero(ws[-16384:]).item()) == 0


def test_staged_bench_inputs_full_oracle(qig):
    """The bench's q4_K inputs (its seed, 512 x 3584 x 3584): every output
    within tolerance of the oracle."""
    import bench
    gm = inputs.WORKLOADS[1][0]
    W, x = inputs.make_gemm_inputs(gm, bench.SEED4)
    Ws = qig.prepare_q4k_staged(dev(W), gm.od, gm.id)
    y = host(qig.mmq_q4k_staged_q8t(Ws, gm.od, gm.id, qig.quantize_q8_tiled(dev(x)), gm.nt))
    ok, worst = oracle.within_tolerance(y, oracle.mmq_q4k(W, gm.od, gm.id, oracle.quantize_q8_pad40(x), gm.nt))
    assert ok, f"worst error/allowance = {worst:.3g}"
