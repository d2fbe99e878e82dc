"""GPU parity of the stream-K GEMM variants against the CPU oracle.

When the output tiles form one round that fills at most three quarters of
the workgroup slots, the stream-K calls share the (tile, super-block)
iterations evenly over all slots; a tile split between workgroups is summed
from their partials in a fixed order.  Other shapes run as whole tiles.
Bars: y within the output tolerance of the oracle's fp64 result;
bit-identical y across calls; the workspace's arrival counters back to zero
after every call.  The shapes give tiles split between 2 and 10 workgroups,
ragged token and row tails, the nt=2630 k/v projection (336 tiles, split)
and workload shapes that run as whole tiles through these entry points; every
output is compared with the oracle.
"""
import numpy as np
import pytest

import oracle
from quant_integer_gemm_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ARMS = ["q4_K", "q4_K_prepared", "q6_K", "q6_K_wexp", "q6_K_prepared"]


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


def _qtype(arm):
    return arm[:4]


class _Weights:
    """Device weights of one arm: raw blocks plus, as the arm needs, the dense
    q6_K plane or the prepared buffer."""

    def __init__(self, qig, arm, W, od, id_):
        self.arm, self.od, self.id = arm, od, id_
        self.Wd = dev(W)
        self.Wexp = qig.expand_q6k_dense(self.Wd, 224, od, id_) if arm == "q6_K_wexp" else None
        if arm == "q4_K_prepared":
            self.Wp = qig.prepare_q4k(self.Wd, od, id_)
        elif arm == "q6_K_prepared":
            self.Wp = qig.prepare_q6k(self.Wd, 224, od, id_)
        else:
            self.Wp = None

    def gemm(self, qig, q8d, nt, ws=None, streamk=True, y=None, ldy=None):
        od, id_ = self.od, self.id
        kw = dict(y=y, ldy=ldy)
        if streamk:
            kw["ws"] = ws
        a = self.arm
        if a == "q4_K":
            f = qig.mmq_q4k_streamk if streamk else qig.mmq_q4k
            return f(self.Wd, od, id_, q8d, nt, **kw)
        if a in ("q6_K", "q6_K_wexp"):
            f = qig.mmq_q6k_streamk if streamk else qig.mmq_q6k
            return f(self.Wd, 224, od, id_, q8d, nt, W_exp=self.Wexp, **kw)
        if a == "q4_K_prepared":
            f = qig.mmq_q4k_prepared_streamk if streamk else qig.mmq_q4k_prepared
        else:
            f = qig.mmq_q6k_prepared_streamk if streamk else qig.mmq_q6k_prepared
        return f(self.Wp, od, id_, q8d, nt, **kw)


def _inputs(arm, nt, od, id_, seed):
    gm = inputs.Gemm("sk", _qtype(arm), od, id_, nt)
    return inputs.make_gemm_inputs(gm, seed)


def _oracle(qtype, W, od, id_, q8, nt):
    if qtype == "q4_K":
        return oracle.mmq_q4k(W, od, id_, q8, nt)
    return oracle.mmq_q6k(W, 224, od, id_, q8, nt)


def _ws_clean(ws):
    """The arrival counters (the workspace's last 16384 bytes) are back to zero."""
    return int(torch.count_nonzero(ws[-16384:]).item()) == 0


# (nt, od, id): 64x64x10240 is one tile shared by 10 workgroups; 100x200x2048
# splits each of 8 tiles in two; 192x320x1792 and 33x700x4096 split tiles at
# uneven super-block boundaries (3 and 4 workgroups); 70x130x768 has ragged
# tails on both sides and too few super-blocks to split (whole tiles);
# 1x1x2560 is a single output split in two.
SPLIT_SHAPES = [(64, 64, 10240), (100, 200, 2048), (192, 320, 1792), (33, 700, 4096),
                (70, 130, 768), (1, 1, 2560)]


@pytest.mark.parametrize("arm", ARMS)
@pytest.mark.parametrize("nt,od,id_", SPLIT_SHAPES)
def test_streamk_matches_oracle(qig, arm, nt, od, id_):
    W, x = _inputs(arm, nt, od, id_, inputs.SEED_BASE + 500 + nt + od)
    q8 = oracle.quantize_q8_pad40(x)
    w = _Weights(qig, arm, W, od, id_)
    ws = qig.new_workspace("cuda")
    y = host(w.gemm(qig, dev(q8), nt, ws=ws))
    ok, worst = oracle.within_tolerance(y, _oracle(_qtype(arm), W, od, id_, q8, nt))
    assert ok, f"{arm} {nt}x{od}x{id_}: worst error/allowance = {worst:.3g}"
    assert _ws_clean(ws), "arrival counters not back to zero"


@pytest.mark.parametrize("arm", ["q4_K", "q6_K"])
def test_streamk_deterministic_and_shared_workspace(qig, arm):
    """Calls in order on one stream share a workspace across shapes; each
    shape's y is bit-identical from call to call."""
    ws = qig.new_workspace("cuda")
    shapes = [(100, 200, 2048), (64, 64, 10240), (192, 320, 1792)]
    first = {}
    for rep in range(2):
        for (nt, od, id_) in shapes:
            W, x = _inputs(arm, nt, od, id_, inputs.SEED_BASE + 600 + nt)
            w = _Weights(qig, arm, W, od, id_)
            y = host(w.gemm(qig, dev(oracle.quantize_q8_pad40(x)), nt, ws=ws))
            if rep == 0:
                first[(nt, od, id_)] = y
            else:
                assert np.array_equal(y.view(np.uint32), first[(nt, od, id_)].view(np.uint32))
            assert _ws_clean(ws)


@pytest.mark.parametrize("arm", ["q4_K", "q6_K"])
def test_streamk_strided_output_and_empty(qig, arm):
    nt, od, id_ = 100, 200, 2048
    W, x = _inputs(arm, nt, od, id_, inputs.SEED_BASE + 700)
    q8 = oracle.quantize_q8_pad40(x)
    w = _Weights(qig, arm, W, od, id_)
    ws = qig.new_workspace("cuda")
    q8d = dev(q8)
    y0 = torch.full((4, od), 7.0, device="cuda")
    w.gemm(qig, q8d, 0, ws=ws, y=y0, ldy=od)
    assert np.all(host(y0) == 7.0)
    ybig = torch.full((nt, od + 13), float("nan"), device="cuda")
    w.gemm(qig, q8d, nt, ws=ws, y=ybig, ldy=od + 13)
    yb = host(ybig)
    assert np.all(np.isnan(yb[:, od:]))
    ok, worst = oracle.within_tolerance(yb[:, :od], _oracle(_qtype(arm), W, od, id_, q8, nt))
    assert ok, f"worst error/allowance = {worst:.3g}"
    assert _ws_clean(ws)


_REF = {}


def _full_check(qig, arm, gm, seed):
    """Every output of the stream-K call and of the whole-tile call against the
    oracle (the tolerance's rms floor from the oracle's y)."""
    W, x = inputs.make_gemm_inputs(gm, seed)
    nt, od, id_ = gm.nt, gm.od, gm.id
    q8d = qig.quantize_q8_pad40(dev(x))
    q8 = host(q8d)
    key = (gm.qtype, nt, od, id_, seed)
    if key not in _REF:
        _REF.clear()
        _REF[key] = _oracle(gm.qtype, W, od, id_, q8, nt)
    y_ref = _REF[key]
    w = _Weights(qig, arm, W, od, id_)
    ws = qig.new_workspace("cuda")
    y = host(w.gemm(qig, q8d, nt, ws=ws))
    y_dp = host(w.gemm(qig, q8d, nt, streamk=False))
    assert _ws_clean(ws)
    for name, v in (("stream-K", y), ("whole tiles", y_dp)):
        assert np.isfinite(v).all(), f"{gm.name} {arm} {name}: non-finite outputs"
        ok, worst = oracle.within_tolerance(v, y_ref)
        assert ok, f"{gm.name} {arm} {name}: worst error/allowance vs oracle = {worst:.3g}"


@pytest.mark.parametrize("arm", ARMS)
def test_streamk_projection_shape(qig, arm):
    """nt=512 x 3584 x 3584: 448 tiles fill 7/8 of the 512 workgroup slots,
    so the call runs whole tiles (the entry point's fallback)."""
    gm = inputs.Gemm("proj", _qtype(arm), 3584, 3584, 512)
    _full_check(qig, arm, gm, inputs.SEED_BASE + 800)


@pytest.mark.parametrize("name", ["attn_k", "attn_q", "ffn_down"])
def test_streamk_layer_shapes(qig, name):
    """nt=2630 layer shapes: k/v (336 tiles, split over all 512 slots); q/o
    and down (several rounds of tiles: whole tiles)."""
    gm = next(g for g in inputs.WORKLOADS[4] if name in g.name)
    _full_check(qig, gm.qtype, gm, inputs.SEED_BASE + 900)
