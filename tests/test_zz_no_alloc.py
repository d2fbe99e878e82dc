"""GPU check of mmq_q4k_q8t_noalloc, the variant of mmq_q4k_q8t whose stream-K
workspace is the library's own device array (for callers that cannot
allocate).  Called through the C ABI with raw device pointers; its y must be
bit-identical to mmq_q4k_q8t with a caller-owned workspace (same split, same
fixed fix-up order) and within tolerance of the oracle, on two calls in a row
with the second input smaller, and on a shape that runs as whole tiles.
"""
import ctypes

import numpy as np
import pytest

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


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _case(qig, nt, od, id_, seed):
    W, x = inputs.make_gemm_inputs(inputs.Gemm("na", "q4_K", od, id_, nt), seed)
    Wd = torch.from_numpy(W).cuda()
    q8t = qig.quantize_q8_tiled(torch.from_numpy(x).cuda())
    y_na = torch.full((nt, od), float("nan"), device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    print(f"noalloc case nt={nt} od={od} id={id_} seed={seed}", flush=True)
    rc = qig.load().mmq_q4k_q8t_noalloc(_ptr(Wd), od, id_, _ptr(q8t), nt, _ptr(y_na), od, stream)
    assert rc == 0, f"mmq_q4k_q8t_noalloc returned {rc}"
    ws = qig.new_workspace("cuda")
    y_ws = qig.mmq_q4k_q8t(Wd, od, id_, q8t, nt, ws=ws)
    torch.cuda.synchronize()
    a, b = y_na.cpu().numpy(), y_ws.cpu().numpy()
    assert np.isfinite(a).all()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "differs from mmq_q4k_q8t with a workspace"
    q8 = oracle.quantize_q8_pad40(x)
    ok, worst = oracle.within_tolerance(a, oracle.mmq_q4k(W, od, id_, q8, nt))
    assert ok, f"worst error/allowance vs oracle = {worst:.3g}"


def test_noalloc_matches_workspace_call(qig):
    # 336 tiles over 512 workgroups (split), then 8 tiles over 16 (split,
    # smaller), then the same large split again (counters cleared each call),
    # then 448 tiles (whole tiles: the scratch is not touched)
    _case(qig, 2630, 512, 3584, inputs.SEED_BASE + 1500)
    _case(qig, 100, 200, 2048, inputs.SEED_BASE + 1501)
    _case(qig, 2630, 512, 3584, inputs.SEED_BASE + 1502)
    _case(qig, 512, 3584, 3584, inputs.SEED_BASE + 1503)


def test_noalloc_argument_checks(qig):
    lib = qig.load()
    A16 = ctypes.c_void_p(0x10000)
    assert lib.mmq_q4k_q8t_noalloc(A16, 8, 300, A16, 4, A16, 8, None) == -1        # id % 256
    assert lib.mmq_q4k_q8t_noalloc(A16, 8, 256, A16, 4, A16, 7, None) == -1        # ldy < od
    assert lib.mmq_q4k_q8t_noalloc(ctypes.c_void_p(0x10001), 8, 256, A16, 4, A16, 8, None) == -2
    assert lib.mmq_q4k_q8t_noalloc(A16, 8, 256, A16, 0, A16, 8, None) == 0         # nt == 0
