"""CPU-only checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import quant_integer_gemm_amd as qig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qig.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s*([A-Za-z_]\w*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for n in ["quantize_q8_pad40", "mmq_q4k", "mmq_q6k", "expand_q6k_dense", "q8_pad40_bytes",
              "qig_strerror", "mmq_q4k_partials", "mmq_q6k_partials", "q4k_prepared_bytes",
              "q6k_prepared_bytes", "prepare_q4k", "prepare_q6k", "mmq_q4k_prepared", "mmq_q6k_prepared",
              "mmq_workspace_bytes", "mmq_q4k_streamk", "mmq_q6k_streamk", "mmq_q4k_prepared_streamk",
              "mmq_q6k_prepared_streamk", "q8_tiled_bytes", "quantize_q8_tiled", "mmq_q4k_q8t", "mmq_q6k_q8t",
              "mmq_q4k_prepared_q8t", "mmq_q6k_prepared_q8t"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = qig.load()
    for n in _declared_functions():
        assert hasattr(lib, n), n
        assert n in qig._lib.SIGNATURES, n


def test_sizes_and_strerror():
    assert qig.q8_pad40_bytes(512, 3584) == 512 * 112 * 40
    assert qig.q8_pad40_bytes(0, 256) == 0
    assert qig.q8_pad40_bytes(3, 33) == 0
    assert qig.q8_pad40_bytes(-1, 32) == 0
    lib = qig.load()
    assert lib.qig_strerror(0) == b"ok"
    assert lib.qig_strerror(-1).startswith(b"invalid")
    assert lib.qig_strerror(-2).startswith(b"pointer")
    assert lib.qig_strerror(-3).startswith(b"HIP")
    assert lib.qig_strerror(7) == b"unknown error"


A16 = ctypes.c_void_p(0x10000)     # aligned fake device addresses, never dereferenced:
B16 = ctypes.c_void_p(0x20000)     # every call below fails its argument check first
MIS = ctypes.c_void_p(0x10004)


@pytest.mark.parametrize("args,rc", [
    ((A16, 4, 100, 100, B16, None), -1),      # id % 32
    ((A16, -1, 64, 64, B16, None), -1),       # nt < 0
    ((A16, 4, 64, 32, B16, None), -1),        # ldx < id
    ((MIS, 4, 64, 64, B16, None), -2),        # x misaligned
    ((A16, 4, 64, 66, B16, None), -2),        # ldx % 4
    ((A16, 4, 64, 64, MIS, None), -2),        # q8 misaligned
    ((A16, 0, 64, 64, B16, None), 0),         # empty: no-op
])
def test_quantize_argument_checks(args, rc):
    assert qig.load().quantize_q8_pad40(*args) == rc


@pytest.mark.parametrize("args,rc", [
    ((A16, 8, 300, B16, 4, A16, 8, None), -1),     # id % 256
    ((A16, 8, 0, B16, 4, A16, 8, None), -1),       # id == 0
    ((A16, -8, 256, B16, 4, A16, 8, None), -1),    # od < 0
    ((A16, 8, 256, B16, 4, A16, 7, None), -1),     # ldy < od
    ((MIS, 8, 256, B16, 4, A16, 8, None), -2),
    ((A16, 8, 256, MIS, 4, A16, 8, None), -2),
    ((A16, 8, 256, B16, 4, ctypes.c_void_p(0x10002), 8, None), -2),
    ((A16, 8, 256, B16, 0, A16, 8, None), 0),      # nt == 0
    ((A16, 0, 256, B16, 4, A16, 0, None), 0),      # od == 0
])
def test_mmq_q4k_argument_checks(args, rc):
    assert qig.load().mmq_q4k(*args) == rc


@pytest.mark.parametrize("args,rc", [
    ((A16, 208, None, 8, 256, B16, 4, A16, 8, None), -1),   # bstride < 210
    ((A16, 216, None, 8, 256, B16, 4, A16, 8, None), -1),   # bstride % 16
    ((A16, 224, MIS, 8, 256, B16, 4, A16, 8, None), -2),    # W_exp misaligned
    ((A16, 224, None, 8, 512, B16, 0, A16, 8, None), 0),
    ((A16, 224, None, 8, 1 << 25, B16, 4, A16, 8, None), -1),      # tile span beyond 32-bit offsets
    ((A16, 1 << 20, None, 8, 1 << 14, B16, 4, A16, 8, None), -1),  # id * bstride / 4 >= 2^31
])
def test_mmq_q6k_argument_checks(args, rc):
    assert qig.load().mmq_q6k(*args) == rc


def test_expand_and_partials_argument_checks():
    lib = qig.load()
    assert lib.expand_q6k_dense(A16, 224, 4, 100, B16, None) == -1
    assert lib.expand_q6k_dense(A16, 200, 4, 256, B16, None) == -1
    assert lib.expand_q6k_dense(MIS, 224, 4, 256, B16, None) == -2
    assert lib.expand_q6k_dense(A16, 224, 0, 256, B16, None) == 0
    # window outside the output
    assert lib.mmq_q4k_partials(A16, 8, 256, B16, 4, 0, 5, 0, 8, A16, None) == -1
    assert lib.mmq_q4k_partials(A16, 8, 256, B16, 4, 2, 1, 0, 8, A16, None) == -1
    assert lib.mmq_q6k_partials(A16, 224, None, 8, 256, B16, 4, 0, 4, 0, 9, A16, None) == -1
    # empty window
    assert lib.mmq_q6k_partials(A16, 224, None, 8, 256, B16, 4, 1, 1, 0, 8, A16, None) == 0


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(2, 32)
    with pytest.raises(qig.QigError):
        qig.quantize_q8_pad40(x)


def test_binding_checks_buffer_sizes_before_any_launch():
    """Tensors too small for the bytes a call touches are refused in the
    binding (before a pointer reaches the library); right-sized host tensors
    pass these checks and are then refused as host memory."""
    torch = pytest.importorskip("torch")
    nt, od, id_ = 5, 3, 512
    W4 = torch.zeros(od * 2 * 144, dtype=torch.uint8)
    W6 = torch.zeros(od * 2 * 224, dtype=torch.uint8)
    q8 = torch.zeros(qig.q8_pad40_bytes(nt, id_), dtype=torch.uint8)
    q8t = torch.zeros(qig.q8_tiled_bytes(nt, id_), dtype=torch.uint8)

    def refused(fn, words):
        with pytest.raises(qig.QigError) as e:
            fn()
        assert all(w in str(e.value) for w in words), str(e.value)

    refused(lambda: qig.mmq_q4k(W4[:-1], od, id_, q8, nt), ["W holds"])
    refused(lambda: qig.mmq_q4k(W4, od, id_, q8[:-1], nt), ["q8 holds"])
    refused(lambda: qig.mmq_q6k(W6, 224, od, id_, q8, nt, W_exp=torch.zeros(od * id_ - 1, dtype=torch.int8)),
            ["W_exp holds"])
    refused(lambda: qig.mmq_q6k(W6, 240, od, id_, q8, nt), ["W holds"])          # wider block stride
    refused(lambda: qig.mmq_q4k_q8t(W4, od, id_, q8t[:-1], nt), ["q8 holds"])
    refused(lambda: qig.mmq_q4k_q8t(W4, od, id_, q8t, nt, ws=torch.zeros(16, dtype=torch.uint8)), ["ws holds"])
    refused(lambda: qig.mmq_q4k(W4, od, id_, q8, nt, y=torch.zeros(nt, od - 1)), ["y must cover"])
    refused(lambda: qig.mmq_q4k(W4, od, id_, q8, nt, y=torch.zeros(nt, od + 4)[:, :od], ldy=od), ["y must cover"])
    refused(lambda: qig.mmq_q4k(W4, od, id_, q8, nt, y=torch.zeros((nt - 1) * 8 + od - 1), ldy=8),
            ["1-D y"])
    refused(lambda: qig.mmq_q4k_prepared(torch.zeros(qig.prepared_bytes("q4_K", od, id_) - 1, dtype=torch.uint8),
                                         od, id_, q8, nt), ["W holds"])
    refused(lambda: qig.quantize_q8_pad40(torch.zeros(nt, id_), out=torch.zeros(8, dtype=torch.uint8)),
            ["out holds"])
    refused(lambda: qig.quantize_q8_tiled(torch.zeros(nt, id_), out=q8t[:-1]), ["out holds"])
    refused(lambda: qig.expand_q6k_dense(W6, 224, od, id_, out=torch.zeros(od, id_ - 1, dtype=torch.int8)),
            ["out holds"])
    refused(lambda: qig.mmq_q4k(torch.zeros(od, 2 * 288, dtype=torch.uint8)[:, ::2], od, id_, q8, nt), ["contiguous"])
    # right sizes: past the checks, refused as host memory
    refused(lambda: qig.mmq_q4k(W4, od, id_, q8, nt), ["GPU tensor"])
    refused(lambda: qig.mmq_q6k_q8t(W6, 224, od, id_, q8t, nt, y=torch.zeros(nt, od + 4), ldy=od + 4),
            ["GPU tensor"])


def test_binding_checks_activation_rows():
    """The quantizers read the first id columns of each of nt rows: id may not
    exceed the width of x (one row, or a column-sliced view alike), and the row
    stride is the tensor's own.  Refused before any pointer reaches the
    library; right-shaped host tensors are then refused as host memory."""
    torch = pytest.importorskip("torch")

    def refused(fn, words):
        with pytest.raises(qig.QigError) as e:
            fn()
        assert all(w in str(e.value) for w in words), str(e.value)

    big = torch.zeros(4, 512)
    for quant in (qig.quantize_q8_pad40, qig.quantize_q8_tiled):
        refused(lambda: quant(torch.zeros(1, 160), id_=256), ["exceeds", "160 columns"])     # one row
        refused(lambda: quant(big[:, :256], id_=512), ["exceeds", "256 columns"])           # sliced view
        refused(lambda: quant(big[1:2, :256], id_=512), ["exceeds"])                        # one sliced row
        refused(lambda: quant(big[:, :256]), ["GPU tensor"])                                # the view itself
        refused(lambda: quant(torch.zeros(1, 256)), ["GPU tensor"])
        refused(lambda: quant(torch.zeros(5, 512, dtype=torch.float64)), ["fp32"])
        refused(lambda: quant(big.t()), ["unit column stride"])


def test_oracle_not_imported_by_product():
    """The product package never imports the oracle."""
    pkg = os.path.join(ROOT, "quant_integer_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "qig_oracle" not in text, f


def test_prepared_sizes_and_argument_checks():
    lib = qig.load()
    assert qig.prepared_bytes("q4_K", 3584, 3584) == 3584 * 1792 + 3584 * 14 * 64
    assert qig.prepared_bytes("q6_K", 256, 512) == 256 * 512 + 256 * 2 * 64
    assert lib.q4k_prepared_bytes(4, 100) == 0
    assert lib.q6k_prepared_bytes(-1, 256) == 0
    assert lib.prepare_q4k(A16, 4, 100, B16, None) == -1          # id % 256
    assert lib.prepare_q4k(MIS, 4, 256, B16, None) == -2
    assert lib.prepare_q4k(A16, 4, 256, MIS, None) == -2
    assert lib.prepare_q4k(A16, 0, 256, B16, None) == 0
    assert lib.prepare_q6k(A16, 200, 4, 256, B16, None) == -1     # bstride
    assert lib.prepare_q6k(A16, 224, 4, 256, MIS, None) == -2
    assert lib.mmq_q4k_prepared(A16, 8, 100, B16, 4, A16, 8, None) == -1   # id % 256
    assert lib.mmq_q4k_prepared(MIS, 8, 256, B16, 4, A16, 8, None) == -2
    assert lib.mmq_q6k_prepared(A16, 8, 256, B16, 4, A16, 4, None) == -1   # ldy < od
    assert lib.mmq_q6k_prepared(A16, 8, 256, B16, 0, A16, 8, None) == 0    # nt == 0


def test_streamk_workspace_and_argument_checks():
    lib = qig.load()
    # two 64x64 fp32 partial slots and four counters per workgroup, 1024 workgroups at most
    assert lib.mmq_workspace_bytes() == 1024 * 2 * 64 * 64 * 4 + 1024 * 16
    assert lib.mmq_q4k_streamk(A16, 8, 256, B16, 4, A16, 8, None, None) == -1          # no workspace
    assert lib.mmq_q4k_streamk(A16, 8, 256, B16, 4, A16, 8, MIS, None) == -2           # misaligned workspace
    assert lib.mmq_q4k_streamk(A16, 8, 300, B16, 4, A16, 8, A16, None) == -1           # id % 256
    assert lib.mmq_q4k_streamk(A16, 8, 256, B16, 0, A16, 8, A16, None) == 0            # nt == 0
    assert lib.mmq_q6k_streamk(A16, 208, None, 8, 256, B16, 4, A16, 8, A16, None) == -1   # bstride
    assert lib.mmq_q6k_streamk(A16, 224, MIS, 8, 256, B16, 4, A16, 8, A16, None) == -2    # W_exp
    assert lib.mmq_q6k_streamk(A16, 224, None, 8, 256, B16, 4, A16, 8, None, None) == -1
    assert lib.mmq_q4k_prepared_streamk(A16, 8, 256, B16, 4, A16, 7, A16, None) == -1   # ldy < od
    assert lib.mmq_q6k_prepared_streamk(A16, 8, 256, B16, 4, A16, 8, MIS, None) == -2
    assert lib.mmq_q6k_prepared_streamk(A16, 0, 256, B16, 4, A16, 0, A16, None) == 0   # od == 0


def test_tiled_sizes_and_argument_checks():
    lib = qig.load()
    assert qig.q8_tiled_bytes(512, 3584) == 8 * 14 * 20480 == qig.q8_pad40_bytes(512, 3584)
    assert qig.q8_tiled_bytes(70, 768) == 2 * 3 * 20480
    assert qig.q8_tiled_bytes(0, 256) == 0
    assert qig.q8_tiled_bytes(5, 100) == 0 and qig.q8_tiled_bytes(5, 288) == 0   # id % 256
    assert lib.quantize_q8_tiled(A16, 4, 288, 288, B16, None) == -1      # id % 256
    assert lib.quantize_q8_tiled(A16, 4, 256, 128, B16, None) == -1      # ldx < id
    assert lib.quantize_q8_tiled(MIS, 4, 256, 256, B16, None) == -2
    assert lib.quantize_q8_tiled(A16, 4, 256, 258, B16, None) == -2      # ldx % 4
    assert lib.quantize_q8_tiled(A16, 0, 256, 256, B16, None) == 0
    assert lib.mmq_q4k_q8t(A16, 8, 300, B16, 4, A16, 8, None, None) == -1
    assert lib.mmq_q4k_q8t(A16, 8, 256, B16, 4, A16, 8, MIS, None) == -2    # misaligned workspace
    assert lib.mmq_q4k_q8t(A16, 8, 256, B16, 0, A16, 8, None, None) == 0
    assert lib.mmq_q6k_q8t(A16, 208, None, 8, 256, B16, 4, A16, 8, None, None) == -1
    assert lib.mmq_q6k_q8t(A16, 224, MIS, 8, 256, B16, 4, A16, 8, None, None) == -2
    assert lib.mmq_q4k_prepared_q8t(A16, 8, 256, B16, 4, A16, 7, None, None) == -1   # ldy < od
    assert lib.mmq_q6k_prepared_q8t(MIS, 8, 256, B16, 4, A16, 8, None, None) == -2


def test_limbs_sizes_and_argument_checks():
    lib = qig.load()
    assert qig.q6k_limbs_bytes(3584, 3584) == 2 * 3584 * 3584 + 3584 * 14 * 4
    assert qig.q6k_limbs_bytes(4, 100) == 0 and qig.q6k_limbs_bytes(-1, 256) == 0
    assert lib.prepare_q6k_limbs(A16, 200, 4, 256, B16, None) == -1       # bstride
    assert lib.prepare_q6k_limbs(A16, 224, 4, 100, B16, None) == -1       # id % 256
    assert lib.prepare_q6k_limbs(MIS, 224, 4, 256, B16, None) == -2
    assert lib.prepare_q6k_limbs(A16, 224, 4, 256, MIS, None) == -2
    assert lib.prepare_q6k_limbs(A16, 224, 0, 256, B16, None) == 0        # od == 0
    assert lib.mmq_q6k_limbs_q8t(A16, 8, 300, B16, 4, A16, 8, None, None) == -1   # id % 256
    assert lib.mmq_q6k_limbs_q8t(A16, 8, 256, B16, 4, A16, 7, None, None) == -1   # ldy < od
    assert lib.mmq_q6k_limbs_q8t(MIS, 8, 256, B16, 4, A16, 8, None, None) == -2
    assert lib.mmq_q6k_limbs_q8t(A16, 8, 256, B16, 4, A16, 8, MIS, None) == -2    # workspace
    assert lib.mmq_q6k_limbs_q8t(A16, 8, 256, B16, 0, A16, 8, None, None) == 0    # nt == 0


def test_xf32_argument_checks():
    lib = qig.load()
    # (W, od, id, x, ldx, nt, y, ldy, ws, stream)
    assert lib.mmq_q4k_xf32(A16, 8, 256, B16, 255, 4, A16, 8, None, None) == -1   # ldx < id
    assert lib.mmq_q4k_xf32(A16, 8, 300, B16, 300, 4, A16, 8, None, None) == -1   # id % 256
    assert lib.mmq_q4k_xf32(A16, 8, 256, B16, 256, 4, A16, 7, None, None) == -1   # ldy < od
    assert lib.mmq_q4k_xf32(A16, 8, 256, B16, 258, 4, A16, 8, None, None) == -2   # ldx % 4
    assert lib.mmq_q4k_xf32(A16, 8, 256, MIS, 256, 4, A16, 8, None, None) == -2   # x
    assert lib.mmq_q4k_xf32(MIS, 8, 256, B16, 256, 4, A16, 8, None, None) == -2   # W
    assert lib.mmq_q4k_xf32(A16, 8, 256, B16, 256, 4, A16, 8, MIS, None) == -2    # workspace
    assert lib.mmq_q4k_xf32(A16, 8, 256, None, 256, 4, A16, 8, None, None) == -1  # no x
    assert lib.mmq_q4k_xf32(A16, 8, 256, B16, 256, 0, A16, 8, None, None) == 0    # nt == 0
    assert lib.mmq_q4k_xf32(A16, 0, 256, B16, 256, 4, A16, 8, None, None) == 0    # od == 0


def test_xf32_binding_checks_activation_rows():
    import torch
    W = torch.zeros(4 * 144, dtype=torch.uint8)
    with pytest.raises(qig.QigError, match="exceeds"):
        qig.mmq_q4k_xf32(W, 4, 512, torch.zeros((2, 256), dtype=torch.float32))
    with pytest.raises(qig.QigError, match="2-D fp32"):
        qig.mmq_q4k_xf32(W, 4, 256, torch.zeros((2, 256), dtype=torch.float64))


def test_staged_sizes_and_argument_checks():
    lib = qig.load()
    assert qig.q4k_staged_bytes(3584, 3584) == 56 * 14 * 14336
    assert qig.q4k_staged_bytes(65, 256) == 2 * 14336
    assert qig.q4k_staged_bytes(4, 100) == 0 and qig.q4k_staged_bytes(-1, 256) == 0
    assert lib.prepare_q4k_staged(A16, 4, 100, B16, None) == -1        # id % 256
    assert lib.prepare_q4k_staged(MIS, 4, 256, B16, None) == -2
    assert lib.prepare_q4k_staged(A16, 4, 256, MIS, None) == -2
    assert lib.prepare_q4k_staged(A16, 0, 256, B16, None) == 0         # od == 0
    assert lib.mmq_q4k_staged_q8t(A16, 8, 300, B16, 4, A16, 8, None, None) == -1   # id % 256
    assert lib.mmq_q4k_staged_q8t(A16, 8, 256, B16, 4, A16, 7, None, None) == -1   # ldy < od
    assert lib.mmq_q4k_staged_q8t(MIS, 8, 256, B16, 4, A16, 8, None, None) == -2
    assert lib.mmq_q4k_staged_q8t(A16, 8, 256, B16, 4, A16, 8, MIS, None) == -2    # workspace
    assert lib.mmq_q4k_staged_q8t(A16, 8, 256, B16, 0, A16, 8, None, None) == 0    # nt == 0
