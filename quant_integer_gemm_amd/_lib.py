"""ctypes binding of libqig.so: argument marshalling only.

Every step of the MMQ runs in the HIP kernels of libqig.so; this module only
turns torch device tensors into raw pointers, picks the current HIP stream and
raises on a non-zero return code.  There is no CPU fallback: if the library is
missing or the tensors are not on the GPU, the call fails loudly.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libqig.so")

_lib = None

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64

# name -> (restype, argtypes), mirroring include/qig.h
SIGNATURES = {
    "q8_pad40_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "qig_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "quantize_q8_pad40": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp]),
    "mmq_q4k": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp]),
    "mmq_q6k": (ctypes.c_int, [_vp, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp]),
    "expand_q6k_dense": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp]),
    "mmq_q4k_partials": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp]),
    "mmq_q6k_partials": (ctypes.c_int, [_vp, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64,
                                        _vp, _vp]),
    "q4k_prepared_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "q6k_prepared_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "prepare_q4k": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp]),
    "prepare_q6k": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp]),
    "mmq_q4k_prepared": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp]),
    "mmq_q6k_prepared": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp]),
    "mmq_workspace_bytes": (ctypes.c_size_t, []),
    "mmq_q4k_streamk": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp]),
    "mmq_q6k_streamk": (ctypes.c_int, [_vp, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp]),
    "mmq_q4k_prepared_streamk": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp]),
    "mmq_q6k_prepared_streamk": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp]),
    "q8_tiled_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "quantize_q8_tiled": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp]),
    "mmq_q4k_q8t": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp]),
    "mmq_q6k_q8t": (ctypes.c_int, [_vp, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp]),
    "mmq_q4k_prepared_q8t": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp]),
    "mmq_q6k_prepared_q8t": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp]),
    "mmq_q4k_q8t_noalloc": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp]),
    "mmq_q4k_xf32": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp, _vp]),
    "q4k_staged_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "prepare_q4k_staged": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp]),
    "mmq_q4k_staged_q8t": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp]),
    "q6k_limbs_bytes": (ctypes.c_size_t, [_i64, _i64]),
    "prepare_q6k_limbs": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp]),
    "mmq_q6k_limbs_q8t": (ctypes.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _vp]),
}


class QigError(RuntimeError):
    pass


def load(path: str | None = None):
    """Load libqig.so (once) and attach the C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise QigError(f"{p} is not built: run `python -m quant_integer_gemm_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = load().qig_strerror(rc).decode()
        raise QigError(f"{what} failed: {msg} (code {rc})")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, nbytes: int, name: str):
    """The library reads and writes through raw pointers: check here that a
    tensor holds the bytes a call will touch (contiguous, large enough)."""
    if t is None:
        return
    if not t.is_contiguous():
        raise QigError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise QigError(f"{name} holds {have} bytes, the call needs {nbytes}")


def _need_y(y, nt: int, od: int, ldy: int):
    """y is addressed as y[t * ldy + j] for t < nt, j < od (fp32)."""
    import torch
    if nt <= 0 or od <= 0:
        return
    if y.dtype != torch.float32:
        raise QigError("y must be fp32")
    if y.dim() == 2:
        if y.stride(1) != 1 or y.stride(0) != ldy or y.shape[0] < nt or y.shape[1] < od:
            raise QigError(f"y must cover [{nt}][{od}] with row stride {ldy} and unit column stride")
    elif y.dim() != 1 or not y.is_contiguous() or y.numel() < (nt - 1) * ldy + od:
        raise QigError(f"a 1-D y must be contiguous with at least {(nt - 1) * ldy + od} elements")


def _raw_bytes(od: int, id_: int, bstride: int) -> int:
    return od * (id_ // 256) * bstride


def _gemm_checks(W, wbytes, q8, q8bytes, nt, od, y, ldy, W_exp=None, id_=0, ws=None):
    _need(W, wbytes, "W")
    _need(q8, q8bytes, "q8")
    _need(W_exp, od * id_, "W_exp")
    if ws is not None:
        _need(ws, int(load().mmq_workspace_bytes()), "ws")
    _need_y(y, nt, od, ldy)


def _dev_ptr(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise QigError(f"{name} must be a GPU tensor")
    return ctypes.c_void_p(t.data_ptr())


def _x_rows(x, id_):
    """(nt, ldx, id) of an activation tensor the quantizers read as
    x[t * ldx + k] for t < nt, k < id.  Only the first id columns of each row
    are read, so id may not exceed the row's width; the row stride is the
    tensor's own (one row: id, which the library accepts as a stride).  The
    last float read must lie inside the tensor's storage."""
    import torch
    if x.dim() != 2 or x.dtype != torch.float32 or (x.numel() > 0 and x.stride(1) != 1):
        raise QigError("x must be a 2-D fp32 tensor with unit column stride")
    nt, width = x.shape
    id_ = width if id_ is None else int(id_)
    if id_ > width:
        raise QigError(f"id = {id_} exceeds the {width} columns of x")
    ldx = x.stride(0) if nt > 1 else id_
    if nt > 0 and id_ > 0:
        last = x.storage_offset() + (nt - 1) * ldx + id_
        if last * 4 > x.untyped_storage().nbytes():
            raise QigError("x's storage does not hold the rows the call reads")
    return nt, ldx, id_


def q8_pad40_bytes(nt: int, id_: int) -> int:
    return int(load().q8_pad40_bytes(nt, id_))


def quantize_q8_pad40(x, id_: int | None = None, out=None, stream=None):
    """fp32 x[nt][ldx] (GPU) -> uint8 pad40 plane of q8_pad40_bytes(nt, id) bytes."""
    import torch
    nt, ldx, id_ = _x_rows(x, id_)
    nbytes = q8_pad40_bytes(nt, id_)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    _need(out, nbytes, "out")
    _check(load().quantize_q8_pad40(_dev_ptr(x, "x"), nt, id_, ldx, _dev_ptr(out, "q8"), _stream(stream)),
           "quantize_q8_pad40")
    return out


def _out_y(y, nt, od, ldy, device):
    import torch
    if y is None:
        y = torch.empty((nt, od), dtype=torch.float32, device=device)
        ldy = od
    elif ldy is None:
        ldy = y.stride(0) if y.dim() == 2 else od
    return y, ldy


def mmq_q4k(W, od: int, id_: int, q8, nt: int, y=None, ldy: int | None = None, stream=None):
    """y[nt][od] = pad40 activations x q4_K weights^T (fp32, overwritten)."""
    y, ldy = _out_y(y, nt, od, ldy, W.device)
    _gemm_checks(W, _raw_bytes(od, id_, 144), q8, q8_pad40_bytes(nt, id_), nt, od, y, ldy)
    _check(load().mmq_q4k(_dev_ptr(W, "W"), od, id_, _dev_ptr(q8, "q8"), nt, _dev_ptr(y, "y"), ldy,
                          _stream(stream)), "mmq_q4k")
    return y


def mmq_q6k(W, bstride: int, od: int, id_: int, q8, nt: int, W_exp=None, y=None, ldy: int | None = None,
            stream=None):
    """y[nt][od] = pad40 activations x q6_K weights^T; W_exp (dense plane) optional."""
    y, ldy = _out_y(y, nt, od, ldy, W.device)
    _gemm_checks(W, _raw_bytes(od, id_, bstride), q8, q8_pad40_bytes(nt, id_), nt, od, y, ldy, W_exp, id_)
    _check(load().mmq_q6k(_dev_ptr(W, "W"), bstride, _dev_ptr(W_exp, "W_exp"), od, id_,
                          _dev_ptr(q8, "q8"), nt, _dev_ptr(y, "y"), ldy, _stream(stream)), "mmq_q6k")
    return y


def expand_q6k_dense(W, bstride: int, od: int, id_: int, out=None, stream=None):
    """Raw q6_K plane -> dense centred int8 W_exp[od][id]."""
    import torch
    if out is None:
        out = torch.empty((od, id_), dtype=torch.int8, device=W.device)
    _need(W, _raw_bytes(od, id_, bstride), "W")
    _need(out, od * id_, "out")
    _check(load().expand_q6k_dense(_dev_ptr(W, "W"), bstride, od, id_, _dev_ptr(out, "W_exp"),
                                   _stream(stream)), "expand_q6k_dense")
    return out


def mmq_q4k_partials(W, od, id_, q8, nt, t0, t1, j0, j1, stream=None):
    """int32 P4[t1-t0][j1-j0][8*nsb] from the q4_K kernel (test export)."""
    import torch
    P = torch.empty((t1 - t0, j1 - j0, 8 * (id_ // 256)), dtype=torch.int32, device=W.device)
    _need(W, _raw_bytes(od, id_, 144), "W")
    _need(q8, q8_pad40_bytes(nt, id_), "q8")
    _check(load().mmq_q4k_partials(_dev_ptr(W, "W"), od, id_, _dev_ptr(q8, "q8"), nt, t0, t1, j0, j1,
                                   _dev_ptr(P, "P"), _stream(stream)), "mmq_q4k_partials")
    return P


def mmq_q6k_partials(W, bstride, od, id_, q8, nt, t0, t1, j0, j1, W_exp=None, stream=None):
    """int32 P6[t1-t0][j1-j0][16*nsb] from the q6_K kernel (test export)."""
    import torch
    P = torch.empty((t1 - t0, j1 - j0, 16 * (id_ // 256)), dtype=torch.int32, device=W.device)
    _need(W, _raw_bytes(od, id_, bstride), "W")
    _need(q8, q8_pad40_bytes(nt, id_), "q8")
    _need(W_exp, od * id_, "W_exp")
    _check(load().mmq_q6k_partials(_dev_ptr(W, "W"), bstride, _dev_ptr(W_exp, "W_exp"), od, id_,
                                   _dev_ptr(q8, "q8"), nt, t0, t1, j0, j1, _dev_ptr(P, "P"),
                                   _stream(stream)), "mmq_q6k_partials")
    return P


def prepared_bytes(qtype: str, od: int, id_: int) -> int:
    """Size of a prepared buffer: od*id quant bytes + od*(id/256)*64 scale bytes."""
    fn = load().q4k_prepared_bytes if qtype == "q4_K" else load().q6k_prepared_bytes
    return int(fn(od, id_))


def prepare_q4k(W, od: int, id_: int, out=None, stream=None):
    """Raw q4_K plane -> prepared buffer (quant plane + fp32 scale plane)."""
    import torch
    if out is None:
        out = torch.empty(prepared_bytes("q4_K", od, id_), dtype=torch.uint8, device=W.device)
    _need(W, _raw_bytes(od, id_, 144), "W")
    _need(out, prepared_bytes("q4_K", od, id_), "out")
    _check(load().prepare_q4k(_dev_ptr(W, "W"), od, id_, _dev_ptr(out, "Wp"), _stream(stream)), "prepare_q4k")
    return out


def prepare_q6k(W, bstride: int, od: int, id_: int, out=None, stream=None):
    """Raw q6_K plane -> prepared buffer (quant plane + fp32 scale plane)."""
    import torch
    if out is None:
        out = torch.empty(prepared_bytes("q6_K", od, id_), dtype=torch.uint8, device=W.device)
    _need(W, _raw_bytes(od, id_, bstride), "W")
    _need(out, prepared_bytes("q6_K", od, id_), "out")
    _check(load().prepare_q6k(_dev_ptr(W, "W"), bstride, od, id_, _dev_ptr(out, "Wp"), _stream(stream)),
           "prepare_q6k")
    return out


def mmq_q4k_prepared(Wp, od: int, id_: int, q8, nt: int, y=None, ldy: int | None = None, stream=None):
    """y[nt][od] from a prepared q4_K buffer (bit-identical to mmq_q4k on the raw blocks)."""
    y, ldy = _out_y(y, nt, od, ldy, Wp.device)
    _gemm_checks(Wp, prepared_bytes("q4_K", od, id_), q8, q8_pad40_bytes(nt, id_), nt, od, y, ldy)
    _check(load().mmq_q4k_prepared(_dev_ptr(Wp, "Wp"), od, id_, _dev_ptr(q8, "q8"), nt, _dev_ptr(y, "y"), ldy,
                                   _stream(stream)), "mmq_q4k_prepared")
    return y


def mmq_q6k_prepared(Wp, od: int, id_: int, q8, nt: int, y=None, ldy: int | None = None, stream=None):
    """y[nt][od] from a prepared q6_K buffer (bit-identical to mmq_q6k on the raw blocks)."""
    y, ldy = _out_y(y, nt, od, ldy, Wp.device)
    _gemm_checks(Wp, prepared_bytes("q6_K", od, id_), q8, q8_pad40_bytes(nt, id_), nt, od, y, ldy)
    _check(load().mmq_q6k_prepared(_dev_ptr(Wp, "Wp"), od, id_, _dev_ptr(q8, "q8"), nt, _dev_ptr(y, "y"), ldy,
                                   _stream(stream)), "mmq_q6k_prepared")
    return y


# --- stream-K variants -------------------------------------------------------

_workspaces = {}


def workspace(device=None, stream=None):
    """The default stream-K workspace of a (device, stream) pair:
    mmq_workspace_bytes() zero bytes, allocated on first use and kept.  Calls on
    one stream run in order and may share it; keying it by stream keeps calls
    that may overlap on different streams from sharing its arrival counters.
    Every call leaves the counters at zero; a call interrupted by a device
    fault does not, but such a fault also ends the HIP context the workspace
    lives in."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    index = dev.index if dev.index is not None else torch.cuda.current_device()
    if stream is None:
        stream = torch.cuda.current_stream(index)
    key = (index, int(stream.cuda_stream))
    ws = _workspaces.get(key)
    if ws is None:
        ws = new_workspace(torch.device("cuda", index))
        _workspaces[key] = ws
    return ws


def new_workspace(device):
    """A fresh zero-filled stream-K workspace (uint8, mmq_workspace_bytes() bytes)."""
    import torch
    return torch.zeros(int(load().mmq_workspace_bytes()), dtype=torch.uint8, device=device)


def mmq_q4k_streamk(W, od: int, id_: int, q8, nt: int, y=None, ldy: int | None = None, ws=None, stream=None):
    """mmq_q4k with the work split by super-block over all CUs (stream-K)."""
    y, ldy = _out_y(y, nt, od, ldy, W.device)
    ws = workspace(W.device, stream) if ws is None else ws
    _gemm_checks(W, _raw_bytes(od, id_, 144), q8, q8_pad40_bytes(nt, id_), nt, od, y, ldy, ws=ws)
    _check(load().mmq_q4k_streamk(_dev_ptr(W, "W"), od, id_, _dev_ptr(q8, "q8"), nt, _dev_ptr(y, "y"), ldy,
                                  _dev_ptr(ws, "ws"), _stream(stream)), "mmq_q4k_streamk")
    return y


def mmq_q6k_streamk(W, bstride: int, od: int, id_: int, q8, nt: int, W_exp=None, y=None, ldy: int | None = None,
                    ws=None, stream=None):
    """mmq_q6k with the work split by super-block over all CUs (stream-K)."""
    y, ldy = _out_y(y, nt, od, ldy, W.device)
    ws = workspace(W.device, stream) if ws is None else ws
    _gemm_checks(W, _raw_bytes(od, id_, bstride), q8, q8_pad40_bytes(nt, id_), nt, od, y, ldy, W_exp, id_, ws)
    _check(load().mmq_q6k_streamk(_dev_ptr(W, "W"), bstride, _dev_ptr(W_exp, "W_exp"), od, id_,
                                  _dev_ptr(q8, "q8"), nt, _dev_ptr(y, "y"), ldy, _dev_ptr(ws, "ws"),
                                  _stream(stream)), "mmq_q6k_streamk")
    return y


def mmq_q4k_prepared_streamk(Wp, od: int, id_: int, q8, nt: int, y=None, ldy: int | None = None, ws=None,
                             stream=None):
    """mmq_q4k_prepared, stream-K."""
    y, ldy = _out_y(y, nt, od, ldy, Wp.device)
    ws = workspace(Wp.device, stream) if ws is None else ws
    _gemm_checks(Wp, prepared_bytes("q4_K", od, id_), q8, q8_pad40_bytes(nt, id_), nt, od, y, ldy, ws=ws)
    _check(load().mmq_q4k_prepared_streamk(_dev_ptr(Wp, "Wp"), od, id_, _dev_ptr(q8, "q8"), nt, _dev_ptr(y, "y"),
                                           ldy, _dev_ptr(ws, "ws"), _stream(stream)), "mmq_q4k_prepared_streamk")
    return y


def mmq_q6k_prepared_streamk(Wp, od: int, id_: int, q8, nt: int, y=None, ldy: int | None = None, ws=None,
                             stream=None):
    """mmq_q6k_prepared, stream-K."""
    y, ldy = _out_y(y, nt, od, ldy, Wp.device)
    ws = workspace(Wp.device, stream) if ws is None else ws
    _gemm_checks(Wp, prepared_bytes("q6_K", od, id_), q8, q8_pad40_bytes(nt, id_), nt, od, y, ldy, ws=ws)
    _check(load().mmq_q6k_prepared_streamk(_dev_ptr(Wp, "Wp"), od, id_, _dev_ptr(q8, "q8"), nt, _dev_ptr(y, "y"),
                                           ldy, _dev_ptr(ws, "ws"), _stream(stream)), "mmq_q6k_prepared_streamk")
    return y


# --- tiled activations (quantization in the GEMM's staging layout) -------------

def q8_tiled_bytes(nt: int, id_: int) -> int:
    return int(load().q8_tiled_bytes(nt, id_))


def quantize_q8_tiled(x, id_: int | None = None, out=None, stream=None):
    """fp32 x[nt][ldx] (GPU) -> uint8 tiled plane of q8_tiled_bytes(nt, id) bytes."""
    import torch
    nt, ldx, id_ = _x_rows(x, id_)
    if out is None:
        out = torch.empty(q8_tiled_bytes(nt, id_), dtype=torch.uint8, device=x.device)
    _need(out, q8_tiled_bytes(nt, id_), "out")
    _check(load().quantize_q8_tiled(_dev_ptr(x, "x"), nt, id_, ldx, _dev_ptr(out, "q8t"), _stream(stream)),
           "quantize_q8_tiled")
    return out


def mmq_q4k_q8t(W, od: int, id_: int, q8t, nt: int, y=None, ldy: int | None = None, ws=None, stream=None):
    """mmq_q4k on a tiled activation plane; ws: None (whole tiles) or a stream-K workspace."""
    y, ldy = _out_y(y, nt, od, ldy, W.device)
    _gemm_checks(W, _raw_bytes(od, id_, 144), q8t, q8_tiled_bytes(nt, id_), nt, od, y, ldy, ws=ws)
    _check(load().mmq_q4k_q8t(_dev_ptr(W, "W"), od, id_, _dev_ptr(q8t, "q8t"), nt, _dev_ptr(y, "y"), ldy,
                              _dev_ptr(ws, "ws"), _stream(stream)), "mmq_q4k_q8t")
    return y


def mmq_q4k_xf32(W, od: int, id_: int, x, y=None, ldy: int | None = None, ws=None, stream=None):
    """The q4_K GEMM on fp32 activations x[nt][ldx] (GPU), quantized inside
    the GEMM: y bit-identical to quantize_q8_tiled then mmq_q4k_q8t.  ws:
    None (whole tiles) or a stream-K workspace."""
    nt, ldx, id_ = _x_rows(x, id_)
    y, ldy = _out_y(y, nt, od, ldy, W.device)
    _gemm_checks(W, _raw_bytes(od, id_, 144), None, 0, nt, od, y, ldy, ws=ws)
    _check(load().mmq_q4k_xf32(_dev_ptr(W, "W"), od, id_, _dev_ptr(x, "x"), ldx, nt, _dev_ptr(y, "y"), ldy,
                               _dev_ptr(ws, "ws"), _stream(stream)), "mmq_q4k_xf32")
    return y


def mmq_q6k_q8t(W, bstride: int, od: int, id_: int, q8t, nt: int, W_exp=None, y=None, ldy: int | None = None,
                ws=None, stream=None):
    """mmq_q6k on a tiled activation plane; ws: None (whole tiles) or a stream-K workspace."""
    y, ldy = _out_y(y, nt, od, ldy, W.device)
    _gemm_checks(W, _raw_bytes(od, id_, bstride), q8t, q8_tiled_bytes(nt, id_), nt, od, y, ldy, W_exp, id_, ws)
    _check(load().mmq_q6k_q8t(_dev_ptr(W, "W"), bstride, _dev_ptr(W_exp, "W_exp"), od, id_, _dev_ptr(q8t, "q8t"),
                              nt, _dev_ptr(y, "y"), ldy, _dev_ptr(ws, "ws"), _stream(stream)), "mmq_q6k_q8t")
    return y


def mmq_q4k_prepared_q8t(Wp, od: int, id_: int, q8t, nt: int, y=None, ldy: int | None = None, ws=None,
                         stream=None):
    """mmq_q4k_prepared on a tiled activation plane."""
    y, ldy = _out_y(y, nt, od, ldy, Wp.device)
    _gemm_checks(Wp, prepared_bytes("q4_K", od, id_), q8t, q8_tiled_bytes(nt, id_), nt, od, y, ldy, ws=ws)
    _check(load().mmq_q4k_prepared_q8t(_dev_ptr(Wp, "Wp"), od, id_, _dev_ptr(q8t, "q8t"), nt, _dev_ptr(y, "y"),
                                       ldy, _dev_ptr(ws, "ws"), _stream(stream)), "mmq_q4k_prepared_q8t")
    return y


def mmq_q6k_prepared_q8t(Wp, od: int, id_: int, q8t, nt: int, y=None, ldy: int | None = None, ws=None,
                         stream=None):
    """mmq_q6k_prepared on a tiled activation plane."""
    y, ldy = _out_y(y, nt, od, ldy, Wp.device)
    _gemm_checks(Wp, prepared_bytes("q6_K", od, id_), q8t, q8_tiled_bytes(nt, id_), nt, od, y, ldy, ws=ws)
    _check(load().mmq_q6k_prepared_q8t(_dev_ptr(Wp, "Wp"), od, id_, _dev_ptr(q8t, "q8t"), nt, _dev_ptr(y, "y"),
                                       ldy, _dev_ptr(ws, "ws"), _stream(stream)), "mmq_q6k_prepared_q8t")
    return y


# --- q6_K limb buffers (sub-block scales folded into two int8 limbs) ------------

def q6k_limbs_bytes(od: int, id_: int) -> int:
    """Size of a q6_K limb buffer: H and L planes (od*id bytes each) + fp32 d plane."""
    return int(load().q6k_limbs_bytes(od, id_))


def prepare_q6k_limbs(W, bstride: int, od: int, id_: int, out=None, stream=None):
    """Raw q6_K plane -> limb buffer (v = sc*c6 = 128 H + L per element, and d)."""
    import torch
    if out is None:
        out = torch.empty(q6k_limbs_bytes(od, id_), dtype=torch.uint8, device=W.device)
    _need(W, _raw_bytes(od, id_, bstride), "W")
    _need(out, q6k_limbs_bytes(od, id_), "out")
    _check(load().prepare_q6k_limbs(_dev_ptr(W, "W"), bstride, od, id_, _dev_ptr(out, "Wl"), _stream(stream)),
           "prepare_q6k_limbs")
    return out


def mmq_q6k_limbs_q8t(Wl, od: int, id_: int, q8t, nt: int, y=None, ldy: int | None = None, ws=None, stream=None):
    """y[nt][od] of the q6_K GEMM from a limb buffer and a tiled activation plane."""
    y, ldy = _out_y(y, nt, od, ldy, Wl.device)
    _gemm_checks(Wl, q6k_limbs_bytes(od, id_), q8t, q8_tiled_bytes(nt, id_), nt, od, y, ldy, ws=ws)
    _check(load().mmq_q6k_limbs_q8t(_dev_ptr(Wl, "Wl"), od, id_, _dev_ptr(q8t, "q8t"), nt, _dev_ptr(y, "y"), ldy,
                                    _dev_ptr(ws, "ws"), _stream(stream)), "mmq_q6k_limbs_q8t")
    return y


def q4k_staged_bytes(od: int, id_: int) -> int:
    """Size of a staged q4_K buffer: ceil(od/64) * (id/256) records of 14336 bytes."""
    return int(load().q4k_staged_bytes(od, id_))


def prepare_q4k_staged(W, od: int, id_: int, out=None, stream=None):
    """Raw q4_K plane -> staged buffer (per 64-row tile and super-block, the
    bytes the GEMM stages into LDS)."""
    import torch
    if out is None:
        out = torch.empty(q4k_staged_bytes(od, id_), dtype=torch.uint8, device=W.device)
    _need(W, _raw_bytes(od, id_, 144), "W")
    _need(out, q4k_staged_bytes(od, id_), "out")
    _check(load().prepare_q4k_staged(_dev_ptr(W, "W"), od, id_, _dev_ptr(out, "Ws"), _stream(stream)),
           "prepare_q4k_staged")
    return out


def mmq_q4k_staged_q8t(Ws, od: int, id_: int, q8t, nt: int, y=None, ldy: int | None = None, ws=None, stream=None):
    """y[nt][od] of the q4_K GEMM from a staged buffer and a tiled activation
    plane (bit-identical to mmq_q4k_q8t)."""
    y, ldy = _out_y(y, nt, od, ldy, Ws.device)
    _gemm_checks(Ws, q4k_staged_bytes(od, id_), q8t, q8_tiled_bytes(nt, id_), nt, od, y, ldy, ws=ws)
    _check(load().mmq_q4k_staged_q8t(_dev_ptr(Ws, "Ws"), od, id_, _dev_ptr(q8t, "q8t"), nt, _dev_ptr(y, "y"), ldy,
                                     _dev_ptr(ws, "ws"), _stream(stream)), "mmq_q4k_staged_q8t")
    return y


def mmq_q4k_q8t_noalloc(W, od: int, id_: int, q8t, nt: int, y, ldy: int | None = None, stream=None):
    """mmq_q4k_q8t with the stream-K split on the library's own scratch: the
    call allocates nothing (y must be given).  Calls that may overlap on one
    GPU race on that scratch."""
    if y is None:
        raise QigError("mmq_q4k_q8t_noalloc allocates nothing: pass y")
    ldy = (y.stride(0) if y.dim() == 2 else od) if ldy is None else ldy
    _gemm_checks(W, _raw_bytes(od, id_, 144), q8t, q8_tiled_bytes(nt, id_), nt, od, y, ldy)
    _check(load().mmq_q4k_q8t_noalloc(_dev_ptr(W, "W"), od, id_, _dev_ptr(q8t, "q8t"), nt, _dev_ptr(y, "y"), ldy,
                                      _stream(stream)), "mmq_q4k_q8t_noalloc")
    return y
