"""Seeded synthetic inputs for the k-quant MMQ (shared by tests, bench, smoke).

This module holds none of the method's arithmetic: it only draws random bytes
and places them at the documented field offsets of the two weight block
formats, and draws fp32 activations.  Both the HIP path and the CPU oracle
consume exactly the bytes produced here.

Recipe (every draw from ``numpy.random.Generator(PCG64(seed))``, in this
order: weight content bytes, then scales, then d (then dmin), then x):

* q6_K block (210 content bytes padded to ``bstride``, 224 by default):
  ql[128] and qh[64] uniform bytes; 16 int8 sub-block scales uniform in
  [-64, 63]; d = fp16(|N(0,1)| * 1e-3) at byte 208; padding bytes zero.
* q4_K block (144 bytes): 128 uniform nibble bytes at 16, 12 uniform packed
  scale/min bytes at 4, d = fp16(|N| * 1e-3) at 0, dmin = fp16(|N| * 1e-4)
  at 2.
* activations: fp32 N(0,1) * ``xscale``.

The workloads (7B-class projection shapes) are named by their sizes.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_BASE = 20260
Q6K_BLOCK = 210
Q6K_BSTRIDE = 224
Q4K_BLOCK = 144


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _f16_bytes(v: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(v.astype(np.float16)).view(np.uint8).reshape(v.shape + (2,))


def q6k_weights(g: np.random.Generator, od: int, id_: int,
                bstride: int = Q6K_BSTRIDE, sc_range=(-64, 63)) -> np.ndarray:
    """Raw q6_K plane uint8[od, nsb*bstride]."""
    assert id_ % 256 == 0 and bstride >= Q6K_BLOCK
    nsb = id_ // 256
    qlqh = g.integers(0, 256, size=(od, nsb, 192), dtype=np.uint8)
    sc = g.integers(sc_range[0], sc_range[1] + 1, size=(od, nsb, 16),
                    dtype=np.int16).astype(np.int8)
    d = (np.abs(g.standard_normal(size=(od, nsb))) * 1e-3).astype(np.float32)
    W = np.zeros((od, nsb, bstride), dtype=np.uint8)
    W[:, :, 0:192] = qlqh
    W[:, :, 192:208] = sc.view(np.uint8)
    W[:, :, 208:210] = _f16_bytes(d)
    return W.reshape(od, nsb * bstride)


def q4k_weights(g: np.random.Generator, od: int, id_: int) -> np.ndarray:
    """Raw q4_K plane uint8[od, nsb*144]."""
    assert id_ % 256 == 0
    nsb = id_ // 256
    qs = g.integers(0, 256, size=(od, nsb, 128), dtype=np.uint8)
    scales = g.integers(0, 256, size=(od, nsb, 12), dtype=np.uint8)
    d = (np.abs(g.standard_normal(size=(od, nsb))) * 1e-3).astype(np.float32)
    dmin = (np.abs(g.standard_normal(size=(od, nsb))) * 1e-4).astype(np.float32)
    W = np.zeros((od, nsb, Q4K_BLOCK), dtype=np.uint8)
    W[:, :, 16:144] = qs
    W[:, :, 4:16] = scales
    W[:, :, 0:2] = _f16_bytes(d)
    W[:, :, 2:4] = _f16_bytes(dmin)
    return W.reshape(od, nsb * Q4K_BLOCK)


def activations(g: np.random.Generator, nt: int, id_: int, xscale: float = 1.0) -> np.ndarray:
    return (g.standard_normal(size=(nt, id_), dtype=np.float32) * np.float32(xscale))


@dataclass(frozen=True)
class Gemm:
    """One GEMM of a workload: quant type, od (rows of W), id, nt."""
    name: str
    qtype: str  # "q4_K" or "q6_K"
    od: int
    id: int
    nt: int
    xscale: float = 1.0


# The five workloads: a small correctness case, the two 3584x3584 nt=512
# q-projection GEMMs, the 7B-class FFN GEMMs at nt=512 and one full 7B-class
# layer at nt=2630.
WORKLOADS = {
    0: [Gemm("q6K_256x512_nt16", "q6_K", 256, 512, 16)],
    1: [Gemm("q4K_3584x3584_nt512", "q4_K", 3584, 3584, 512)],
    2: [Gemm("q6K_3584x3584_nt512", "q6_K", 3584, 3584, 512)],
    3: [Gemm("q4K_ffn_up_18944x3584_nt512", "q4_K", 18944, 3584, 512, 2.0),
        Gemm("q6K_ffn_down_3584x18944_nt512", "q6_K", 3584, 18944, 512, 2.0)],
    4: [Gemm("q4K_attn_q_3584x3584_nt2630", "q4_K", 3584, 3584, 2630),
        Gemm("q4K_attn_k_512x3584_nt2630", "q4_K", 512, 3584, 2630),
        Gemm("q4K_attn_v_512x3584_nt2630", "q4_K", 512, 3584, 2630),
        Gemm("q4K_attn_o_3584x3584_nt2630", "q4_K", 3584, 3584, 2630),
        Gemm("q4K_ffn_gate_18944x3584_nt2630", "q4_K", 18944, 3584, 2630),
        Gemm("q4K_ffn_up_18944x3584_nt2630", "q4_K", 18944, 3584, 2630),
        Gemm("q6K_ffn_down_3584x18944_nt2630", "q6_K", 3584, 18944, 2630)],
}

# The layer's v projection as q6_K: the pages' model keeps attn_v in q6_K in
# some layers (r44 page "W_exp stride mismatch root cause", s2.4).
LAYER_Q6K_ATTN_V = Gemm("q6K_attn_v_512x3584_nt2630", "q6_K", 512, 3584, 2630)


def make_gemm_inputs(gm: Gemm, seed: int):
    """(W uint8 2-D, x fp32 [nt, id]) for one GEMM, drawn in recipe order."""
    g = rng(seed)
    if gm.qtype == "q6_K":
        W = q6k_weights(g, gm.od, gm.id)
    else:
        W = q4k_weights(g, gm.od, gm.id)
    x = activations(g, gm.nt, gm.id, gm.xscale)
    return W, x
