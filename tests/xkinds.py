"""Activation inputs of different kinds for the quantizer's byte-exact tests.

The quantizer rounds x / d32 half away from zero, d32 = max|x| / 127 in fp32
(the r21 page "Coalesced block-linear A staging", s2.1, pad40 producer).  Most
random inputs never land near a rounding tie, so two kinds here place them
there on purpose:

- "halves": every 32-element chunk has a power-of-two d32 (its amax is
  127 * 2^e) and every other element is (k + 1/2) 2^e, so x / d32 is an exact
  tie for all of them.
- "neartie": the same ties moved by 0, 1 or 2 ulps either way, plus chunks
  whose d32 is not a power of two with elements at the fp32 value nearest
  (k + 1/2) d32 and its neighbours, so each quotient sits on or within a few
  ulps of a tie and the rounding depends on its last bits.

Expected bytes always come from the oracle; nothing here computes them.
"""
import numpy as np


def _halves(g, nt, id_):
    nb32 = id_ // 32
    e = g.integers(-12, 7, size=(nt, nb32, 1))
    d = np.ldexp(np.float32(1.0), e).astype(np.float32)
    k = g.integers(-126, 126, size=(nt, nb32, 32))
    x = ((k + 0.5) * d).astype(np.float32)                  # exact: k + 1/2 has 9 bits
    pos = g.integers(0, 32, size=(nt, nb32))
    sign = np.where(g.random((nt, nb32)) < 0.5, -1.0, 1.0).astype(np.float32)
    amax = (np.float32(127.0) * d[:, :, 0] * sign).astype(np.float32)
    np.put_along_axis(x, pos[:, :, None], amax[:, :, None], axis=2)
    return x, pos


def _nudge(g, x, keep):
    """Move each element by 0, +-1 or +-2 ulps (elements where keep is set stay)."""
    steps = g.integers(-2, 3, size=x.shape)
    out = x.copy()
    for s in (-2, -1, 1, 2):
        sel = (steps == s) & ~keep
        v = out[sel]
        for _ in range(abs(s)):
            v = np.nextafter(v, np.float32(np.inf) if s > 0 else np.float32(-np.inf)).astype(np.float32)
        out[sel] = v
    return out


def x_variant(g, nt, id_, kind):
    if kind == "halves":
        return _halves(g, nt, id_)[0].reshape(nt, id_)
    if kind == "neartie":
        nb32 = id_ // 32
        x, pos = _halves(g, nt, id_)
        keep = np.zeros(x.shape, dtype=bool)
        np.put_along_axis(keep, pos[:, :, None], True, axis=2)
        x = _nudge(g, x, keep)
        # every other chunk: a d32 that is not a power of two
        amax = (g.random((nt, nb32)) * 50 + 0.01).astype(np.float32)
        d32 = (amax / np.float32(127.0)).astype(np.float32)
        k = g.integers(-126, 126, size=(nt, nb32, 32))
        y = ((k + 0.5) * d32[:, :, None].astype(np.float64)).astype(np.float32)
        np.put_along_axis(y, pos[:, :, None], amax[:, :, None], axis=2)
        y = _nudge(g, y, keep)
        odd = (np.arange(nb32) % 2 == 1)[None, :, None]
        return np.where(odd, y, x).reshape(nt, id_).astype(np.float32)
    x = g.standard_normal((nt, id_), dtype=np.float32)
    if kind == "scaled2":
        x *= np.float32(2.0)
    elif kind == "tiny":                    # fp16-subnormal scales
        x *= np.float32(1e-6)
    elif kind == "ties":                    # integer inputs
        x = np.round(x * 40).astype(np.float32)
    elif kind == "zeros":                   # whole zero chunks
        x[::3, : min(id_, 64)] = 0.0
    elif kind == "heavy":
        x = (g.standard_t(2.0, size=(nt, id_)) * 3).astype(np.float32)
    return x
