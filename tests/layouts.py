"""Byte layouts of the registration-time and prepass buffers, built in numpy
from the oracle's decoders, per the layouts include/qig.h states.  Test
infrastructure: the GPU tests compare the library's buffers with these bytes,
and the CPU stage simulation reads them as the kernels' LDS stages."""
import numpy as np

import oracle

Q8T_RECORD = 20480      # tiled activation record per (64-token tile, super-block)
Q4S_RECORD = 14336      # staged q4_K record per (64-row tile, super-block)
MAGIC = np.float32(12582912.0)


def bf16_rne(v):
    """float32 array -> bf16 bits (round to nearest even), as uint32 in the low half."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32)


def tiled_plane(q8, nt, id_):
    """The tiled plane from a pad40 plane, per the layout the header states."""
    nb32, nsb, ntt = id_ // 32, id_ // 256, (nt + 63) // 64
    blk = np.zeros((ntt * 64, nb32, 40), dtype=np.uint8)
    blk[:nt] = q8.reshape(nt, nb32, 40)                  # padding tokens: quantized zeros
    d = blk[:, :, 0:2].copy().view(np.float16)[:, :, 0].astype(np.float32)
    qs = blk[:, :, 4:36]
    ssum = blk[:, :, 36:40].copy().view(np.float32)[:, :, 0]
    out = np.zeros((ntt, nsb, Q8T_RECORD), dtype=np.uint8)
    u = np.arange(64)
    s = ((u >> 2) ^ (u >> 3)) & 1
    slot = (u & 32) + 16 * ((u >> 2) & 1) + 4 * ((u & 31) >> 3) + (u & 3)
    for T in range(ntt):
        tok = slice(64 * T, 64 * T + 64)
        for sb in range(nsb):
            rec = out[T, sb]
            for c in range(8):
                ch = 8 * sb + c
                rows = qs[tok, ch]                                    # [64][32]
                for h in range(2):
                    base = 2048 * c + 32 * u + 16 * (h ^ s)
                    idx = base[:, None] + np.arange(16)[None, :]
                    rec[idx] = rows[:, 16 * h:16 * h + 16]
                dv = np.zeros(64, dtype=np.float32)
                dv[slot] = d[tok, ch]
                rec[16384 + 256 * c:16384 + 256 * c + 256] = dv.view(np.uint8)
                v = (-ssum[tok, ch]).astype(np.float32)
                hi = bf16_rne(v)
                lo = bf16_rne(v - (hi << 16).astype(np.uint32).view(np.float32))
                m = rec[18432:20480].view(np.uint16).reshape(64, 2, 8)
                m[:, c // 4, c % 4] = hi.astype(np.uint16)
                m[:, c // 4, 4 + c % 4] = lo.astype(np.uint16)
    return out.reshape(-1)


def staged_records(W, od, id_):
    nsb = id_ // 256
    ntile = (od + 63) // 64
    out = np.zeros((ntile, nsb, Q4S_RECORD), dtype=np.uint8)
    Wb = W.reshape(od, nsb, 144)
    for j in range(od):
        T, r = divmod(j, 64)
        for sb in range(nsb):
            blk = Wb[j, sb]
            q, sc, m, d, dmin = oracle.q4k_decode_block(blk)
            # the packed bytes decode to the oracle's quants (low nibble of
            # byte 32g + i: element 64g + i; high: element 64g + 32 + i)
            nib = blk[16:144]
            g, i = np.divmod(np.arange(128), 32)
            assert np.array_equal(nib & 15, q[64 * g + i]) and np.array_equal(nib >> 4, q[64 * g + 32 + i])
            rec = out[T, sb]
            for u in range(8):
                pos = 128 * r + 16 * (u ^ ((r >> 1) & 7))
                rec[pos:pos + 16] = nib[16 * u:16 * u + 16]
            w = np.float32(d) * sc.astype(np.float32)            # d is an fp16 value: exact in fp32
            mm = np.float32(dmin) * m.astype(np.float32)
            for c in range(8):
                pair = np.array([w[c], -MAGIC * w[c]], dtype=np.float32)
                rec[8192 + 8 * (64 * c + r):8192 + 8 * (64 * c + r) + 8] = pair.view(np.uint8)
            for h in range(2):
                v = mm[4 * h:4 * h + 4]
                hi = bf16_rne(v)
                lo = bf16_rne(v - (hi << 16).astype(np.uint32).view(np.float32))
                ent = np.zeros(8, dtype=np.uint16)
                ent[:4] = hi
                ent[4:] = lo
                rec[12288 + 16 * (2 * r + h):12288 + 16 * (2 * r + h) + 16] = ent.view(np.uint8)
    return out.reshape(-1)


def limb_planes(W, bstride, od, id_):
    """H, L (int8 [od][id]) and d (fp32 [od][nsb]) from the oracle's decoder."""
    nsb = id_ // 256
    Wb = W.reshape(od, nsb, bstride)
    v = np.zeros((od, id_), dtype=np.int32)
    d = np.zeros((od, nsb), dtype=np.float32)
    for j in range(od):
        for sb in range(nsb):
            c6, sc, dd = oracle.q6k_decode_block(Wb[j, sb])
            v[j, 256 * sb:256 * sb + 256] = sc.astype(np.int32).repeat(16) * c6.astype(np.int32)
            d[j, sb] = dd
    H = v >> 7
    L = v & 127
    assert np.array_equal(128 * H + L, v)
    assert H.min() >= -32 and H.max() <= 32 and L.min() >= 0 and L.max() <= 127
    return H.astype(np.int8), L.astype(np.int8), d
