"""CPU simulation of the LDS stages of the two bench kernels: the staged
q4_K GEMM on the tiled activation plane and the q6_K limb GEMM.

The stage bytes come from the buffers' byte layouts (tests/layouts.py, built
from the oracle's decoders); the simulation then makes every LDS read a
wave's lanes make -- the MFMA operands with their swizzles, the nibble
split, the scale and min-term operands -- with the address expressions of
csrc/mmq.hip, and multiplies the operands with the documented lane layout of
v_mfma_i32_32x32x32_i8 (csrc/qig_device.h).  Each simulated MFMA result must
equal the oracle's integer chunk sum for the (token, row) its register holds,
and each scale register the oracle's factor for that register's row or
token: a byte-exact gate on the staging and read layouts that needs no GPU.
"""
import numpy as np
import pytest

import layouts
import oracle
from quant_integer_gemm_amd import inputs

Q8T = layouts.Q8T_RECORD


def swz(r):
    return ((r >> 2) ^ (r >> 3)) & 1


def mfma_row(i, hh):
    return 8 * (i >> 2) + 4 * hh + (i & 3)


def row_slot(tau):
    return 16 * ((tau >> 2) & 1) + 4 * (tau >> 3) + (tau & 3)


def x_slot(t):
    return (t & 32) + row_slot(t & 31)


def mfma(a_lanes, b_lanes, k_per_lane=16):
    """A 32x32 MFMA per the lane layout: lane l gives k_per_lane values of A
    row l % 32 and of B column l % 32, for k in its half (l // 32); returns
    D[lane][register], register i of lane l holding row mfma_row(i, l // 32)
    and column l % 32."""
    A = np.zeros((32, 2 * k_per_lane), dtype=np.float64)
    B = np.zeros((32, 2 * k_per_lane), dtype=np.float64)
    for l in range(64):
        h = l // 32
        A[l % 32, k_per_lane * h:k_per_lane * (h + 1)] = a_lanes[l]
        B[l % 32, k_per_lane * h:k_per_lane * (h + 1)] = b_lanes[l]
    C = A @ B.T
    D = np.zeros((64, 16))
    for l in range(64):
        for i in range(16):
            D[l, i] = C[mfma_row(i, l // 32), l % 32]
    return D


def f32_at(buf, off, n=1):
    return buf[off:off + 4 * n].view(np.float32)


def bf16_words(buf, off):
    """Eight bf16 values (a 16-byte MinOp entry) as float64."""
    u = buf[off:off + 16].view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _activations(seed, nt, id_):
    g = inputs.rng(seed)
    x = g.standard_normal((nt, id_)).astype(np.float32)
    q8 = oracle.quantize_q8_pad40(x)
    d_bits, qs, ssum, _ = oracle.q8_fields(q8, nt, id_)
    d = d_bits.view(np.float16).astype(np.float32)
    return q8, qs.astype(np.int64), d, ssum


@pytest.mark.parametrize("nt,od", [(64, 64), (40, 50)])
def test_staged_q4k_stage_reads(nt, od):
    id_ = 512
    nsb = id_ // 256
    W = inputs.q4k_weights(inputs.rng(11 + od), od, id_)
    q8, qs, dx, ssum = _activations(12 + nt, nt, id_)
    act = layouts.tiled_plane(q8, nt, id_).reshape(-1, nsb, Q8T)[0]             # token tile 0
    wrec = layouts.staged_records(W, od, id_).reshape(-1, nsb, layouts.Q4S_RECORD)[0]   # row tile 0
    dec = [[oracle.q4k_decode_block(W.reshape(od, nsb, 144)[j, sb]) for sb in range(nsb)] for j in range(od)]
    P = oracle.q4k_partials(W, od, id_, q8, nt, 0, nt, 0, od)
    checked = 0
    for sb in range(nsb):
        stage = np.concatenate([act[sb], wrec[sb]])        # the stage is the two records back to back
        for wave in range(4):
            wt, wr = wave & 1, wave >> 1
            lanes = np.arange(64)
            hh = lanes >> 5
            ta = 32 * wt + (lanes & 31)
            jb = 32 * wr + (lanes & 31)
            for c in range(8):
                a = [stage[2048 * c + 32 * ta[l] + 16 * (hh[l] ^ swz(ta[l])):][:16].view(np.int8) for l in lanes]
                unit = ((c & ~1) + hh) ^ ((jb >> 1) & 7)
                pk = [stage[Q8T + 128 * jb[l] + 16 * unit[l]:][:16] for l in lanes]
                b = [(p >> 4) & 15 if c & 1 else p & 15 for p in pk]
                D = mfma(a, b)
                w0 = np.array([f32_at(stage, Q8T + 8192 + 8 * (64 * c + jb[l]))[0] for l in lanes])
                w1 = np.array([f32_at(stage, Q8T + 8192 + 8 * (64 * c + jb[l]) + 4)[0] for l in lanes])
                x = np.array([f32_at(stage, 16384 + 256 * c + 4 * (32 * wt + 16 * hh[l]), 16) for l in lanes])
                for l in lanes:
                    j = jb[l]
                    if j >= od:
                        continue
                    _, sc, _, d, _ = dec[j][sb]
                    assert w0[l] == np.float32(d) * np.float32(sc[c]) and w1[l] == -layouts.MAGIC * w0[l]
                    for i in range(16):
                        t = 32 * wt + mfma_row(i, hh[l])
                        if t >= nt:
                            continue
                        assert D[l, i] == P[t, j, 8 * sb + c], (sb, wave, c, l, i)
                        assert x[l, i] == dx[t, 8 * sb + c]
                        checked += 1
            # the min-term operands: three bf16 MFMAs (hi*hi, hi*lo, lo*hi) over the super-block's 8 chunks
            mA = [bf16_words(stage, 18432 + 16 * (2 * ta[l] + hh[l])) for l in lanes]
            mB = [bf16_words(stage, Q8T + 12288 + 16 * (2 * jb[l] + hh[l])) for l in lanes]
            acc = (mfma([m[:4] for m in mA], [m[:4] for m in mB], 4) + mfma([m[:4] for m in mA], [m[4:] for m in mB], 4)
                   + mfma([m[4:] for m in mA], [m[:4] for m in mB], 4))
            for l in lanes:
                j = jb[l]
                if j >= od:
                    continue
                _, _, m, _, dmin = dec[j][sb]
                for i in range(16):
                    t = 32 * wt + mfma_row(i, hh[l])
                    if t >= nt:
                        continue
                    terms = -ssum[t, 8 * sb:8 * sb + 8].astype(np.float64) * (np.float32(dmin) * m.astype(np.float32))
                    assert abs(acc[l, i] - terms.sum()) <= 2.0 ** -14 * np.abs(terms).sum() + 1e-30
    assert checked == nsb * 8 * min(nt, 64) * od


@pytest.mark.parametrize("nt,od", [(64, 64), (40, 50)])
def test_limb_stage_reads(nt, od):
    id_ = 512
    nsb = id_ // 256
    W = inputs.q6k_weights(inputs.rng(21 + od), od, id_)
    q8, qs, dx, _ = _activations(22 + nt, nt, id_)
    act = layouts.tiled_plane(q8, nt, id_).reshape(-1, nsb, Q8T)[0]
    H, L, dw = layouts.limb_planes(W, 224, od, id_)
    v = 128 * H.astype(np.int64) + L.astype(np.int64)                   # sc * c6
    Hb, Lb = H.view(np.uint8), L.view(np.uint8)
    checked = 0
    for sb in range(nsb):
        for hs in range(2):
            # the stage of step (sb, hs), filled as the kernel's copies fill it
            a = np.zeros(8192, np.uint8)
            hst = np.zeros(8192, np.uint8)
            lst = np.zeros(8192, np.uint8)
            ax = act[sb][16384 + 1024 * hs:16384 + 1024 * hs + 1024]
            for w in range(4):
                c = 4 * hs + w
                a[2048 * w:2048 * w + 2048] = act[sb][2048 * c:2048 * c + 2048]
                for jh in range(2):
                    for l in range(64):
                        r = 32 * jh + (l >> 1)
                        rl = min(r, od - 1)                                    # rows past od: the last row
                        src = 256 * sb + 32 * c + 16 * ((l & 1) ^ swz(r))
                        dst = 2048 * w + 1024 * jh + 16 * l
                        hst[dst:dst + 16] = Hb[rl, src:src + 16]
                        lst[dst:dst + 16] = Lb[rl, src:src + 16]
            dws = np.zeros(64, np.float32)
            for rr in range(64):
                dws[32 * (rr >> 5) + row_slot(rr & 31)] = dw[min(rr, od - 1), sb]
            for wave in range(4):
                wt, wr = wave & 1, wave >> 1
                lanes = np.arange(64)
                hh = lanes >> 5
                tok = 32 * wt + (lanes & 31)
                row = 32 * wr + (lanes & 31)
                pa = 32 * tok + 16 * (hh ^ swz(tok))
                pw = 32 * row + 16 * (hh ^ swz(row))
                for c in range(4):
                    ah = [hst[2048 * c + pw[l]:][:16].view(np.int8) for l in lanes]
                    al = [lst[2048 * c + pw[l]:][:16].view(np.int8) for l in lanes]
                    ab = [a[2048 * c + pa[l]:][:16].view(np.int8) for l in lanes]
                    DH, DL = mfma(ah, ab), mfma(al, ab)                        # rows: weight rows, columns: tokens
                    xv = np.array([f32_at(ax, 4 * (64 * c + x_slot(tok[l])))[0] for l in lanes])
                    ch = 8 * sb + 4 * hs + c
                    for l in lanes:
                        t = tok[l]
                        if t >= nt:
                            continue
                        assert xv[l] == dx[t, ch]
                        for i in range(16):
                            j = 32 * wr + mfma_row(i, hh[l])
                            if j >= od:
                                continue
                            want = int(v[j, 32 * ch:32 * ch + 32] @ qs[t, 32 * ch:32 * ch + 32])
                            assert 128 * DH[l, i] + DL[l, i] == want, (sb, hs, wave, c, l, i)
                            checked += 1
                if hs == 1:
                    for l in lanes:
                        d16 = dws[32 * wr + 16 * hh[l]:32 * wr + 16 * hh[l] + 16]
                        for i in range(16):
                            j = 32 * wr + mfma_row(i, hh[l])
                            if j < od:
                                assert d16[i] == dw[j, sb]
    assert checked == nsb * 8 * min(nt, 64) * od
