// mmq.hip -- k-quant prefill MMQ on gfx950: int8 MFMA sub-block dot products
// with a fused fp32 rescale epilogue.
//
// Operation (minfer pages: r44 "W_exp stride mismatch root cause" s1.1/s2.1
// for q6_K sub-block scaling, s3.2 for the element map; r20/r21 pages for the
// pad40 activation blocks):
//   q6_K: y[t][j] = sum_sb d(j,sb) sum_s sc(j,sb,s) da(t,8sb+s/2) P6(t,j,sb,s)
//   q4_K: y[t][j] = sum_sb sum_b [ d sc_b da(t,c) P4(t,j,c) - dmin m_b ssum(t,c) ]
// with int32 P over a 16- (q6_K) or 32-element (q4_K) sub-block.
//
// Design (MI355X-first; the pages' IMMA kernels are prior art only):
//  * Workgroup of 256 threads = 4 waves computes a 64-token x 128-row tile;
//    each wave a 32-token x 64-row tile = two 32x32 MFMA tiles that share the
//    token-side per-row scales.
//  * MFMA rows are tokens, columns are weight rows, so each lane owns one
//    weight row: the per-(row, chunk) weight scale is a lane constant and the
//    per-(token, chunk) fp16 activation scale is a per-register value read
//    straight from LDS as fp16 (v_fma_mix consumes it without conversion).
//  * K advances one super-block (256) per step.  The raw blocks of step k+1
//    are loaded into registers with 16-byte loads while step k computes, then
//    decoded (nibble / 2-bit recombination to int8) into the other half of a
//    double-buffered LDS stage: one barrier per super-block.
//  * Epilogue per 32-chunk and MFMA tile: the int8 MFMA accumulates onto the
//    1.5*2^23 bias so one fma turns the int32 partial into P*w exactly once
//    rounded; a v_fma_mix folds in the fp16 activation scale.  2 VALU ops per
//    output and chunk (q4_K), 4 for q6_K (two 16-element sub-blocks, each its
//    own MFMA with the other half of K zeroed).
//  * q4_K min term: -dmin*m*ssum summed over chunks is a K = id/32 fp32 matrix
//    product, done on the fp32 MFMA (32x32x2) into a second accumulator.
#include "qig_device.h"
#include "qig_launch.h"

namespace qig {

constexpr int NTHR = 256;
constexpr int TT = 64;    // tokens per workgroup tile
constexpr int TJ = 128;   // weight rows per workgroup tile
constexpr int NCH = 8;    // 32-element chunks per super-block

// One super-block of staged operands.
template <int QT>
struct Stage;

template <>
struct Stage<4> {
    uint8_t a[NCH][TT][32];     // activation quants (16-byte halves swizzled)
    uint16_t ad[NCH][TT];       // activation fp16 d, row_slot order per 32 tokens
    float as[NCH][TT];          // activation ssum
    uint8_t b[NCH][TJ][32];     // weight nibbles 0..15 as int8
    float bs[NCH][TJ];          // d * sc
    float bm[NCH][TJ];          // dmin * m
};

template <>
struct Stage<6> {
    uint8_t a[NCH][TT][32];
    uint16_t ad[NCH][TT];
    uint8_t b[NCH][TJ][32];     // centred int8 weights
    float bs[NCH][TJ][2];       // d * sc of the two 16-element sub-blocks
};

// 16-byte half h of row r lives at half (h ^ swz(r)) so that the 16 lanes of
// one LDS access phase touch 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 1; }

struct MmqArgs {
    const uint8_t *W;
    const uint8_t *Wexp;
    const uint8_t *q8;
    float *y;
    int32_t *P;
    int64_t bstride, od, id, nt, ldy;
    int64_t t0, t1, j0, j1;   // output window (all of y for the GEMM)
    int nbt;                  // token tiles in the window
};

// ---------------------------------------------------------------------------
// global -> register loads of one super-block, and register -> LDS decode
// ---------------------------------------------------------------------------
template <int QT, bool WEXP>
struct Regs;

template <>
struct Regs<4, false> {
    u32x4 a[5];   // two pad40 blocks of one token (80 bytes)
    u32x4 h;      // q4_K header: d, dmin, 12 scale bytes
    u32x4 q[4];   // 64 nibble bytes
};

template <bool WEXP>
struct Regs6 {
    u32x4 a[5];
    u32x4 q[WEXP ? 8 : 6];   // W_exp: 128 centred bytes; raw: ql 64 B + qh 32 B
    u32x4 sc;                // 16 int8 scales
    uint32_t d;              // fp16 d in the low half
};
template <>
struct Regs<6, false> : Regs6<false> {};
template <>
struct Regs<6, true> : Regs6<true> {};

__device__ __forceinline__ u32x4 ld16(const uint8_t *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

// Activations: thread -> (token tau = tid/4, block pair p = tid%4).
template <typename R>
__device__ __forceinline__ void load_a(R &r, const MmqArgs &g, int64_t tw0, int64_t sb)
{
    const int tid = threadIdx.x;
    const int tau = tid >> 2, p = tid & 3;
    const int64_t t = tw0 + tau;
    const int64_t nb32 = g.id / 32;
    if (t < g.nt) {
        const uint8_t *src = g.q8 + ((t * nb32) + 8 * sb + 2 * p) * 40;
#pragma unroll
        for (int k = 0; k < 5; ++k) r.a[k] = ld16(src + 16 * k);
    } else {
#pragma unroll
        for (int k = 0; k < 5; ++k) r.a[k] = u32x4{0, 0, 0, 0};
    }
}

template <int QT, typename R>
__device__ __forceinline__ void store_a(Stage<QT> &s, const R &r)
{
    const int tid = threadIdx.x;
    const int tau = tid >> 2, p = tid & 3;
    uint32_t w[20];
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        w[4 * k + 0] = r.a[k][0];
        w[4 * k + 1] = r.a[k][1];
        w[4 * k + 2] = r.a[k][2];
        w[4 * k + 3] = r.a[k][3];
    }
    const int sl = (tau & 32) + row_slot(tau & 31);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int c = 2 * p + k;
        const uint32_t *b = w + 10 * k;
        s.ad[c][sl] = (uint16_t)(b[0] & 0xffffu);
        u32x4 lo = {b[1], b[2], b[3], b[4]};
        u32x4 hi = {b[5], b[6], b[7], b[8]};
        *reinterpret_cast<u32x4 *>(&s.a[c][tau][16 * (0 ^ swz(tau))]) = lo;
        *reinterpret_cast<u32x4 *>(&s.a[c][tau][16 * (1 ^ swz(tau))]) = hi;
        if constexpr (QT == 4) s.as[c][tau] = __builtin_bit_cast(float, b[9]);
    }
}

// q4_K weights: thread -> (row r = tid/2, half g2 = tid%2: nibble groups 2g2, 2g2+1)
__device__ __forceinline__ void load_b(Regs<4, false> &r, const MmqArgs &g, int64_t jw0, int64_t sb)
{
    const int tid = threadIdx.x;
    const int row = tid >> 1, g2 = tid & 1;
    const int64_t j = jw0 + row;
    const int64_t nsb = g.id / 256;
    if (j < g.od) {
        const uint8_t *blk = g.W + (j * nsb + sb) * 144;
        r.h = ld16(blk);
#pragma unroll
        for (int k = 0; k < 4; ++k) r.q[k] = ld16(blk + 16 + 64 * g2 + 16 * k);
    } else {
        r.h = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < 4; ++k) r.q[k] = u32x4{0, 0, 0, 0};
    }
}

__device__ __forceinline__ void store_b(Stage<4> &s, const Regs<4, false> &r)
{
    const int tid = threadIdx.x;
    const int row = tid >> 1, g2 = tid & 1;
    const int sw = swz(row);
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
        const int grp = 2 * g2 + gg;          // nibble group: chunks 2grp (low), 2grp+1 (high)
        const u32x4 w0 = r.q[2 * gg], w1 = r.q[2 * gg + 1];
        u32x4 lo0 = w0 & 0x0F0F0F0Fu, lo1 = w1 & 0x0F0F0F0Fu;
        u32x4 hi0 = (w0 >> 4) & 0x0F0F0F0Fu, hi1 = (w1 >> 4) & 0x0F0F0F0Fu;
        *reinterpret_cast<u32x4 *>(&s.b[2 * grp][row][16 * (0 ^ sw)]) = lo0;
        *reinterpret_cast<u32x4 *>(&s.b[2 * grp][row][16 * (1 ^ sw)]) = lo1;
        *reinterpret_cast<u32x4 *>(&s.b[2 * grp + 1][row][16 * (0 ^ sw)]) = hi0;
        *reinterpret_cast<u32x4 *>(&s.b[2 * grp + 1][row][16 * (1 ^ sw)]) = hi1;
    }
    uint8_t S[12];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const uint32_t v = r.h[1 + k];
        S[4 * k + 0] = v & 0xff;
        S[4 * k + 1] = (v >> 8) & 0xff;
        S[4 * k + 2] = (v >> 16) & 0xff;
        S[4 * k + 3] = v >> 24;
    }
    const float d = h2f(r.h[0]), dmin = h2f(r.h[0] >> 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int b = 4 * g2 + k;
        int sc, m;
        q4_scale_min(S, b, sc, m);
        s.bs[b][row] = d * (float)sc;
        s.bm[b][row] = dmin * (float)m;
    }
}

// q6_K weights: thread -> (row r = tid/2, half h = tid%2: chunks 4h..4h+3)
template <bool WEXP>
__device__ __forceinline__ void load_b(Regs<6, WEXP> &r, const MmqArgs &g, int64_t jw0, int64_t sb)
{
    const int tid = threadIdx.x;
    const int row = tid >> 1, h = tid & 1;
    const int64_t j = jw0 + row;
    const int64_t nsb = g.id / 256;
    if (j < g.od) {
        const uint8_t *blk = g.W + j * nsb * g.bstride + sb * g.bstride;
        if constexpr (WEXP) {
            const uint8_t *src = g.Wexp + j * g.id + 256 * sb + 128 * h;
#pragma unroll
            for (int k = 0; k < 8; ++k) r.q[k] = ld16(src + 16 * k);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) r.q[k] = ld16(blk + 64 * h + 16 * k);
#pragma unroll
            for (int k = 0; k < 2; ++k) r.q[4 + k] = ld16(blk + 128 + 32 * h + 16 * k);
        }
        r.sc = ld16(blk + 192);
        r.d = *reinterpret_cast<const uint32_t *>(blk + 208);
    } else {
#pragma unroll
        for (int k = 0; k < (WEXP ? 8 : 6); ++k) r.q[k] = u32x4{0, 0, 0, 0};
        r.sc = u32x4{0, 0, 0, 0};
        r.d = 0;
    }
}

template <bool WEXP>
__device__ __forceinline__ void store_b(Stage<6> &s, const Regs<6, WEXP> &r)
{
    const int tid = threadIdx.x;
    const int row = tid >> 1, h = tid & 1;
    const int sw = swz(row);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
        const int c = 4 * h + qq;
        u32x4 o[2];
        if constexpr (WEXP) {
            o[0] = r.q[2 * qq];
            o[1] = r.q[2 * qq + 1];
        } else {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k = 4 * hh + e;   // output dword 0..7 of the chunk
                    const uint32_t qlw = r.q[2 * (qq & 1) + (k >> 2)][k & 3];
                    const uint32_t qhw = r.q[4 + (k >> 2)][k & 3];
                    o[hh][e] = q6_centred(qlw, qhw, qq);
                }
        }
        *reinterpret_cast<u32x4 *>(&s.b[c][row][16 * (0 ^ sw)]) = o[0];
        *reinterpret_cast<u32x4 *>(&s.b[c][row][16 * (1 ^ sw)]) = o[1];
    }
    const float d = h2f(r.d);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
        const int c = 4 * h + qq;
        const uint32_t v = r.sc[c >> 1];            // scale bytes 2c, 2c+1
        const int sh = 16 * (c & 1);
        const float s0 = (float)(int8_t)((v >> sh) & 0xff);
        const float s1 = (float)(int8_t)((v >> (sh + 8)) & 0xff);
        s.bs[c][row][0] = d * s0;
        s.bs[c][row][1] = d * s1;
    }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int QT, bool WEXP, int MODE>
__global__ __launch_bounds__(NTHR, 1) void mmq_kernel(MmqArgs g)
{
    __shared__ Stage<QT> st[2];

    const int bt = blockIdx.x % g.nbt;
    const int bj = blockIdx.x / g.nbt;
    const int64_t tw0 = g.t0 + (int64_t)TT * bt;   // workgroup tile origin
    const int64_t jw0 = g.j0 + (int64_t)TJ * bj;
    const int64_t nsb = g.id / 256;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wt = wave & 1;          // 32-token group of this wave
    const int wj = wave >> 1;         // 64-row group of this wave
    const int l32 = lane & 31;
    const int hh = lane >> 5;
    const int ta = 32 * wt + l32;     // token (tile-local) this lane loads for MFMA a
    const int jb[2] = {64 * wj + l32, 64 * wj + 32 + l32};   // weight rows of the lane

    i32x16 bias;
#pragma unroll
    for (int i = 0; i < 16; ++i) bias[i] = MAGIC_I;
    f32x16 acc[2], accm[2];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc[n][i] = 0.0f;
            accm[n][i] = 0.0f;
        }

    Regs<QT, WEXP> rg;
    load_a(rg, g, tw0, 0);
    load_b(rg, g, jw0, 0);
    store_a<QT>(st[0], rg);
    store_b(st[0], rg);
    __syncthreads();

    for (int64_t sb = 0; sb < nsb; ++sb) {
        Stage<QT> &s = st[sb & 1];
        const bool more = sb + 1 < nsb;
        if (more) {
            load_a(rg, g, tw0, sb + 1);
            load_b(rg, g, jw0, sb + 1);
        }
#pragma unroll 2
        for (int c = 0; c < NCH; ++c) {
            const i32x4 av = *reinterpret_cast<const i32x4 *>(&s.a[c][ta][16 * (hh ^ swz(ta))]);
            i32x4 bv[2];
#pragma unroll
            for (int n = 0; n < 2; ++n)
                bv[n] = *reinterpret_cast<const i32x4 *>(&s.b[c][jb[n]][16 * (hh ^ swz(jb[n]))]);
            // fp16 activation scales of this lane's 16 token rows, register order
            _Float16 da[16];
            {
                const u32x4 d0 = *reinterpret_cast<const u32x4 *>(&s.ad[c][32 * wt + 16 * hh]);
                const u32x4 d1 = *reinterpret_cast<const u32x4 *>(&s.ad[c][32 * wt + 16 * hh + 8]);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    da[2 * k] = __builtin_bit_cast(_Float16, (uint16_t)(d0[k] & 0xffff));
                    da[2 * k + 1] = __builtin_bit_cast(_Float16, (uint16_t)(d0[k] >> 16));
                    da[8 + 2 * k] = __builtin_bit_cast(_Float16, (uint16_t)(d1[k] & 0xffff));
                    da[8 + 2 * k + 1] = __builtin_bit_cast(_Float16, (uint16_t)(d1[k] >> 16));
                }
            }
            if constexpr (QT == 4) {
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const i32x16 D = mfma_i8(av, bv[n], bias);
                    if constexpr (MODE == 0) {
                        const float w = s.bs[c][jb[n]];
                        const float nw = -MAGIC_F * w;
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const float u = __builtin_fmaf(as_float(D[i]), w, nw);
                            acc[n][i] = __builtin_fmaf(u, (float)da[i], acc[n][i]);
                        }
                    } else {
                        const int64_t j = jw0 + jb[n];
                        const int64_t nsub = 8 * nsb, sub = 8 * sb + c;
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int64_t t = tw0 + 32 * wt + mfma_row(i, hh);
                            if (t < g.t1 && j < g.j1)
                                g.P[((t - g.t0) * (g.j1 - g.j0) + (j - g.j0)) * nsub + sub] = D[i] - MAGIC_I;
                        }
                    }
                }
                if constexpr (MODE == 0) {
                    if (c & 1) {   // min term for chunks c-1, c on the fp32 MFMA
                        const int ck = c - 1 + hh;
                        const float am = -s.as[ck][ta];
#pragma unroll
                        for (int n = 0; n < 2; ++n) accm[n] = mfma_f32(am, s.bm[ck][jb[n]], accm[n]);
                    }
                }
            } else {
                const i32x4 zero = {0, 0, 0, 0};
                const i32x4 a0 = hh ? zero : av;   // first 16 elements of the chunk
                const i32x4 a1 = hh ? av : zero;   // last 16
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const i32x16 D0 = mfma_i8(a0, bv[n], bias);
                    const i32x16 D1 = mfma_i8(a1, bv[n], bias);
                    if constexpr (MODE == 0) {
                        const float w0 = s.bs[c][jb[n]][0], w1 = s.bs[c][jb[n]][1];
                        const float nw0 = -MAGIC_F * w0, nw1 = -MAGIC_F * w1;
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const float u0 = __builtin_fmaf(as_float(D0[i]), w0, nw0);
                            acc[n][i] = __builtin_fmaf(u0, (float)da[i], acc[n][i]);
                            const float u1 = __builtin_fmaf(as_float(D1[i]), w1, nw1);
                            acc[n][i] = __builtin_fmaf(u1, (float)da[i], acc[n][i]);
                        }
                    } else {
                        const int64_t j = jw0 + jb[n];
                        const int64_t nsub = 16 * nsb, sub = 2 * (8 * sb + c);
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int64_t t = tw0 + 32 * wt + mfma_row(i, hh);
                            if (t < g.t1 && j < g.j1) {
                                int32_t *dst = g.P + ((t - g.t0) * (g.j1 - g.j0) + (j - g.j0)) * nsub + sub;
                                dst[0] = D0[i] - MAGIC_I;
                                dst[1] = D1[i] - MAGIC_I;
                            }
                        }
                    }
                }
            }
        }
        if (more) {
            store_a<QT>(st[(sb + 1) & 1], rg);
            store_b(st[(sb + 1) & 1], rg);
        }
        __syncthreads();
    }

    if constexpr (MODE == 0) {
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int64_t j = jw0 + jb[n];
            if (j >= g.j1) continue;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t t = tw0 + 32 * wt + mfma_row(i, hh);
                if (t < g.t1) g.y[t * g.ldy + j] = acc[n][i] + accm[n][i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// host-side launchers (argument checking is done by the C ABI layer)
// ---------------------------------------------------------------------------
template <int QT, bool WEXP, int MODE>
static int launch(MmqArgs g, hipStream_t stream)
{
    const int64_t nbt = (g.t1 - g.t0 + TT - 1) / TT;
    const int64_t nbj = (g.j1 - g.j0 + TJ - 1) / TJ;
    if (nbt <= 0 || nbj <= 0) return 0;
    if (nbt * nbj > 0x7fffffff) return -1;
    g.nbt = (int)nbt;
    hipLaunchKernelGGL((mmq_kernel<QT, WEXP, MODE>), dim3((unsigned)(nbt * nbj)), dim3(NTHR), 0,
                       stream, g);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_mmq(const MmqLaunch &L, hipStream_t stream)
{
    MmqArgs g;
    g.W = static_cast<const uint8_t *>(L.W);
    g.Wexp = reinterpret_cast<const uint8_t *>(L.Wexp);
    g.q8 = static_cast<const uint8_t *>(L.q8);
    g.y = L.y;
    g.P = L.P;
    g.bstride = L.bstride;
    g.od = L.od;
    g.id = L.id;
    g.nt = L.nt;
    g.ldy = L.ldy;
    g.t0 = L.t0;
    g.t1 = L.t1;
    g.j0 = L.j0;
    g.j1 = L.j1;
    g.nbt = 0;
    const bool part = L.P != nullptr;
    if (L.qtype == 4)
        return part ? launch<4, false, 1>(g, stream) : launch<4, false, 0>(g, stream);
    if (L.Wexp)
        return part ? launch<6, true, 1>(g, stream) : launch<6, true, 0>(g, stream);
    return part ? launch<6, false, 1>(g, stream) : launch<6, false, 0>(g, stream);
}

}  // namespace qig
