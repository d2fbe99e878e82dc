// prepare.hip -- registration-time "prepared" weight buffers for the MMQ.
//
// A prepared buffer trades device memory for work in the GEMM: its scales
// are already fp32 products and its quants need no bit-field recombination.
// Layout:
//   quant plane  q6_K: Q[j*id + 256*sb + e], one centred int8 per element
//                (as expand_q6k_dense writes it), row stride id;
//                q4_K: the 128 packed nibble bytes of each block, as in the
//                raw block, at Q[j*id/2 + 128*sb + i] (row stride id/2) --
//                a byte per element would double the bytes the GEMM loads
//                and measured slower than splitting nibbles in registers
//   scale plane  S[(j*nsb + sb)*16 + k]          fp32, 64 bytes per block
//     q4_K: k = 2b     -> d * sc_b     (b = 0..7, 32-element sub-blocks)
//           k = 2b + 1 -> dmin * m_b   (so each 16-byte piece is complete
//                                       for two sub-blocks)
//     q6_K: k = s      -> d * sc_s     (s = 0..15, 16-element sub-blocks)
// The products are formed exactly as the raw-block GEMM forms them (fp16 d
// widened to fp32, times the integer scale, one fp32 rounding), so a GEMM on
// a prepared buffer gives bit-identical output to one on the raw blocks.
#include "qig_device.h"
#include "qig_launch.h"

namespace qig {

// q4_K: one thread per (row, super-block, 64-element group g): the group's 32
// nibble bytes copied, plus the scales of sub-blocks 2g and 2g+1.
__global__ __launch_bounds__(256) void prepare_q4k_kernel(const uint8_t *__restrict__ W, int64_t od,
                                                           int64_t id, uint8_t *__restrict__ Q,
                                                           float *__restrict__ S)
{
    const int64_t nsb = id / 256;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= od * nsb * 4) return;
    const int grp = (int)(gid & 3);
    const int64_t blkno = gid >> 2;                 // j * nsb + sb
    const int64_t j = blkno / nsb, sb = blkno % nsb;
    const uint8_t *blk = W + blkno * 144;
    const u32x4 hdr = *reinterpret_cast<const u32x4 *>(blk);
    const u32x4 q0 = *reinterpret_cast<const u32x4 *>(blk + 16 + 32 * grp);
    const u32x4 q1 = *reinterpret_cast<const u32x4 *>(blk + 32 + 32 * grp);
    uint8_t *dst = Q + j * (id / 2) + 128 * sb + 32 * grp;
    *reinterpret_cast<u32x4 *>(dst) = q0;
    *reinterpret_cast<u32x4 *>(dst + 16) = q1;
    uint8_t sbytes[12];
#pragma unroll
    for (int k = 0; k < 12; ++k) sbytes[k] = (uint8_t)(hdr[1 + (k >> 2)] >> (8 * (k & 3)));
    const float d = h2f(hdr[0]), dmin = h2f(hdr[0] >> 16);
    float *s = S + blkno * 16;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int b = 2 * grp + k;
        int sc, m;
        q4_scale_min(sbytes, b, sc, m);
        s[2 * b] = d * (float)sc;
        s[2 * b + 1] = dmin * (float)m;
    }
}

// q6_K scale plane: one thread per (row, super-block).
__global__ __launch_bounds__(256) void prepare_q6k_scales_kernel(const uint8_t *__restrict__ W, int64_t bstride,
                                                                  int64_t od, int64_t id, float *__restrict__ S)
{
    const int64_t nsb = id / 256;
    const int64_t blkno = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // j * nsb + sb
    if (blkno >= od * nsb) return;
    const uint8_t *blk = W + blkno * bstride;
    const u32x4 sc = *reinterpret_cast<const u32x4 *>(blk + 192);
    const float d = h2f(*reinterpret_cast<const uint32_t *>(blk + 208));
    float *s = S + blkno * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = d * (float)(int8_t)((sc[q] >> (8 * e)) & 0xff);
        *reinterpret_cast<f32x4 *>(s + 4 * q) = v;
    }
}

// q6_K limb planes: one thread per (row, super-block, 16-element sub-block
// s).  Each element's centred quant c6 (the element map of the r44 page
// "W_exp stride mismatch root cause", s3.2) is multiplied by its sub-block's
// int8 scale, and the product v = sc * c6 (|v| <= 4096) is split exactly into
// two int8 limbs, H = v >> 7 (floor, in [-32, 32]) and L = v & 127, so that
// v = 128 H + L.  The fp16 d of the super-block goes to the d plane as fp32.
__global__ __launch_bounds__(256) void prepare_q6k_limbs_kernel(const uint8_t *__restrict__ W, int64_t bstride,
                                                                 int64_t od, int64_t id, uint8_t *__restrict__ H,
                                                                 uint8_t *__restrict__ L, float *__restrict__ D)
{
    const int64_t nsb = id / 256;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= od * nsb * 16) return;
    const int s = (int)(gid & 15);
    const int64_t blkno = gid >> 4;                 // j * nsb + sb
    const int64_t j = blkno / nsb, sb = blkno % nsb;
    const uint8_t *blk = W + blkno * bstride;
    const int sc = (int8_t)blk[192 + s];
    uint32_t hw[4] = {0, 0, 0, 0}, lw[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = 16 * s + i, n = e & 127, half = e >> 7;
        const int lo = (blk[64 * half + (n & 63)] >> (4 * (n >> 6))) & 15;
        const int hi = (blk[128 + 32 * half + (e & 31)] >> (2 * ((n >> 5) & 3))) & 3;
        const int v = sc * ((lo | (hi << 4)) - 32);
        hw[i >> 2] |= ((uint32_t)(v >> 7) & 0xffu) << (8 * (i & 3));
        lw[i >> 2] |= (uint32_t)(v & 127) << (8 * (i & 3));
    }
    const int64_t off = j * id + 256 * sb + 16 * s;
    *reinterpret_cast<u32x4 *>(H + off) = u32x4{hw[0], hw[1], hw[2], hw[3]};
    *reinterpret_cast<u32x4 *>(L + off) = u32x4{lw[0], lw[1], lw[2], lw[3]};
    if (s == 0) D[blkno] = h2f(*reinterpret_cast<const uint32_t *>(blk + 208));
}

int launch_prepare_q6k_limbs(const void *W, int64_t bstride, int64_t od, int64_t id, void *Wl, hipStream_t stream)
{
    const int64_t n = od * (id / 256) * 16;
    if (n == 0) return 0;
    const int64_t grid = (n + 255) / 256;
    if (grid > 0x7fffffff) return -1;
    uint8_t *H = static_cast<uint8_t *>(Wl);
    return launch_kernel(prepare_q6k_limbs_kernel, dim3((unsigned)grid), dim3(256), stream,
                         static_cast<const uint8_t *>(W), bstride, od, id, H, H + od * id,
                         reinterpret_cast<float *>(H + 2 * od * id));
}

// q4_K staged buffer: per 64-row tile T and super-block sb a record of
// Q4S_RECORD bytes at (T * nsb + sb) * Q4S_RECORD, the byte image of the
// weight part of the GEMM's LDS stage:
//   [0, 8192)      the packed nibble bytes (block bytes 16..143) of rows
//                  r = 0..63 of the tile: 16-byte unit u of row r at
//                  128 r + 16 (u ^ ((r >> 1) & 7))
//   [8192, 12288)  for chunk (sub-block) c and row r, at 8192 + 8 (64 c + r):
//                  w = d * sc_c and -M w (fp32; M = 1.5 * 2^23, the
//                  epilogue's magic bias)
//   [12288, 14336) for row r and K half h, at 12288 + 16 (2 r + h): dmin *
//                  m of chunks 4h .. 4h+3 split as bf16 hi (16-bit indices
//                  0-3) and lo = bf16(v - hi) (indices 4-7)
// Rows past od are zero.  One workgroup per record: thread (r, p) = (tid %
// 64, tid / 64) writes nibble units 2p, 2p+1 and the scales of sub-blocks
// p and p + 4 of row r, with the raw-block GEMM's arithmetic, so y is
// bit-identical to mmq_q4k_q8t.
__global__ __launch_bounds__(256) void prepare_q4k_staged_kernel(const uint8_t *__restrict__ W, int64_t od,
                                                                  int64_t id, uint8_t *__restrict__ R)
{
    const int64_t nsb = id / 256;
    const int64_t rec = blockIdx.x;
    const int64_t T = rec / nsb, sb = rec - T * nsb;
    const int r = threadIdx.x & 63, p = threadIdx.x >> 6;
    const int64_t j = 64 * T + r;
    uint8_t *out = R + rec * Q4S_RECORD;
    u32x4 q[2] = {u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}};
    float w[2] = {0.0f, 0.0f}, mm[2] = {0.0f, 0.0f};
    if (j < od) {
        const uint8_t *blk = W + (j * nsb + sb) * 144;
        const u32x4 hdr = *reinterpret_cast<const u32x4 *>(blk);
        q[0] = *reinterpret_cast<const u32x4 *>(blk + 16 + 32 * p);
        q[1] = *reinterpret_cast<const u32x4 *>(blk + 32 + 32 * p);
        uint8_t sbytes[12];
#pragma unroll
        for (int k = 0; k < 12; ++k) sbytes[k] = (uint8_t)(hdr[1 + (k >> 2)] >> (8 * (k & 3)));
        const float d = h2f(hdr[0]), dmin = h2f(hdr[0] >> 16);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            int sc, m;
            q4_scale_min(sbytes, p + 4 * k, sc, m);
            w[k] = d * (float)sc;
            mm[k] = dmin * (float)m;
        }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int u = 2 * p + k;
        *reinterpret_cast<u32x4 *>(out + 128 * r + 16 * (u ^ ((r >> 1) & 7))) = q[k];
        const int c = p + 4 * k;
        float *ws = reinterpret_cast<float *>(out + 8192 + 8 * (64 * c + r));
        ws[0] = w[k];
        ws[1] = j < od ? -MAGIC_F * w[k] : 0.0f;   // +0 in the zero rows past od
        uint16_t hi, lo;
        bf16_split(mm[k], hi, lo);
        uint16_t *mb = reinterpret_cast<uint16_t *>(out + 12288 + 16 * (2 * r + k));
        mb[p] = hi;
        mb[4 + p] = lo;
    }
}

int launch_prepare_q4k_staged(const void *W, int64_t od, int64_t id, void *R, hipStream_t stream)
{
    const int64_t nrec = (od + 63) / 64 * (id / 256);
    if (nrec == 0) return 0;
    if (nrec > 0x7fffffff) return -1;
    return launch_kernel(prepare_q4k_staged_kernel, dim3((unsigned)nrec), dim3(256), stream,
                         static_cast<const uint8_t *>(W), od, id, static_cast<uint8_t *>(R));
}

int launch_prepare_q4k(const void *W, int64_t od, int64_t id, int8_t *Q, float *S, hipStream_t stream)
{
    const int64_t n = od * (id / 256) * 4;
    if (n == 0) return 0;
    const int64_t grid = (n + 255) / 256;
    if (grid > 0x7fffffff) return -1;
    return launch_kernel(prepare_q4k_kernel, dim3((unsigned)grid), dim3(256), stream,
                         static_cast<const uint8_t *>(W), od, id, reinterpret_cast<uint8_t *>(Q), S);
}

int launch_prepare_q6k_scales(const void *W, int64_t bstride, int64_t od, int64_t id, float *S,
                              hipStream_t stream)
{
    const int64_t n = od * (id / 256);
    if (n == 0) return 0;
    const int64_t grid = (n + 255) / 256;
    if (grid > 0x7fffffff) return -1;
    return launch_kernel(prepare_q6k_scales_kernel, dim3((unsigned)grid), dim3(256), stream,
                         static_cast<const uint8_t *>(W), bstride, od, id, S);
}

}  // namespace qig
