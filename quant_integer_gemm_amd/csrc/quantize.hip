// quantize.hip -- fp32 activations -> q8 pad40 blocks on gfx950.
//
// Block (t, c) of 32 elements lives at byte (t*id/32 + c)*40: fp16 d at 0,
// zero at 2, 32 int8 quants at 4, fp32 ssum at 36 (pad40 layout of the r21
// page "Coalesced block-linear A staging", s2.1, addressed as on the r20 page
// "Split-phase A staging", s3.2).  d32 = max|x|/127 with IEEE division,
// q = round-half-away(x/d32) clamped to +-127, d = fp16(d32) round-to-even,
// ssum = d*sum(q) (exact in fp32).
//
// 8 lanes own one block, each lane one float4; max and sum reduce over the 8
// lanes with DPP moves.  The per-element division is the costly part of the
// arithmetic, so the rounding decision is taken from a reciprocal product and
// only values within reach of a rounding tie go through IEEE division
// (round_fast); the bytes are those of the IEEE definition either way.
//
// quantize_tiled_kernel writes the same quantization in the layout the GEMM's
// LDS stage uses (the quantize-transpose prepass the r21 page, s5, reports
// the campaign moving to), so the GEMM stages activations by plain copies.
#include "qig_device.h"
#include "qig_launch.h"

namespace qig {

__device__ __forceinline__ float round_half_away(float v)
{
    float r = __builtin_truncf(v);
    if (__builtin_fabsf(v - r) >= 0.5f) r += __builtin_copysignf(1.0f, v);
    return r;
}

// Reductions over the 8 lanes of a group (lanes 8g .. 8g+7) with DPP moves:
// swap neighbours, swap pairs in a quad, then mirror within the half row.
template <int CTRL>
__device__ __forceinline__ int dpp(int v)
{
    return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float group8_max(float v)
{
    v = __builtin_fmaxf(v, __builtin_bit_cast(float, dpp<0xB1>(__builtin_bit_cast(int, v))));
    v = __builtin_fmaxf(v, __builtin_bit_cast(float, dpp<0x4E>(__builtin_bit_cast(int, v))));
    return __builtin_fmaxf(v, __builtin_bit_cast(float, dpp<0x141>(__builtin_bit_cast(int, v))));
}
__device__ __forceinline__ int group8_sum(int v)
{
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    return v + dpp<0x141>(v);
}

// round-half-away(x / d) for d > 0 from the product with an approximate
// reciprocal r.  With r within 2 ulps of 1/d, x * r rounded differs from the
// correctly rounded quotient by less than 1.5 * 2^-22 relative, so by less
// than 2^-14 for |x / d| <= 128.  Unless x * r lies within 2^-13 of a tie
// (k + 1/2), both are in the same rounding interval and give the same
// integer; *near is set otherwise and the caller takes the IEEE quotient.
__device__ __forceinline__ float round_fast(float x, float r, bool &near)
{
    const float qa = x * r;
    const float t = __builtin_truncf(qa);
    const float f = __builtin_fabsf(qa - t);
    near = __builtin_fabsf(f - 0.5f) < 0x1p-13f;
    return f >= 0.5f ? t + __builtin_copysignf(1.0f, qa) : t;
}

// One 32-element block, eight lanes each holding four of its values (lane l8
// holds elements 4*l8 .. 4*l8+3): the lane's four quant bytes, and on every
// lane the fp16 d bits and ssum.
struct QBlock {
    uint32_t packed;   // this lane's four int8 quants
    uint32_t dbits;    // fp16 d (low half)
    float ssum;        // d * sum(q), exact
};

__device__ __forceinline__ QBlock quant_block(float4 v)
{
    float amax = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v.x), __builtin_fabsf(v.y)),
                                 __builtin_fmaxf(__builtin_fabsf(v.z), __builtin_fabsf(v.w)));
    amax = group8_max(amax);
    const float d32 = amax / 127.0f;
    float k[4];
    const float xs[4] = {v.x, v.y, v.z, v.w};
    // d32 below 2^-100 (and 0) takes the IEEE path: its reciprocal may not
    // be finite.
    const bool tiny = d32 < 0x1p-100f;
    const float r = __builtin_amdgcn_rcpf(tiny ? 1.0f : d32);
    bool slow = tiny;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bool nr;
        k[i] = round_fast(xs[i], r, nr);
        slow |= nr;
    }
    if (slow) {
#pragma unroll
        for (int i = 0; i < 4; ++i) k[i] = d32 == 0.0f ? 0.0f : round_half_away(xs[i] / d32);
    }
    int q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = (int)__builtin_amdgcn_fmed3f(k[i], -127.0f, 127.0f);
    const int s = group8_sum(q[0] + q[1] + q[2] + q[3]);
    QBlock o;
    o.packed = (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) | ((uint32_t)(q[2] & 0xff) << 16) |
               ((uint32_t)(q[3] & 0xff) << 24);
    const _Float16 dh = (_Float16)d32;
    o.dbits = (uint32_t)__builtin_bit_cast(uint16_t, dh);
    o.ssum = (float)dh * (float)s;
    return o;
}

__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ x, int64_t nblk,
                                                        int64_t nb32, int64_t ldx,
                                                        uint8_t *__restrict__ q8)
{
    // the workgroup's first block (t0, c0) in scalar registers; lane group i
    // takes block b0 + i, which wraps to the next token at most once when
    // nb32 >= 32
    const int64_t b0 = (int64_t)blockIdx.x * 32;
    const int64_t t0 = b0 / nb32, c0 = b0 - t0 * nb32;
    const int i = threadIdx.x >> 3;
    const int64_t blk = b0 + i;
    const int l8 = threadIdx.x & 7;
    const bool valid = blk < nblk;
    int64_t t, c;
    if (nb32 >= 32) {
        c = c0 + i;
        const bool w = c >= nb32;
        t = t0 + w;
        c -= w ? nb32 : 0;
    } else {
        t = blk / nb32;
        c = blk - t * nb32;
    }
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) v = *reinterpret_cast<const float4 *>(x + t * ldx + 32 * c + 4 * l8);
    const QBlock q = quant_block(v);
    if (!valid) return;
    uint8_t *dst = q8 + blk * 40;
    *reinterpret_cast<uint32_t *>(dst + 4 + 4 * l8) = q.packed;
    if (l8 == 0)
        *reinterpret_cast<uint32_t *>(dst) = q.dbits;
    else if (l8 == 7)
        *reinterpret_cast<float *>(dst + 36) = q.ssum;
}

// Tiled plane: one Q8T_RECORD-byte record per (64-token tile T, super-block
// sb), at ((T * nsb) + sb) * Q8T_RECORD, holding for its 64 tokens t and 8
// chunks c (global chunk 8 sb + c):
//   [0, 16384)      quants, row (c, t) of 32 bytes at 2048 c + 32 t, its
//                   16-byte halves h at 16 (h ^ swz(t))
//   [16384, 18432)  d widened to fp32 at 16384 + 256 c + 4 x_slot(t)
//   [18432, 20480)  -ssum split as bf16 hi + lo: 16-byte entry (t, c / 4)
//                   at 18432 + 16 (2 t + c / 4), hi at 16-bit index c % 4,
//                   lo at 4 + c % 4
// Tokens past nt are quantized from zeros (d = 0, quants 0, -ssum = -0).
// A workgroup quantizes one chunk c of one record for 32 tokens (U = 1, two
// workgroups per chunk) or all 64 (U = 2: each lane group takes tokens i and
// 32 + i, both loads issued first), so the quant rows it writes are
// contiguous and the record, chunk and token half are workgroup-uniform.
template <int U>
__global__ __launch_bounds__(256) void quantize_tiled_kernel(const float *__restrict__ x, int64_t nt,
                                                              int64_t nsb, int64_t ldx,
                                                              uint8_t *__restrict__ q8t)
{
    const uint32_t wg = blockIdx.x;
    const int l8 = threadIdx.x & 7;
    const int cc = (int)((wg >> (U == 1 ? 1 : 0)) & 7);
    const uint32_t rec = wg >> (U == 1 ? 4 : 3);   // T * nsb + sb
    const uint32_t T = rec / (uint32_t)nsb, sb = rec - T * (uint32_t)nsb;
    const int tl0 = (U == 1 ? 32 * (int)(wg & 1) : 0) + (int)(threadIdx.x >> 3);
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t t = 64 * (int64_t)T + tl0 + 32 * u;
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < nt) v[u] = *reinterpret_cast<const float4 *>(x + t * ldx + 256 * (int64_t)sb + 32 * cc + 4 * l8);
    }
    uint8_t *r = q8t + (int64_t)rec * Q8T_RECORD;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int tl = tl0 + 32 * u;
        const QBlock q = quant_block(v[u]);
        const int h = l8 >> 2;
        *reinterpret_cast<uint32_t *>(r + 2048 * cc + 32 * tl + 16 * (h ^ swz(tl)) + 4 * (l8 & 3)) = q.packed;
        if (l8 == 0) {
            *reinterpret_cast<float *>(r + 16384 + 256 * cc + 4 * x_slot(tl)) = h2f(q.dbits);
        } else if (l8 == 7) {
            uint16_t hi, lo;
            bf16_split(-q.ssum, hi, lo);
            uint16_t *m = reinterpret_cast<uint16_t *>(r + 18432 + 16 * (2 * tl + (cc >> 2)));
            m[cc & 3] = hi;
            m[4 + (cc & 3)] = lo;
        }
    }
}

int launch_quantize(const float *x, int64_t nt, int64_t id, int64_t ldx, void *q8, hipStream_t stream)
{
    const int64_t nb32 = id / 32;
    const int64_t nblk = nt * nb32;
    if (nblk == 0) return 0;
    const int64_t grid = (nblk + 31) / 32;
    if (grid > 0x7fffffff) return -1;
    return launch_kernel(quantize_kernel, dim3((unsigned)grid), dim3(256), stream, x, nblk, nb32, ldx,
                         static_cast<uint8_t *>(q8));
}

int launch_quantize_tiled(const float *x, int64_t nt, int64_t id, int64_t ldx, void *q8t, hipStream_t stream)
{
    const int64_t nsb = id / 256;
    const int64_t nrec = (nt + 63) / 64 * nsb;
    if (nrec == 0) return 0;
    if (nrec * 16 > 0x7fffffff) return -1;
    // Two tokens per lane group once the plane has 1024 records or more:
    // measured 6% faster at 2630x18944 and 7% slower at 512x3584, where the
    // halved grid no longer covers the load latency.
    if (nrec >= 1024)
        return launch_kernel(quantize_tiled_kernel<2>, dim3((unsigned)(nrec * 8)), dim3(256), stream, x, nt, nsb,
                             ldx, static_cast<uint8_t *>(q8t));
    return launch_kernel(quantize_tiled_kernel<1>, dim3((unsigned)(nrec * 16)), dim3(256), stream, x, nt, nsb, ldx,
                         static_cast<uint8_t *>(q8t));
}

}  // namespace qig
