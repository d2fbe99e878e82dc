// qig_quant.h -- quantization of one 32-element activation block into the
// q8 pad40 fields (quant bytes, fp16 d, ssum), as the r21 page "Coalesced
// block-linear A staging", s2.1, defines the block: d32 = max|x|/127 with
// IEEE division, q = round-half-away(x/d32) clamped to +-127, d =
// fp16(d32) round-to-even, ssum = d*sum(q) (exact in fp32).  Eight lanes own
// one block, each lane one float4; max and sum reduce over the eight lanes
// with DPP moves.  Used by the quantize kernels and by the GEMM's
// fp32-activation source, which quantizes its stage in the prologue.
#pragma once
#include "qig_device.h"

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


// Lane l8 of the group that quantized chunk cc (0..7) of tile-local token tl
// (0..63) stores its share of the block into a tiled record at r (global
// memory, or the GEMM's LDS stage, which has the same bytes):
//   [0, 16384)      quants, row (cc, tl) of 32 bytes at 2048 cc + 32 tl, its
//                   16-byte halves h at 16 (h ^ swz(tl))
//   [16384, 18432)  d widened to fp32 at 16384 + 256 cc + 4 x_slot(tl)
//   [18432, 20480)  -ssum split as bf16 hi + lo: 16-byte entry (tl, cc / 4)
//                   at 18432 + 16 (2 tl + cc / 4), hi at 16-bit index cc % 4,
//                   lo at 4 + cc % 4
__device__ __forceinline__ void put_tiled(uint8_t *r, int cc, int tl, int l8, const QBlock &q)
{
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

}  // namespace qig
