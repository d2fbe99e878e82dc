// quantize.hip -- fp32 activations -> q8 pad40 blocks on gfx950.
//
// Block (t, c) of 32 elements lives at byte (t*id/32 + c)*40: fp16 d at 0,
// zero at 2, 32 int8 quants at 4, fp32 ssum at 36 (pad40 layout of the r21
// page "Coalesced block-linear A staging", s2.1, addressed as on the r20 page
// "Split-phase A staging", s3.2).  d32 = max|x|/127 with IEEE division,
// q = round-half-away(x/d32) clamped to +-127, d = fp16(d32) round-to-even,
// ssum = d*sum(q) (exact in fp32).
//
// HBM-bound: 8 lanes own one block, each lane one float4, so one wave reads
// 1 KB of contiguous x per instruction; max and sum reduce over the 8 lanes
// with cross-lane shuffles.
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

__device__ __forceinline__ int quant1(float x, float d32)
{
    if (d32 == 0.0f) return 0;
    float r = round_half_away(x / d32);
    r = __builtin_fminf(__builtin_fmaxf(r, -127.0f), 127.0f);
    return (int)r;
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
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, 8));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2, 8));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 4, 8));
    const float d32 = amax / 127.0f;
    const int q0 = quant1(v.x, d32), q1 = quant1(v.y, d32), q2 = quant1(v.z, d32), q3 = quant1(v.w, d32);
    int s = q0 + q1 + q2 + q3;
    s += __shfl_xor(s, 1, 8);
    s += __shfl_xor(s, 2, 8);
    s += __shfl_xor(s, 4, 8);
    QBlock r;
    r.packed = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) | ((uint32_t)(q2 & 0xff) << 16) |
               ((uint32_t)(q3 & 0xff) << 24);
    const _Float16 dh = (_Float16)d32;
    r.dbits = (uint32_t)__builtin_bit_cast(uint16_t, dh);
    r.ssum = (float)dh * (float)s;
    return r;
}

__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ x, int64_t nblk,
                                                        int64_t nb32, int64_t ldx,
                                                        uint8_t *__restrict__ q8)
{
    const int64_t blk = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    const int l8 = threadIdx.x & 7;
    const bool valid = blk < nblk;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) {
        const int64_t t = blk / nb32, c = blk - (blk / nb32) * nb32;
        v = *reinterpret_cast<const float4 *>(x + t * ldx + 32 * c + 4 * l8);
    }
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
// Blocks are visited token fastest within a (T, sb, c) run of 64, so the
// quant rows of consecutive blocks are contiguous.
__global__ __launch_bounds__(256) void quantize_tiled_kernel(const float *__restrict__ x, int64_t nt,
                                                              int64_t nsb, int64_t ldx, int64_t nblk,
                                                              uint8_t *__restrict__ q8t)
{
    const int64_t blk = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    const int l8 = threadIdx.x & 7;
    const bool valid = blk < nblk;
    const int tl = (int)(blk & 63);
    const int cc = (int)((blk >> 6) & 7);
    const int64_t rec = blk >> 9;                  // T * nsb + sb
    const int64_t T = rec / nsb, sb = rec - T * nsb;
    const int64_t t = 64 * T + tl;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid && t < nt) v = *reinterpret_cast<const float4 *>(x + t * ldx + 256 * sb + 32 * cc + 4 * l8);
    const QBlock q = quant_block(v);
    if (!valid) return;
    uint8_t *r = q8t + rec * Q8T_RECORD;
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

int launch_quantize(const float *x, int64_t nt, int64_t id, int64_t ldx, void *q8, hipStream_t stream)
{
    const int64_t nb32 = id / 32;
    const int64_t nblk = nt * nb32;
    if (nblk == 0) return 0;
    const int64_t grid = (nblk + 31) / 32;
    if (grid > 0x7fffffff) return -1;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, nblk, nb32, ldx,
                       static_cast<uint8_t *>(q8));
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_quantize_tiled(const float *x, int64_t nt, int64_t id, int64_t ldx, void *q8t, hipStream_t stream)
{
    const int64_t nsb = id / 256;
    const int64_t ntt = (nt + 63) / 64;
    const int64_t nblk = ntt * nsb * 512;          // 64 tokens x 8 chunks per record
    if (nblk == 0) return 0;
    const int64_t grid = (nblk + 31) / 32;
    if (grid > 0x7fffffff) return -1;
    hipLaunchKernelGGL(quantize_tiled_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, nt, nsb, ldx, nblk,
                       static_cast<uint8_t *>(q8t));
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace qig
