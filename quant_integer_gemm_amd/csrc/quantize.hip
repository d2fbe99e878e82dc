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
#include "qig_quant.h"

namespace qig {

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
    for (int u = 0; u < U; ++u) put_tiled(r, cc, tl0 + 32 * u, l8, quant_block(v[u]));
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
