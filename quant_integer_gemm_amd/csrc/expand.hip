// expand.hip -- raw q6_K (padded stride) -> dense centred-int8 plane W_exp.
//
// W_exp[j*id + 256*sb + e] = centred element e of super-block sb of row j
// (r43 page "PC-sampling attribution", s3.2; r44 page "W_exp stride mismatch
// root cause", s2.2: dense row stride id and super-block stride 256, against
// the raw plane's row stride nsb*bstride and block stride bstride).
// One thread per (row, super-block, 128-element half): 96 bytes of ql/qh in,
// 128 bytes out, all as 16-byte accesses.  HBM-bound.
#include "qig_device.h"
#include "qig_launch.h"

namespace qig {

__global__ __launch_bounds__(256) void expand_q6k_kernel(const uint8_t *__restrict__ W, int64_t bstride,
                                                          int64_t od, int64_t id, uint8_t *__restrict__ out)
{
    const int64_t nsb = id / 256;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= od * nsb * 2) return;
    const int h = (int)(gid & 1);
    const int64_t sb = (gid >> 1) % nsb;
    const int64_t j = (gid >> 1) / nsb;
    const uint8_t *blk = W + j * nsb * bstride + sb * bstride;
    u32x4 ql[4], qh[2];
#pragma unroll
    for (int k = 0; k < 4; ++k) ql[k] = *reinterpret_cast<const u32x4 *>(blk + 64 * h + 16 * k);
#pragma unroll
    for (int k = 0; k < 2; ++k) qh[k] = *reinterpret_cast<const u32x4 *>(blk + 128 + 32 * h + 16 * k);
    uint8_t *dst = out + j * id + 256 * sb + 128 * h;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = 4 * hh + e;
                o[e] = q6_centred(ql[2 * (qq & 1) + (k >> 2)][k & 3], qh[k >> 2][k & 3], qq);
            }
            *reinterpret_cast<u32x4 *>(dst + 32 * qq + 16 * hh) = o;
        }
}

int launch_expand_q6k(const void *W, int64_t bstride, int64_t od, int64_t id, int8_t *Wexp,
                      hipStream_t stream)
{
    const int64_t n = od * (id / 256) * 2;
    if (n == 0) return 0;
    const int64_t grid = (n + 255) / 256;
    if (grid > 0x7fffffff) return -1;
    return launch_kernel(expand_q6k_kernel, dim3((unsigned)grid), dim3(256), stream,
                         static_cast<const uint8_t *>(W), bstride, od, id, reinterpret_cast<uint8_t *>(Wexp));
}

}  // namespace qig
