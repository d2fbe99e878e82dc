// qig_launch.h -- internal launchers behind the C ABI (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qig {

struct MmqLaunch {
    int qtype;               // 4 (q4_K) or 6 (q6_K)
    const void *W;           // raw blocks
    const int8_t *Wexp;      // q6_K dense plane or nullptr
    const void *q8;          // pad40 activations
    float *y;                // output (GEMM mode) or nullptr
    int32_t *P;              // partials (test mode) or nullptr
    int64_t bstride, od, id, nt, ldy;
    int64_t t0, t1, j0, j1;  // output window
};

// All return 0, -1 (grid too large) or -3 (launch error).
int launch_mmq(const MmqLaunch &L, hipStream_t stream);
int launch_quantize(const float *x, int64_t nt, int64_t id, int64_t ldx, void *q8,
                    hipStream_t stream);
int launch_expand_q6k(const void *W, int64_t bstride, int64_t od, int64_t id, int8_t *Wexp,
                      hipStream_t stream);

}  // namespace qig
