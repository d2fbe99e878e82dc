// qig_launch.h -- internal launchers behind the C ABI (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

namespace qig {

// Enqueue kernel<<<grid, block, 0, stream>>>(args...) and return 0, or -3 if
// the runtime refused this launch.  The status is hipLaunchKernel's own: a
// triple-chevron launch followed by hipGetLastError() would also report, and
// clear, an error left on the calling thread by an earlier, unrelated call.
template <typename... Params, typename... Args>
inline int launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, hipStream_t stream, Args... args)
{
    static_assert(sizeof...(Params) == sizeof...(Args), "argument count");
    std::tuple<Params...> held(static_cast<Params>(args)...);
    const hipError_t e = std::apply(
        [&](auto &...a) {
            void *ptrs[] = {static_cast<void *>(&a)...};
            return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, 0, stream);
        },
        held);
    return e == hipSuccess ? 0 : -3;
}

struct MmqLaunch {
    int qtype;               // 4 (q4_K) or 6 (q6_K)
    const void *W;           // raw blocks; prepared: the scale plane
    const int8_t *Wexp;      // q6_K dense plane or nullptr; prepared: the quant plane
    const void *q8;          // pad40 activations
    float *y;                // output (GEMM mode) or nullptr
    int32_t *P;              // partials (test mode) or nullptr
    int64_t bstride, od, id, nt, ldy;
    int64_t t0, t1, j0, j1;  // output window
    bool prepared = false;   // W / Wexp point into a prepared buffer
    void *ws = nullptr;      // stream-K workspace (mmq_ws_bytes(ws_workers), zeroed once) or nullptr
    bool q8_tiled = false;   // q8 is a tiled plane (launch_quantize_tiled), not pad40
    int64_t ws_workers = 1024;     // workgroups the workspace has partial slots and counters for
    bool clear_counters = false;   // zero the arrival counters before a split launch
    bool limbs = false;      // q6_K limb buffer: W = its d plane, Wexp = its H plane (L plane follows)
    bool x_f32 = false;      // q8 points to fp32 activations (ldx floats per token), quantized in the GEMM
    int64_t ldx = 0;
    bool staged = false;     // q4_K staged buffer: Wexp = its records (W unused)
};

// Stream-K workspace: two 64 x 64 fp32 partial-sum slots per worker, then
// four uint32 arrival counters (one per wave's quarter tile) per worker.  At most MMQ_MAX_WORKERS workers (two
// per CU); a split needs at least MMQ_MIN_SPLIT_ITERS super-blocks per worker.
constexpr int64_t MMQ_MAX_WORKERS = 1024;
constexpr int64_t MMQ_MIN_SPLIT_ITERS = 4;
// stream-K only for a single round of tiles filling at most NUM/DEN of the slots
constexpr int64_t MMQ_SK_FILL_NUM = 3, MMQ_SK_FILL_DEN = 4;
// Bytes of a workspace for `workers` workgroups: the partial slots, then the
// counters.
constexpr int64_t mmq_ws_partial_bytes(int64_t workers) { return workers * 2 * 64 * 64 * 4; }
constexpr int64_t mmq_ws_bytes(int64_t workers) { return mmq_ws_partial_bytes(workers) + workers * 16; }
constexpr int64_t MMQ_WS_BYTES = mmq_ws_bytes(MMQ_MAX_WORKERS);
// The library's own workspace for calls that cannot allocate: a file-scope
// device array sized for two workgroups on each of 256 CUs.
constexpr int64_t MMQ_SCRATCH_WORKERS = 512;
constexpr int64_t MMQ_SCRATCH_BYTES = mmq_ws_bytes(MMQ_SCRATCH_WORKERS);

// All return 0, -1 (grid too large) or -3 (launch error).
int launch_mmq(const MmqLaunch &L, hipStream_t stream);
// Device address of this device's library scratch (MMQ_SCRATCH_BYTES), found
// once per device; nullptr if the runtime cannot resolve it.
void *mmq_scratch(void);
int launch_quantize(const float *x, int64_t nt, int64_t id, int64_t ldx, void *q8,
                    hipStream_t stream);
int launch_expand_q6k(const void *W, int64_t bstride, int64_t od, int64_t id, int8_t *Wexp,
                      hipStream_t stream);
// Tiled activation plane: one record of Q8T_RECORD bytes per (64-token tile,
// super-block) -- quants [8][64][32] (halves swizzled), fp32 d [8][64] in
// register order, bf16 hi/lo pairs of -ssum [64][2][8] -- the first bytes of
// the GEMM's LDS stage, so the GEMM copies it without conversion.
constexpr int64_t Q8T_RECORD = 20480;
// Staged q4_K weights: one record of Q4S_RECORD bytes per (64-row tile,
// super-block), the byte image of the weight part of the GEMM's LDS stage.
constexpr int64_t Q4S_RECORD = 14336;
int launch_quantize_tiled(const float *x, int64_t nt, int64_t id, int64_t ldx, void *q8t, hipStream_t stream);
// Prepared buffers: quant plane (q6_K: [od][id] centred int8; q4_K:
// [od][id/2] packed nibble bytes), then scale plane [od][id/256][16] fp32
// (q4_K: d*sc and dmin*m of each of the 8 sub-blocks, in pairs; q6_K: d*sc
// of the 16).
int launch_prepare_q4k(const void *W, int64_t od, int64_t id, int8_t *Q, float *S, hipStream_t stream);
// q6_K limb buffer: H plane int8 [od][id], L plane int8 [od][id], then d
// plane fp32 [od][id/256]; v = sc * c6 = 128 H + L per element.
int launch_prepare_q4k_staged(const void *W, int64_t od, int64_t id, void *R, hipStream_t stream);
int launch_prepare_q6k_limbs(const void *W, int64_t bstride, int64_t od, int64_t id, void *Wl, hipStream_t stream);
int launch_prepare_q6k_scales(const void *W, int64_t bstride, int64_t od, int64_t id, float *S,
                              hipStream_t stream);

}  // namespace qig
