// abi.hip -- the C ABI of libqig.so: argument checks, then one launch on the
// caller's stream.  Declarations and the full contract are in include/qig.h.
#include <qig.h>

#include "qig_launch.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int rc_from_launch(int r) { return r == 0 ? QIG_OK : (r == -1 ? QIG_EINVAL : QIG_ELAUNCH); }

// The GEMM kernels address the bytes of one 64-token, 64-row tile with
// 32-bit offsets: 64 pad40 rows (80 * id bytes), 64 raw weight rows
// (id * bstride / 4) and 64 dense-plane rows (64 * id).
bool tile_span_ok(int64_t id, int64_t bstride)
{
    const int64_t lim = int64_t(1) << 31;
    return id < lim / 80 && id / 4 < lim / bstride && id < lim / 64;
}

int check_gemm(const void *W, int64_t od, int64_t id, const void *q8, int64_t nt, const void *out,
               int64_t ldy, int64_t bstride)
{
    if (nt < 0 || od < 0 || id <= 0 || id % 256 != 0) return QIG_EINVAL;
    if (!tile_span_ok(id, bstride)) return QIG_EINVAL;
    if (ldy < od) return QIG_EINVAL;
    if (nt == 0 || od == 0) return QIG_OK;
    if (!W || !q8 || !out) return QIG_EINVAL;
    if (!aligned(W, 16) || !aligned(q8, 16) || !aligned(out, 4)) return QIG_EALIGN;
    return QIG_OK;
}

bool bad_bstride(int64_t bstride) { return bstride < 210 || bstride % 16 != 0; }

bool bad_window(int64_t nt, int64_t od, int64_t t0, int64_t t1, int64_t j0, int64_t j1)
{
    return t0 < 0 || t1 < t0 || t1 > nt || j0 < 0 || j1 < j0 || j1 > od;
}

}  // namespace

extern "C" {

size_t q8_pad40_bytes(int64_t nt, int64_t id)
{
    if (nt < 0 || id <= 0 || id % 32 != 0) return 0;
    return (size_t)nt * (size_t)(id / 32) * 40u;
}

const char *qig_strerror(int code)
{
    switch (code) {
    case QIG_OK: return "ok";
    case QIG_EINVAL: return "invalid shape, stride or size";
    case QIG_EALIGN: return "pointer or leading dimension misaligned";
    case QIG_ELAUNCH: return "HIP launch error";
    default: return "unknown error";
    }
}

int quantize_q8_pad40(const float *x, int64_t nt, int64_t id, int64_t ldx, void *q8, hipStream_t stream)
{
    if (nt < 0 || id <= 0 || id % 32 != 0 || ldx < id) return QIG_EINVAL;
    if (nt == 0) return QIG_OK;
    if (!x || !q8) return QIG_EINVAL;
    if (!aligned(x, 16) || !aligned(q8, 16) || ldx % 4 != 0) return QIG_EALIGN;
    return rc_from_launch(qig::launch_quantize(x, nt, id, ldx, q8, stream));
}

// ws: the stream-K workspace, or nullptr for whole tiles only.  tiled: q8 is
// a tiled plane (quantize_q8_tiled) instead of pad40.
static int gemm_q4k(const void *W, int64_t od, int64_t id, const void *q8, int64_t nt, float *y, int64_t ldy,
                    void *ws, bool tiled, hipStream_t stream)
{
    int rc = check_gemm(W, od, id, q8, nt, y, ldy, 144);
    if (rc != QIG_OK || nt == 0 || od == 0) return rc;
    if (ws && !aligned(ws, 16)) return QIG_EALIGN;
    qig::MmqLaunch L = {4, W, nullptr, q8, y, nullptr, 144, od, id, nt, ldy, 0, nt, 0, od};
    L.ws = ws;
    L.q8_tiled = tiled;
    return rc_from_launch(qig::launch_mmq(L, stream));
}

static int gemm_q6k(const void *W, int64_t bstride, const int8_t *W_exp, int64_t od, int64_t id,
                    const void *q8, int64_t nt, float *y, int64_t ldy, void *ws, bool tiled, hipStream_t stream)
{
    if (bad_bstride(bstride)) return QIG_EINVAL;
    int rc = check_gemm(W, od, id, q8, nt, y, ldy, bstride);
    if (rc != QIG_OK || nt == 0 || od == 0) return rc;
    if (W_exp && !aligned(W_exp, 16)) return QIG_EALIGN;
    if (ws && !aligned(ws, 16)) return QIG_EALIGN;
    qig::MmqLaunch L = {6, W, W_exp, q8, y, nullptr, bstride, od, id, nt, ldy, 0, nt, 0, od};
    L.ws = ws;
    L.q8_tiled = tiled;
    return rc_from_launch(qig::launch_mmq(L, stream));
}

int mmq_q4k(const void *W, int64_t od, int64_t id, const void *q8, int64_t nt, float *y, int64_t ldy,
            hipStream_t stream)
{
    return gemm_q4k(W, od, id, q8, nt, y, ldy, nullptr, false, stream);
}

int mmq_q6k(const void *W, int64_t bstride, const int8_t *W_exp, int64_t od, int64_t id, const void *q8,
            int64_t nt, float *y, int64_t ldy, hipStream_t stream)
{
    return gemm_q6k(W, bstride, W_exp, od, id, q8, nt, y, ldy, nullptr, false, stream);
}

size_t mmq_workspace_bytes(void) { return (size_t)qig::MMQ_WS_BYTES; }

int mmq_q4k_streamk(const void *W, int64_t od, int64_t id, const void *q8, int64_t nt, float *y, int64_t ldy,
                    void *ws, hipStream_t stream)
{
    if (!ws) return QIG_EINVAL;
    if (!aligned(ws, 16)) return QIG_EALIGN;
    return gemm_q4k(W, od, id, q8, nt, y, ldy, ws, false, stream);
}

int mmq_q6k_streamk(const void *W, int64_t bstride, const int8_t *W_exp, int64_t od, int64_t id,
                    const void *q8, int64_t nt, float *y, int64_t ldy, void *ws, hipStream_t stream)
{
    if (!ws) return QIG_EINVAL;
    if (!aligned(ws, 16)) return QIG_EALIGN;
    return gemm_q6k(W, bstride, W_exp, od, id, q8, nt, y, ldy, ws, false, stream);
}

int expand_q6k_dense(const void *W, int64_t bstride, int64_t od, int64_t id, int8_t *W_exp,
                     hipStream_t stream)
{
    if (bad_bstride(bstride) || od < 0 || id <= 0 || id % 256 != 0) return QIG_EINVAL;
    if (od == 0) return QIG_OK;
    if (!W || !W_exp) return QIG_EINVAL;
    if (!aligned(W, 16) || !aligned(W_exp, 16)) return QIG_EALIGN;
    return rc_from_launch(qig::launch_expand_q6k(W, bstride, od, id, W_exp, stream));
}

// quant plane bytes of a prepared buffer: q4_K keeps packed nibbles
static int64_t prepared_quant_bytes(int qtype, int64_t od, int64_t id) { return qtype == 4 ? od * (id / 2) : od * id; }

static size_t prepared_bytes(int qtype, int64_t od, int64_t id)
{
    if (od < 0 || id <= 0 || id % 256 != 0) return 0;
    return (size_t)prepared_quant_bytes(qtype, od, id) + (size_t)od * (size_t)(id / 256) * 64u;
}

size_t q4k_prepared_bytes(int64_t od, int64_t id) { return prepared_bytes(4, od, id); }

size_t q6k_prepared_bytes(int64_t od, int64_t id) { return prepared_bytes(6, od, id); }

int prepare_q4k(const void *W, int64_t od, int64_t id, void *Wp, hipStream_t stream)
{
    if (od < 0 || id <= 0 || id % 256 != 0) return QIG_EINVAL;
    if (od == 0) return QIG_OK;
    if (!W || !Wp) return QIG_EINVAL;
    if (!aligned(W, 16) || !aligned(Wp, 16)) return QIG_EALIGN;
    int8_t *Q = static_cast<int8_t *>(Wp);
    float *S = reinterpret_cast<float *>(static_cast<uint8_t *>(Wp) + prepared_quant_bytes(4, od, id));
    return rc_from_launch(qig::launch_prepare_q4k(W, od, id, Q, S, stream));
}

int prepare_q6k(const void *W, int64_t bstride, int64_t od, int64_t id, void *Wp, hipStream_t stream)
{
    if (bad_bstride(bstride) || od < 0 || id <= 0 || id % 256 != 0) return QIG_EINVAL;
    if (od == 0) return QIG_OK;
    if (!W || !Wp) return QIG_EINVAL;
    if (!aligned(W, 16) || !aligned(Wp, 16)) return QIG_EALIGN;
    int8_t *Q = static_cast<int8_t *>(Wp);
    float *S = reinterpret_cast<float *>(static_cast<uint8_t *>(Wp) + od * id);
    int rc = rc_from_launch(qig::launch_expand_q6k(W, bstride, od, id, Q, stream));
    if (rc != QIG_OK) return rc;
    return rc_from_launch(qig::launch_prepare_q6k_scales(W, bstride, od, id, S, stream));
}

static int mmq_prepared(int qtype, const void *Wp, int64_t od, int64_t id, const void *q8, int64_t nt, float *y,
                        int64_t ldy, void *ws, hipStream_t stream, bool tiled = false)
{
    int rc = check_gemm(Wp, od, id, q8, nt, y, ldy, 64);
    if (rc != QIG_OK || nt == 0 || od == 0) return rc;
    if (ws && !aligned(ws, 16)) return QIG_EALIGN;
    const int8_t *Q = static_cast<const int8_t *>(Wp);
    const void *S = static_cast<const uint8_t *>(Wp) + prepared_quant_bytes(qtype, od, id);
    qig::MmqLaunch L = {qtype, S, Q, q8, y, nullptr, 64, od, id, nt, ldy, 0, nt, 0, od, true};
    L.ws = ws;
    L.q8_tiled = tiled;
    return rc_from_launch(qig::launch_mmq(L, stream));
}

int mmq_q4k_prepared(const void *Wp, int64_t od, int64_t id, const void *q8, int64_t nt, float *y, int64_t ldy,
                     hipStream_t stream)
{
    return mmq_prepared(4, Wp, od, id, q8, nt, y, ldy, nullptr, stream);
}

int mmq_q6k_prepared(const void *Wp, int64_t od, int64_t id, const void *q8, int64_t nt, float *y, int64_t ldy,
                     hipStream_t stream)
{
    return mmq_prepared(6, Wp, od, id, q8, nt, y, ldy, nullptr, stream);
}

int mmq_q4k_prepared_streamk(const void *Wp, int64_t od, int64_t id, const void *q8, int64_t nt, float *y,
                             int64_t ldy, void *ws, hipStream_t stream)
{
    if (!ws) return QIG_EINVAL;
    if (!aligned(ws, 16)) return QIG_EALIGN;
    return mmq_prepared(4, Wp, od, id, q8, nt, y, ldy, ws, stream);
}

int mmq_q6k_prepared_streamk(const void *Wp, int64_t od, int64_t id, const void *q8, int64_t nt, float *y,
                             int64_t ldy, void *ws, hipStream_t stream)
{
    if (!ws) return QIG_EINVAL;
    if (!aligned(ws, 16)) return QIG_EALIGN;
    return mmq_prepared(6, Wp, od, id, q8, nt, y, ldy, ws, stream);
}

size_t q8_tiled_bytes(int64_t nt, int64_t id)
{
    if (nt < 0 || id <= 0 || id % 256 != 0) return 0;
    return (size_t)((nt + 63) / 64) * (size_t)(id / 256) * (size_t)qig::Q8T_RECORD;
}

int quantize_q8_tiled(const float *x, int64_t nt, int64_t id, int64_t ldx, void *q8t, hipStream_t stream)
{
    if (nt < 0 || id <= 0 || id % 256 != 0 || ldx < id) return QIG_EINVAL;
    if (nt == 0) return QIG_OK;
    if (!x || !q8t) return QIG_EINVAL;
    if (!aligned(x, 16) || !aligned(q8t, 16) || ldx % 4 != 0) return QIG_EALIGN;
    return rc_from_launch(qig::launch_quantize_tiled(x, nt, id, ldx, q8t, stream));
}

int mmq_q4k_q8t(const void *W, int64_t od, int64_t id, const void *q8t, int64_t nt, float *y, int64_t ldy, void *ws,
                hipStream_t stream)
{
    return gemm_q4k(W, od, id, q8t, nt, y, ldy, ws, true, stream);
}

int mmq_q4k_xf32(const void *W, int64_t od, int64_t id, const float *x, int64_t ldx, int64_t nt, float *y,
                 int64_t ldy, void *ws, hipStream_t stream)
{
    if (ldx < id) return QIG_EINVAL;
    int rc = check_gemm(W, od, id, x, nt, y, ldy, 144);
    if (rc != QIG_OK || nt == 0 || od == 0) return rc;
    if (ldx % 4 != 0) return QIG_EALIGN;
    if (ws && !aligned(ws, 16)) return QIG_EALIGN;
    qig::MmqLaunch L = {4, W, nullptr, x, y, nullptr, 144, od, id, nt, ldy, 0, nt, 0, od};
    L.ws = ws;
    L.x_f32 = true;
    L.ldx = ldx;
    return rc_from_launch(qig::launch_mmq(L, stream));
}

int mmq_q6k_q8t(const void *W, int64_t bstride, const int8_t *W_exp, int64_t od, int64_t id, const void *q8t,
                int64_t nt, float *y, int64_t ldy, void *ws, hipStream_t stream)
{
    return gemm_q6k(W, bstride, W_exp, od, id, q8t, nt, y, ldy, ws, true, stream);
}

size_t q4k_staged_bytes(int64_t od, int64_t id)
{
    if (od < 0 || id <= 0 || id % 256 != 0) return 0;
    return (size_t)((od + 63) / 64) * (size_t)(id / 256) * (size_t)qig::Q4S_RECORD;
}

int prepare_q4k_staged(const void *W, int64_t od, int64_t id, void *Ws, hipStream_t stream)
{
    if (od < 0 || id <= 0 || id % 256 != 0) return QIG_EINVAL;
    if (od == 0) return QIG_OK;
    if (!W || !Ws) return QIG_EINVAL;
    if (!aligned(W, 16) || !aligned(Ws, 16)) return QIG_EALIGN;
    return rc_from_launch(qig::launch_prepare_q4k_staged(W, od, id, Ws, stream));
}

int mmq_q4k_staged_q8t(const void *Ws, int64_t od, int64_t id, const void *q8t, int64_t nt, float *y, int64_t ldy,
                       void *ws, hipStream_t stream)
{
    // a record spans 64 rows of id/256 super-blocks: its byte offsets stay
    // below 2^31 when the raw blocks' do
    int rc = check_gemm(Ws, od, id, q8t, nt, y, ldy, 144);
    if (rc != QIG_OK || nt == 0 || od == 0) return rc;
    if (ws && !aligned(ws, 16)) return QIG_EALIGN;
    qig::MmqLaunch L = {4, nullptr, static_cast<const int8_t *>(Ws), q8t, y, nullptr, 144, od, id, nt, ldy,
                        0, nt, 0, od};
    L.ws = ws;
    L.q8_tiled = true;
    L.staged = true;
    return rc_from_launch(qig::launch_mmq(L, stream));
}

size_t q6k_limbs_bytes(int64_t od, int64_t id)
{
    if (od < 0 || id <= 0 || id % 256 != 0) return 0;
    return 2 * (size_t)od * (size_t)id + (size_t)od * (size_t)(id / 256) * 4u;
}

int prepare_q6k_limbs(const void *W, int64_t bstride, int64_t od, int64_t id, void *Wl, hipStream_t stream)
{
    if (bad_bstride(bstride) || od < 0 || id <= 0 || id % 256 != 0) return QIG_EINVAL;
    if (od == 0) return QIG_OK;
    if (!W || !Wl) return QIG_EINVAL;
    if (!aligned(W, 16) || !aligned(Wl, 16)) return QIG_EALIGN;
    return rc_from_launch(qig::launch_prepare_q6k_limbs(W, bstride, od, id, Wl, stream));
}

int mmq_q6k_limbs_q8t(const void *Wl, int64_t od, int64_t id, const void *q8t, int64_t nt, float *y, int64_t ldy,
                      void *ws, hipStream_t stream)
{
    int rc = check_gemm(Wl, od, id, q8t, nt, y, ldy, 64);
    if (rc != QIG_OK || nt == 0 || od == 0) return rc;
    if (ws && !aligned(ws, 16)) return QIG_EALIGN;
    const uint8_t *H = static_cast<const uint8_t *>(Wl);
    const void *D = H + 2 * od * id;
    qig::MmqLaunch L = {6, D, reinterpret_cast<const int8_t *>(H), q8t, y, nullptr, 64, od, id, nt, ldy, 0, nt, 0, od};
    L.ws = ws;
    L.q8_tiled = true;
    L.limbs = true;
    return rc_from_launch(qig::launch_mmq(L, stream));
}

int mmq_q4k_q8t_noalloc(const void *W, int64_t od, int64_t id, const void *q8t, int64_t nt, float *y, int64_t ldy,
                        hipStream_t stream)
{
    int rc = check_gemm(W, od, id, q8t, nt, y, ldy, 144);
    if (rc != QIG_OK || nt == 0 || od == 0) return rc;
    void *ws = qig::mmq_scratch();
    if (!ws) return QIG_ELAUNCH;
    qig::MmqLaunch L = {4, W, nullptr, q8t, y, nullptr, 144, od, id, nt, ldy, 0, nt, 0, od};
    L.ws = ws;
    L.q8_tiled = true;
    L.ws_workers = qig::MMQ_SCRATCH_WORKERS;
    L.clear_counters = true;
    return rc_from_launch(qig::launch_mmq(L, stream));
}

int mmq_q4k_prepared_q8t(const void *Wp, int64_t od, int64_t id, const void *q8t, int64_t nt, float *y, int64_t ldy,
                         void *ws, hipStream_t stream)
{
    return mmq_prepared(4, Wp, od, id, q8t, nt, y, ldy, ws, stream, true);
}

int mmq_q6k_prepared_q8t(const void *Wp, int64_t od, int64_t id, const void *q8t, int64_t nt, float *y, int64_t ldy,
                         void *ws, hipStream_t stream)
{
    return mmq_prepared(6, Wp, od, id, q8t, nt, y, ldy, ws, stream, true);
}

int mmq_q4k_partials(const void *W, int64_t od, int64_t id, const void *q8, int64_t nt, int64_t t0,
                     int64_t t1, int64_t j0, int64_t j1, int32_t *P, hipStream_t stream)
{
    int rc = check_gemm(W, od, id, q8, nt, P, od, 144);
    if (rc != QIG_OK) return rc;
    if (bad_window(nt, od, t0, t1, j0, j1)) return QIG_EINVAL;
    if (t1 == t0 || j1 == j0) return QIG_OK;
    qig::MmqLaunch L = {4, W, nullptr, q8, nullptr, P, 144, od, id, nt, 0, t0, t1, j0, j1};
    return rc_from_launch(qig::launch_mmq(L, stream));
}

int mmq_q6k_partials(const void *W, int64_t bstride, const int8_t *W_exp, int64_t od, int64_t id,
                     const void *q8, int64_t nt, int64_t t0, int64_t t1, int64_t j0, int64_t j1, int32_t *P,
                     hipStream_t stream)
{
    if (bad_bstride(bstride)) return QIG_EINVAL;
    int rc = check_gemm(W, od, id, q8, nt, P, od, bstride);
    if (rc != QIG_OK) return rc;
    if (W_exp && !aligned(W_exp, 16)) return QIG_EALIGN;
    if (bad_window(nt, od, t0, t1, j0, j1)) return QIG_EINVAL;
    if (t1 == t0 || j1 == j0) return QIG_OK;
    qig::MmqLaunch L = {6, W, W_exp, q8, nullptr, P, bstride, od, id, nt, 0, t0, t1, j0, j1};
    return rc_from_launch(qig::launch_mmq(L, stream));
}

}  // extern "C"
