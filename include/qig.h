/*
 * qig.h -- C ABI of libqig.so, the MI355X (gfx950) k-quant prefill MMQ.
 *
 * The operation (the "minfer CUDA optimization steps" pages, r20/r21/r43/r44):
 * weights stored as 256-element k-quant super-blocks (q6_K or q4_K) times
 * activations quantized per token into q8 "pad40" blocks, contracted as
 * int8 x int8 -> int32 sub-block dot products and rescaled to an fp32
 * output y[nt][od] = x[nt][id] . W[od][id]^T.
 *
 * Conventions shared by every entry point
 *  - All buffer pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or synchronises inside a call; work is enqueued on
 *    `stream` (0 = the null stream) and the call returns at once.
 *  - Shapes are element counts.  nt (tokens) and od (weight rows) may be 0:
 *    the call then does nothing and returns QIG_OK.  id (the contraction
 *    length) must be a positive multiple of 256 for the GEMMs (one super-
 *    block) and of 32 for the quantizer (one pad40 chunk).
 *  - Return value: QIG_OK, or a negative QIG_E* code; nothing is enqueued
 *    when an argument check fails.  qig_strerror() names a code.
 *  - Outputs never alias inputs.  NaN/Inf inputs give unspecified output.
 *  - Calls on one stream run in order; calls on different streams that write
 *    the same buffer race.
 */
#ifndef QIG_H
#define QIG_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QIG_OK 0
#define QIG_EINVAL (-1)   /* bad shape, stride or size */
#define QIG_EALIGN (-2)   /* pointer or leading dimension misaligned */
#define QIG_ELAUNCH (-3)  /* the HIP runtime reported a launch error */

/* Size in bytes of a pad40 plane for nt tokens of id elements:
 * nt * (id / 32) * 40.  Returns 0 for invalid arguments. */
size_t q8_pad40_bytes(int64_t nt, int64_t id);

/* Human-readable name of a return code (static string, never NULL). */
const char *qig_strerror(int code);

/*
 * quantize_q8_pad40 -- per-token activation quantization into pad40 blocks.
 * Layout (r21 page "Coalesced block-linear A staging", s2.1; r20 page
 * "Split-phase A staging", s3.2): one 40-byte block per (token t, chunk c of
 * 32 elements) at byte offset (t * id/32 + c) * 40, holding fp16 d at bytes
 * 0-1, zero at 2-3, 32 int8 quants at 4-35 and fp32 ssum at 36-39.
 * Fill rule: d32 = max|x| / 127 (fp32 division), q = round-half-away(x / d32)
 * clamped to [-127, 127] (all 0 when d32 == 0), d = fp16 of d32 (round to
 * nearest even, subnormals kept), ssum = d * sum(q) in fp32 (exact).
 *
 *   x      [nt][ldx] fp32, 16-byte aligned, ldx >= id, ldx % 4 == 0
 *   q8     q8_pad40_bytes(nt, id) bytes, 16-byte aligned; every byte written
 * Errors: QIG_EINVAL (nt < 0, id <= 0 or id % 32, ldx < id),
 *         QIG_EALIGN (x or q8 not 16-byte aligned, ldx % 4).
 */
int quantize_q8_pad40(const float *x, int64_t nt, int64_t id, int64_t ldx,
                      void *q8, hipStream_t stream);

/*
 * mmq_q4k -- y[nt][od] = pad40(x) . W^T for q4_K weights.
 * W is [od][id/256] blocks of 144 bytes, contiguous: fp16 d at 0, fp16 dmin
 * at 2, twelve bytes of packed 6-bit (scale, min) pairs at 4, 128 bytes of
 * 4-bit quants at 16 (GGUF block_q4_K; the pages name the format but do not
 * print its layout).  Per 32-element sub-block b of super-block sb:
 *   y += da(t,c) * d * sc_b * P4(t,j,c) - dmin * m_b * ssum(t,c),
 *   P4 = int32 sum over the chunk of q8 quants times 4-bit quants,
 * c = 8*sb + b being the matching pad40 chunk.
 *
 *   W      16-byte aligned
 *   q8     pad40 plane of nt tokens x id, 16-byte aligned
 *   y      [nt][ldy] fp32, ldy >= od; overwritten (not accumulated),
 *          4-byte aligned
 * Errors: QIG_EINVAL (nt < 0, od < 0, id <= 0 or id % 256, ldy < od, or
 *         id too large for 32-bit offsets within one 64-token, 64-row tile:
 *         80*id, id*bstride/4 (bstride = 144 here) and 64*id must stay below
 *         2^31), QIG_EALIGN, QIG_ELAUNCH.
 */
int mmq_q4k(const void *W, int64_t od, int64_t id, const void *q8, int64_t nt,
            float *y, int64_t ldy, hipStream_t stream);

/*
 * mmq_q6k -- y[nt][od] = pad40(x) . W^T for q6_K weights.
 * W is the padded raw plane (r44 page "W_exp stride mismatch root cause",
 * s2.2): row j, super-block sb at W + j*nsb*bstride + sb*bstride, nsb =
 * id/256; each block holds ql[128] at 0, qh[64] at 128, 16 int8 sub-block
 * scales at 192 and fp16 d at 208; bytes 210..bstride-1 are ignored.
 * Sixteen 16-element sub-blocks, each with its own d*sc (r44 page s1.1):
 *   y += da(t, 8*sb + s/2) * d * sc_s * P6(t,j,sb,s).
 * Element map of the 6-bit quants: r44 page s3.2 (centred value in
 * [-32, 31]).
 *
 *   bstride  >= 210 and a multiple of 16 (224 for the padded in-VRAM form)
 *   W_exp    NULL: quants are decoded from W.  Non-NULL: the dense centred
 *            plane made by expand_q6k_dense (od x id int8, row stride id,
 *            super-block stride 256, 16-byte aligned) supplies the quants;
 *            d and the scales are still read from W.  Both arms give
 *            bit-identical y.
 *   W, q8, y as for mmq_q4k.
 * Errors: QIG_EINVAL (shapes as mmq_q4k, bad bstride), QIG_EALIGN,
 *         QIG_ELAUNCH.
 */
int mmq_q6k(const void *W, int64_t bstride, const int8_t *W_exp, int64_t od,
            int64_t id, const void *q8, int64_t nt, float *y, int64_t ldy,
            hipStream_t stream);

/*
 * expand_q6k_dense -- registration-time expansion of raw q6_K into the dense
 * centred-int8 plane W_exp (r43 page "PC-sampling attribution", s3.2; r44
 * page s2.2 and s3.2): W_exp[j*id + 256*sb + e] = centred element e of
 * super-block sb of row j.
 *
 *   W      padded raw plane as for mmq_q6k, 16-byte aligned
 *   W_exp  od * id bytes, 16-byte aligned; every byte written
 * Errors: QIG_EINVAL (od < 0, id <= 0 or id % 256, bad bstride),
 *         QIG_EALIGN, QIG_ELAUNCH.
 */
int expand_q6k_dense(const void *W, int64_t bstride, int64_t od, int64_t id,
                     int8_t *W_exp, hipStream_t stream);

/*
 * Prepared weights -- registration-time planes that let the GEMM stage its
 * weights without decoding them (device memory traded for work, as the
 * dense-plane arm above does for q6_K quants; r44 page s2.4 weighs that
 * trade).  A prepared buffer of qNk_prepared_bytes(od, id) = Qb +
 * od*(id/256)*64 bytes holds
 *   quant plane  at offset 0, Qb bytes.  q6_K: int8 [od][id], the values
 *                centred to [-32, 31] (the same bytes as expand_q6k_dense),
 *                Qb = od*id.  q4_K: the packed 4-bit quants of each block
 *                as in the raw block, [od][id/2] with 128 bytes per
 *                super-block, Qb = od*id/2 (a byte per element measured
 *                slower: it doubles the bytes the GEMM loads)
 *   scale plane  fp32 [od][id/256][16] at offset Qb:
 *                q4_K: d*sc_b, dmin*m_b for b = 0..7, in pairs;
 *                q6_K: d*sc of the 16 sub-blocks,
 * each product formed as the raw-block GEMM forms it (one fp32 rounding of
 * fp16 d times the integer scale), so mmq_qNk_prepared gives bit-identical y
 * to mmq_qNk on the raw blocks.  The layout is part of this contract.  The
 * q6_K buffer removes all weight decoding from the GEMM; the q4_K buffer
 * removes the 6-bit scale/min unpacking and keeps the nibble split.
 *
 *   W     raw blocks as for mmq_q4k / mmq_q6k, 16-byte aligned
 *   Wp    the prepared buffer, 16-byte aligned; every byte written
 * qNk_prepared_bytes returns 0 for invalid shapes.  prepare_*: QIG_EINVAL
 * (od < 0, id <= 0 or id % 256, bad bstride), QIG_EALIGN, QIG_ELAUNCH.
 * mmq_qNk_prepared: arguments and errors as mmq_q4k with W replaced by Wp.
 */
size_t q4k_prepared_bytes(int64_t od, int64_t id);
size_t q6k_prepared_bytes(int64_t od, int64_t id);
int prepare_q4k(const void *W, int64_t od, int64_t id, void *Wp, hipStream_t stream);
int prepare_q6k(const void *W, int64_t bstride, int64_t od, int64_t id, void *Wp,
                hipStream_t stream);
int mmq_q4k_prepared(const void *Wp, int64_t od, int64_t id, const void *q8,
                     int64_t nt, float *y, int64_t ldy, hipStream_t stream);
int mmq_q6k_prepared(const void *Wp, int64_t od, int64_t id, const void *q8,
                     int64_t nt, float *y, int64_t ldy, hipStream_t stream);

/*
 * Stream-K variants -- the same GEMMs, with the work split by super-block
 * when the 64 x 64 output tiles leave much of the GPU idle (the pages'
 * reference launches a stream-k grid plus a fix-up kernel for the q-proj
 * shape: r20 page "Split-phase A staging", s1 and s2.2).  When the tiles
 * form a single round that fills at most three quarters of the workgroup
 * slots (two per CU), the (tile, super-block) iterations are shared evenly
 * by all slots, and a tile split between workgroups is summed from their
 * partial sums in a fixed order, so y is the same on every call (it may
 * differ from the plain call's y by fp32 rounding order, within the output
 * tolerance).  Other shapes, and id < 512, run exactly as the plain calls:
 * on them whole tiles measured faster.
 *
 *   ws     mmq_workspace_bytes() bytes of device memory, 16-byte aligned,
 *          owned by the caller and ZERO-FILLED ONCE before its first use.
 *          It holds partial sums (written before they are read) and, in
 *          its last 16384 bytes, arrival counters that every call returns to
 *          zero; do not write to it between calls.  Calls that may run at
 *          the same time (different streams) need different workspaces;
 *          calls in order on one stream may share one.
 *   other arguments as the plain call of the same name.
 * Errors: as the plain call, plus QIG_EINVAL for ws == NULL and QIG_EALIGN
 *         for a misaligned ws.
 */
size_t mmq_workspace_bytes(void);
int mmq_q4k_streamk(const void *W, int64_t od, int64_t id, const void *q8,
                    int64_t nt, float *y, int64_t ldy, void *ws,
                    hipStream_t stream);
int mmq_q6k_streamk(const void *W, int64_t bstride, const int8_t *W_exp,
                    int64_t od, int64_t id, const void *q8, int64_t nt,
                    float *y, int64_t ldy, void *ws, hipStream_t stream);
int mmq_q4k_prepared_streamk(const void *Wp, int64_t od, int64_t id,
                             const void *q8, int64_t nt, float *y, int64_t ldy,
                             void *ws, hipStream_t stream);
int mmq_q6k_prepared_streamk(const void *Wp, int64_t od, int64_t id,
                             const void *q8, int64_t nt, float *y, int64_t ldy,
                             void *ws, hipStream_t stream);

/*
 * Tiled activations -- quantization straight into the layout the GEMM stages
 * (the quantize-transpose prepass the r21 page "Coalesced block-linear A
 * staging", s5, reports the campaign moving to), so the GEMMs' activation
 * staging is a plain copy.  The quantization is the pad40 one (same d, quants
 * and ssum); only the layout differs.  For 64-token tile T = t / 64 and
 * super-block sb, a record of 20480 bytes at ((T * (id/256)) + sb) * 20480
 * holds, for its tokens u = t % 64 and chunks c = 0..7 (pad40 chunk
 * 8 sb + c):
 *   quants   the 32 int8 of (t, c) at 2048 c + 32 u, each 16-byte half h
 *            stored at offset 16 (h ^ s(u)), s(u) = ((u >> 2) ^ (u >> 3)) & 1
 *   d        fp16 d widened to fp32 at 16384 + 256 c + 4 slot(u), slot(u) =
 *            (u & 32) + 16 ((u >> 2) & 1) + 4 ((u & 31) >> 3) + (u & 3)
 *   -ssum    split as hi = bf16(-ssum), lo = bf16(-ssum - hi) (round to
 *            nearest even): 16-byte entry at 18432 + 16 (2 u + c / 4), hi at
 *            its 16-bit index c % 4, lo at index 4 + c % 4
 * Tokens nt .. 64 * ceil(nt/64) - 1 are quantized from zeros: d = 0, quants
 * 0, -ssum = -0 (hi 0x8000, lo 0).  The GEMMs below give y bit-identical to
 * the pad40 calls of the same name.
 *
 *   x      as quantize_q8_pad40; id must be a multiple of 256
 *   q8t    q8_tiled_bytes(nt, id) = ceil(nt/64) * (id/256) * 20480 bytes,
 *          16-byte aligned; every byte written
 *   ws     NULL (whole tiles, as the plain calls) or a stream-K workspace (as
 *          the *_streamk calls)
 * Errors: as quantize_q8_pad40 and the GEMM of the same name (QIG_EINVAL also
 *         for id % 256 in quantize_q8_tiled; QIG_EALIGN for a misaligned ws).
 */
size_t q8_tiled_bytes(int64_t nt, int64_t id);
int quantize_q8_tiled(const float *x, int64_t nt, int64_t id, int64_t ldx,
                      void *q8t, hipStream_t stream);
int mmq_q4k_q8t(const void *W, int64_t od, int64_t id, const void *q8t,
                int64_t nt, float *y, int64_t ldy, void *ws,
                hipStream_t stream);
int mmq_q6k_q8t(const void *W, int64_t bstride, const int8_t *W_exp,
                int64_t od, int64_t id, const void *q8t, int64_t nt, float *y,
                int64_t ldy, void *ws, hipStream_t stream);
int mmq_q4k_prepared_q8t(const void *Wp, int64_t od, int64_t id,
                         const void *q8t, int64_t nt, float *y, int64_t ldy,
                         void *ws, hipStream_t stream);
int mmq_q6k_prepared_q8t(const void *Wp, int64_t od, int64_t id,
                         const void *q8t, int64_t nt, float *y, int64_t ldy,
                         void *ws, hipStream_t stream);

/*
 * q6_K limb buffers -- a registration-time form of q6_K weights in which each
 * 16-element sub-block's int8 scale is folded into the quants (the pages'
 * pre-expansion of r43 "PC-sampling attribution" s3.2 and r44 "W_exp stride
 * mismatch root cause" s2.1-s2.4, carried one step further: the sub-block
 * scales of r44 s1.1 leave the GEMM's epilogue).  Per element, with c6 the
 * centred quant (r44 s3.2) and sc its sub-block's scale,
 *   v = sc * c6 (|v| <= 4096) = 128 * H + L,  H = floor(v / 128) in
 *   [-32, 32], L = v - 128 * H in [0, 127],
 * both stored as int8.  A buffer of q6k_limbs_bytes(od, id) =
 * 2*od*id + od*(id/256)*4 bytes holds
 *   H plane   int8 [od][id] at offset 0 (row stride id)
 *   L plane   int8 [od][id] at offset od*id
 *   d plane   fp32 [od][id/256] at offset 2*od*id: the super-block's fp16 d
 * The layout is part of this contract.  It takes 2.3 times the raw blocks'
 * memory (25.7 MB against 11.2 MB at 3584 x 3584).
 *
 * mmq_q6k_limbs_q8t -- y[nt][od] of the q6_K GEMM from a limb buffer and a
 * tiled activation plane (quantize_q8_tiled).  Per 32-element chunk the
 * exact integer Q = sum(qa * v) = 128 P_H + P_L comes from two int8 MFMAs;
 *   y = sum_sb d * sum_c da(t, c) * Q(t, j, c),
 * in fp32 (the same value as mmq_q6k up to rounding order: within the
 * output tolerance, not bit-identical).
 *   W      raw q6_K plane as for mmq_q6k (prepare only), 16-byte aligned
 *   Wl     the limb buffer, 16-byte aligned; prepare writes every byte
 *   q8t, nt, y, ldy, ws as for mmq_q6k_q8t
 * q6k_limbs_bytes returns 0 for invalid shapes.  prepare_q6k_limbs:
 * QIG_EINVAL (od < 0, id <= 0 or id % 256, bad bstride), QIG_EALIGN,
 * QIG_ELAUNCH.  mmq_q6k_limbs_q8t: as mmq_q6k_q8t.
 */
size_t q6k_limbs_bytes(int64_t od, int64_t id);
int prepare_q6k_limbs(const void *W, int64_t bstride, int64_t od, int64_t id,
                      void *Wl, hipStream_t stream);
int mmq_q6k_limbs_q8t(const void *Wl, int64_t od, int64_t id,
                      const void *q8t, int64_t nt, float *y, int64_t ldy,
                      void *ws, hipStream_t stream);

/*
 * Staged q4_K weights -- a registration-time buffer whose records are the
 * bytes the q4_K GEMM stages into LDS for each 64-row tile and super-block
 * (the registration-time direction of the pages' prepared planes: r43 page
 * "PC-sampling attribution + pre-expand-B parity FAIL", s3.2), so that with
 * the tiled activation plane the GEMM's whole stage is plain copies and no
 * scale is decoded in the GEMM.  For tile T = j / 64 and super-block sb, a
 * record of 14336 bytes at ((T * (id/256)) + sb) * 14336 holds, for rows
 * r = j % 64:
 *   nibbles  block bytes 16..143 of row r, 16-byte unit u at
 *            128 r + 16 (u ^ ((r >> 1) & 7))
 *   scales   for sub-block c (0..7): w = d * sc_c and -1.5 * 2^23 * w,
 *            fp32, at 8192 + 8 (64 c + r)
 *   mins     dmin * m of sub-blocks 4h .. 4h+3 (h = 0, 1) split as
 *            hi = bf16(v) and lo = bf16(v - hi) (round to nearest even):
 *            16-byte entry at 12288 + 16 (2 r + h), hi at 16-bit index
 *            c % 4, lo at 4 + c % 4
 * Rows od .. 64 * ceil(od/64) - 1 are zero.  The layout is part of this
 * contract.  The buffer takes 1.56 times the raw blocks' memory.
 *
 * mmq_q4k_staged_q8t -- y[nt][od] of the q4_K GEMM from a staged buffer and
 * a tiled activation plane: bit-identical to mmq_q4k_q8t on the same blocks.
 *   W      raw q4_K blocks as for mmq_q4k (prepare only), 16-byte aligned
 *   Ws     the staged buffer, q4k_staged_bytes(od, id) bytes, 16-byte
 *          aligned; prepare writes every byte
 *   q8t, nt, y, ldy, ws as for mmq_q4k_q8t
 * q4k_staged_bytes returns 0 for invalid shapes.  prepare_q4k_staged:
 * QIG_EINVAL (od < 0, id <= 0 or id % 256), QIG_EALIGN, QIG_ELAUNCH.
 * mmq_q4k_staged_q8t: as mmq_q4k_q8t.
 */
size_t q4k_staged_bytes(int64_t od, int64_t id);
int prepare_q4k_staged(const void *W, int64_t od, int64_t id, void *Ws,
                       hipStream_t stream);
int mmq_q4k_staged_q8t(const void *Ws, int64_t od, int64_t id,
                       const void *q8t, int64_t nt, float *y, int64_t ldy,
                       void *ws, hipStream_t stream);

/*
 * mmq_q4k_xf32 -- the q4_K GEMM on fp32 activations, quantized inside the
 * GEMM (the "quantization fused into the GEMM prologue" direction after the
 * quantize-transpose prepass, r21 page "Coalesced block-linear A staging",
 * s5): each workgroup quantizes its 64 tokens of the next super-block
 * straight into its LDS stage, with the pad40 quantization of
 * quantize_q8_pad40, so no q8 plane is written or read.  y is bit-identical
 * to quantize_q8_tiled followed by mmq_q4k_q8t (with the same ws).  Every
 * row tile of the output quantizes the same tokens again: ceil(od/64) times
 * the quantization work of the prepass.
 *   W, od, id, nt, y, ldy, ws as for mmq_q4k_q8t
 *   x      fp32 activations [nt][ldx], ldx >= id and ldx % 4 == 0, 16-byte
 *          aligned; read only
 * Errors: QIG_EINVAL (as mmq_q4k_q8t, or ldx < id), QIG_EALIGN (x, W, y or
 *         ws misaligned, ldx % 4), QIG_ELAUNCH.
 */
int mmq_q4k_xf32(const void *W, int64_t od, int64_t id, const float *x,
                 int64_t ldx, int64_t nt, float *y, int64_t ldy, void *ws,
                 hipStream_t stream);

/*
 * mmq_q4k_q8t_noalloc -- mmq_q4k_q8t with a stream-K workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The call itself
 * allocates nothing: its workspace is the library's own, a file-scope
 * device array of 16 MiB + 8 KiB that each GPU holds from the library's
 * load until the process ends (partial-sum slots and arrival counters for
 * 512 workgroups, two on each of 256 CUs).  No shape needs more: the
 * stream-K split never uses more than 512 workgroups, so no size is refused
 * for want of scratch.  Each call first zeroes the counters it will use
 * (with a kernel, not hipMemsetAsync); the partial slots are written before
 * they are read.  y is bit-identical to mmq_q4k_q8t with a workspace on a
 * GPU with 256 CUs.
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or different host threads) race and give
 * wrong y; calls in order on one stream are safe.
 *   arguments as mmq_q4k_q8t (ws omitted)
 * Errors: as mmq_q4k_q8t, plus QIG_ELAUNCH when the runtime cannot give the
 *         array's device address.
 */
int mmq_q4k_q8t_noalloc(const void *W, int64_t od, int64_t id,
                        const void *q8t, int64_t nt, float *y, int64_t ldy,
                        hipStream_t stream);

/*
 * Test exports: the int32 sub-block partials of the same kernels, for the
 * window of tokens [t0, t1) and rows [j0, j1), written to
 * P[(t - t0)][(j - j0)][sub] (int32, 4-byte aligned), where sub runs over all
 * 8*nsb q4_K sub-blocks of 32 (P4) or 16*nsb q6_K sub-blocks of 16 (P6).
 * Same argument rules as the GEMMs plus 0 <= t0 <= t1 <= nt and
 * 0 <= j0 <= j1 <= od (QIG_EINVAL otherwise).
 */
int mmq_q4k_partials(const void *W, int64_t od, int64_t id, const void *q8,
                     int64_t nt, int64_t t0, int64_t t1, int64_t j0, int64_t j1,
                     int32_t *P, hipStream_t stream);
int mmq_q6k_partials(const void *W, int64_t bstride, const int8_t *W_exp,
                     int64_t od, int64_t id, const void *q8, int64_t nt,
                     int64_t t0, int64_t t1, int64_t j0, int64_t j1, int32_t *P,
                     hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QIG_H */
