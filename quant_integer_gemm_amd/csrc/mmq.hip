// mmq.hip -- k-quant prefill MMQ on gfx950: int8 MFMA sub-block dot products
// with a fused fp32 rescale epilogue.
//
// Operation (minfer pages: r44 "W_exp stride mismatch root cause" s1.1/s2.1
// for q6_K sub-block scaling, s3.2 for the element map; r20/r21 pages for the
// pad40 activation blocks):
//   q6_K: y[t][j] = sum_sb d(j,sb) sum_s sc(j,sb,s) da(t,8sb+s/2) P6(t,j,sb,s)
//   q4_K: y[t][j] = sum_sb sum_b [ d sc_b da(t,c) P4(t,j,c) - dmin m_b ssum(t,c) ]
// with int32 P over a 16- (q6_K) or 32-element (q4_K) sub-block.
//
// Design (MI355X-first; the pages' IMMA kernels are prior art only):
//  * A workgroup of 256 threads = 4 waves owns a 64-token x 64-row output
//    tile, one 32x32 MFMA tile per wave.  Its double-buffered LDS stage is
//    80 KB at most, so two workgroups share a CU and each SIMD runs two waves
//    of different workgroups that do not move in lock-step.
//  * MFMA rows are tokens and columns weight rows, so each lane owns one
//    weight row: the per-(row, chunk) weight scale is a lane constant and the
//    per-(token, chunk) activation scale a per-register value, read from an
//    fp32 table in LDS laid out in register order.
//  * K advances one super-block (256) per step.  Step k+1's activation quants
//    (and the q4_K packed nibbles, and the dense planes' quants) are copied
//    global->LDS directly while step k computes; the rest of its weights
//    (q6_K raw quants, recombined to centred int8; the scales, to fp32) goes
//    through registers into the other half of the LDS stage: one barrier per
//    step.  q4_K nibbles are split after the LDS read, one read per pair of
//    chunks (low nibbles, then high).
//  * Within a step a wave runs its 8 chunks as a software pipeline: the MFMA
//    of chunk c+1 is issued before the VALU epilogue of chunk c, chunk c+2's
//    MFMA operands and chunk c+1's scales are fetched from LDS while it runs,
//    and value pins keep the compiler from collapsing the pipeline.
//  * Epilogue per 32-chunk: the int8 MFMA accumulates onto the 1.5*2^23 bias
//    so one fma turns the int32 partial into P*w, rounded once; a second fma
//    (three-operand form) folds in the activation scale: 2 VALU ops per
//    output and chunk for q4_K, 4 for q6_K (two 16-element sub-blocks, each
//    its own MFMA with the other half of K zeroed).
//  * q4_K min term: -dmin*m*ssum summed over chunks is a K = id/32 matrix
//    product, run per super-block on the bf16 MFMA with both factors split
//    into bf16 hi/lo pairs, into a second accumulator.
//  * Work: each workgroup (worker) runs a list of (tile, super-block range)
//    items; whole tiles normally, or stream-K splits with a fixed-order
//    fix-up when the tiles leave many workgroup slots empty.  Tiles are
//    numbered in groups of 8 row tiles and workers XCD by XCD, so the tiles
//    running on one XCD at a time share operands in its L2.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <cstddef>
#include <utility>

#include "qig_device.h"
#include "qig_launch.h"
#include "qig_quant.h"

namespace qig {

constexpr int NTHR = 256;
constexpr int TT = 64;    // tokens per workgroup tile
constexpr int TJ = 64;    // weight rows per workgroup tile
constexpr int NCH = 8;    // 32-element chunks per super-block

// Weight sources ("arms").  RAW: raw blocks (q4_K: packed nibbles copied
// into LDS, scales decoded; q6_K: decoded on the way into LDS).  WEXP (q6_K):
// quants from the dense plane W_exp, copied straight into LDS; d and the
// scales from the raw blocks.  PREP: a prepared buffer made once at
// registration, with the scales as an fp32 plane loaded as they are; its
// quants are copied straight into LDS (q6_K, one centred byte per element;
// q4_K, the nibble plane, split after the LDS read as in RAW).
constexpr int ARM_RAW = 0, ARM_WEXP = 1, ARM_PREP = 2;
// LIMB (q6_K, tiled activations only): a limb buffer (prepare_q6k_limbs) run
// by mmq_limbs_kernel, below.
constexpr int ARM_LIMB = 3;
// STAGED (q4_K, tiled activations only): a staged buffer (prepare_q4k_staged)
// whose records are the byte image of the weight part of the stage, so the
// whole stage -- activations and weights -- arrives by plain copies.
constexpr int ARM_STAGED = 4;

// Activation sources.  PAD40: the pad40 plane; quants are copied into LDS,
// d and ssum go through registers (d widened, -ssum split into bf16 pairs).
// TILED: the tiled plane of quantize_q8_tiled, whose records already hold
// the LDS image of all three, so the whole activation stage is a copy.
// F32 (q4_K): the fp32 activations themselves; each workgroup quantizes its
// 64 tokens of the next super-block into the stage it will compute from
// (quant_stage), the bytes the tiled record would hold, so no q8 plane goes
// through memory.
constexpr int ACT_PAD40 = 0, ACT_TILED = 1, ACT_F32 = 2;

// One super-block of staged operands.
template <int QT>
struct Stage;

// Activation quants, q4_K's packed nibbles and the dense planes' quants
// arrive by direct global->LDS copies (load_act, load_bq, load_wexp); pad40
// activation d and ssum values, the weight scales and q6_K's raw quants go
// through registers (load_raw / store_raw): d is widened to fp32, ssum and
// the weights' dmin*m are split into bf16 pairs for the min-term MFMA, the
// scales are decoded and q6_K's quants recombined.

// q4_K min term.  -sum_c ssum(t,c) * dmin*m(j,c) is a matrix product with
// K = 8 per super-block, run on v_mfma_f32_32x32x8_bf16 with both factors
// split as v = hi + lo (hi = bf16(v), lo = bf16(v - hi)): hi*hi + hi*lo +
// lo*hi carries v*w to about 2^-16 relative, far inside the output tolerance
// and at a fraction of the fp32 MFMA's cost.  A MinOp holds the four values
// of chunks 4h .. 4h+3 of one token or row: hi in dwords 0-1, lo in 2-3, in
// the element order of the MFMA's K half h.
struct MinOp {
    uint32_t w[4];
};
template <>
struct Stage<4> {
    __attribute__((aligned(16))) uint8_t a[NCH][TT][32];   // activation quants (halves swizzled)
    float ax[NCH][TT];          // activation d as fp32, token rows in register order (x_slot)
    MinOp ma[TT][2];            // -ssum of token t, chunks 4h .. 4h+3
    // packed nibble bytes of row j as in the block (byte 32g + i holds
    // element 64g + i low and 64g + 32 + i high), its 16-byte unit u at
    // position u ^ ((j / 2) % 8)
    __attribute__((aligned(16))) uint8_t bq[TJ][128];
    float bs[NCH][TJ][2];       // d * sc, and -M d * sc (the magic term of the epilogue's first fma)
    MinOp mb[TJ][2];            // dmin * m of row j, chunks 4h .. 4h+3
};

static_assert(offsetof(Stage<4>, a) == 0 && offsetof(Stage<4>, ax) == 16384 && offsetof(Stage<4>, ma) == 18432 &&
                  offsetof(Stage<4>, bq) == Q8T_RECORD,
              "the tiled activation record is the byte image of the first Q8T_RECORD bytes of Stage<4>");
static_assert(offsetof(Stage<4>, bs) == Q8T_RECORD + 8192 && offsetof(Stage<4>, mb) == Q8T_RECORD + 12288 &&
                  sizeof(Stage<4>) == Q8T_RECORD + Q4S_RECORD,
              "a staged q4_K record is the byte image of the last Q4S_RECORD bytes of Stage<4>");

// q6_K: row TT of every chunk plane of a is all zero.  Each 16-element
// sub-block has its own MFMA, which must see zeros in the lanes that carry
// the other half of the chunk; those lanes read the zero row instead of
// selecting zeros with VALU instructions.
template <>
struct Stage<6> {
    __attribute__((aligned(16))) uint8_t a[NCH][TT + 1][32];
    float ax[NCH][TT];
    uint8_t b[NCH][TJ][32];     // centred int8 weights
    float bs[NCH][TJ][2];       // d * sc of the two 16-element sub-blocks
};


struct MmqArgs {
    const uint8_t *W;
    const uint8_t *Wexp;
    const uint8_t *q8;        // F32 source: the fp32 activations, ldx floats per token
    int64_t ldx;
    float *y;
    int32_t *P;
    int64_t bstride, od, id, nt, ldy;
    int64_t t0, t1, j0, j1;   // output window (all of y for the GEMM)
    int nbt, nbj;             // token and row tiles in the window
    // Work decomposition (tiles numbered as tile_origin does): tiles below dp_tiles are
    // whole-tile work items; the next sk_tiles are split into (tile,
    // super-block) iterations shared evenly by the workers.
    int dp_tiles, sk_tiles;   // both below 2^31, as is sk_tiles * (id / 256)
    float *ws;                // split tiles: partial-sum slots, 2 per worker
    uint32_t *cnt;            // split tiles: arrival counters, 1 per worker
};

__device__ __forceinline__ u32x4 ld16(const uint8_t *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ void st16(uint8_t *p, u32x4 v)
{
    *reinterpret_cast<u32x4 *>(p) = v;
}

// Ordering points for the software pipeline.  MFMAs and VALU arithmetic are
// free-floating in the compiler's instruction DAG, which tends to hoist all
// MFMAs of a step and sink all epilogues, keeping every result live.  An empty
// volatile asm is ordered with the LDS operations around it; making it read
// one value and redefine another pins "this MFMA is issued before that
// epilogue starts" and "this epilogue is done before the next loads".
template <typename T>
__device__ __forceinline__ void pin(T &x) { asm volatile("" : "+v"(x)); }
template <typename T, typename U>
__device__ __forceinline__ void pin_after(T &x, const U &y) { asm volatile("" : "+v"(x) : "v"(y)); }


// ---------------------------------------------------------------------------
// Staging.  Activations and q4_K's packed nibbles are copied straight into
// LDS (make_src, load_act, load_bq).  The scales, and q6_K's raw quants, go
// through registers and are decoded on the way into LDS: row = 16 * wave +
// lane % 16 and part = (lane / 16) % 4, a quarter of the super-block:
//   q4_K: scale and min of sub-blocks `part` and `part` + 4;
//   q6_K: half h = part/2 and pair pp = part%2 -> chunks 4h+pp and 4h+pp+2,
//         which share the same ql bytes (low / high nibble) and qh bytes.
// Each 16-lane group walks 16 consecutive rows, so the LDS writes are free of
// bank conflicts.  Rows and tokens past the end are clamped to the last valid
// one: the loads stay unconditional and a clamped row only feeds outputs that
// are never stored.
// ---------------------------------------------------------------------------
template <int QT, int ARM>
struct Raw {
    static constexpr int NQ = QT == 4 ? 1 : (ARM != ARM_RAW ? 1 : 4);
    u32x4 h;       // q4_K header (d, dmin, 12 scale bytes) | q6_K: 16 int8 scales |
                   // PREP: 16 bytes of the row's scale block
    u32x4 q[NQ];   // q6_K raw: ql 32 B, qh 32 B | other arms: unused
    uint32_t d;    // q6_K fp16 d (low half)
    uint32_t ad[2];   // two activation block dwords (fp16 d in the low half)
    uint32_t as[2];   // q4_K: ssum of the same two blocks
};

// Staging sources: workgroup-uniform bases (the tile's first token / row, so
// they live in scalar registers and advance per super-block with scalar
// adds) plus 32-bit per-lane byte offsets, which the loads take as their
// vector offset.  A tile spans 64 tokens and 64 rows, so every offset is
// below 64 * (id / 32) * 40 or 64 * (id / 256) * bstride.
struct Src {
    const uint8_t *q8;   // pad40 plane at the tile's first token
    const uint8_t *w;    // raw weight rows at the tile's first row
    const uint8_t *x;    // W_exp rows at the tile's first row (q6_K dense arm)
    uint32_t aq[2];      // this lane's quant-half sources, token halves 0/1 of the tile
    uint32_t ad[2];      // blocks of this lane's two activation d (and ssum) loads
    uint32_t wo;         // this lane's weight row
    uint32_t xq[2];      // this lane's weight copy sources: W_exp row halves 0/1 (q6_K), nibble copies 0/1 (q4_K)
    int64_t wstep;       // bytes per super-block along w
};

template <int QT, int ARM, int ACT>
__device__ __forceinline__ Src make_src(const MmqArgs &g, int64_t tw0, int64_t jw0, int tid)
{
    Src s;
    const int64_t nb32 = g.id / 32, nsb = g.id / 256;
    // Activation copies (one super-block = 16 quant copies of 1 KB and 8 (q6_K)
    // or 16 (q4_K) dword copies of 256 bytes per workgroup).  Quant copy q of
    // Stage::a (wave w issues q = 4w .. 4w+3) fills a[c][32*th .. +31] with
    // c = q / 2, th = q % 2: lane l brings half h' = l % 2 of token
    // 32*th + l/2, i.e. quant bytes 16*(h' ^ swz(t)) .. +15 of its block.
    // The d (and q4_K ssum) loads of wave w take tokens 8q + l%8 (q = 2w,
    // 2w+1), chunk l/8: eight tokens of one chunk per lane octet, which keeps
    // their LDS stores (store_raw) free of conflicts.
    const uint32_t tok = (uint32_t)(nb32 * 40);      // bytes per token
    if constexpr (ACT == ACT_TILED) {
        // the tile's records (tiles start at multiples of 64 tokens); lane l
        // copies bytes 16 l .. 16 l + 15 of every 1 KB piece
        s.q8 = g.q8 + (tw0 / 64) * nsb * Q8T_RECORD;
        s.aq[0] = s.aq[1] = 16u * (uint32_t)(tid & 63);
        s.ad[0] = s.ad[1] = 0;
    } else if constexpr (ACT == ACT_F32) {
        s.q8 = nullptr;   // quant_stage reads the activations
        s.aq[0] = s.aq[1] = 0;
        s.ad[0] = s.ad[1] = 0;
    } else {
        s.q8 = g.q8 + tw0 * (int64_t)tok;
        const int l = tid & 63, w = tid >> 6;
#pragma unroll
        for (int th = 0; th < 2; ++th) {
            const int t = 32 * th + (l >> 1);
            const uint32_t tl = (uint32_t)(min(tw0 + t, g.nt - 1) - tw0);
            s.aq[th] = tl * tok + 4 + 16 * ((l & 1) ^ swz(t));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int td = 8 * (2 * w + i) + (l & 7);
            const uint32_t tl = (uint32_t)(min(tw0 + td, g.nt - 1) - tw0);
            s.ad[i] = tl * tok + (l >> 3) * 40;
        }
    }
    // Weight staging: lanes l and l+16k of a wave take rows 16w + l%16, so a
    // load covers 16 rows (not 64) and the LDS writes stay conflict free.
    const uint32_t jl = (uint32_t)(min(jw0 + 16 * (tid >> 6) + (tid & 15), g.od - 1) - jw0);
    // PREP: W is the scale plane, 64 bytes per (row, super-block)
    s.wstep = ARM == ARM_PREP ? 64 : (QT == 4 ? 144 : g.bstride);
    s.w = g.W + jw0 * nsb * s.wstep;
    s.wo = jl * (uint32_t)(nsb * s.wstep);
    // W_exp copies: the same mapping as the activation quant copies, with
    // weight rows in place of tokens (a row's chunk is 32 plain bytes).
    // q4_K PREP: nibble plane, id/2 bytes per row, 128 per super-block
    s.x = ARM == ARM_RAW ? nullptr : g.Wexp + jw0 * (QT == 4 ? g.id / 2 : g.id);
    if constexpr (ARM == ARM_STAGED) {
        // the row tile's records (tiles start at multiples of 64 rows); lane l
        // copies bytes 16 l .. 16 l + 15 of every 1 KB piece
        s.x = g.Wexp + (jw0 / 64) * nsb * Q4S_RECORD;
        s.xq[0] = s.xq[1] = 16u * (uint32_t)(tid & 63);
    } else if constexpr (QT == 4) {
        // packed nibble copies: wave w's copy i fills rows 16w + 8i .. +7 of
        // Stage::bq; lane l writes position l % 8 of row 16w + 8i + l / 8,
        // which holds unit (l % 8) ^ ((row / 2) % 8) of the row's 128 bytes
        const int l = tid & 63, w = tid >> 6;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 16 * w + 8 * i + (l >> 3);
            const int u = (l & 7) ^ ((r >> 1) & 7);
            const uint32_t rl = (uint32_t)(min(jw0 + r, g.od - 1) - jw0);
            s.xq[i] = ARM == ARM_PREP ? rl * (uint32_t)(g.id / 2) + 16 * u
                                      : rl * (uint32_t)(nsb * 144) + 16 + 16 * u;
        }
    } else {
        const int l = tid & 63;
#pragma unroll
        for (int jh = 0; jh < 2; ++jh) {
            const int r = 32 * jh + (l >> 1);
            const uint32_t rl = (uint32_t)(min(jw0 + r, g.od - 1) - jw0);
            s.xq[jh] = rl * (uint32_t)g.id + 16 * ((l & 1) ^ swz(r));
        }
    }
    return s;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global->LDS copies of 16 bytes per lane.  dma16n<N> copies N
// consecutive 1 KB pieces: lane l's bytes at base + voff + 1024 i land at LDS
// byte address lds + 1024 i + 16 l (base and lds wave-uniform).  The
// instruction's offset field moves the global and the LDS address alike (a
// probe on the device confirmed it), so a run of pieces laid out the same in
// memory and in the stage needs one M0 (the LDS address register) and one
// base for up to four pieces.  The copies are issued from inline assembly
// because the compiler, unable to tell the copy's LDS bytes from those the
// compute reads, otherwise waits for every outstanding global load at the
// first such read, which kept each step's loads from overlapping its compute.
// The compiler therefore does not know about these copies: their data is
// read only after an explicit vmcnt(0) wait and a barrier, and since loads
// complete in order, extra untracked loads only make the compiler's own
// counted waits stricter.  M0 is an input operand, so the compiler writes it
// and knows its value.  The compiler inserts no wait states before inline
// assembly, so the copy brings its own: a VMEM instruction must follow a VALU
// write of an SGPR it reads by 5 wait states (the scalar base often comes
// from v_readfirstlane_b32 right before; read early, the copy takes the
// register's previous value as its address), and an LDS copy must follow an
// M0 write by 1.  The leading s_nop 4 gives 5.
template <int N>
__device__ __forceinline__ void dma16n(const uint8_t *base, uint32_t voff, uint32_t lds)
{
    static_assert(N >= 1 && N <= 4, "the offset field reaches 4095 bytes: at most four 1 KB pieces");
    // base and lds are wave-uniform; readfirstlane puts them in scalar
    // registers, as the instruction requires, whatever the compiler infers.
    // (readfirstlane returns a signed int: each half goes through uint32_t
    // before it is widened, or an address with bit 31 set would sign-extend.)
    const uint64_t b = reinterpret_cast<uintptr_t>(base);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const uint64_t sbase = (uint64_t)lo | ((uint64_t)hi << 32);
    const uint32_t m0v = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
    if constexpr (N == 1)
        asm volatile("s_nop 4\n\t"
                     "global_load_lds_dwordx4 %0, %1"
                     :
                     : "v"(voff), "s"(sbase), "{m0}"(m0v)
                     : "memory");
    else if constexpr (N == 2)
        asm volatile("s_nop 4\n\t"
                     "global_load_lds_dwordx4 %0, %1\n\t"
                     "global_load_lds_dwordx4 %0, %1 offset:1024"
                     :
                     : "v"(voff), "s"(sbase), "{m0}"(m0v)
                     : "memory");
    else if constexpr (N == 3)
        asm volatile("s_nop 4\n\t"
                     "global_load_lds_dwordx4 %0, %1\n\t"
                     "global_load_lds_dwordx4 %0, %1 offset:1024\n\t"
                     "global_load_lds_dwordx4 %0, %1 offset:2048"
                     :
                     : "v"(voff), "s"(sbase), "{m0}"(m0v)
                     : "memory");
    else
        asm volatile("s_nop 4\n\t"
                     "global_load_lds_dwordx4 %0, %1\n\t"
                     "global_load_lds_dwordx4 %0, %1 offset:1024\n\t"
                     "global_load_lds_dwordx4 %0, %1 offset:2048\n\t"
                     "global_load_lds_dwordx4 %0, %1 offset:3072"
                     :
                     : "v"(voff), "s"(sbase), "{m0}"(m0v)
                     : "memory");
}

__device__ __forceinline__ void dma16(const uint8_t *base, uint32_t voff, uint32_t lds)
{
    dma16n<1>(base, voff, lds);
}

// LDS byte addresses: the copies take the stage's address (sl, computed
// once per kernel from the __shared__ array) plus field offsets, so their
// destinations are scalar integer arithmetic.
template <int QT>
constexpr uint32_t A_PLANE = sizeof(Stage<QT>::a[0]);   // bytes per chunk plane of a

// Direct global->LDS copies of super-block sb's activations into the stage at
// LDS address sl.  The data lands asynchronously; a vmcnt(0) wait plus a
// barrier must come before any wave reads it.
template <int QT>
__device__ __forceinline__ void load_act(uint32_t sl, const Src &s, int64_t sb, int tid)
{
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const uint8_t *q8 = s.q8 + sb * 320;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = 4 * w + i, c = q >> 1;
        dma16(q8 + 40 * c, s.aq[i & 1], sl + offsetof(Stage<QT>, a) + c * A_PLANE<QT> + 1024 * (q & 1));
    }
}

// Tiled activations: the record of super-block sb holds the first
// Q8T_RECORD bytes of the q4_K stage (quants, d table, min-term operands)
// byte for byte; q6_K takes the quants, into its chunk planes (which keep a
// zero row after each), and the d table.  Pieces of 1 KB.  q4_K: wave w
// copies the record's pieces 5w .. 5w + 4, which land at the same offsets in
// the stage.  q6_K: wave w copies chunks 2w and 2w + 1 (two pieces each),
// waves 0 and 1 also piece 16 + w (the d table).
template <int QT>
__device__ __forceinline__ void load_act_tiled(uint32_t sl, const Src &s, int64_t sb, int tid)
{
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const uint8_t *rec = s.q8 + sb * Q8T_RECORD;
    if constexpr (QT == 4) {
        dma16n<4>(rec + 5120 * w, s.aq[0], sl + 5120 * w);
        dma16n<1>(rec + 5120 * w + 4096, s.aq[0], sl + 5120 * w + 4096);
    } else {
#pragma unroll
        for (int k = 0; k < 2; ++k)
            dma16n<2>(rec + 2048 * (2 * w + k), s.aq[0], sl + offsetof(Stage<QT>, a) + (2 * w + k) * A_PLANE<QT>);
        if (w < 2) dma16(rec + 1024 * (16 + w), s.aq[0], sl + offsetof(Stage<QT>, ax) + 1024 * w);
    }
}

template <int QT, int ACT>
__device__ __forceinline__ void stage_act(uint32_t sl, const Src &s, int64_t sb, int tid)
{
    if constexpr (ACT == ACT_TILED)
        load_act_tiled<QT>(sl, s, sb, tid);
    else if constexpr (ACT == ACT_PAD40)
        load_act<QT>(sl, s, sb, tid);
    // F32: quant_stage, called where the stage is free to write
}

// F32 source: quantize super-block sb of the 64 tokens from tw0 into the
// activation part of stage s (q4_K), the bytes of the tiled record
// (put_tiled).  Lane group i = tid / 8 takes token i (passes 0-7) and 32 + i
// (passes 8-15), chunk pass % 8; each lane one float4 of the block.  All 16
// loads are issued before the first block is quantized.  Tokens past nt are
// quantized from zeros, as the tiled plane holds them.  The caller makes the
// stores visible with a barrier before any wave reads the stage.
__device__ __forceinline__ void quant_stage(const MmqArgs &g, Stage<4> &s, int64_t tw0, int64_t sb, int tid)
{
    const int l8 = tid & 7, tg = tid >> 3;
    float4 v[16];
#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const int64_t t = tw0 + tg + 32 * (p >> 3);
        v[p] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < g.nt)
            v[p] = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(g.q8) + t * g.ldx +
                                                     256 * sb + 32 * (p & 7) + 4 * l8);
    }
    uint8_t *r = reinterpret_cast<uint8_t *>(&s);
#pragma unroll
    for (int p = 0; p < 16; ++p) put_tiled(r, p & 7, tg + 32 * (p >> 3), l8, quant_block(v[p]));
}

// Dense arms: direct global->LDS copies of super-block sb's quants from the
// quant plane into stage b (same completion rule as load_act).
template <int QT>
__device__ __forceinline__ void load_wexp(uint32_t sl, const Src &s, int64_t sb, int tid)
{
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const uint8_t *x = s.x + sb * 256;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = 4 * w + i, c = q >> 1;
        dma16(x + 32 * c, s.xq[i & 1], sl + offsetof(Stage<QT>, b) + c * (TJ * 32) + 1024 * (q & 1));
    }
}

// q4_K: direct global->LDS copies of super-block sb's packed nibbles (raw
// blocks or the prepared nibble plane) into Stage::bq, two per wave.
template <int ARM>
__device__ __forceinline__ void load_bq(uint32_t sl, const Src &s, int64_t sb, int tid)
{
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    if constexpr (ARM == ARM_STAGED) {
        // the record's 14 pieces of 1 KB, which land at the same offsets in
        // the stage: waves 0 and 1 copy pieces 4w .. 4w + 3, waves 2 and 3
        // pieces 8 + 3 (w - 2) .. + 2
        static_assert(Q4S_RECORD == 14 * 1024, "the staged record is 14 pieces");
        const uint8_t *rec = s.x + sb * Q4S_RECORD;
        const uint32_t lb = sl + offsetof(Stage<4>, bq);
        if (w < 2)
            dma16n<4>(rec + 4096 * w, s.xq[0], lb + 4096 * w);
        else
            dma16n<3>(rec + 8192 + 3072 * (w - 2), s.xq[0], lb + 8192 + 3072 * (w - 2));
        return;
    }
    const uint8_t *base = ARM == ARM_PREP ? s.x + sb * 128 : s.w + sb * 144;
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(base, s.xq[i], sl + offsetof(Stage<4>, bq) + (16 * w + 8 * i) * 128);
}

template <int QT, int ARM, int ACT>
__device__ __forceinline__ void load_raw(Raw<QT, ARM> &r, const Src &s, int64_t sb, int tid)
{
    const int part = (tid >> 4) & 3;
    if constexpr (ACT == ACT_PAD40) {
        const uint8_t *q8 = s.q8 + sb * 320;
        r.ad[0] = *reinterpret_cast<const uint32_t *>(q8 + s.ad[0]);
        r.ad[1] = *reinterpret_cast<const uint32_t *>(q8 + s.ad[1]);
        if constexpr (QT == 4) {
            r.as[0] = *reinterpret_cast<const uint32_t *>(q8 + 36 + s.ad[0]);
            r.as[1] = *reinterpret_cast<const uint32_t *>(q8 + 36 + s.ad[1]);
        }
    }
    if constexpr (ARM == ARM_STAGED) return;   // the weight stage is all copies (load_bq)
    const uint8_t *blk = s.w + sb * s.wstep + s.wo;
    if constexpr (ARM == ARM_PREP) {
        r.h = ld16(blk + 16 * part);
    } else if constexpr (QT == 4) {
        r.h = ld16(blk);
    } else {
        const int h = part >> 1, pp = part & 1;
        if constexpr (ARM == ARM_RAW) {
            r.q[0] = ld16(blk + 64 * h + 32 * pp);        // ql bytes of quarters pp, pp+2
            r.q[1] = ld16(blk + 64 * h + 32 * pp + 16);
            r.q[2] = ld16(blk + 128 + 32 * h);            // qh bytes of this half
            r.q[3] = ld16(blk + 128 + 32 * h + 16);
        }
        // the 8 scale bytes of this half (sub-blocks 8h .. 8h+7)
        const uint2 sv = *reinterpret_cast<const uint2 *>(blk + 192 + 8 * h);
        r.h[0] = sv.x;
        r.h[1] = sv.y;
        r.d = *reinterpret_cast<const uint32_t *>(blk + 208);
    }
}

template <int QT, int ARM, int ACT>
__device__ __forceinline__ void store_raw(Stage<QT> &s, const Raw<QT, ARM> &r, int tid)
{
    const int row = 16 * (tid >> 6) + (tid & 15), part = (tid >> 4) & 3;
    const int sw = swz(row);
#pragma unroll
    for (int i = 0; i < (ACT == ACT_PAD40 ? 2 : 0); ++i) {
        const int l = tid & 63, t = 8 * (2 * (tid >> 6) + i) + (l & 7);
        s.ax[l >> 3][x_slot(t)] = h2f(r.ad[i]);
        if constexpr (QT == 4) {
            const int c = l >> 3;
            uint16_t hi, lo;
            bf16_split(-__builtin_bit_cast(float, r.as[i]), hi, lo);
            uint16_t *m = reinterpret_cast<uint16_t *>(&s.ma[t][c >> 2]);
            m[c & 3] = hi;
            m[4 + (c & 3)] = lo;
        }
    }
    if constexpr (ARM == ARM_STAGED) {
        // the weight stage came with the copies
    } else if constexpr (ARM == ARM_PREP) {
        // this lane's 16 bytes of the row's scale block
        if constexpr (QT == 4) {
            // part p: (d*sc, dmin*m) of sub-blocks 2p and 2p+1; the min-term
            // pair lands in K half p/2, elements 2(p%2), 2(p%2)+1
            uint16_t hi0, lo0, hi1, lo1;
            const float w0 = as_float((int)r.h[0]), w1 = as_float((int)r.h[2]);
            s.bs[2 * part][row][0] = w0;
            s.bs[2 * part][row][1] = -MAGIC_F * w0;
            s.bs[2 * part + 1][row][0] = w1;
            s.bs[2 * part + 1][row][1] = -MAGIC_F * w1;
            bf16_split(as_float((int)r.h[1]), hi0, lo0);
            bf16_split(as_float((int)r.h[3]), hi1, lo1);
            uint32_t *mm = s.mb[row][part >> 1].w;
            mm[part & 1] = hi0 | (uint32_t)hi1 << 16;
            mm[2 + (part & 1)] = lo0 | (uint32_t)lo1 << 16;
        } else {
            // part p: d*sc of sub-blocks 4p .. 4p+3 = chunks 2p, 2p+1
#pragma unroll
            for (int k = 0; k < 4; ++k) s.bs[2 * part + (k >> 1)][row][k & 1] = as_float((int)r.h[k]);
        }
    } else if constexpr (QT == 4) {
        // scale/min of sub-blocks part (< 4) and part + 4 from the twelve
        // packed bytes S[0..11] = header bytes 4..15: byte `part` of each of
        // the three scale dwords.
        const float d = h2f(r.h[0]), dmin = h2f(r.h[0] >> 16);
        const uint32_t s0 = __builtin_amdgcn_ubfe(r.h[1], 8 * part, 8);   // S[part]
        const uint32_t s1 = __builtin_amdgcn_ubfe(r.h[2], 8 * part, 8);   // S[part + 4]
        const uint32_t s2 = __builtin_amdgcn_ubfe(r.h[3], 8 * part, 8);   // S[part + 8]
        const uint32_t sc0 = s0 & 63, m0 = s1 & 63;
        const uint32_t sc1 = (s2 & 15) | ((s0 >> 2) & 0x30), m1 = (s2 >> 4) | ((s1 >> 2) & 0x30);
        const float w0 = d * (float)sc0, w1 = d * (float)sc1;
        s.bs[part][row][0] = w0;
        s.bs[part][row][1] = -MAGIC_F * w0;
        s.bs[part + 4][row][0] = w1;
        s.bs[part + 4][row][1] = -MAGIC_F * w1;
        uint16_t hi, lo;
        uint16_t *mm0 = reinterpret_cast<uint16_t *>(&s.mb[row][0]);
        uint16_t *mm1 = reinterpret_cast<uint16_t *>(&s.mb[row][1]);
        bf16_split(dmin * (float)m0, hi, lo);
        mm0[part] = hi;
        mm0[4 + part] = lo;
        bf16_split(dmin * (float)m1, hi, lo);
        mm1[part] = hi;
        mm1[4 + part] = lo;
    } else {
        const int h = part >> 1, pp = part & 1;
#pragma unroll
        for (int z = 0; z < 2; ++z) {
            const int qq = pp + 2 * z;          // quarter of the half
            const int c = 4 * h + qq;
            if constexpr (ARM == ARM_RAW) {
                u32x4 o[2];
                // quarter qq: nibble z of ql; the 2-bit field f of qh at bits
                // 2qq..2qq+1 selects the centred high bits 16 f - 32 (mod 256)
                // of each byte from a byte table {E0, F0, 00, 10}.
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {   // output dword 4h2+e of the chunk
                        const uint32_t ql = r.q[h2][e], qh = r.q[2 + h2][e];
                        const uint32_t sel = (qh >> (2 * qq)) & 0x03030303u;
                        const uint32_t hi = __builtin_amdgcn_perm(0u, 0x1000F0E0u, sel);
                        const uint32_t nib = z == 0 ? ql : (ql >> 4);
                        o[h2][e] = (nib & 0x0F0F0F0Fu) | hi;
                    }
                st16(&s.b[c][row][16 * (0 ^ sw)], o[0]);
                st16(&s.b[c][row][16 * (1 ^ sw)], o[1]);
            }
            const uint32_t v = r.h[z];                  // scale bytes 2c, 2c+1 (c / 2 = 2h + z)
            const int sh = 16 * (c & 1);
            const float d = h2f(r.d);
            s.bs[c][row][0] = d * (float)(int8_t)((v >> sh) & 0xff);
            s.bs[c][row][1] = d * (float)(int8_t)((v >> (sh + 8)) & 0xff);
        }
    }
}

// ---------------------------------------------------------------------------
// Per-wave compute
// ---------------------------------------------------------------------------
template <int QT>
struct Ab {                          // MFMA operands of one chunk
    i32x4 a0, a1;                    // q4_K: a0 = activation operand; q6_K: the two K halves
    i32x4 b;                         // weight operand
};

template <int QT>
struct Sc {                          // epilogue scales of one chunk
    float w0, w1;                    // weight scale (q6_K: of both sub-blocks; q4_K: w1 = -M w0)
};

template <int QT>
struct ChunkD {                      // MFMA results of one chunk
    i32x16 v[QT == 4 ? 1 : 2];
};

struct Lane {
    int ta, hh, wt, jb, l16;
    int pa0, pa1;  // q6_K: byte offsets in a chunk plane of the two sub-block operands (one is the zero row)
};

// Chunks are fetched in order; q4_K reads the packed unit of a chunk pair at
// its even chunk into pk and takes the low nibbles, its odd chunk the high
// nibbles of the same pk.
template <int QT>
__device__ __forceinline__ void load_ab(Ab<QT> &o, const Stage<QT> &s, int c, const Lane &L, u32x4 &pk)
{
    if constexpr (QT == 4) {
        o.a0 = *reinterpret_cast<const i32x4 *>(&s.a[c][L.ta][16 * (L.hh ^ swz(L.ta))]);
        if ((c & 1) == 0)
            pk = *reinterpret_cast<const u32x4 *>(&s.bq[L.jb][16 * ((c + L.hh) ^ ((L.jb >> 1) & 7))]);
        o.b = __builtin_bit_cast(i32x4, (c & 1) ? ((pk >> 4) & 0x0F0F0F0Fu) : (pk & 0x0F0F0F0Fu));
    } else {
        o.a0 = *reinterpret_cast<const i32x4 *>(&s.a[c][0][0] + L.pa0);   // first 16 elements
        o.a1 = *reinterpret_cast<const i32x4 *>(&s.a[c][0][0] + L.pa1);   // last 16
        o.b = *reinterpret_cast<const i32x4 *>(&s.b[c][L.jb][16 * (L.hh ^ swz(L.jb))]);
    }
}

template <int QT>
__device__ __forceinline__ void load_sc(Sc<QT> &o, const Stage<QT> &s, int c, const Lane &L)
{
    if constexpr (QT == 4) {
        o.w0 = s.bs[c][L.jb][0];
        o.w1 = s.bs[c][L.jb][1];
    } else {
        o.w0 = s.bs[c][L.jb][0];
        o.w1 = s.bs[c][L.jb][1];
    }
}

template <int QT>
__device__ __forceinline__ ChunkD<QT> mfma_chunk(const Ab<QT> &o, const i32x16 &bias)
{
    ChunkD<QT> r;
    r.v[0] = mfma_i8(o.a0, o.b, bias);
    if constexpr (QT == 6) r.v[1] = mfma_i8(o.a1, o.b, bias);
    return r;
}

// The activation scales of the sixteen token rows that this lane's result
// registers hold, in register order (four 16-byte LDS reads).
template <int QT>
__device__ __forceinline__ f32x16 load_x(const Stage<QT> &s, int c, const Lane &L)
{
    const f32x4 *p = reinterpret_cast<const f32x4 *>(&s.ax[c][32 * L.wt + 16 * L.hh]);
    const f32x4 v0 = p[0], v1 = p[1], v2 = p[2], v3 = p[3];
    return __builtin_shufflevector(__builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7),
                                   __builtin_shufflevector(v2, v3, 0, 1, 2, 3, 4, 5, 6, 7),
                                   0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
}

// acc + a * b in the three-operand (VOP3) encoding.  With two waves per SIMD
// the two-operand v_fmac_f32 form, which the compiler prefers for an
// accumulation, issues markedly slower on gfx950.
__device__ __forceinline__ float fma3(float a, float b, float acc)
{
    asm("v_fma_f32 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
    return acc;
}

template <int... I>
__device__ __forceinline__ void scale_rows(f32x16 &acc, const i32x16 &D, float w, float nw, const f32x16 &x,
                                           std::integer_sequence<int, I...>)
{
    // All sixteen products first, each in its own register (the pin keeps the
    // compiler from pairing every product with its accumulation through one
    // scratch register, which would make the 32 instructions one serial
    // dependency chain); each accumulation then finds its operand long done.
    f32x16 u;
    ((u[I] = __builtin_fmaf(as_float(D[I]), w, nw)), ...);
    pin(u);
    ((acc[I] = fma3(u[I], x[I], acc[I])), ...);
}

template <int QT, int MODE>
__device__ __forceinline__ void epilogue(const ChunkD<QT> &D, const Sc<QT> &o, const f32x16 &x, f32x16 &acc,
                                         const MmqArgs &g, int64_t tw0, int64_t j, int64_t sb, int c,
                                         const Lane &L)
{
    if constexpr (MODE == 0) {
        constexpr auto rows = std::make_integer_sequence<int, 16>{};
        if constexpr (QT == 4) {
            scale_rows(acc, D.v[0], o.w0, o.w1, x, rows);
        } else {
            scale_rows(acc, D.v[0], o.w0, -MAGIC_F * o.w0, x, rows);
            scale_rows(acc, D.v[1], o.w1, -MAGIC_F * o.w1, x, rows);
        }
    } else {
        const int64_t nsb = g.id / 256;
        const int64_t nsub = (QT == 4 ? 8 : 16) * nsb;
        const int64_t sub = QT == 4 ? 8 * sb + c : 2 * (8 * sb + c);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t t = tw0 + 32 * L.wt + mfma_row(i, L.hh);
            if (t < g.t1 && j < g.j1) {
                int32_t *dst = g.P + ((t - g.t0) * (g.j1 - g.j0) + (j - g.j0)) * nsub + sub;
                dst[0] = D.v[0][i] - MAGIC_I;
                if constexpr (QT == 6) dst[1] = D.v[1][i] - MAGIC_I;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Work items and the output of a tile.
//
// A worker (workgroup) runs a list of work items, each a tile and a run
// [k0, k1) of its super-blocks: first whole tiles v, v + G, .. below
// dp_tiles, then its share of the I = sk_tiles * nsb split-phase iterations
// (stream-K), worker w taking iterations [floor(w I / G), floor((w+1) I / G))
// in tile-major order.  A tile done by one item is stored straight to y.  A
// split tile has contributors fw .. lw, consecutive workers.  Each wave owns
// a 32 x 32 quarter of the tile and finishes it on its own: it writes its
// partial sum to its worker's workspace slot and adds one to the quarter's
// counter; the wave that brings the count to lw - fw + 1 adds the partials in
// worker order fw, fw + 1, .., lw (its own from registers), stores y and puts
// the counter back to zero.  The sum therefore does not depend on which
// contributor finished last, and nothing waits on another workgroup.
// ---------------------------------------------------------------------------
struct Work {
    int tile, k0, k1;   // k1 == 0: no more work
};

__device__ __forceinline__ Work next_work(const MmqArgs &g, int &dpt, int &it, int it_end, int G, int nsb)
{
    Work w;
    if (dpt < g.dp_tiles) {
        w.tile = dpt;
        w.k0 = 0;
        w.k1 = nsb;
        dpt += G;
    } else if (it < it_end) {
        const int u = it / nsb;
        w.tile = g.dp_tiles + u;
        w.k0 = it - u * nsb;
        w.k1 = min(nsb, w.k0 + (it_end - it));
        it += w.k1 - w.k0;
    } else {
        w.tile = 0;
        w.k0 = 0;
        w.k1 = 0;
    }
    return w;
}

// Tile numbering: groups of TGROUP row tiles (the last group may be
// narrower); within a group the row tile runs fastest.  Consecutive tile
// numbers go to one XCD (see the worker numbering), so the 64 tiles an XCD
// runs at once form an 8 x 8 block of token and row tiles that share their
// activation and weight super-blocks in that XCD's L2, instead of one row
// tile against every token tile (which made each XCD read the whole
// activation plane).
constexpr int TGROUP = 8;

__device__ __forceinline__ void tile_origin(const MmqArgs &g, int tile, int64_t &tw0, int64_t &jw0)
{
    const int per = TGROUP * g.nbt;
    const int grp = tile / per, r = tile - grp * per;
    const int first = grp * TGROUP;
    const int w = min(g.nbj - first, TGROUP);
    tw0 = g.t0 + (int64_t)TT * (r / w);
    jw0 = g.j0 + (int64_t)TJ * (first + r % w);
}

__device__ __forceinline__ void store_tile(const MmqArgs &g, const f32x16 &v, int64_t tw0, int64_t j,
                                           const Lane &L)
{
    if (j < g.j1) {
        // register i holds row tb + 8 (i / 4) + i % 4: walk a pointer down
        // the rows; all 16 exist unless the tile reaches past t1
        const int64_t tb = tw0 + 32 * L.wt + 4 * L.hh;
        const int64_t ld = g.ldy;
        float *p = g.y + tb * ld + j;
        const int64_t rem = g.t1 - tb;
        const int n = (int)(rem < 0 ? 0 : (rem > 32 ? 32 : rem));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (8 * k + e < n) *p = v[4 * k + e];
                p += ld;
            }
            p += 4 * ld;
        }
    }
}

// Worker owning split-phase iteration i.
__device__ __forceinline__ int sk_worker(int i, int I, int G) { return (int)((((int64_t)i + 1) * G - 1) / I); }

// Workspace slot of worker w's partial of split tile u (counted from the
// first split tile): 2w for the tile holding w's first iteration, else 2w + 1
// (a worker's iterations are contiguous, so only its first and last tiles can
// be split).
__device__ __forceinline__ int sk_slot(int u, int w, int I, int G, int nsb)
{
    return 2 * w + (u == (int)((int64_t)w * I / G) / nsb ? 0 : 1);
}

// The partial sums cross XCDs, whose L2 caches are not kept coherent with
// each other.  Every access to them is an agent-scope atomic access, which
// carries its own cache policy (stores write through to the device coherence
// point, loads read from it), and a vmcnt(0) wait completes the stores before
// the counter update.  A device-scope fence would do the same by writing back
// and invalidating the whole L2 of the XCD, which measured several times the
// cost of the GEMM itself when every split tile did it.
__device__ __forceinline__ void st_agent(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(float *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

__device__ __forceinline__ void finish_tile(const MmqArgs &g, const f32x16 &p, const Work &w, int v, int G,
                                            int nsb, const Lane &L, int wave, int lane)
{
    int64_t tw0, jw0;
    tile_origin(g, w.tile, tw0, jw0);
    const int64_t j = jw0 + L.jb;
    if (w.k0 == 0 && w.k1 == nsb) {
        store_tile(g, p, tw0, j, L);
        return;
    }
    const int u = w.tile - g.dp_tiles;
    const int I = g.sk_tiles * nsb;
    const int fw = sk_worker(u * nsb, I, G), lw = sk_worker((u + 1) * nsb - 1, I, G);
    const int64_t quarter = 1024 * wave + lane;   // this lane's floats of the wave's quarter: + 64 i
    float *mine = g.ws + (int64_t)sk_slot(u, v, I, G, nsb) * (TT * TJ) + quarter;
#pragma unroll
    for (int i = 0; i < 16; ++i) st_agent(mine + 64 * i, p[i]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the partial is at the coherence point
    uint32_t *cnt = g.cnt + 4 * fw + wave;
    uint32_t before = 0;
    if (lane == 0) before = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    before = __builtin_amdgcn_readfirstlane(before);
    if (before != (uint32_t)(lw - fw)) return;   // another contributor finishes the quarter
    f32x16 sum;
    for (int c = fw; c <= lw; ++c) {
        f32x16 q;
        if (c == v) {
            q = p;
        } else {
            float *src = g.ws + (int64_t)sk_slot(u, c, I, G, nsb) * (TT * TJ) + quarter;
#pragma unroll
            for (int i = 0; i < 16; ++i) q[i] = ld_agent(src + 64 * i);
        }
        if (c == fw) {
            sum = q;
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) sum[i] += q[i];
        }
    }
    store_tile(g, sum, tw0, j, L);
    if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int QT, int ARM, int MODE, int ACT>
__global__ __launch_bounds__(NTHR, 2) void mmq_kernel(MmqArgs g)
{
    static_assert(ACT != ACT_F32 || (QT == 4 && MODE == 0), "the fp32 source is built for the q4_K GEMM");
    static_assert(ARM != ARM_STAGED || (QT == 4 && MODE == 0 && ACT == ACT_TILED),
                  "the staged buffer is built for the q4_K GEMM on the tiled plane");
    __shared__ Stage<QT> st[2];
    const uint32_t sl0 = (uint32_t)(uintptr_t)(lds_void_t *)&st[0];   // LDS address of stage 0

    // XCD-aware worker numbering: consecutive blocks go round-robin to the 8
    // XCDs, so hand each XCD a contiguous run of worker numbers (and so of
    // tiles).
    const int G = gridDim.x, b = blockIdx.x;
    const int q = G / 8, r = G % 8, x = b % 8;
    const int v = x * q + min(x, r) + b / 8;
    const int nsb = (int)(g.id / 256);
    const int I = g.sk_tiles * nsb;   // the host keeps tile counts and I below 2^31
    int it = (int)((int64_t)v * I / G);
    const int it_end = (int)((int64_t)(v + 1) * I / G);
    int dpt = v;
    Work cur = next_work(g, dpt, it, it_end, G, nsb);
    if (cur.k1 == 0) return;

    if constexpr (QT == 6) {
        // the zero rows of both stages (2 x 8 x 32 bytes); no copy writes them
        if (threadIdx.x < 32) {
            const int k = threadIdx.x;
            *reinterpret_cast<u32x4 *>(&st[k >> 4].a[(k >> 1) & 7][TT][16 * (k & 1)]) = u32x4{0, 0, 0, 0};
        }
    }

    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    int64_t tw0, jw0;
    tile_origin(g, cur.tile, tw0, jw0);
    Src src = make_src<QT, ARM, ACT>(g, tw0, jw0, tid);
    Raw<QT, ARM> rw;
    stage_act<QT, ACT>(sl0, src, cur.k0, tid);
    if constexpr (ACT == ACT_F32) quant_stage(g, st[0], tw0, cur.k0, tid);
    if constexpr (ARM != ARM_RAW && QT == 6) load_wexp<QT>(sl0, src, cur.k0, tid);
    if constexpr (QT == 4) load_bq<ARM>(sl0, src, cur.k0, tid);
    load_raw<QT, ARM, ACT>(rw, src, cur.k0, tid);
    int ph = 0;   // stage holding the next super-block to compute
    for (;;) {
        store_raw<QT, ARM, ACT>(st[ph], rw, tid);
        const int lane = tid & 63;
        const int wave = tid >> 6;
        Lane L;
        L.wt = wave & 1;                       // 32-token group of this wave
        L.hh = lane >> 5;
        L.ta = 32 * L.wt + (lane & 31);        // token (tile-local) this lane feeds to MFMA a
        L.jb = 32 * (wave >> 1) + (lane & 31); // weight row (tile-local) of the lane
        L.l16 = lane & 15;
        {
            const int own = 32 * L.ta + 16 * (L.hh ^ swz(L.ta)), zrow = 32 * TT;
            L.pa0 = L.hh ? zrow : own;
            L.pa1 = L.hh ? own : zrow;
        }
        i32x16 bias;
#pragma unroll
        for (int i = 0; i < 16; ++i) bias[i] = MAGIC_I;
        // kept live across the super-blocks instead of rebuilt (8 moves) in
        // each: about 1.5% faster.  Not in the q6_K raw pad40 build, which
        // has no registers to spare for it (it spilled).
        if constexpr (!(QT == 6 && ARM == ARM_RAW && ACT == ACT_PAD40)) asm volatile("" : "+v"(bias));
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the activation copy has landed
        __syncthreads();

        f32x16 acc, accm;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc[i] = 0.0f;
            accm[i] = 0.0f;
        }
        for (int sb = cur.k0; sb < cur.k1; ++sb) {
            const Stage<QT> &s = st[ph];
            Stage<QT> &sn = st[ph ^ 1];
            const bool more = sb + 1 < cur.k1;
            if (more) {
                const uint32_t sln = sl0 + (ph ^ 1) * (uint32_t)sizeof(Stage<QT>);
                stage_act<QT, ACT>(sln, src, sb + 1, tid);
                if constexpr (ARM != ARM_RAW && QT == 6) load_wexp<QT>(sln, src, sb + 1, tid);
                if constexpr (QT == 4) load_bq<ARM>(sln, src, sb + 1, tid);
                load_raw<QT, ARM, ACT>(rw, src, sb + 1, tid);
            }

            // Operand rings: chunk c+DA's MFMA operands and weight scales and
            // chunk c+DX's activation scales are fetched from LDS while chunk
            // c's epilogue runs.  q4_K has the registers for one chunk more of
            // lead (measured 1-2% faster); q6_K does not.
            constexpr int DA = QT == 4 ? 3 : 2;
            constexpr int DX = QT == 4 ? 2 : 1;
            Ab<QT> ab[DA + 1];
            u32x4 pk;
            Sc<QT> sc[DA + 1];
            f32x16 xr[DX + 1];
            ChunkD<QT> dd[2];
#pragma unroll
            for (int k = 0; k < DA; ++k) {
                load_ab(ab[k], s, k, L, pk);
                load_sc(sc[k], s, k, L);
            }
#pragma unroll
            for (int k = 0; k < DX; ++k) xr[k] = load_x(s, k, L);
            MinOp mA, mB;
            if constexpr (QT == 4 && MODE == 0) {
                mA = s.ma[L.ta][L.hh];
                mB = s.mb[L.jb][L.hh];
            }
            dd[0] = mfma_chunk(ab[0], bias);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                if (c + DA < NCH) {
                    load_ab(ab[(c + DA) % (DA + 1)], s, c + DA, L, pk);
                    load_sc(sc[(c + DA) % (DA + 1)], s, c + DA, L);
                }
                if (c + DX < NCH) xr[(c + DX) % (DX + 1)] = load_x(s, c + DX, L);
                ChunkD<QT> &cd = dd[c & 1];
                if (c + 1 < NCH) {
                    ChunkD<QT> &nd = dd[(c + 1) & 1];
                    nd = mfma_chunk(ab[(c + 1) % (DA + 1)], bias);
                    pin_after(cd.v[0], nd.v[QT == 4 ? 0 : 1]);   // issue MFMA c+1 first
                    if constexpr (QT == 6) pin(cd.v[1]);
                }
                epilogue<QT, MODE>(cd, sc[c % (DA + 1)], xr[c % (DX + 1)], acc, g, tw0, jw0 + L.jb, sb, c, L);
                if constexpr (QT == 4 && MODE == 0) {
                    // the super-block's min term: hi*hi, hi*lo, lo*hi
                    if (c == 2) accm = mfma_bf16(mA.w[0], mA.w[1], mB.w[0], mB.w[1], accm);
                    if (c == 4) accm = mfma_bf16(mA.w[0], mA.w[1], mB.w[2], mB.w[3], accm);
                    if (c == 6) accm = mfma_bf16(mA.w[2], mA.w[3], mB.w[0], mB.w[1], accm);
                }
                if constexpr (MODE == 0) pin(acc);                  // epilogue c done here
            }
            if (more) {
                if constexpr (ACT == ACT_F32) quant_stage(g, sn, tw0, sb + 1, tid);
                store_raw<QT, ARM, ACT>(sn, rw, tid);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            ph ^= 1;
        }

        // Issue the next item's first loads, then finish this tile while they
        // are in flight.  Its per-lane offsets come from a thread index the
        // compiler cannot see through, so that they are not hoisted out of
        // the loop and kept live across the super-block loop.
        const Work nxt = next_work(g, dpt, it, it_end, G, nsb);
        if (nxt.k1 != 0) {
            tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            int64_t nt0, nj0;
            tile_origin(g, nxt.tile, nt0, nj0);
            src = make_src<QT, ARM, ACT>(g, nt0, nj0, tid);
            const uint32_t slp = sl0 + ph * (uint32_t)sizeof(Stage<QT>);
            stage_act<QT, ACT>(slp, src, nxt.k0, tid);
            if constexpr (ACT == ACT_F32) quant_stage(g, st[ph], nt0, nxt.k0, tid);
            if constexpr (ARM != ARM_RAW && QT == 6) load_wexp<QT>(slp, src, nxt.k0, tid);
            if constexpr (QT == 4) load_bq<ARM>(slp, src, nxt.k0, tid);
            load_raw<QT, ARM, ACT>(rw, src, nxt.k0, tid);
        }
        if constexpr (MODE == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] += accm[i];
            finish_tile(g, acc, cur, v, G, nsb, L, wave, lane);
        }
        if (nxt.k1 == 0) break;
        cur = nxt;
        tile_origin(g, cur.tile, tw0, jw0);
    }
}


// ---------------------------------------------------------------------------
// q6_K limb arm (a registration-time limb buffer; tiled activations).
//
// The limb buffer folds each 16-element sub-block's int8 scale into the
// quants: v = sc * c6 = 128 H + L with int8 limbs H in [-32, 32] and L in
// [0, 127].  For a 32-element chunk the exact integer Q = sum qa * v =
// 128 P_H + P_L comes from two MFMAs, and the chunk's weight scale is d alone,
// applied once per super-block.  The MFMA is transposed here (weight rows are
// its rows, tokens its columns), so the activation scale of a chunk is one
// value per lane rather than sixteen per lane from LDS.  Per chunk and output:
//   t = fma(D_H, 128, -129 M) = 128 P_H - M          (D = M + P, M = 1.5 2^23;
//   u = D_L + t                = 128 P_H + P_L = Q    both exact: |Q| < 2^24)
//   acc = fma(u, da, acc)                            (rounded once)
// and per super-block y = fma(acc, d, y).  Steps are half super-blocks (four
// chunks): the limbs double the weight bytes, and a full super-block stage
// pair would not leave room for two workgroups per CU.
// ---------------------------------------------------------------------------
constexpr int LCH = 4;   // chunks per step

struct StageL {
    __attribute__((aligned(16))) uint8_t a[LCH][TT][32];   // activation quants (token rows, halves swizzled)
    float ax[LCH][TT];                                      // activation d (fp32), x_slot order
    __attribute__((aligned(16))) uint8_t h[LCH][TJ][32];   // H limbs (weight rows, halves swizzled)
    __attribute__((aligned(16))) uint8_t l[LCH][TJ][32];   // L limbs
    __attribute__((aligned(16))) float dw[TJ];             // the super-block's weight d, row-slot order (odd steps)
};
static_assert(sizeof(StageL) >= 4 * 32 * 33 * 4, "a stage holds the four waves' transpose scratch");

struct SrcL {
    const uint8_t *q8;    // the tile's tiled activation records
    const uint8_t *hl;    // H plane at the tile's first row (L plane: + od * id)
    const float *d;       // d plane at the tile's first row
    uint32_t xq[2];       // this lane's limb copy sources: rows 32 jh + l / 2, half (l & 1) ^ swz(row)
    uint32_t dro;         // d of row tid (< 64), clamped: its offset in rows of the d plane
};

__device__ __forceinline__ SrcL make_src_l(const MmqArgs &g, int64_t tw0, int64_t jw0, int tid)
{
    SrcL s;
    const int64_t nsb = g.id / 256;
    s.q8 = g.q8 + (tw0 / 64) * nsb * Q8T_RECORD;
    s.hl = g.Wexp + jw0 * g.id;
    s.d = reinterpret_cast<const float *>(g.W) + jw0 * nsb;
    const int l = tid & 63;
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
        const int r = 32 * jh + (l >> 1);
        const uint32_t rl = (uint32_t)(min(jw0 + r, g.od - 1) - jw0);
        s.xq[jh] = rl * (uint32_t)g.id + 16 * ((l & 1) ^ swz(r));
    }
    s.dro = (uint32_t)(min(jw0 + (tid & 63), g.od - 1) - jw0);
    return s;
}

// Half P (0 or 1) of step (sb, hs)'s copies into the stage at LDS address sl.
// Wave w brings chunk w of the half: its activation quants (two 1 KB pieces
// of the record), and its H and L limbs (two 1 KB copies each, one per
// 32-row half); wave 0 also the activation d of the half.
template <int P>
__device__ __forceinline__ void issue_l(uint32_t sl, const SrcL &s, const MmqArgs &g, int64_t sb, int hs, int tid)
{
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t lo = 16u * (uint32_t)(tid & 63);
    const int c = 4 * hs + w;   // chunk of the super-block
    const uint8_t *rec = s.q8 + sb * Q8T_RECORD;
    const uint8_t *hb = s.hl + 256 * sb + 32 * c;
    if constexpr (P == 0) {
        dma16n<2>(rec + 2048 * c, lo, sl + offsetof(StageL, a) + 2048 * w);
        dma16(hb, s.xq[0], sl + offsetof(StageL, h) + 2048 * w);
        if (w == 0) dma16(rec + 16384 + 1024 * hs, lo, sl + offsetof(StageL, ax));
    } else {
        const uint8_t *lb = hb + g.od * g.id;
        dma16(hb, s.xq[1], sl + offsetof(StageL, h) + 2048 * w + 1024);
        dma16(lb, s.xq[0], sl + offsetof(StageL, l) + 2048 * w);
        dma16(lb, s.xq[1], sl + offsetof(StageL, l) + 2048 * w + 1024);
    }
}

__device__ __forceinline__ float fma3c(float a, float b, float c)
{
    asm("v_fma_f32 %0, %1, %2, %3" : "=v"(a) : "v"(a), "v"(b), "v"(c));
    return a;
}

// OCC: workgroups per CU the register allocation is made for.  Three (168
// VGPRs) measured 5% faster where the tiles make several rounds (the layer's
// down projection) and 3% slower where they make one round of at most two
// per CU (the 3584 x 3584, nt = 512 shape), so the launch picks by tile count.
template <int OCC>
__global__ __launch_bounds__(NTHR, OCC) void mmq_limbs_kernel(MmqArgs g)
{
    __shared__ StageL st[2];
    const uint32_t sl0 = (uint32_t)(uintptr_t)(lds_void_t *)&st[0];

    const int G = gridDim.x, b = blockIdx.x;
    const int q = G / 8, r = G % 8, x = b % 8;
    const int v = x * q + min(x, r) + b / 8;
    const int nsb = (int)(g.id / 256);
    const int I = g.sk_tiles * nsb;
    int it = (int)((int64_t)v * I / G);
    const int it_end = (int)((int64_t)(v + 1) * I / G);
    int dpt = v;
    Work cur = next_work(g, dpt, it, it_end, G, nsb);
    if (cur.k1 == 0) return;

    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6, hh = lane >> 5;
    const int wt = wave & 1, wr = wave >> 1;   // token group, row group (the layout finish_tile expects)
    const int tok = 32 * wt + (lane & 31), row = 32 * wr + (lane & 31);
    const int pa = 32 * tok + 16 * (hh ^ swz(tok));    // byte offsets within a chunk plane
    const int pw = 32 * row + 16 * (hh ^ swz(row));
    const int xs = x_slot(tok);
    const float c128 = 128.0f, cm = -129.0f * MAGIC_F;
    int64_t tw0, jw0;
    tile_origin(g, cur.tile, tw0, jw0);
    SrcL src = make_src_l(g, tw0, jw0, tid);
    issue_l<0>(sl0, src, g, cur.k0, 0, tid);
    issue_l<1>(sl0, src, g, cur.k0, 0, tid);
    int ph = 0;
    for (;;) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        i32x16 bias;
#pragma unroll
        for (int i = 0; i < 16; ++i) bias[i] = MAGIC_I;
        // With the two-per-CU register budget the bias stays live across the
        // steps instead of being rebuilt (8 moves) in each: 2-3% faster.  The
        // three-per-CU build has no room for it (it spilled, 12% slower).
        if constexpr (OCC == 2) asm volatile("" : "+v"(bias));
        f32x16 acc, y;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc[i] = 0.0f;
            y[i] = 0.0f;
        }
        const int nsteps = 2 * (cur.k1 - cur.k0);
        float dnext = 0.0f;
        for (int stp = 0; stp < nsteps; ++stp) {
            const int hs = stp & 1;   // half of super-block cur.k0 + stp / 2
            const StageL &s = st[ph];
            const bool more = stp + 1 < nsteps;
            const uint32_t sln = sl0 + (ph ^ 1) * (uint32_t)sizeof(StageL);
            const int64_t sbn = cur.k0 + ((stp + 1) >> 1);
            if (more) {
                issue_l<0>(sln, src, g, sbn, hs ^ 1, tid);
                issue_l<1>(sln, src, g, sbn, hs ^ 1, tid);
                // the next step is the second half of a super-block: its d
                if (hs == 0 && tid < 64) dnext = src.d[src.dro * nsb + sbn];
            }
            i32x4 ah[LCH], al[LCH], ab[LCH];
            float xv[LCH];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                ah[c] = *reinterpret_cast<const i32x4 *>(&s.h[c][0][0] + pw);
                al[c] = *reinterpret_cast<const i32x4 *>(&s.l[c][0][0] + pw);
                ab[c] = *reinterpret_cast<const i32x4 *>(&s.a[c][0][0] + pa);
                xv[c] = s.ax[c][xs];
            }
            i32x16 dh[2], dl[2];
            dh[0] = mfma_i8(ah[0], ab[0], bias);
            dl[0] = mfma_i8(al[0], ab[0], bias);
#pragma unroll
            for (int c = 0; c < LCH; ++c) {
                if (c + 2 < LCH) {
                    ah[c + 2] = *reinterpret_cast<const i32x4 *>(&s.h[c + 2][0][0] + pw);
                    al[c + 2] = *reinterpret_cast<const i32x4 *>(&s.l[c + 2][0][0] + pw);
                    ab[c + 2] = *reinterpret_cast<const i32x4 *>(&s.a[c + 2][0][0] + pa);
                    xv[c + 2] = s.ax[c + 2][xs];
                }
                i32x16 &ch = dh[c & 1], &cl = dl[c & 1];
                // The epilogue's fmas are inline assembly, and the compiler
                // inserts no wait states for an inline-asm read of an MFMA
                // result: read right after its own MFMA, a result is wrong.
                // Chunk c's results are read only after chunk c+1's MFMAs
                // have issued (the matrix core runs them one after another,
                // so c's are written back by then) or, for the last chunk,
                // after the whole previous epilogue.  A CPU test checks this
                // order in the built assembly.  (Explicit s_nop padding
                // instead costs 7-9%.)
                if (c + 1 < LCH) {
                    i32x16 &nh = dh[(c + 1) & 1], &nl = dl[(c + 1) & 1];
                    nh = mfma_i8(ah[c + 1], ab[c + 1], bias);
                    nl = mfma_i8(al[c + 1], ab[c + 1], bias);
                    pin_after(ch, nl);
                    pin(cl);
                }
                f32x16 t;
#pragma unroll
                for (int i = 0; i < 16; ++i) t[i] = fma3c(as_float(ch[i]), c128, cm);
                pin(t);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float u;
                    asm("v_add_f32 %0, %1, %2" : "=v"(u) : "v"(as_float(cl[i])), "v"(t[i]));
                    t[i] = u;
                }
                pin(t);
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = fma3(t[i], xv[c], acc[i]);
                pin(acc);
            }
            if (hs == 1) {
                // end of the super-block: y += d * acc, with this lane's 16 rows' d
                const f32x4 *pd = reinterpret_cast<const f32x4 *>(&s.dw[32 * wr + 16 * hh]);
                const f32x4 d0 = pd[0], d1 = pd[1], d2 = pd[2], d3 = pd[3];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    y[i] = fma3(acc[i], d0[i], y[i]);
                    y[4 + i] = fma3(acc[4 + i], d1[i], y[4 + i]);
                    y[8 + i] = fma3(acc[8 + i], d2[i], y[8 + i]);
                    y[12 + i] = fma3(acc[12 + i], d3[i], y[12 + i]);
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
            }
            if (more && hs == 0 && tid < 64) {
                const int rr = tid;
                st[ph ^ 1].dw[32 * (rr >> 5) + row_slot(rr & 31)] = dnext;
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            ph ^= 1;
        }

        // Issue the next item's first step, then transpose this wave's 32 x 32
        // block through the stage just computed (free after the barrier) into
        // finish_tile's layout (lane = weight row, registers = tokens).
        const Work nxt = next_work(g, dpt, it, it_end, G, nsb);
        if (nxt.k1 != 0) {
            tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            int64_t nt0, nj0;
            tile_origin(g, nxt.tile, nt0, nj0);
            src = make_src_l(g, nt0, nj0, tid);
            const uint32_t slp = sl0 + ph * (uint32_t)sizeof(StageL);
            issue_l<0>(slp, src, g, nxt.k0, 0, tid);
            issue_l<1>(slp, src, g, nxt.k0, 0, tid);
        }
        float *tp = reinterpret_cast<float *>(&st[ph ^ 1]) + wave * (32 * 33);
#pragma unroll
        for (int i = 0; i < 16; ++i) tp[mfma_row(i, hh) * 33 + (lane & 31)] = y[i];
        f32x16 ys;
#pragma unroll
        for (int i = 0; i < 16; ++i) ys[i] = tp[(lane & 31) * 33 + mfma_row(i, hh)];
        Lane L;
        L.wt = wt;
        L.hh = hh;
        L.ta = tok;
        L.jb = row;
        L.l16 = lane & 15;
        L.pa0 = L.pa1 = 0;
        finish_tile(g, ys, cur, v, G, nsb, L, wave, lane);
        if (nxt.k1 == 0) break;
        cur = nxt;
        tile_origin(g, cur.tile, tw0, jw0);
    }
}

// ---------------------------------------------------------------------------
// host-side launchers (argument checking is done by the C ABI layer)
// ---------------------------------------------------------------------------

// Workgroups that run at once: two per CU.  The CU count of each device is
// queried once; host threads may race to fill the cache, with equal values.
static int64_t worker_slots(int64_t cap)
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return cap;
    if (dev < 0 || dev >= 64) return cap;
    int cus = cached[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return cap;
        cached[dev].store(cus, std::memory_order_relaxed);
    }
    return std::min<int64_t>(2 * (int64_t)cus, cap);
}

// Zero the n arrival counters of a workspace (a kernel rather than
// hipMemsetAsync, so that the call can be captured in a HIP graph).
__global__ __launch_bounds__(256) void clear_counters_kernel(uint32_t *cnt, int n)
{
    for (int i = threadIdx.x; i < n; i += 256) cnt[i] = 0;
}

template <int QT, int ARM, int MODE, int ACT = ACT_PAD40>
static int launch(MmqArgs g, int64_t ws_workers, bool clear_counters, hipStream_t stream)
{
    const int64_t nbt = (g.t1 - g.t0 + TT - 1) / TT;
    const int64_t nbj = (g.j1 - g.j0 + TJ - 1) / TJ;
    if (nbt <= 0 || nbj <= 0) return 0;
    const int64_t ntiles = nbt * nbj;
    if (ntiles > 0x7fffffff) return -1;
    g.nbt = (int)nbt;
    g.nbj = (int)nbj;
    // Whole tiles, one per workgroup, unless a workspace is given and the
    // tiles make one round that leaves a quarter or more of the workgroup
    // slots (two per CU) empty: then the (tile, super-block) iterations are
    // shared evenly by all slots (stream-K).  A fuller round, or a shape with
    // several rounds, measured faster as whole tiles: a second workgroup adds
    // only about half a CU's throughput, so the CUs left with one workgroup
    // lose less than the tile count suggests, and each split tile pays a
    // fix-up of a few microseconds.  (The work list also supports whole-tile
    // rounds followed by a split remainder: dp_tiles > 0.)
    int64_t G = ntiles;
    g.dp_tiles = (int)ntiles;
    g.sk_tiles = 0;
    const int64_t nsb = g.id / 256;
    if (MODE == 0 && g.ws != nullptr && nsb >= 2) {
        const int64_t S = worker_slots(ws_workers);
        const int64_t workers = std::min<int64_t>(S, ntiles * nsb / MMQ_MIN_SPLIT_ITERS);
        if (ntiles * MMQ_SK_FILL_DEN <= S * MMQ_SK_FILL_NUM && workers > ntiles && ntiles * nsb < 0x7fffffff) {
            g.dp_tiles = 0;
            g.sk_tiles = (int)ntiles;
            G = workers;
        }
    }
    if (g.sk_tiles > 0 && clear_counters) {
        const int rc = launch_kernel(clear_counters_kernel, dim3(1), dim3(256), stream, g.cnt, (int)(4 * G));
        if (rc != 0) return rc;
    }
    if constexpr (ARM == ARM_LIMB) {
        if (g.sk_tiles == 0 && G > worker_slots(MMQ_MAX_WORKERS))
            return launch_kernel(mmq_limbs_kernel<3>, dim3((unsigned)G), dim3(NTHR), stream, g);
        return launch_kernel(mmq_limbs_kernel<2>, dim3((unsigned)G), dim3(NTHR), stream, g);
    } else
        return launch_kernel(mmq_kernel<QT, ARM, MODE, ACT>, dim3((unsigned)G), dim3(NTHR), stream, g);
}

int launch_mmq(const MmqLaunch &Lc, hipStream_t stream)
{
    MmqArgs g;
    g.W = static_cast<const uint8_t *>(Lc.W);
    g.Wexp = reinterpret_cast<const uint8_t *>(Lc.Wexp);
    g.q8 = static_cast<const uint8_t *>(Lc.q8);
    g.ldx = Lc.ldx;
    g.y = Lc.y;
    g.P = Lc.P;
    g.bstride = Lc.bstride;
    g.od = Lc.od;
    g.id = Lc.id;
    g.nt = Lc.nt;
    g.ldy = Lc.ldy;
    g.t0 = Lc.t0;
    g.t1 = Lc.t1;
    g.j0 = Lc.j0;
    g.j1 = Lc.j1;
    g.nbt = 0;
    g.nbj = 0;
    g.ws = static_cast<float *>(Lc.ws);
    g.cnt = Lc.ws ? reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(Lc.ws) + mmq_ws_partial_bytes(Lc.ws_workers))
                  : nullptr;
    const int64_t wsw = Lc.ws_workers;
    const bool clr = Lc.clear_counters;
    const bool part = Lc.P != nullptr;
    if (Lc.limbs) {
        if (part || !Lc.q8_tiled || Lc.qtype != 6) return -1;
        return launch<6, ARM_LIMB, 0, ACT_TILED>(g, wsw, clr, stream);
    }
    if (Lc.x_f32) {
        if (part || Lc.qtype != 4 || Lc.prepared || Lc.q8_tiled) return -1;
        return launch<4, ARM_RAW, 0, ACT_F32>(g, wsw, clr, stream);
    }
    if (Lc.staged) {
        // records are per 64-row tile: the output window must start at row 0
        if (part || Lc.qtype != 4 || !Lc.q8_tiled || Lc.j0 != 0) return -1;
        return launch<4, ARM_STAGED, 0, ACT_TILED>(g, wsw, clr, stream);
    }
    if (Lc.q8_tiled) {
        // whole-output GEMMs only (the partials exports read pad40)
        if (part) return -1;
        if (Lc.qtype == 4)
            return Lc.prepared ? launch<4, ARM_PREP, 0, ACT_TILED>(g, wsw, clr, stream)
                               : launch<4, ARM_RAW, 0, ACT_TILED>(g, wsw, clr, stream);
        if (Lc.prepared) return launch<6, ARM_PREP, 0, ACT_TILED>(g, wsw, clr, stream);
        return Lc.Wexp ? launch<6, ARM_WEXP, 0, ACT_TILED>(g, wsw, clr, stream)
                       : launch<6, ARM_RAW, 0, ACT_TILED>(g, wsw, clr, stream);
    }
    if (Lc.qtype == 4) {
        if (Lc.prepared)
            return part ? launch<4, ARM_PREP, 1>(g, wsw, clr, stream) : launch<4, ARM_PREP, 0>(g, wsw, clr, stream);
        return part ? launch<4, ARM_RAW, 1>(g, wsw, clr, stream) : launch<4, ARM_RAW, 0>(g, wsw, clr, stream);
    }
    if (Lc.prepared)
        return part ? launch<6, ARM_PREP, 1>(g, wsw, clr, stream) : launch<6, ARM_PREP, 0>(g, wsw, clr, stream);
    if (Lc.Wexp)
        return part ? launch<6, ARM_WEXP, 1>(g, wsw, clr, stream) : launch<6, ARM_WEXP, 0>(g, wsw, clr, stream);
    return part ? launch<6, ARM_RAW, 1>(g, wsw, clr, stream) : launch<6, ARM_RAW, 0>(g, wsw, clr, stream);
}

// ---------------------------------------------------------------------------
// The library's own stream-K workspace, for callers that cannot allocate.
// Each device holds its own copy of this array from load to process exit; the
// host resolves its device address once per device (with that device
// current) and passes that address to the kernels -- the array's name in host
// code is only a host-side stand-in.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[MMQ_SCRATCH_BYTES];

void *mmq_scratch(void)
{
    static std::atomic<void *> addr[64];
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace qig
