// qig_device.h -- device-side helpers shared by the gfx950 kernels of libqig.
//
// CDNA4 facts relied on (checked on the device by the parity tests):
//  * v_mfma_i32_32x32x32_i8: a wave multiplies a 32x32 int8 A (rows m) by a
//    32x32 int8 B (columns n) over K = 32.  Lane l supplies 16 bytes of row
//    m = l % 32 of A and 16 bytes of column n = l % 32 of B; the same
//    (lane half l / 32, byte) position of A and B meets in the sum, so loading
//    bytes 16*(l/32) .. +15 of a 32-wide chunk into lane l makes lanes 0-31
//    carry k = 0..15 and lanes 32-63 carry k = 16..31.
//  * The 32x32 result: lane l, register i holds column n = l % 32 and row
//    m = 8*(i/4) + 4*(l/32) + i%4 (the same for the f32 32x32x2 form).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qig {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Starting an int32 MFMA accumulator at the bit pattern of 1.5*2^23 makes the
// result, read as fp32, equal 1.5*2^23 + P exactly while |P| < 2^22.  Then
// fma(D, s, -1.5*2^23*s) == round(P*s) in one instruction whenever
// 1.5*2^23*s is exact (s with at most 22 significant bits).
constexpr int MAGIC_I = 0x4B400000;
constexpr float MAGIC_F = 12582912.0f;

__device__ __forceinline__ i32x16 mfma_i8(i32x4 a, i32x4 b, i32x16 c)
{
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// 32x32x8 bf16 -> fp32; each operand is four bf16 packed in two dwords.
__device__ __forceinline__ f32x16 mfma_bf16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x16 c)
{
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const s16x4 a = __builtin_bit_cast(s16x4, u32x2{a0, a1});
    const s16x4 b = __builtin_bit_cast(s16x4, u32x2{b0, b1});
    return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a, b, c, 0, 0, 0);
}

// Reinterpret an int32 as fp32.  Takes the value by copy: clang's
// __builtin_bit_cast applied directly to an ext-vector element (v[i]) reads
// element 0 whatever i is, so vector elements must pass through a scalar.
__device__ __forceinline__ float as_float(int v)
{
    return __builtin_bit_cast(float, v);
}

__device__ __forceinline__ float h2f(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xffffu));
}

// Row of the 32x32 MFMA result held by register i of a lane in half `hh`.
__device__ __forceinline__ int mfma_row(int i, int hh)
{
    return 8 * (i >> 2) + 4 * hh + (i & 3);
}

// Position of token row tau (0..31) in a per-row scale vector laid out so
// that each lane half reads its 16 rows contiguously, in register order.
__device__ __forceinline__ int row_slot(int tau)
{
    return 16 * ((tau >> 2) & 1) + 4 * (tau >> 3) + (tau & 3);
}

// Position of tile token t (0..63) in a row of a per-token scale table: each
// 32-token group in register order, so the 16 rows a lane half holds are 16
// consecutive entries.
__device__ __forceinline__ int x_slot(int t) { return (t & 32) + row_slot(t & 31); }

// The 16-byte half h of quant row r (32 bytes) is stored at half h ^ swz(r).
// An LDS access phase serves 8 (32 banks) or 16 (64 banks) lanes reading 16
// bytes of consecutive rows 32 bytes apart; flipping the half on bit 2 xor
// bit 3 of the row spreads both kinds of phase over distinct 16-byte bank
// groups.
__device__ __forceinline__ int swz(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }

// v = hi + lo + O(2^-16 v) with hi, lo bf16 (round to nearest even).
__device__ __forceinline__ void bf16_split(float v, uint16_t &hi, uint16_t &lo)
{
    const __bf16 h = (__bf16)v;
    const __bf16 l = (__bf16)(v - (float)h);
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, l);
}

// Four 6-bit values v in [0, 63], one per byte, to the two's-complement
// bytes of v - 32: v + 0x60 stays below 0x100 (no carry between bytes) and
// flipping bit 7 then gives v - 32 modulo 256.
__device__ __forceinline__ uint32_t q6_centre(uint32_t v)
{
    return (v + 0x60606060u) ^ 0x80808080u;
}

// q6_K: four centred int8 weights from one ql dword and one qh dword.
// quarter qq (0..3) picks the nibble (low for 0,1; high for 2,3) and the
// 2-bit field of qh, which lands in bits 4-5 of each byte.
__device__ __forceinline__ uint32_t q6_centred(uint32_t qlw, uint32_t qhw, int qq)
{
    const uint32_t nib = (qq < 2) ? (qlw & 0x0F0F0F0Fu) : ((qlw >> 4) & 0x0F0F0F0Fu);
    const uint32_t hi2 = ((qhw >> (2 * qq)) << 4) & 0x30303030u;
    return q6_centre(nib + hi2);
}

// q4_K 6-bit scale and min of sub-block b from the twelve packed bytes S.
__device__ __forceinline__ void q4_scale_min(const uint8_t *S, int b, int &sc, int &m)
{
    if (b < 4) {
        sc = S[b] & 63;
        m = S[b + 4] & 63;
    } else {
        sc = (S[b + 4] & 15) | ((S[b - 4] >> 6) << 4);
        m = (S[b + 4] >> 4) | ((S[b] >> 6) << 4);
    }
}

}  // namespace qig
