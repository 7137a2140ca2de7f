// qoq_device.hpp -- device-side helpers shared by the libqoq kernels (gfx950).
//
// Internal to the GPU library; the CPU oracle has its own, independent code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qoq {

typedef int int32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kGroup = 128;

// binary16 bits <-> float. Widening is exact; narrowing rounds to nearest even
// (v_cvt_f16_f32 under the default round-to-nearest-even mode).
__device__ __forceinline__ float h2f(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}
__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Wave-wide reductions over 64 lanes.
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
__device__ __forceinline__ unsigned wave_max_u(unsigned v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, (unsigned)__shfl_xor((int)v, o, kWave));
    return v;
}
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ float wave_min_f(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Largest |x| among the FP16 values held in a 32-bit word, as magnitude bits.
// With the sign bit cleared, FP16 bit patterns of finite values order like
// the values themselves, so the maximum can be taken on the integers.
__device__ __forceinline__ unsigned absmax_bits2(uint32_t w) {
    return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
}

// Per-lane constants of the g128 unpack for one group: the integer scale in
// both 16-bit halves, and the biased zero-point compensation
// C = (128 - z*s_g) * 257 mod 2^16 in both halves. The parameter byte holds
// (s_g - 1) in its high nibble and z in its low nibble.
struct GroupConst {
    uint32_t mul;
    uint32_t add;
};
__device__ __forceinline__ GroupConst group_const(uint32_t pbyte) {
    const uint32_t sg = (pbyte >> 4) + 1u;
    const uint32_t zs = (pbyte & 15u) * sg;
    const uint32_t c16 = ((128u - zs) * 257u) & 0xFFFFu;
    return {sg * 0x00010001u, c16 * 0x00010001u};
}

// Four codes (one per byte, 0..15) -> four INT8 values (q - z) * s_g:
// per 16-bit half, codes*s_g + C (no carry between bytes because every byte of
// the exact result lies in [0, 255] thanks to the [-119, 119] headroom), then
// the XOR maps each biased byte b to the two's-complement byte of b - 128.
__device__ __forceinline__ uint32_t unpack4_g128(uint32_t codes, GroupConst gc) {
    uint32_t r;
    asm("v_pk_mad_u16 %0, %1, %2, %3" : "=v"(r) : "v"(codes), "v"(gc.mul), "v"(gc.add));
    return r ^ 0x80808080u;
}

// The same unpack with both constants in one 32-bit group word: s_g in the low
// half and C in the high half. The packed multiply-add reads the scale from
// the low half and the addend from the high half for both result halves
// (op_sel / op_sel_hi), so no per-step duplication of the constants is needed.
__device__ __forceinline__ uint32_t group_word(uint32_t pbyte) {
    const uint32_t sg = (pbyte >> 4) + 1u;
    const uint32_t zs = (pbyte & 15u) * sg;
    const uint32_t c16 = ((128u - zs) * 257u) & 0xFFFFu;
    return sg | (c16 << 16);
}
__device__ __forceinline__ uint32_t unpack4_g128w(uint32_t codes, uint32_t gw) {
    uint32_t r;
    asm("v_pk_mad_u16 %0, %1, %2, %2 op_sel:[0,0,1] op_sel_hi:[1,0,1]"
        : "=v"(r)
        : "v"(codes), "v"(gw));
    return r ^ 0x80808080u;
}

// One k-step (KS = 0 or 1) of a lane's 32 packed codes -> one MFMA B operand.
template <bool kG128, int KS>
__device__ __forceinline__ int32x4 unpack_half(u32x4 p, uint32_t gw) {
    const uint32_t w0 = KS ? p.z : p.x, w1 = KS ? p.w : p.y;
    uint32_t a0 = w0 & 0x0F0F0F0Fu, a1 = (w0 >> 4) & 0x0F0F0F0Fu;
    uint32_t a2 = w1 & 0x0F0F0F0Fu, a3 = (w1 >> 4) & 0x0F0F0F0Fu;
    if (kG128) {
        a0 = unpack4_g128w(a0, gw); a1 = unpack4_g128w(a1, gw);
        a2 = unpack4_g128w(a2, gw); a3 = unpack4_g128w(a3, gw);
    }
    return int32x4{(int)a0, (int)a1, (int)a2, (int)a3};
}

// Packed 16 bytes of one lane (32 codes) -> the two MFMA B operands (k-steps
// s = 0 and 1) of 16 INT8 values each, in the byte order of the A operand.
template <bool kG128>
__device__ __forceinline__ void unpack_lane(u32x4 p, GroupConst gc, int32x4& b0, int32x4& b1) {
    uint32_t a0 = p.x & 0x0F0F0F0Fu, a1 = (p.x >> 4) & 0x0F0F0F0Fu;
    uint32_t a2 = p.y & 0x0F0F0F0Fu, a3 = (p.y >> 4) & 0x0F0F0F0Fu;
    uint32_t c0 = p.z & 0x0F0F0F0Fu, c1 = (p.z >> 4) & 0x0F0F0F0Fu;
    uint32_t c2 = p.w & 0x0F0F0F0Fu, c3 = (p.w >> 4) & 0x0F0F0F0Fu;
    if (kG128) {
        a0 = unpack4_g128(a0, gc); a1 = unpack4_g128(a1, gc);
        a2 = unpack4_g128(a2, gc); a3 = unpack4_g128(a3, gc);
        c0 = unpack4_g128(c0, gc); c1 = unpack4_g128(c1, gc);
        c2 = unpack4_g128(c2, gc); c3 = unpack4_g128(c3, gc);
    }
    b0 = int32x4{(int)a0, (int)a1, (int)a2, (int)a3};
    b1 = int32x4{(int)c0, (int)c1, (int)c2, (int)c3};
}

__device__ __forceinline__ int32x4 mfma16x16x64(int32x4 a, int32x4 b, int32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

}  // namespace qoq
