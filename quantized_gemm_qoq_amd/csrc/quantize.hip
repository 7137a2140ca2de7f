// quantize.hip -- per-token INT8 activation quantization, its fused producers
// (SiLU(gate) * up and RMSNorm in front of the quantization), and the offline
// weight quantizers (progressive g128 and per-channel UINT4, and the INT8
// weights of the W8A8 sibling), for gfx950.
//
// Method: QServe / QoQ (arXiv 2405.04532).
//   Activations: "QServe Guide: W4A8KV4 Quantization for LLM Serving", Deep Dive
//   part 1 -- per-token symmetric INT8 with scale max|X|/127.
//   Weights: "QServe: Low Bit Width Does Not Guarantee High Throughput",
//   section 4 -- stage 1 (per-channel INT8 in [-119, 119], scale max|W|/119)
//   and stage 2 (groups of 128 inputs, integer scale, UINT4 zero and codes).
// Rounding follows the library contract in qoq.h: round half to even, scales
// computed in IEEE fp32 with correctly rounded division, stored as FP16, and
// the stored FP16 scale is the one used to quantize.
#include <algorithm>

#include "qoq_device.hpp"
#include "qoq.h"
#include "qoq_launch.hpp"

namespace qoq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <typename T, typename Op, int kNW = kWaves>
__device__ __forceinline__ T block_reduce(T v, T* smem, Op wave_op) {
    v = wave_op(v);
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) smem[wave] = v;
    __syncthreads();
    T r = smem[0];
#pragma unroll
    for (int i = 1; i < kNW; ++i) r = wave_op.combine(r, smem[i]);
    __syncthreads();
    return r;
}

struct MaxU {
    __device__ unsigned operator()(unsigned v) const { return wave_max_u(v); }
    __device__ unsigned combine(unsigned a, unsigned b) const { return max(a, b); }
};
struct SumI {
    __device__ int operator()(int v) const { return wave_sum_i(v); }
    __device__ int combine(int a, int b) const { return a + b; }
};
struct MaxF {
    __device__ float operator()(float v) const { return wave_max_f(v); }
    __device__ float combine(float a, float b) const { return fmaxf(a, b); }
};
struct MinF {
    __device__ float operator()(float v) const { return wave_min_f(v); }
    __device__ float combine(float a, float b) const { return fminf(a, b); }
};

// Quantize one FP16 value with the row's FP16 scale (given as float, non-zero).
__device__ __forceinline__ int quant_act1(uint32_t hbits, float sf) {
    const float r = rintf(h2f(hbits) / sf);
    return (int)fminf(fmaxf(r, -128.0f), 127.0f);
}

// One workgroup per token row (the grid covers the padded rows too, which are
// written as zeros). Pass 1 takes the row's largest magnitude on the FP16 bit
// patterns; pass 2 re-reads the row (an L2 hit) and writes each run of 16
// codes to its 16-byte slot of the packed tile order.
__global__ __launch_bounds__(kThreads) void k_quantize_act(const uint16_t* __restrict__ x, int M,
                                                           int K, int8_t* __restrict__ xq,
                                                           uint16_t* __restrict__ s_x,
                                                           int32_t* __restrict__ rowsum) {
    __shared__ unsigned red_u[kWaves];
    __shared__ int red_i[kWaves];
    const int m = blockIdx.x;
    const int U = gridDim.x / 16;  // grid = Mp rows
    const int u = m / 16, r = m % 16;
    const int nchunk = K / 16;
    uint4* out = reinterpret_cast<uint4*>(xq);
    // 16-byte slot of chunk c (inputs 16c .. 16c+15) of this row.
    auto slot = [&](int c) {
        const int g = c / 8, s = (c / 4) % 2, j = c % 4;
        return ((size_t)g * U + u) * 128 + 64 * s + 16 * j + r;
    };
    if (m >= M) {
        for (int c = threadIdx.x; c < nchunk; c += kThreads) out[slot(c)] = make_uint4(0, 0, 0, 0);
        return;
    }
    const uint4* row = reinterpret_cast<const uint4*>(x + (size_t)m * K);
    const int nvec = K / 8;

    unsigned amax = 0;
    for (int i = threadIdx.x; i < nvec; i += kThreads) {
        const uint4 v = row[i];
        amax = max(amax, max(max(absmax_bits2(v.x), absmax_bits2(v.y)),
                             max(absmax_bits2(v.z), absmax_bits2(v.w))));
    }
    amax = block_reduce(amax, red_u, MaxU{});
    const uint16_t sbits = f2h(h2f(amax) / 127.0f);
    const float sf = h2f(sbits);

    int sum = 0;
    for (int c = threadIdx.x; c < nchunk; c += kThreads) {
        uint4 o = make_uint4(0, 0, 0, 0);
        if (sf != 0.0f) {
            const uint4 v0 = row[2 * c], v1 = row[2 * c + 1];
            const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t hb = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
                const int q = quant_act1(hb, sf);
                sum += q;
                packed[e >> 2] |= (uint32_t)(q & 0xFF) << (8 * (e & 3));
            }
            o = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        }
        out[slot(c)] = o;
    }
    if (rowsum) sum = block_reduce(sum, red_i, SumI{});
    if (threadIdx.x == 0) {
        s_x[m] = sbits;
        if (rowsum) rowsum[m] = sum;
    }
}

// The same quantization with the row held in registers (CH runs of 16 inputs
// per thread, THR threads per row): one read of the row instead of two. Used
// for K <= 16 * THR * CH.
template <int THR, int CH>
__global__ __launch_bounds__(THR) void k_quantize_act_reg(const uint16_t* __restrict__ x, int M,
                                                          int K, int8_t* __restrict__ xq,
                                                          uint16_t* __restrict__ s_x,
                                                          int32_t* __restrict__ rowsum) {
    constexpr int kNW = THR / kWave;
    __shared__ unsigned red_u[kNW];
    __shared__ int red_i[kNW];
    const int m = blockIdx.x;
    const int U = gridDim.x / 16;  // grid = Mp rows
    const int u = m / 16, r = m % 16;
    const int nchunk = K / 16;
    u32x4* out = reinterpret_cast<u32x4*>(xq);
    // 16-byte slot of chunk c (inputs 16c .. 16c+15) of this row.
    auto slot = [&](int c) {
        const int g = c / 8, s = (c / 4) % 2, j = c % 4;
        return ((size_t)g * U + u) * 128 + 64 * s + 16 * j + r;
    };
    if (m >= M) {
        for (int c = threadIdx.x; c < nchunk; c += THR) out[slot(c)] = u32x4{0u, 0u, 0u, 0u};
        return;
    }
    const u32x4* row = reinterpret_cast<const u32x4*>(x + (size_t)m * K);
    u32x4 v0[CH], v1[CH];
    unsigned amax = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = threadIdx.x + THR * i;
        v0[i] = u32x4{0u, 0u, 0u, 0u};
        v1[i] = u32x4{0u, 0u, 0u, 0u};
        if (c < nchunk) {
            v0[i] = row[2 * c];
            v1[i] = row[2 * c + 1];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            amax = max(amax, max(absmax_bits2(v0[i][e]), absmax_bits2(v1[i][e])));
    }
    amax = block_reduce<unsigned, MaxU, kNW>(amax, red_u, MaxU{});
    const uint16_t sbits = f2h(h2f(amax) / 127.0f);
    const float sf = h2f(sbits);

    int sum = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = threadIdx.x + THR * i;
        if (c < nchunk) {
            u32x4 o = u32x4{0u, 0u, 0u, 0u};
            if (sf != 0.0f) {
                const uint32_t w[8] = {v0[i][0], v0[i][1], v0[i][2], v0[i][3],
                                       v1[i][0], v1[i][1], v1[i][2], v1[i][3]};
                uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t hb = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
                    const int q = quant_act1(hb, sf);
                    sum += q;
                    packed[e >> 2] |= (uint32_t)(q & 0xFF) << (8 * (e & 3));
                }
                o = u32x4{packed[0], packed[1], packed[2], packed[3]};
            }
            out[slot(c)] = o;
        }
    }
    if (rowsum) sum = block_reduce<int, SumI, kNW>(sum, red_i, SumI{});
    if (threadIdx.x == 0) {
        s_x[m] = sbits;
        if (rowsum) rowsum[m] = sum;
    }
}

// Many rows: one wave per (padded) row, four rows per workgroup. A lane holds
// CH runs of 16 inputs (runs lane, lane + 64, ...) in registers, so the whole
// row's loads are in flight at once, and both reductions stay inside the wave
// (no LDS table, no barrier). The arithmetic is k_quantize_act_reg's.
template <int CH>
__global__ __launch_bounds__(256) void k_quantize_act_wave(const uint16_t* __restrict__ x, int M, int K,
                                                           int Mp, int8_t* __restrict__ xq,
                                                           uint16_t* __restrict__ s_x,
                                                           int32_t* __restrict__ rowsum) {
    const int lane = threadIdx.x % kWave;
    const int m = blockIdx.x * 4 + threadIdx.x / kWave;
    if (m >= Mp) return;  // the whole wave
    const int U = Mp / 16;
    const int u = m / 16, r = m % 16;
    const int nchunk = K / 16;
    u32x4* out = reinterpret_cast<u32x4*>(xq);
    auto slot = [&](int c) {
        const int g = c / 8, s = (c / 4) % 2, j = c % 4;
        return ((size_t)g * U + u) * 128 + 64 * s + 16 * j + r;
    };
    if (m >= M) {
        for (int c = lane; c < nchunk; c += kWave) out[slot(c)] = u32x4{0u, 0u, 0u, 0u};
        return;
    }
    const u32x4* row = reinterpret_cast<const u32x4*>(x + (size_t)m * K);
    u32x4 v0[CH], v1[CH];
    unsigned amax = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = lane + kWave * i;
        v0[i] = u32x4{0u, 0u, 0u, 0u};
        v1[i] = u32x4{0u, 0u, 0u, 0u};
        if (c < nchunk) {
            v0[i] = row[2 * c];
            v1[i] = row[2 * c + 1];
        }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            amax = max(amax, max(absmax_bits2(v0[i][e]), absmax_bits2(v1[i][e])));
    amax = wave_max_u(amax);
    const uint16_t sbits = f2h(h2f(amax) / 127.0f);
    const float sf = h2f(sbits);

    int sum = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = lane + kWave * i;
        if (c < nchunk) {
            u32x4 o = u32x4{0u, 0u, 0u, 0u};
            if (sf != 0.0f) {
                const uint32_t w[8] = {v0[i][0], v0[i][1], v0[i][2], v0[i][3],
                                       v1[i][0], v1[i][1], v1[i][2], v1[i][3]};
                uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t hb = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
                    const int q = quant_act1(hb, sf);
                    sum += q;
                    packed[e >> 2] |= (uint32_t)(q & 0xFF) << (8 * (e & 3));
                }
                o = u32x4{packed[0], packed[1], packed[2], packed[3]};
            }
            out[slot(c)] = o;
        }
    }
    if (rowsum) sum = wave_sum_i(sum);
    if (lane == 0) {
        s_x[m] = sbits;
        if (rowsum) rowsum[m] = sum;
    }
}

// Progressive group quantization, one workgroup per output channel.
// Stage 1 needs the row's largest magnitude; stage 2 runs one wave per group
// of 128, two inputs per lane.
__global__ __launch_bounds__(kThreads) void k_quantize_weights_g128(
    const uint16_t* __restrict__ w, int K, uint8_t* __restrict__ q, uint16_t* __restrict__ s_c,
    uint8_t* __restrict__ s_g, uint8_t* __restrict__ zp) {
    __shared__ unsigned red_u[kWaves];
    const size_t n = blockIdx.x;
    const uint16_t* row = w + n * (size_t)K;
    const uint4* rowv = reinterpret_cast<const uint4*>(row);
    const int nvec = K / 8;
    const int G = K / kGroup;

    unsigned amax = 0;
    for (int i = threadIdx.x; i < nvec; i += kThreads) {
        const uint4 v = rowv[i];
        amax = max(amax, max(max(absmax_bits2(v.x), absmax_bits2(v.y)),
                             max(absmax_bits2(v.z), absmax_bits2(v.w))));
    }
    amax = block_reduce(amax, red_u, MaxU{});
    const uint16_t scbits = f2h(h2f(amax) / 119.0f);
    const float scf = h2f(scbits);
    if (threadIdx.x == 0) s_c[n] = scbits;

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    for (int g = wave; g < G; g += kWaves) {
        const uint32_t pair = reinterpret_cast<const uint32_t*>(row + g * kGroup)[lane];
        int w8[2] = {0, 0};
        if (scf != 0.0f) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float r = rintf(h2f(e ? pair >> 16 : pair & 0xFFFFu) / scf);
                w8[e] = (int)fminf(fmaxf(r, -119.0f), 119.0f);
            }
        }
        const int mn = wave_min_i(min(0, min(w8[0], w8[1])));
        const int mx = wave_max_i(max(0, max(w8[0], w8[1])));
        const int sg = max(1, (mx - mn + 14) / 15);
        // Quotients of small integers: the fp32 division is exact at ties and
        // cannot cross a half-integer otherwise, so rintf rounds the rational.
        const float sgf = (float)sg;
        const int zz = (int)rintf((float)(-mn) / sgf);
        uint32_t codes = 0;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = min(15, max(0, (int)rintf((float)w8[e] / sgf) + zz));
            codes |= (uint32_t)c << (8 * e);
        }
        reinterpret_cast<uint16_t*>(q + n * (size_t)K + g * kGroup)[lane] = (uint16_t)codes;
        if (lane == 0) {
            s_g[n * (size_t)G + g] = (uint8_t)sg;
            zp[n * (size_t)G + g] = (uint8_t)zz;
        }
    }
}

// Per-channel UINT4: one asymmetric range per output channel, spanning zero.
__global__ __launch_bounds__(kThreads) void k_quantize_weights_pc(
    const uint16_t* __restrict__ w, int K, uint8_t* __restrict__ q, uint16_t* __restrict__ s_c,
    uint8_t* __restrict__ zp) {
    __shared__ float red_f[kWaves];
    const size_t n = blockIdx.x;
    const uint4* rowv = reinterpret_cast<const uint4*>(w + n * (size_t)K);
    const int nvec = K / 8;

    float mn = 0.0f, mx = 0.0f;
    for (int i = threadIdx.x; i < nvec; i += kThreads) {
        const uint4 v = rowv[i];
        const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float f = h2f((e & 1) ? (ws[e >> 1] >> 16) : (ws[e >> 1] & 0xFFFFu));
            mn = fminf(mn, f);
            mx = fmaxf(mx, f);
        }
    }
    mn = block_reduce(mn, red_f, MinF{});
    mx = block_reduce(mx, red_f, MaxF{});
    const float range = mx - mn;
    const uint16_t scbits = f2h(range / 15.0f);
    const float scf = h2f(scbits);
    int zz = 0;
    if (scf != 0.0f) zz = (int)fminf(fmaxf(rintf(-mn / scf), 0.0f), 15.0f);
    if (threadIdx.x == 0) {
        s_c[n] = scbits;
        zp[n] = (uint8_t)zz;
    }

    uint2* out = reinterpret_cast<uint2*>(q + n * (size_t)K);
    for (int i = threadIdx.x; i < nvec; i += kThreads) {
        uint2 o = {0u, 0u};
        if (scf != 0.0f) {
            const uint4 v = rowv[i];
            const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
            uint32_t packed[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = h2f((e & 1) ? (ws[e >> 1] >> 16) : (ws[e >> 1] & 0xFFFFu));
                const int c = min(15, max(0, (int)rintf(f / scf) + zz));
                packed[e >> 2] |= (uint32_t)c << (8 * (e & 3));
            }
            o = make_uint2(packed[0], packed[1]);
        }
        out[i] = o;
    }
}

// ---------------------------------------------------------------------------
// Fused producer of the down projection's input: h = f16(SiLU(gate) * up)
// from the fused gate_up output [M, 2I] (gate in columns 0..I-1, up in
// columns I..2I-1), then the per-token quantization above -- one pass over
// the gate_up rows instead of a SiLU pass that writes h and a quantization
// pass that reads it back.
//
// The exponential is computed step by step so that the result is a fixed
// function of the input (the codes depend on it): Cody and Waite's range
// reduction x = n ln2 + r with ln2 split in two (the first part has trailing
// zero bits, so n * ln2_hi is exact), the Taylor polynomial of exp(r) to degree
// 7 in Horner form, and the scaling by 2^n built as an exponent field. Each
// line is one IEEE fp32 operation (the build forbids contraction into fused
// multiply-adds); inputs above 88 give +inf and below -86 give 0, which keeps
// 2^n and the result normal numbers.
__device__ __forceinline__ float exp_steps(float x) {
    if (x > 88.0f) return __builtin_inff();
    if (x < -86.0f) return 0.0f;
    const float log2e = (float)1.4426950408889634;  // 1 / ln 2
    const float ln2_hi = 0.693145751953125f;          // ln 2 to 16 significant bits
    const float ln2_lo = (float)(0.6931471805599453 - 0.693145751953125);
    const float n = rintf(x * log2e);
    const float r = (x - n * ln2_hi) - n * ln2_lo;
    float p = (float)(1.0 / 5040.0);
    p = p * r + (float)(1.0 / 720.0);
    p = p * r + (float)(1.0 / 120.0);
    p = p * r + (float)(1.0 / 24.0);
    p = p * r + (float)(1.0 / 6.0);
    p = p * r + 0.5f;
    p = p * r + 1.0f;
    p = p * r + 1.0f;
    const uint32_t bits = (uint32_t)((int)n + 127) << 23;
    return p * __builtin_bit_cast(float, bits);
}

// h = f16((g / (1 + exp(-g))) * u) for one FP16 pair; the barrier keeps the
// product and the conversion two roundings.
__device__ __forceinline__ uint32_t silu_mul1(uint32_t gbits, uint32_t ubits) {
    const float g = h2f(gbits);
    const float t = 1.0f + exp_steps(-g);
    float v = (g / t) * h2f(ubits);
    asm("" : "+v"(v));
    return f2h(v);
}

// Eight outputs from four words of gate and four of up (two FP16 per word).
__device__ __forceinline__ u32x4 silu_mul8(u32x4 g, u32x4 u) {
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = silu_mul1(g[e] & 0xFFFFu, u[e] & 0xFFFFu) | (silu_mul1(g[e] >> 16, u[e] >> 16) << 16);
    return o;
}

// Row held in registers (CH runs of 16 outputs per thread, THR threads per
// row), for I <= 16 * THR * CH; h (FP16 [M, I]) is written too when asked for.
template <int THR, int CH>
__global__ __launch_bounds__(THR) void k_silu_quant_reg(const uint16_t* __restrict__ gu, int M,
                                                        int I, int8_t* __restrict__ xq,
                                                        uint16_t* __restrict__ s_x,
                                                        int32_t* __restrict__ rowsum,
                                                        uint16_t* __restrict__ h_out) {
    constexpr int kNW = THR / kWave;
    __shared__ unsigned red_u[kNW];
    __shared__ int red_i[kNW];
    const int m = blockIdx.x;
    const int U = gridDim.x / 16;
    const int u = m / 16, r = m % 16;
    const int nchunk = I / 16;
    u32x4* out = reinterpret_cast<u32x4*>(xq);
    auto slot = [&](int c) {
        const int g = c / 8, s = (c / 4) % 2, j = c % 4;
        return ((size_t)g * U + u) * 128 + 64 * s + 16 * j + r;
    };
    if (m >= M) {
        for (int c = threadIdx.x; c < nchunk; c += THR) out[slot(c)] = u32x4{0u, 0u, 0u, 0u};
        return;
    }
    const u32x4* grow = reinterpret_cast<const u32x4*>(gu + (size_t)m * 2 * I);
    const u32x4* urow = reinterpret_cast<const u32x4*>(gu + (size_t)m * 2 * I + I);
    u32x4* hrow = h_out ? reinterpret_cast<u32x4*>(h_out + (size_t)m * I) : nullptr;
    u32x4 v0[CH], v1[CH];
    unsigned amax = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = threadIdx.x + THR * i;
        v0[i] = u32x4{0u, 0u, 0u, 0u};
        v1[i] = u32x4{0u, 0u, 0u, 0u};
        if (c < nchunk) {
            v0[i] = silu_mul8(grow[2 * c], urow[2 * c]);
            v1[i] = silu_mul8(grow[2 * c + 1], urow[2 * c + 1]);
            if (hrow) {
                hrow[2 * c] = v0[i];
                hrow[2 * c + 1] = v1[i];
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            amax = max(amax, max(absmax_bits2(v0[i][e]), absmax_bits2(v1[i][e])));
    }
    amax = block_reduce<unsigned, MaxU, kNW>(amax, red_u, MaxU{});
    const uint16_t sbits = f2h(h2f(amax) / 127.0f);
    const float sf = h2f(sbits);

    int sum = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = threadIdx.x + THR * i;
        if (c < nchunk) {
            u32x4 o = u32x4{0u, 0u, 0u, 0u};
            if (sf != 0.0f) {
                const uint32_t w[8] = {v0[i][0], v0[i][1], v0[i][2], v0[i][3],
                                       v1[i][0], v1[i][1], v1[i][2], v1[i][3]};
                uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t hb = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
                    const int q = quant_act1(hb, sf);
                    sum += q;
                    packed[e >> 2] |= (uint32_t)(q & 0xFF) << (8 * (e & 3));
                }
                o = u32x4{packed[0], packed[1], packed[2], packed[3]};
            }
            out[slot(c)] = o;
        }
    }
    if (rowsum) sum = block_reduce<int, SumI, kNW>(sum, red_i, SumI{});
    if (threadIdx.x == 0) {
        s_x[m] = sbits;
        if (rowsum) rowsum[m] = sum;
    }
}

// ---------------------------------------------------------------------------
// RMSNorm producer of a GEMM input: y = f16((x * r) * gamma) with
// r = 1 / sqrt(f32(f64(S) / K) + eps), S the exact sum of squares of the
// row, then the per-token INT8 quantization of y exactly as
// k_quantize_act_reg does it. Each FP16 x = M 2^(e - 24) squares to an
// integer multiple of 2^-48, so S is kept exactly as a 128-bit integer
// (K <= 32768 values below 2^80) and the rounding of the mean is unique,
// which makes y, and with it every code, independent of the summation order.
// The fp64 division, the fp32 square root and the fp32 reciprocal are
// correctly rounded, the products separate fp32 multiplies.
__device__ __forceinline__ unsigned __int128 square_fp16(uint32_t bits) {
    const uint32_t e = (bits >> 10) & 31u, f = bits & 1023u;
    const uint32_t mant = e ? (f | 1024u) : f;  // |x| = mant 2^(max(e, 1) - 25)
    const uint32_t shift = e ? 2u * (e - 1u) : 0u;
    return (unsigned __int128)(mant * mant) << shift;  // x^2 in units of 2^-48
}

struct SumU128 {
    __device__ unsigned __int128 operator()(unsigned __int128 v) const {
        uint64_t lo = (uint64_t)v, hi = (uint64_t)(v >> 64);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const uint64_t olo = __shfl_xor(lo, o, kWave), ohi = __shfl_xor(hi, o, kWave);
            const uint64_t nlo = lo + olo;
            hi += ohi + (nlo < lo ? 1u : 0u);
            lo = nlo;
        }
        return ((unsigned __int128)hi << 64) | lo;
    }
    __device__ unsigned __int128 combine(unsigned __int128 a, unsigned __int128 b) const { return a + b; }
};

// y of 8 inputs (one 16-byte vector of x and of gamma)
__device__ __forceinline__ u32x4 rms_scale8(u32x4 xv, u32x4 gv, float r) {
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float lo = (h2f(xv[e] & 0xFFFFu) * r) * h2f(gv[e] & 0xFFFFu);
        float hi = (h2f(xv[e] >> 16) * r) * h2f(gv[e] >> 16);
        // keep the fp32 product: the backend would otherwise form one
        // mixed-precision multiply rounding straight to FP16
        asm("" : "+v"(lo), "+v"(hi));
        out[e] = (uint32_t)f2h(lo) | ((uint32_t)f2h(hi) << 16);
    }
    return out;
}

// Row held in registers (CH runs of 16 inputs per thread, THR threads per
// row), K <= 16 * THR * CH; y (FP16 [M, K]) is written too when asked for.
template <int THR, int CH>
__global__ __launch_bounds__(THR) void k_rmsnorm_quant_reg(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ gamma,
                                                          float eps, int M, int K,
                                                          int8_t* __restrict__ xq,
                                                          uint16_t* __restrict__ s_x,
                                                          int32_t* __restrict__ rowsum,
                                                          uint16_t* __restrict__ y_out) {
    constexpr int kNW = THR / kWave;
    __shared__ unsigned __int128 red_s[kNW];
    __shared__ unsigned red_u[kNW];
    __shared__ int red_i[kNW];
    const int m = blockIdx.x;
    const int U = gridDim.x / 16;
    const int u = m / 16, rr = m % 16;
    const int nchunk = K / 16;
    u32x4* out = reinterpret_cast<u32x4*>(xq);
    auto slot = [&](int c) {
        const int g = c / 8, s = (c / 4) % 2, j = c % 4;
        return ((size_t)g * U + u) * 128 + 64 * s + 16 * j + rr;
    };
    if (m >= M) {
        for (int c = threadIdx.x; c < nchunk; c += THR) out[slot(c)] = u32x4{0u, 0u, 0u, 0u};
        return;
    }
    const u32x4* xrow = reinterpret_cast<const u32x4*>(x + (size_t)m * K);
    const u32x4* grow = reinterpret_cast<const u32x4*>(gamma);
    u32x4* yrow = y_out ? reinterpret_cast<u32x4*>(y_out + (size_t)m * K) : nullptr;
    u32x4 v0[CH], v1[CH];
    unsigned __int128 S = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = threadIdx.x + THR * i;
        v0[i] = u32x4{0u, 0u, 0u, 0u};
        v1[i] = u32x4{0u, 0u, 0u, 0u};
        if (c < nchunk) {
            v0[i] = xrow[2 * c];
            v1[i] = xrow[2 * c + 1];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            S += square_fp16(v0[i][e] & 0xFFFFu) + square_fp16(v0[i][e] >> 16);
            S += square_fp16(v1[i][e] & 0xFFFFu) + square_fp16(v1[i][e] >> 16);
        }
    }
    S = block_reduce<unsigned __int128, SumU128, kNW>(S, red_s, SumU128{});
    const double s64 = (double)S * 0x1p-48;
    const float ms = (float)(s64 / (double)K);
    const float r = 1.0f / sqrtf(ms + eps);

    unsigned amax = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = threadIdx.x + THR * i;
        if (c < nchunk) {
            v0[i] = rms_scale8(v0[i], grow[2 * c], r);
            v1[i] = rms_scale8(v1[i], grow[2 * c + 1], r);
            if (yrow) {
                yrow[2 * c] = v0[i];
                yrow[2 * c + 1] = v1[i];
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            amax = max(amax, max(absmax_bits2(v0[i][e]), absmax_bits2(v1[i][e])));
    }
    amax = block_reduce<unsigned, MaxU, kNW>(amax, red_u, MaxU{});
    const uint16_t sbits = f2h(h2f(amax) / 127.0f);
    const float sf = h2f(sbits);

    int sum = 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int c = threadIdx.x + THR * i;
        if (c < nchunk) {
            u32x4 o = u32x4{0u, 0u, 0u, 0u};
            if (sf != 0.0f) {
                const uint32_t w[8] = {v0[i][0], v0[i][1], v0[i][2], v0[i][3],
                                       v1[i][0], v1[i][1], v1[i][2], v1[i][3]};
                uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t hb = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
                    const int q = quant_act1(hb, sf);
                    sum += q;
                    packed[e >> 2] |= (uint32_t)(q & 0xFF) << (8 * (e & 3));
                }
                o = u32x4{packed[0], packed[1], packed[2], packed[3]};
            }
            out[slot(c)] = o;
        }
    }
    if (rowsum) sum = block_reduce<int, SumI, kNW>(sum, red_i, SumI{});
    if (threadIdx.x == 0) {
        s_x[m] = sbits;
        if (rowsum) rowsum[m] = sum;
    }
}

// Split rows, for few rows: S workgroups share a row (grid Mp x S, the
// row's quads of 4 inputs split evenly, one quad per thread and step, so a
// thread's chain of exponentials and divisions stays short). Part 1 computes
// h for its share and writes its largest magnitude (FP16 bits) to the
// workspace, and the share-0 workgroup clears the row's tally; part 2 takes
// the row's maximum over the S shares, computes h again and writes the codes
// of its share (4 bytes of a 16-byte run slot per thread). The row sum is
// gathered without a separate pass: each part-2 workgroup adds (1 << 32) plus
// its share's sum biased by 128 per input to the row's 64-bit tally (one
// atomic per workgroup, each row's tally on its own 256-byte line, so rows do
// not queue on one line), and the workgroup that finds S - 1 shares already
// counted writes the row sum, the tally's low word less 128 I. Integer adds:
// exact in any order. h, codes, scale and row sum are the single-pass
// kernel's bit for bit.
constexpr int kTallyStride = 32;  // 64-bit words: 256 bytes per row
static_assert(255LL * QOQ_MAX_K < (1LL << 32), "the biased row tally must fit its low word");

__device__ __forceinline__ void split_range(int n, int S, int s, int& q0, int& q1) {
    q0 = (int)((int64_t)n * s / S);
    q1 = (int)((int64_t)n * (s + 1) / S);
}

// h of 4 inputs: two words of gate and two of up
__device__ __forceinline__ uint2 silu_mul4(uint2 g, uint2 u) {
    return uint2{silu_mul1(g.x & 0xFFFFu, u.x & 0xFFFFu) | (silu_mul1(g.x >> 16, u.x >> 16) << 16),
                 silu_mul1(g.y & 0xFFFFu, u.y & 0xFFFFu) | (silu_mul1(g.y >> 16, u.y >> 16) << 16)};
}

__global__ __launch_bounds__(kThreads) void k_silu_max_part(const uint16_t* __restrict__ gu, int M,
                                                            int I, int S,
                                                            uint32_t* __restrict__ part_max,
                                                            unsigned long long* __restrict__ tally) {
    __shared__ unsigned red_u[kWaves];
    const int m = blockIdx.x / S, s = blockIdx.x % S;
    if (m >= M) return;
    int q0, q1;
    split_range(I / 4, S, s, q0, q1);
    const uint2* grow = reinterpret_cast<const uint2*>(gu + (size_t)m * 2 * I);
    const uint2* urow = reinterpret_cast<const uint2*>(gu + (size_t)m * 2 * I + I);
    unsigned amax = 0;
    for (int q = q0 + threadIdx.x; q < q1; q += kThreads) {
        const uint2 h = silu_mul4(grow[q], urow[q]);
        amax = max(amax, max(absmax_bits2(h.x), absmax_bits2(h.y)));
    }
    amax = block_reduce(amax, red_u, MaxU{});
    if (threadIdx.x == 0) {
        part_max[blockIdx.x] = amax;
        if (s == 0) tally[(size_t)m * kTallyStride] = 0ull;
    }
}

__global__ __launch_bounds__(kThreads) void k_silu_quant_part(const uint16_t* __restrict__ gu, int M,
                                                              int I, int S,
                                                              const uint32_t* __restrict__ part_max,
                                                              unsigned long long* __restrict__ tally,
                                                              int8_t* __restrict__ xq,
                                                              uint16_t* __restrict__ s_x,
                                                              int32_t* __restrict__ rowsum,
                                                              uint16_t* __restrict__ h_out) {
    __shared__ int red_i[kWaves];
    const int m = blockIdx.x / S, s = blockIdx.x % S;
    const int U = gridDim.x / S / 16;
    const int u = m / 16, r = m % 16;
    int q0, q1;
    split_range(I / 4, S, s, q0, q1);
    // byte offset of quad q's 4 codes: its run's 16-byte slot in the packed
    // tile order, plus 4 bytes per quad within the run
    auto dst = [&](int q) {
        const int c = q / 4, g = c / 8, sl = (c / 4) % 2, j = c % 4;
        return ((((size_t)g * U + u) * 128 + 64 * sl + 16 * j + r) << 4) + 4 * (q % 4);
    };
    if (m >= M) {
        for (int q = q0 + threadIdx.x; q < q1; q += kThreads)
            *reinterpret_cast<uint32_t*>(xq + dst(q)) = 0u;
        return;
    }
    const uint2* grow = reinterpret_cast<const uint2*>(gu + (size_t)m * 2 * I);
    const uint2* urow = reinterpret_cast<const uint2*>(gu + (size_t)m * 2 * I + I);
    uint2* hrow = h_out ? reinterpret_cast<uint2*>(h_out + (size_t)m * I) : nullptr;
    // h of the first quad is computed while the shares' maxima are read (each
    // wave reads them across its lanes)
    int q = q0 + threadIdx.x;
    uint2 h = uint2{0u, 0u};
    if (q < q1) h = silu_mul4(grow[q], urow[q]);
    unsigned amax = 0;
    for (int i = threadIdx.x % kWave; i < S; i += kWave) amax = max(amax, part_max[(size_t)m * S + i]);
    amax = wave_max_u(amax);
    const uint16_t sbits = f2h(h2f(amax) / 127.0f);
    const float sf = h2f(sbits);
    int sum = 0;
    // the last quad's codes are stored after the row-sum reduction, so its
    // barriers do not wait on them
    uint32_t held = 0u;
    int held_q = -1;
    for (; q < q1; q += kThreads) {
        if (q != q0 + (int)threadIdx.x) h = silu_mul4(grow[q], urow[q]);
        if (hrow) hrow[q] = h;
        uint32_t packed = 0u;
        if (sf != 0.0f) {
            const uint32_t w[4] = {h.x & 0xFFFFu, h.x >> 16, h.y & 0xFFFFu, h.y >> 16};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int qv = quant_act1(w[e], sf);
                sum += qv;
                packed |= (uint32_t)(qv & 0xFF) << (8 * e);
            }
        }
        if (held_q >= 0) *reinterpret_cast<uint32_t*>(xq + dst(held_q)) = held;
        held = packed;
        held_q = q;
    }
    if (rowsum) {
        sum = block_reduce(sum, red_i, SumI{});
        if (threadIdx.x == 0) {
            const unsigned long long add =
                (1ull << 32) + (unsigned long long)(uint32_t)(sum + 128 * 4 * (q1 - q0));
            const unsigned long long old = atomicAdd(&tally[(size_t)m * kTallyStride], add);
            if ((int)(old >> 32) == S - 1)
                rowsum[m] = (int32_t)((uint32_t)(old + add) - (uint32_t)(128 * I));
        }
    }
    if (held_q >= 0) *reinterpret_cast<uint32_t*>(xq + dst(held_q)) = held;
    if (threadIdx.x == 0 && s == 0) s_x[m] = sbits;
}

// Larger I: two passes over the gate_up row (the second recomputes h).
__global__ __launch_bounds__(kThreads) void k_silu_quant(const uint16_t* __restrict__ gu, int M,
                                                         int I, int8_t* __restrict__ xq,
                                                         uint16_t* __restrict__ s_x,
                                                         int32_t* __restrict__ rowsum,
                                                         uint16_t* __restrict__ h_out) {
    __shared__ unsigned red_u[kWaves];
    __shared__ int red_i[kWaves];
    const int m = blockIdx.x;
    const int U = gridDim.x / 16;
    const int u = m / 16, r = m % 16;
    const int nchunk = I / 16;
    uint4* out = reinterpret_cast<uint4*>(xq);
    auto slot = [&](int c) {
        const int g = c / 8, s = (c / 4) % 2, j = c % 4;
        return ((size_t)g * U + u) * 128 + 64 * s + 16 * j + r;
    };
    if (m >= M) {
        for (int c = threadIdx.x; c < nchunk; c += kThreads) out[slot(c)] = make_uint4(0, 0, 0, 0);
        return;
    }
    const u32x4* grow = reinterpret_cast<const u32x4*>(gu + (size_t)m * 2 * I);
    const u32x4* urow = reinterpret_cast<const u32x4*>(gu + (size_t)m * 2 * I + I);
    u32x4* hrow = h_out ? reinterpret_cast<u32x4*>(h_out + (size_t)m * I) : nullptr;
    unsigned amax = 0;
    for (int i = threadIdx.x; i < I / 8; i += kThreads) {
        const u32x4 h = silu_mul8(grow[i], urow[i]);
        if (hrow) hrow[i] = h;
#pragma unroll
        for (int e = 0; e < 4; ++e) amax = max(amax, absmax_bits2(h[e]));
    }
    amax = block_reduce(amax, red_u, MaxU{});
    const uint16_t sbits = f2h(h2f(amax) / 127.0f);
    const float sf = h2f(sbits);
    int sum = 0;
    for (int c = threadIdx.x; c < nchunk; c += kThreads) {
        uint4 o = make_uint4(0, 0, 0, 0);
        if (sf != 0.0f) {
            const u32x4 h0 = silu_mul8(grow[2 * c], urow[2 * c]);
            const u32x4 h1 = silu_mul8(grow[2 * c + 1], urow[2 * c + 1]);
            const uint32_t w[8] = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
            uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t hb = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
                const int q = quant_act1(hb, sf);
                sum += q;
                packed[e >> 2] |= (uint32_t)(q & 0xFF) << (8 * (e & 3));
            }
            o = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        }
        out[slot(c)] = o;
    }
    if (rowsum) sum = block_reduce(sum, red_i, SumI{});
    if (threadIdx.x == 0) {
        s_x[m] = sbits;
        if (rowsum) rowsum[m] = sum;
    }
}

// W8A8 sibling: per-channel symmetric INT8 ("QServe Guide: W4A8KV4
// Quantization for LLM Serving", "The Problem" item 2, with the per-channel
// symmetric scaling of "Deep Dive" part 1 at 8 bits): s_c = f16(max|W|/127),
// q = clamp(round(W / s_c), -128, 127). One workgroup per output channel.
__global__ __launch_bounds__(kThreads) void k_quantize_weights_w8(const uint16_t* __restrict__ w,
                                                                  int K, int8_t* __restrict__ q,
                                                                  uint16_t* __restrict__ s_c) {
    __shared__ unsigned red_u[kWaves];
    const size_t n = blockIdx.x;
    const uint4* rowv = reinterpret_cast<const uint4*>(w + n * (size_t)K);
    const int nvec = K / 8;

    unsigned amax = 0;
    for (int i = threadIdx.x; i < nvec; i += kThreads) {
        const uint4 v = rowv[i];
        amax = max(amax, max(max(absmax_bits2(v.x), absmax_bits2(v.y)),
                             max(absmax_bits2(v.z), absmax_bits2(v.w))));
    }
    amax = block_reduce(amax, red_u, MaxU{});
    const uint16_t scbits = f2h(h2f(amax) / 127.0f);
    const float scf = h2f(scbits);
    if (threadIdx.x == 0) s_c[n] = scbits;

    uint2* out = reinterpret_cast<uint2*>(q + n * (size_t)K);
    for (int i = threadIdx.x; i < nvec; i += kThreads) {
        uint2 o = {0u, 0u};
        if (scf != 0.0f) {
            const uint4 v = rowv[i];
            const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
            uint32_t packed[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                packed[e >> 2] |= (uint32_t)(quant_act1((e & 1) ? (ws[e >> 1] >> 16)
                                                                : (ws[e >> 1] & 0xFFFFu),
                                                        scf) & 0xFF)
                                  << (8 * (e & 3));
            o = make_uint2(packed[0], packed[1]);
        }
        out[i] = o;
    }
}

}  // namespace

void launch_silu_mul_quantize_act(const uint16_t* gate_up, int64_t M, int64_t I, int8_t* xq,
                                  uint16_t* s_x, int32_t* rowsum, uint16_t* h,
                                  hipStream_t stream) {
    const unsigned mp = (unsigned)((M + 15) / 16 * 16);
    const int64_t runs = I / 16;
#define QOQ_SQ(THRV, CHV)                                                                     \
    hipLaunchKernelGGL((k_silu_quant_reg<THRV, CHV>), dim3(mp), dim3(THRV), 0, stream, gate_up, \
                       (int)M, (int)I, xq, s_x, rowsum, h)
    if (runs <= 256) QOQ_SQ(256, 1);
    else if (runs <= 512) QOQ_SQ(256, 2);
    else if (runs <= 1024) QOQ_SQ(1024, 1);
    else if (runs <= 2048) QOQ_SQ(1024, 2);
    else
        hipLaunchKernelGGL(k_silu_quant, dim3(mp), dim3(kThreads), 0, stream, gate_up, (int)M,
                           (int)I, xq, s_x, rowsum, h);
#undef QOQ_SQ
}

void launch_rmsnorm_quantize_act(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M,
                                 int64_t K, int8_t* xq, uint16_t* s_x, int32_t* rowsum,
                                 uint16_t* y, hipStream_t stream) {
    const unsigned mp = (unsigned)((M + 15) / 16 * 16);
    const int64_t runs = K / 16;
#define QOQ_RQ(THRV, CHV)                                                                      \
    hipLaunchKernelGGL((k_rmsnorm_quant_reg<THRV, CHV>), dim3(mp), dim3(THRV), 0, stream, x,      \
                       gamma, eps, (int)M, (int)K, xq, s_x, rowsum, y)
    if (runs <= 256) QOQ_RQ(256, 1);
    else if (runs <= 512) QOQ_RQ(256, 2);
    else if (runs <= 1024) QOQ_RQ(1024, 1);
    else QOQ_RQ(1024, 2);  // K <= 32768, checked by the caller
#undef QOQ_RQ
}

// Shares per row of the split path: about 512 workgroups in all, each share
// at least 1024 inputs (one quad per thread); 1 means the one-pass kernels
// are used. The split pays its second launch back only where the one-pass
// kernel leaves most compute units idle (at most 32 rows) and its threads
// carry long chains (rows of 12288 inputs or more).
int64_t silu_split_shares(int64_t M, int64_t I) {
    const int64_t mp = (M + 15) / 16 * 16;
    if (M <= 0 || mp > 32 || I < 12288) return 1;
    return std::max<int64_t>(1, std::min<int64_t>((512 + mp - 1) / mp, I / 1024));
}

// Workspace of the split path: the shares' maxima, then one 256-byte line
// per row for its tally.
static int64_t silu_tally_offset(int64_t mp, int64_t S) { return (mp * S * 4 + 255) / 256 * 256; }

int64_t silu_mul_workspace_bytes(int64_t M, int64_t I) {
    const int64_t S = silu_split_shares(M, I);
    const int64_t mp = (M + 15) / 16 * 16;
    return S > 1 ? silu_tally_offset(mp, S) + mp * kTallyStride * 8 : 0;
}

void launch_silu_mul_quantize_act_ws(const uint16_t* gate_up, int64_t M, int64_t I, int8_t* xq,
                                     uint16_t* s_x, int32_t* rowsum, uint16_t* h, void* ws,
                                     hipStream_t stream) {
    const int64_t S = silu_split_shares(M, I);
    if (S <= 1 || !ws) {
        launch_silu_mul_quantize_act(gate_up, M, I, xq, s_x, rowsum, h, stream);
        return;
    }
    const unsigned mp = (unsigned)((M + 15) / 16 * 16);
    uint32_t* part = static_cast<uint32_t*>(ws);
    auto* tally = reinterpret_cast<unsigned long long*>(static_cast<char*>(ws) +
                                                        silu_tally_offset(mp, S));
    hipLaunchKernelGGL(k_silu_max_part, dim3(mp * (unsigned)S), dim3(kThreads), 0, stream, gate_up,
                       (int)M, (int)I, (int)S, part, tally);
    hipLaunchKernelGGL(k_silu_quant_part, dim3(mp * (unsigned)S), dim3(kThreads), 0, stream, gate_up,
                       (int)M, (int)I, (int)S, part, tally, xq, s_x, rowsum, h);
}

void launch_quantize_weights_w8(const uint16_t* w, int64_t N, int64_t K, int8_t* q, uint16_t* s_c,
                                hipStream_t stream) {
    hipLaunchKernelGGL(k_quantize_weights_w8, dim3((unsigned)N), dim3(kThreads), 0, stream, w,
                       (int)K, q, s_c);
}

// Rows from which the one-wave-per-row kernel is used (K <= 16384). Measured
// over the benchmark layers: at M >= 1024 it was 2-30% faster than one
// workgroup per row; at M <= 256 it was 30-95% slower (each compute unit then
// carries four rows' loads, and few compute units are busy).
constexpr int64_t kQuantWaveRows = 1024;

void launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, uint16_t* s_x,
                         int32_t* rowsum, hipStream_t stream) {
    const unsigned mp = (unsigned)((M + 15) / 16 * 16);
    const int64_t runs = K / 16;  // 16-input runs per row
#define QOQ_REG(THRV, CHV)                                                                    \
    hipLaunchKernelGGL((k_quantize_act_reg<THRV, CHV>), dim3(mp), dim3(THRV), 0, stream, x,      \
                       (int)M, (int)K, xq, s_x, rowsum)
#define QOQ_WAVE(CHV)                                                                         \
    hipLaunchKernelGGL((k_quantize_act_wave<CHV>), dim3(mp / 4), dim3(256), 0, stream, x, (int)M, \
                       (int)K, (int)mp, xq, s_x, rowsum)
    if (M >= kQuantWaveRows && runs <= 16 * kWave) {
        if (runs <= 2 * kWave) QOQ_WAVE(2);
        else if (runs <= 4 * kWave) QOQ_WAVE(4);
        else if (runs <= 8 * kWave) QOQ_WAVE(8);
        else QOQ_WAVE(16);
        return;
    }
#undef QOQ_WAVE
    // One or two 16-input runs per thread: 256 threads per row up to K = 8192,
    // then 1024 (more loads in flight per row, few registers per thread).
    if (runs <= 256) QOQ_REG(256, 1);
    else if (runs <= 512) QOQ_REG(256, 2);
    else if (runs <= 1024) QOQ_REG(1024, 1);
    else if (runs <= 2048) QOQ_REG(1024, 2);
    else
        hipLaunchKernelGGL(k_quantize_act, dim3(mp), dim3(kThreads), 0, stream, x, (int)M, (int)K,
                           xq, s_x, rowsum);
#undef QOQ_REG
}

void launch_quantize_weights(int mode, const uint16_t* w, int64_t N, int64_t K, uint8_t* q,
                             uint16_t* s_c, uint8_t* s_g, uint8_t* z, hipStream_t stream) {
    if (mode == 0)
        hipLaunchKernelGGL(k_quantize_weights_g128, dim3((unsigned)N), dim3(kThreads), 0, stream, w,
                           (int)K, q, s_c, s_g, z);
    else
        hipLaunchKernelGGL(k_quantize_weights_pc, dim3((unsigned)N), dim3(kThreads), 0, stream, w,
                           (int)K, q, s_c, z);
}

}  // namespace qoq
