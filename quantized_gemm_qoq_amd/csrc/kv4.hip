// kv4.hip -- KV4 decode attention with SmoothAttention, for gfx950.
//
// SmoothAttention ("QServe: Low Bit Width Does Not Guarantee High Throughput",
// section 4, the SmoothAttention paragraph; "QServe Guide: W4A8KV4
// Quantization for LLM Serving", part 3): a per-channel scale lambda moves key
// outliers into the queries, K' = K / lambda and Q' = Q * lambda, so that
// Q' K'^T = Q K^T; lambda = max|K|^alpha with alpha = 0.5 over calibration
// keys, here per (KV head, channel) and stored as FP16. Keys (after smoothing)
// and values are cached as 4-bit codes, one asymmetric range per (token, head)
// vector with an FP16 scale and a UINT4 zero, so that the decode attention
// streams a quarter of the FP16 cache ("QServe: Low Bit Width ...", section 3,
// judgment C: the KV4 gain needs the attention kernel's support).
//
// Cache layouts (d = 128, two codes per byte, channel 2j in the low nibble of
// byte j and 2j + 1 in the high nibble):
//   kq [B][H][Tcap][64]          token-major: one token's key is 64 contiguous bytes
//   vq [B][H][Tcap/16][64][16]   blocks of 16 tokens: byte j of the 16 tokens of a
//                                block are 16 contiguous bytes
//   ks, vs [B][H][Tcap] FP16 scales; kz, vz [B][H][Tcap] zeros (0..15)
//
// The decode kernel keeps the codes' dequantization out of its inner loops,
// the way the W4A8 GEMM keeps the zero point out of its: with k^ = s (c - z),
//   q' . k^ = s (q' . c - z sum(q')),   sum_t w_t v^_t = sum_t (w_t s_t) c_t - sum_t w_t s_t z_t
// so the codes c are converted to FP16 integers and multiplied as they are
// (QK on the FP16 matrix cores with FP32 accumulation, the FP16 QK of the
// pages; SV in FP32 on the vector units), and each token's scale and zero are
// applied once.
#include <math.h>

#include <algorithm>

#include "qoq_device.hpp"
#include "qoq_launch.hpp"

namespace qoq {
namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kD = 128;        // head dimension
constexpr int kKvThreads = 256;
constexpr int kAttnWaves = 4;  // waves per attention workgroup

// ---------------------------------------------------------------------------
// lambda[h, j] = f16(sqrt(max_t |k[t, h, j]|)), 1 where the maximum is 0.
// One workgroup of 16 waves per 64 consecutive (head, channel) indices: lane l
// of a wave reads the 8 channels 8 (l % 8) .. +7 (one 16-byte load) of token
// 8 w + l / 8 + 128 s at step s, so every step of the workgroup covers 128
// tokens with 128-byte runs; the magnitudes are maximised on their FP16 bit
// patterns (which order like the values), across the token lanes of a wave
// with shuffles and across the waves in LDS.
constexpr int kSmoothWaves = 16;
__global__ __launch_bounds__(kSmoothWaves * kWave) void k_kv4_smooth_scales(
    const uint16_t* __restrict__ k, int T, int H, uint16_t* __restrict__ lambda) {
    __shared__ uint32_t part[kSmoothWaves][64];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int c8 = lane % 8;
    const int i0 = blockIdx.x * 64 + c8 * 8;  // first (head, channel) index of this lane
    const size_t row = (size_t)H * kD;         // elements per token
    uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int t = wave * 8 + lane / 8; t < T; t += 8 * kSmoothWaves) {
        const uint4 v = *reinterpret_cast<const uint4*>(k + (size_t)t * row + i0);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            m[2 * q] = max(m[2 * q], w[q] & 0x7FFFu);
            m[2 * q + 1] = max(m[2 * q + 1], (w[q] >> 16) & 0x7FFFu);
        }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int o = 8; o < kWave; o <<= 1) m[q] = max(m[q], (uint32_t)__shfl_xor((int)m[q], o, kWave));
    if (lane < 8)
#pragma unroll
        for (int q = 0; q < 8; ++q) part[wave][c8 * 8 + q] = m[q];
    __syncthreads();
    if (threadIdx.x < 64) {
        uint32_t mx = 0;
#pragma unroll
        for (int w2 = 0; w2 < kSmoothWaves; ++w2) mx = max(mx, part[w2][threadIdx.x]);
        const float mf = h2f(mx);
        lambda[blockIdx.x * 64 + threadIdx.x] = mf > 0.0f ? f2h(sqrtf(mf)) : f2h(1.0f);
    }
}

// ---------------------------------------------------------------------------
// Append T tokens at positions t0 .. t0+T-1.
//
// Quantization of one key or value vector held by a row of 16 lanes, eight
// channels per lane (8g .. 8g+7 in lane g of the row): the range includes 0,
// s = f16((max - min) / 15), z = clamp(rne(-min / s), 0, 15), codes
// clamp(rne(x / s) + z, 0, 15); returns the lane's four code bytes, byte p
// holding channel 8g + 2p in its low and 8g + 2p + 1 in its high nibble.
__device__ __forceinline__ uint32_t kv4_quant_row8(const float (&x)[8], uint16_t& sbits, int& zz) {
    float mn = 0.0f, mx = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        mn = fminf(mn, x[e]);
        mx = fmaxf(mx, x[e]);
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o, 16));
        mx = fmaxf(mx, __shfl_xor(mx, o, 16));
    }
    sbits = f2h((mx - mn) / 15.0f);
    const float sf = h2f(sbits);
    zz = 0;
    uint32_t w = 0;
    if (sf != 0.0f) {
        zz = (int)fminf(fmaxf(rintf(-mn / sf), 0.0f), 15.0f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = min(15, max(0, (int)rintf(x[e] / sf) + zz));
            w |= (uint32_t)c << (4 * e);
        }
    }
    return w;
}

// One wave per (b, h, 16-token block of the cache) that the appended tokens
// touch, in four steps of four tokens: lane l takes token 4q + l/16 of step q
// and channels 8(l%16) .. +7, one 16-byte load per tensor, so each load
// instruction moves 1 KB and the per-token reductions stay inside a row of
// 16 lanes. Key codes leave as 4 bytes per lane (a token's 64-byte row per
// row of lanes); value codes are gathered in a 1 KB LDS slice of the wave in
// the value layout (channel pair major, 16 tokens per pair) and leave as one
// 16-byte slot per lane. A block that the append covers only in part keeps
// its other tokens' value codes (its slots are read into LDS first).
__global__ __launch_bounds__(kKvThreads) void k_kv4_append(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ lambda, int B, int T, int H, int Tcap, int t0, int blk0, int nblk,
    uint8_t* __restrict__ kq, uint16_t* __restrict__ ks, uint8_t* __restrict__ kz,
    uint8_t* __restrict__ vq, uint16_t* __restrict__ vs, uint8_t* __restrict__ vz) {
    __shared__ u32x4 vt[kKvThreads / kWave][kWave];
    const int lane = threadIdx.x % kWave;
    const int wv = threadIdx.x / kWave;
    const int64_t item = (int64_t)blockIdx.x * (kKvThreads / kWave) + wv;
    if (item >= (int64_t)B * H * nblk) return;  // the whole wave
    const int cb = blk0 + (int)(item % nblk);
    const int h = (int)((item / nblk) % H);
    const int b = (int)(item / ((int64_t)nblk * H));
    const int lo = max(16 * cb, t0), hi = min(16 * cb + 16, t0 + T);  // appended tokens of the block
    const size_t row0 = ((size_t)b * H + h) * Tcap + 16 * cb;        // cache row of the block's token 0
    const int g = lane % 16, r = lane / 16;

    const u32x4 lw = *reinterpret_cast<const u32x4*>(lambda + (size_t)h * kD + 8 * g);
    u32x4 kin[4], vin[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int t = min(max(16 * cb + 4 * q + r, lo), hi - 1) - t0;  // clamped: outside tokens unused
        const size_t src = (((size_t)b * T + t) * H + h) * kD + 8 * g;  // [B][T][H][d]
        kin[q] = *reinterpret_cast<const u32x4*>(k + src);
        vin[q] = *reinterpret_cast<const u32x4*>(v + src);
    }
    const size_t blk = ((size_t)b * H + h) * (Tcap / 16) + cb;
    u32x4* vslot = reinterpret_cast<u32x4*>(vq + blk * 1024) + lane;  // channel pair `lane`, 16 tokens
    uint8_t* vtb = reinterpret_cast<uint8_t*>(vt[wv]);
    if (lo > 16 * cb || hi < 16 * cb + 16) vt[wv][lane] = *vslot;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = 4 * q + r;
        const bool in = 16 * cb + i >= lo && 16 * cb + i < hi;
        float x[8];
        uint16_t sb;
        int zz;
        // keys, smoothed
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t kw = kin[q][e / 2] >> (16 * (e % 2)), lwe = lw[e / 2] >> (16 * (e % 2));
            x[e] = h2f(kw & 0xFFFFu) / h2f(lwe & 0xFFFFu);
        }
        uint32_t w = kv4_quant_row8(x, sb, zz);  // byte p: channels 8g + 2p (low), 8g + 2p + 1
        if (in) {
            *reinterpret_cast<uint32_t*>(kq + (row0 + i) * 64 + 4 * g) = w;
            if (g == 0) {
                ks[row0 + i] = sb;
                kz[row0 + i] = (uint8_t)zz;
            }
        }
        // values
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = h2f((vin[q][e / 2] >> (16 * (e % 2))) & 0xFFFFu);
        w = kv4_quant_row8(x, sb, zz);
        if (in) {
#pragma unroll
            for (int p = 0; p < 4; ++p)
                vtb[(4 * g + p) * 16 + i] = (uint8_t)(w >> (8 * p));
            if (g == 0) {
                vs[row0 + i] = sb;
                vz[row0 + i] = (uint8_t)zz;
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
    *vslot = vt[wv][lane];
}

// ---------------------------------------------------------------------------
// Decode attention, part 1: one workgroup per (b, KV head h, chunk of C
// tokens) for all G query heads of the group; wave w takes C/4 of the chunk's
// tokens in steps of 32, the loads of a step issued while the step before is
// computed, with an online softmax across steps. Scores are kept in log2
// units (the 1/sqrt(128) and log2(e) factors folded into s_k), p = 2^(s - m).
// Both contractions run on v_mfma_f32_16x16x32_f16 (16 x 16 output, K = 32):
//   Key codes enter the matrix cores as FP16 subnormals: the bit pattern c is
//   the value c 2^-24, exact, so a code needs only a mask and a shift; the
//   2^24 is folded into the scales, and the queries are scaled by a power of
//   two so that the largest of a row lies in [2^14, 2^15). The K order of each
//   lane's 8 elements is permuted to what the masks give, and the queries use
//   the same order. Value codes are normal FP16 integers (1024 + c - 1024):
//   with the much smaller weights as the other operand, subnormal codes lose
//   bits of the products on the matrix cores.
//   Rows: query g sits on MFMA row 4 j + v (j = (g / NV) 4 / GR, v = g % NV,
//   GR = min(G, 4) row groups of NV = G / GR queries), so that every lane of a
//   row group holds its queries' results in registers v < NV and the softmax
//   work is not repeated on padding rows.
//   Scores: S[g][t] = q'_g . c_t for 16 tokens is four MFMAs with the queries as
//   A and the key codes as B. Lane l reads 16 bytes of token l % 16 (channels
//   32(l/16) .. +31: the four lanes of a token cover its 64 bytes, the wave
//   reads 1 KB in one instruction). s = s_k (S - z_k sum q').
//   Values: with w = p s_v, O[g][ch] = sum_t w_t c_t[ch] is P (16 x 32 tokens)
//   times the codes (32 tokens x 16 channels) per MFMA. The weights are scaled
//   by 2^E and split as w 2^E = hi + lo, both FP16 (hi: w 2^E cut to 11
//   significant bits, lo: the remainder rounded toward zero); two MFMAs with
//   exact products carry w to about 22 bits; each step is summed from zero on
//   the matrix cores and added to FP32 running sums. E only decreases,
//   from the step maxima of s_v, so that max(s_v) 2^E < 2^7; the running
//   maximum m moves only when a step's maximum exceeds it by more than 8, so
//   p <= 2^8 and w 2^E < 2^15 stays finite in FP16. hi and lo pass through LDS
//   to the A layout (row 4 j + v, 8 tokens per lane); lane l reads bytes j =
//   16m + l % 16 of the same 8 tokens from one 16-token value block (low
//   nibbles: channel 2j, high: 2j + 1) for m = 0..3: eight output blocks of 16
//   channels. sum_t w_t z_t is subtracted at the end.
// The four waves' states are merged through LDS; the chunk's (max, sum,
// output) go to the workspace for part 2, or, when the sequence is a single
// chunk, the normalised FP16 output is written directly and part 2 is skipped.
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4t __attribute__((ext_vector_type(4)));

constexpr float kLog2eRsqrtD = 0.12751743082459868f;  // log2(e) / sqrt(128)
constexpr float kLazyMax = 8.0f;  // log2 units the running maximum may lag
constexpr int kPrefetch = 1;      // steps whose loads are in flight ahead of the one computed

// One DPP move within rows of 16 lanes.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}
// Maximum and sum over the 16 lanes of a row (the same value on all of them):
// swap neighbours, swap pairs, mirror the half rows, mirror the row.
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));
    x = fmaxf(x, dpp_f<0x4E>(x));
    x = fmaxf(x, dpp_f<0x141>(x));
    return fmaxf(x, dpp_f<0x140>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x141>(x);
    return x + dpp_f<0x140>(x);
}

__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(127 + e) << 23); }

// One 32-bit word of key codes (bytes i = 0..3: channels 2i low, 2i + 1 high)
// as an 8-element FP16 operand in channel order 0, 4, 2, 6, 1, 5, 3, 7.
__device__ __forceinline__ half8v key_word_f16(uint32_t w) {
    const uint32_t m = 0x000F000Fu;
    return __builtin_bit_cast(half8v, u32x4{w & m, (w >> 8) & m, (w >> 4) & m, (w >> 12) & m});
}
// Bytes of 8 tokens (x0: tokens 0..3, x1: 4..7) -> two 8-element FP16
// operands in token order: the low nibbles c and the high nibbles as 16 c, both
// as normal FP16 integers (bytes [n, 0x64] are 1024 + n; 1024 is subtracted).
__device__ __forceinline__ void value_bytes_f16(uint32_t x0, uint32_t x1, half8v& lo, half8v& hi) {
    const uint32_t k64 = 0x64646464u;
    const half2v off = half2v{(_Float16)1024.0f, (_Float16)1024.0f};
    auto cv = [&](uint32_t nib, uint32_t sel) {
        return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, __builtin_amdgcn_perm(k64, nib, sel)) - off);
    };
    const uint32_t l0 = x0 & 0x0F0F0F0Fu, l1 = x1 & 0x0F0F0F0Fu;
    const uint32_t h0 = x0 & 0xF0F0F0F0u, h1 = x1 & 0xF0F0F0F0u;
    lo = __builtin_bit_cast(half8v, u32x4{cv(l0, 0x04010400u), cv(l0, 0x04030402u), cv(l1, 0x04010400u),
                                          cv(l1, 0x04030402u)});
    hi = __builtin_bit_cast(half8v, u32x4{cv(h0, 0x04010400u), cv(h0, 0x04030402u), cv(h1, 0x04010400u),
                                          cv(h1, 0x04030402u)});
}

template <int G>
__global__ __launch_bounds__(kAttnWaves * 64) __attribute__((amdgpu_waves_per_eu(3))) void k_kv4_attn_chunk(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ lambda,
    const uint8_t* __restrict__ kq, const uint16_t* __restrict__ ks, const uint8_t* __restrict__ kz,
    const uint8_t* __restrict__ vq, const uint16_t* __restrict__ vs, const uint8_t* __restrict__ vz,
    const int32_t* __restrict__ lens, int H, int Tcap, int C, int nchunks,
    float* __restrict__ part_o, float* __restrict__ part_ml, uint16_t* __restrict__ out) {
    constexpr int GR = G < 4 ? G : 4;  // row groups that hold queries
    constexpr int NV = G / GR;         // queries per row group
    constexpr int JS = 4 / GR;         // stride between those row groups
    __shared__ __align__(16) uint16_t wh_lds[kAttnWaves][16][32];  // hi parts of w 2^E, by row
    __shared__ __align__(16) uint16_t wl_lds[kAttnWaves][16][32];  // lo parts
    __shared__ float qs_lds[kAttnWaves][16], qf_lds[kAttnWaves][16];
    __shared__ float mrg_m[kAttnWaves][G], mrg_l[kAttnWaves][G], mrg_z[kAttnWaves][G];
    __shared__ float mrg_o[kAttnWaves][G][kD];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar branches
    const int chunk = blockIdx.x % nchunks;
    const int bh = blockIdx.x / nchunks;  // b * H + h
    const int h = bh % H, b = bh / H;
    const int Hq = H * G;
    const int len = min(max(lens[b], 0), Tcap);
    const int c0 = chunk * C;
    // Part 2 reads a chunk's record only when the chunk starts before len; a
    // sequence of length 0 that is one chunk gets its zeros here.
    if (c0 >= len) {
        if (nchunks == 1)
            for (int g = wave; g < G; g += kAttnWaves)
                reinterpret_cast<uint32_t*>(out + ((size_t)b * Hq + h * G + g) * kD)[lane] = 0u;
        return;
    }

    const size_t rowbase = (size_t)bh * Tcap;
    const int wstart = c0 + wave * (C / kAttnWaves);  // a multiple of 32
    const int wend = min(wstart + C / kAttnWaves, len);
    const int ntotal = wend > wstart ? (wend - wstart + 31) / 32 : 0;  // steps of this wave
    const int r16 = lane % 16, jg = lane / 16;
    const uint8_t* vbase = vq + (size_t)bh * (Tcap / 16) * 1024;
    const int vlast = (wend - 1) / 16;  // last value block with a valid token
    const bool lane_q = jg % JS == 0;   // rows 4 jg + v (v < NV) of this lane are queries
    const int gbase = (jg / JS) * NV;   // the query on row 4 jg

    // One step: 32 tokens.
    struct StepData {
        u32x4 kb[2];  // key bytes of token 16 hs + r16, channels 32 jg ..
        uint2 vb[4];  // value bytes j = 16m + r16 of tokens 8 jg .. +7
        // raw scales and zeros: converted only when the step is computed, so
        // that no use waits for a load of the step ahead
        uint16_t sk[2], sv[2];
        uint8_t zk[2], zv[2];
    };
    auto load_step = [&](int st, StepData& d) {
        const int bstart = wstart + 32 * st;
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            const int t = min(bstart + 16 * hs + r16, wend - 1);  // masked tokens read a valid row
            d.kb[hs] = *reinterpret_cast<const u32x4*>(kq + (rowbase + t) * 64 + 16 * jg);
        }
        const int blk = min(bstart / 16 + jg / 2, vlast);
        const uint8_t* vp = vbase + (size_t)blk * 1024 + r16 * 16 + 8 * (jg % 2);
#pragma unroll
        for (int m = 0; m < 4; ++m) d.vb[m] = *reinterpret_cast<const uint2*>(vp + 256 * m);
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            const int t = min(bstart + 16 * hs + r16, wend - 1);
            d.sk[hs] = ks[rowbase + t];
            d.zk[hs] = kz[rowbase + t];
            d.sv[hs] = vs[rowbase + t];
            d.zv[hs] = vz[rowbase + t];
        }
    };
    StepData d[kPrefetch + 1];

    // ---- A operands of the scores: row r16 (zeros where it holds no query),
    // channels 32 jg + 8f + {0, 4, 2, 6, 1, 5, 3, 7}; q' = f16(q * lambda) from
    // an FP32 product (the barrier keeps the backend from forming one
    // mixed-precision multiply that rounds once), times 2^s_r per row so that
    // the row's largest |q'| 2^s_r lies in [2^14, 2^15) (s_r >= 0, exact): the
    // products with the subnormal codes then stay far above the smallest FP16
    // magnitudes, where the matrix cores lose bits of such products.
    half8v qa[4];
    {
        const int rj = r16 / 4, rv = r16 % 4;
        const bool row_q = rj % JS == 0 && rv < NV;
        const int rg = (rj / JS) * NV + rv;
        // all query and lambda loads in flight together (rows without a query
        // read row 0 and give zeros)
        const size_t qoff = ((size_t)b * Hq + h * G + (row_q ? rg : 0)) * kD + 32 * jg;
        u32x4 qw[4], lw[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            qw[f] = *reinterpret_cast<const u32x4*>(q + qoff + 8 * f);
            lw[f] = *reinterpret_cast<const u32x4*>(lambda + (size_t)h * kD + 32 * jg + 8 * f);
        }
        uint16_t e8[4][8];
        float qpart = 0.0f, qmax = 0.0f;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float pa = h2f(qw[f][e] & 0xFFFFu) * h2f(lw[f][e] & 0xFFFFu);
                float pb = h2f(qw[f][e] >> 16) * h2f(lw[f][e] >> 16);
                asm("" : "+v"(pa), "+v"(pb));
                e8[f][2 * e] = row_q ? f2h(pa) : (uint16_t)0;
                e8[f][2 * e + 1] = row_q ? f2h(pb) : (uint16_t)0;
                const float a = h2f(e8[f][2 * e]), c = h2f(e8[f][2 * e + 1]);
                qpart += a + c;
                qmax = fmaxf(qmax, fmaxf(fabsf(a), fabsf(c)));
            }
        }
        // sum(q') and max|q'| of row r16 over the four lanes of the row (jg = 0..3)
        qpart += __shfl_xor(qpart, 16, kWave);
        qpart += __shfl_xor(qpart, 32, kWave);
        qmax = fmaxf(qmax, __shfl_xor(qmax, 16, kWave));
        qmax = fmaxf(qmax, __shfl_xor(qmax, 32, kWave));
        const int srow = qmax > 0.0f ? max(0, 141 - (int)((__float_as_uint(qmax) >> 23) & 0xFF)) : 0;
        const float qscale = pow2f(srow);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            uint32_t e2[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) e2[e] = f2h(h2f(e8[f][e]) * qscale);
            qa[f] = __builtin_bit_cast(half8v, u32x4{e2[0] | (e2[4] << 16), e2[2] | (e2[6] << 16),
                                                     e2[1] | (e2[5] << 16), e2[3] | (e2[7] << 16)});
        }
        if (lane < 16) {
            qs_lds[wave][lane] = qpart;
            qf_lds[wave][lane] = pow2f(24 - srow);  // undoes 2^s_r and the codes' 2^-24
        }
    }
    __builtin_amdgcn_wave_barrier();
    float qsum[NV], qfac[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        qsum[v] = qs_lds[wave][4 * jg + v];
        qfac[v] = qf_lds[wave][4 * jg + v];
    }

    float mrun[NV], lp[NV], zp[NV];  // running maximum (log2 units), sum of p, sum of w z_v
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        mrun[v] = -INFINITY;
        lp[v] = zp[v] = 0.0f;
    }
    float acc[8][NV];  // output block 2m + n: channels 2(16m + r16) + n, rows 4 jg + v
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[i][v] = 0.0f;
    int ecur = 64;  // the exponent E the accumulators carry (64: none yet)

    auto compute_step = [&](int st, const StepData& d) {
        const int bstart = wstart + 32 * st;
        float sk[2], zk[2], sv[2], zv[2];
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            sk[hs] = h2f(d.sk[hs]) * kLog2eRsqrtD;
            zk[hs] = (float)d.zk[hs];
            sv[hs] = h2f(d.sv[hs]);
            zv[hs] = (float)d.zv[hs];
        }
        // ---- scores of 16 tokens per half step: lane l holds token l % 16
        float sc[2][NV];
        float bmx[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) bmx[v] = -INFINITY;
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            float4t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int f = 0; f < 4; ++f)
                s4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[f], key_word_f16(d.kb[hs][f]), s4, 0, 0, 0);
            const bool valid = bstart + 16 * hs + r16 < wend;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                sc[hs][v] = valid ? sk[hs] * __builtin_fmaf(-zk[hs], qsum[v], s4[v] * qfac[v]) : -INFINITY;
                bmx[v] = fmaxf(bmx[v], sc[hs][v]);
            }
        }
        float msv = row16_max(fmaxf(sv[0], sv[1]));
        // E: max(s_v) 2^E < 2^7 with s_v an FP16 value (at least 2^-24 when
        // not 0); the same on every lane, never increased
        const int ebits = __builtin_amdgcn_readfirstlane((int)((__float_as_uint(msv) >> 23) & 0xFF));
        const int enew = min(ecur, 133 - max(ebits, 103));
        bool need = enew != ecur;
        const float erescale = pow2f(enew - ecur);
        float rs[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            bmx[v] = row16_max(bmx[v]);  // finite: the step has a valid token
            const float mn = bmx[v] > mrun[v] + kLazyMax ? bmx[v] : mrun[v];
            const float r = __builtin_amdgcn_exp2f(mrun[v] - mn);  // 0 on the first step
            need |= mn != mrun[v];
            lp[v] *= r;
            zp[v] *= r;
            rs[v] = r * erescale;
            mrun[v] = mn;
        }
        ecur = enew;
        if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int v = 0; v < NV; ++v) acc[i][v] *= rs[v];
        }

        // ---- p = 2^(s - m); sums of p and of w z_v; w 2^E = hi + lo into LDS
        const float wscale = pow2f(enew);
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            const float svs = sv[hs] * wscale, svz = sv[hs] * zv[hs];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const float p = __builtin_amdgcn_exp2f(sc[hs][v] - mrun[v]);  // 0 for masked tokens
                lp[v] += p;
                zp[v] = __builtin_fmaf(p, svz, zp[v]);
                const float w = p * svs;
                const float whi = __uint_as_float(__float_as_uint(w) & 0xFFFFE000u);
                const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(whi, w - whi));
                wh_lds[wave][4 * jg + v][16 * hs + r16] = (uint16_t)pk;
                wl_lds[wave][4 * jg + v][16 * hs + r16] = (uint16_t)(pk >> 16);
            }
        }
        __builtin_amdgcn_wave_barrier();

        // ---- values: O += (hi + lo) x codes. Each step's products are summed
        // on the matrix cores from zero (the lo products first, so that their
        // small sum is the addend of the hi ones), then added to the running
        // sums in FP32 on the vector units: the matrix cores align their
        // addends to the largest one, which would cut the bits of a step's
        // contribution against a long running sum.
        const half8v ah = *reinterpret_cast<const half8v*>(&wh_lds[wave][r16][8 * jg]);
        const half8v al = *reinterpret_cast<const half8v*>(&wl_lds[wave][r16][8 * jg]);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            half8v blo, bhi;
            value_bytes_f16(d.vb[m].x, d.vb[m].y, blo, bhi);
            const float4t zero = {0.f, 0.f, 0.f, 0.f};
            float4t t0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, blo, zero, 0, 0, 0);
            float4t t1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bhi, zero, 0, 0, 0);
            t0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, blo, t0, 0, 0, 0);
            t1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bhi, t1, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                acc[2 * m][v] += t0[v];
                acc[2 * m + 1][v] += t1[v];
            }
        }
        __builtin_amdgcn_wave_barrier();  // the next step rewrites the LDS weights
    };

    // Loads run kPrefetch steps ahead of their use; a load beyond the last
    // step repeats the last step (cached, unused), so that the count of loads
    // in flight, and with it each wait, is the same at every step.
    if (ntotal > 0) {
#pragma unroll
        for (int i = 0; i < kPrefetch; ++i) load_step(min(i, ntotal - 1), d[i]);
        for (int st = 0;; st += kPrefetch + 1) {
#pragma unroll
            for (int ph = 0; ph <= kPrefetch; ++ph) {
                load_step(min(st + ph + kPrefetch, ntotal - 1), d[(ph + kPrefetch) % (kPrefetch + 1)]);
                compute_step(st + ph, d[ph]);
                if (st + ph + 1 >= ntotal) goto steps_done;
            }
        }
    }
steps_done:

    // ---- merge the waves' states; a wave without tokens has l = 0
    // undo 2^E (and the 16 of the high-nibble codes)
    const float unscale_lo = ntotal > 0 ? pow2f(-ecur) : 1.0f, unscale_hi = unscale_lo * 0.0625f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const float l = row16_sum(lp[v]), z = row16_sum(zp[v]);
        if (lane_q) {
            const int g = gbase + v;
            if (r16 == 0) {
                mrg_m[wave][g] = ntotal > 0 ? mrun[v] : -INFINITY;
                mrg_l[wave][g] = l;
                mrg_z[wave][g] = z;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                mrg_o[wave][g][2 * (16 * (i / 2) + r16) + (i % 2)] = acc[i][v] * (i % 2 ? unscale_hi : unscale_lo);
        }
    }
    __syncthreads();
    // wave w finishes query heads g = w, w + 4, ...; a sequence that is one
    // chunk writes its FP16 output here, otherwise the chunk's record for part 2
    for (int g = wave; g < G; g += kAttnWaves) {
        float M = -INFINITY;
        for (int w = 0; w < kAttnWaves; ++w)
            if (mrg_l[w][g] > 0.0f) M = fmaxf(M, mrg_m[w][g]);
        float L = 0.0f, Z = 0.0f, o0 = 0.0f, o1 = 0.0f;
        for (int w = 0; w < kAttnWaves; ++w) {
            const float e = mrg_l[w][g] > 0.0f ? __builtin_amdgcn_exp2f(mrg_m[w][g] - M) : 0.0f;
            L += e * mrg_l[w][g];
            Z += e * mrg_z[w][g];
            o0 += e * mrg_o[w][g][2 * lane];
            o1 += e * mrg_o[w][g][2 * lane + 1];
        }
        const size_t qrow = (size_t)b * Hq + h * G + g;
        if (nchunks == 1) {
            const float inv = 1.0f / L;  // L > 0: the chunk has a valid token
            reinterpret_cast<uint32_t*>(out + qrow * kD)[lane] =
                (uint32_t)f2h((o0 - Z) * inv) | ((uint32_t)f2h((o1 - Z) * inv) << 16);
        } else {
            const size_t rec = qrow * nchunks + chunk;
            part_o[rec * kD + 2 * lane] = o0 - Z;
            part_o[rec * kD + 2 * lane + 1] = o1 - Z;
            if (lane == 0) {
                part_ml[rec * 2] = M;
                part_ml[rec * 2 + 1] = L;
            }
        }
    }
}

// Part 2: one wave per (b, query head): combine the chunks that start before
// len[b]; o = sum_c 2^(M_c - M) O_c / sum_c 2^(M_c - M) L_c (maxima in log2
// units, M their maximum, taken as a running maximum), rounded to FP16 (a
// sequence of length 0 gives zeros).
__global__ __launch_bounds__(kKvThreads) void k_kv4_attn_combine(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ lens, int B, int Hq, int Tcap, int C, int nchunks,
    uint16_t* __restrict__ o) {
    const int lane = threadIdx.x % kWave;
    const int64_t w = (int64_t)blockIdx.x * (kKvThreads / kWave) + threadIdx.x / kWave;
    if (w >= (int64_t)B * Hq) return;
    const int b = (int)(w / Hq);
    const int len = min(max(lens[b], 0), Tcap);
    const int used = (len + C - 1) / C;
    // One pass with a running maximum; the records of four chunks are read
    // together, independently of len (chunks past it are read but not used),
    // so the loads of a batch overlap each other and the load of len.
    float M = -INFINITY, L = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int cb = 0; cb < nchunks; cb += 4) {
        float mc[4], lc[4];
        float2 oc[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const size_t rec = (size_t)w * nchunks + min(cb + k, nchunks - 1);
            mc[k] = part_ml[rec * 2];
            lc[k] = part_ml[rec * 2 + 1];
            oc[k] = *reinterpret_cast<const float2*>(part_o + rec * kD + 2 * lane);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (cb + k < used) {
                const float mn = fmaxf(M, mc[k]);
                const float r = __builtin_amdgcn_exp2f(M - mn);  // 0 for the first chunk
                const float e = __builtin_amdgcn_exp2f(mc[k] - mn);
                L = L * r + e * lc[k];
                o0 = o0 * r + e * oc[k].x;
                o1 = o1 * r + e * oc[k].y;
                M = mn;
            }
        }
        if (cb + 4 >= used) break;
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    reinterpret_cast<uint32_t*>(o + (size_t)w * kD)[lane] =
        (uint32_t)f2h(o0 * inv) | ((uint32_t)f2h(o1 * inv) << 16);
}

unsigned blocks_of(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

void launch_kv4_smooth_scales(const uint16_t* k, int64_t T, int64_t H, uint16_t* lambda,
                              hipStream_t stream) {
    hipLaunchKernelGGL(k_kv4_smooth_scales, dim3((unsigned)(H * kD / 64)), dim3(kSmoothWaves * kWave), 0,
                       stream, k, (int)T, (int)H, lambda);
}

void launch_kv4_append(const uint16_t* k, const uint16_t* v, const uint16_t* lambda, int64_t B,
                       int64_t T, int64_t H, int64_t Tcap, int64_t t0, uint8_t* kq, uint16_t* ks,
                       uint8_t* kz, uint8_t* vq, uint16_t* vs, uint8_t* vz, hipStream_t stream) {
    // the 16-token cache blocks the tokens t0 .. t0+T-1 fall in
    const int64_t blk0 = t0 / 16, nblk = (t0 + T - 1) / 16 - blk0 + 1;
    const int64_t items = B * H * nblk;
    hipLaunchKernelGGL(k_kv4_append, dim3(blocks_of(items, kKvThreads / kWave)), dim3(kKvThreads), 0,
                       stream, k, v, lambda, (int)B, (int)T, (int)H, (int)Tcap, (int)t0, (int)blk0,
                       (int)nblk, kq, ks, kz, vq, vs, vz);
}

// Chunk length: the sequence is cut into n = ceil(256 / (B H)) chunks (at
// least one workgroup per compute unit; one chunk when B H >= 256, which
// skips the combine kernel), each a multiple of 128 tokens so that every wave
// takes whole 32-token steps.

int64_t kv4_chunk(int64_t B, int64_t H, int64_t Tcap) {
    const int64_t bh = std::max<int64_t>(B * H, 1);
    const int64_t n = std::min<int64_t>((256 + bh - 1) / bh, std::max<int64_t>((Tcap + 127) / 128, 1));
    return std::max<int64_t>(((Tcap + n - 1) / n + 127) / 128 * 128, 128);
}

int64_t kv4_workspace_bytes(int64_t B, int64_t Hq, int64_t H, int64_t Tcap) {
    const int64_t n = (Tcap + kv4_chunk(B, H, Tcap) - 1) / kv4_chunk(B, H, Tcap);
    return B * Hq * n * (kD + 2) * 4;
}

void launch_kv4_decode_attention(const uint16_t* q, const uint16_t* lambda, const uint8_t* kq,
                                 const uint16_t* ks, const uint8_t* kz, const uint8_t* vq,
                                 const uint16_t* vs, const uint8_t* vz, const int32_t* lens,
                                 int64_t B, int64_t Hq, int64_t H, int64_t Tcap, uint16_t* o,
                                 void* ws, hipStream_t stream) {
    const int64_t C = kv4_chunk(B, H, Tcap);
    const int64_t n = (Tcap + C - 1) / C;
    float* part_o = static_cast<float*>(ws);
    float* part_ml = part_o + B * Hq * n * kD;
    const unsigned grid = (unsigned)(B * H * n);
    const int G = (int)(Hq / H);
#define QOQ_ATTN(GV)                                                                                 \
    hipLaunchKernelGGL((k_kv4_attn_chunk<GV>), dim3(grid), dim3(kAttnWaves * 64), 0, stream, q,     \
                       lambda, kq, ks, kz, vq, vs, vz, lens, (int)H, (int)Tcap, (int)C, (int)n, part_o, \
                       part_ml, o)
    if (G == 1) QOQ_ATTN(1);
    else if (G == 2) QOQ_ATTN(2);
    else if (G == 4) QOQ_ATTN(4);
    else QOQ_ATTN(8);
#undef QOQ_ATTN
    if (n == 1) return;  // part 1 wrote the output
    hipLaunchKernelGGL(k_kv4_attn_combine, dim3(blocks_of(B * Hq, kKvThreads / kWave)),
                       dim3(kKvThreads), 0, stream, part_o, part_ml, lens, (int)B, (int)Hq, (int)Tcap,
                       (int)C, (int)n, o);
}

}  // namespace qoq
