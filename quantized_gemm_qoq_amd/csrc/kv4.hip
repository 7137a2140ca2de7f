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
__global__ __launch_bounds__(kKvThreads) void k_kv4_smooth_scales(const uint16_t* __restrict__ k,
                                                                  int T, int H,
                                                                  uint16_t* __restrict__ lambda) {
    const int i = blockIdx.x * kKvThreads + threadIdx.x;  // h * kD + j
    if (i >= H * kD) return;
    unsigned mx = 0;  // magnitude bits of FP16 values order like the values
    for (int t = 0; t < T; ++t) mx = max(mx, (unsigned)(k[(size_t)t * H * kD + i] & 0x7FFFu));
    const float m = h2f(mx);
    lambda[i] = m > 0.0f ? f2h(sqrtf(m)) : f2h(1.0f);
}

// ---------------------------------------------------------------------------
// Append T tokens at positions t0 .. t0+T-1: one wave per (b, t, h) vector of
// the keys and one of the values; lane l handles channels 2l and 2l + 1.
__device__ __forceinline__ void kv4_quant_pair(float x0, float x1, int& c0, int& c1,
                                               uint16_t& sbits, int& zz) {
    const float mn = wave_min_f(fminf(0.0f, fminf(x0, x1)));
    const float mx = wave_max_f(fmaxf(0.0f, fmaxf(x0, x1)));
    sbits = f2h((mx - mn) / 15.0f);
    const float sf = h2f(sbits);
    zz = 0;
    c0 = c1 = 0;
    if (sf != 0.0f) {
        zz = (int)fminf(fmaxf(rintf(-mn / sf), 0.0f), 15.0f);
        c0 = min(15, max(0, (int)rintf(x0 / sf) + zz));
        c1 = min(15, max(0, (int)rintf(x1 / sf) + zz));
    }
}

__global__ __launch_bounds__(kKvThreads) void k_kv4_append(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ lambda, int B, int T, int H, int Tcap, int t0,
    uint8_t* __restrict__ kq, uint16_t* __restrict__ ks, uint8_t* __restrict__ kz,
    uint8_t* __restrict__ vq, uint16_t* __restrict__ vs, uint8_t* __restrict__ vz) {
    const int lane = threadIdx.x % kWave;
    const int64_t vec = (int64_t)blockIdx.x * (kKvThreads / kWave) + threadIdx.x / kWave;
    const int64_t total = (int64_t)B * T * H;
    if (vec >= total) return;
    const int h = (int)(vec % H);
    const int t = (int)((vec / H) % T);
    const int b = (int)(vec / ((int64_t)H * T));
    const size_t src = (size_t)vec * kD + 2 * lane;  // [B][T][H][d] is vec-major
    const int tc = t0 + t;
    const size_t row = ((size_t)b * H + h) * Tcap + tc;

    // keys, smoothed
    const uint32_t kw = *reinterpret_cast<const uint32_t*>(k + src);
    const uint32_t lw = *reinterpret_cast<const uint32_t*>(lambda + (size_t)h * kD + 2 * lane);
    int c0, c1, zz;
    uint16_t sb;
    kv4_quant_pair(h2f(kw & 0xFFFFu) / h2f(lw & 0xFFFFu), h2f(kw >> 16) / h2f(lw >> 16), c0, c1,
                   sb, zz);
    kq[row * 64 + lane] = (uint8_t)(c0 | (c1 << 4));
    if (lane == 0) {
        ks[row] = sb;
        kz[row] = (uint8_t)zz;
    }
    // values
    const uint32_t vw = *reinterpret_cast<const uint32_t*>(v + src);
    kv4_quant_pair(h2f(vw & 0xFFFFu), h2f(vw >> 16), c0, c1, sb, zz);
    const size_t blk = ((size_t)b * H + h) * (Tcap / 16) + tc / 16;
    vq[blk * 1024 + lane * 16 + tc % 16] = (uint8_t)(c0 | (c1 << 4));
    if (lane == 0) {
        vs[row] = sb;
        vz[row] = (uint8_t)zz;
    }
}

// ---------------------------------------------------------------------------
// Decode attention, part 1: one workgroup per (b, KV head h, chunk of C
// tokens) for all G query heads of the group; wave w takes C/4 of the chunk's
// tokens (at most 128) in steps of 16, in two passes.
//   Pass 1, scores on the matrix cores: S[g][t] = q'_g . c_t for 16 tokens is
//   four v_mfma_f32_16x16x32_f16 with the G queries as A (rows g, padded with
//   zeros to 16) and the raw codes as B. Lane l reads 16 bytes of token l % 16
//   (channels 32(l/16) .. +31, the four lanes of a token cover its 64 bytes,
//   the wave reads 1 KB in one instruction); operation f uses channels
//   32(l/16) + 8f .. +7 of A and B alike. Scores s = s_k (S - z_k sum q') /
//   sqrt(128) go to LDS, and the chunk maximum of each query is taken once.
//   Pass 2: p = exp(s - m) and u = p s_v per (query, token) into LDS; then lane
//   l owns channels 2l, 2l + 1 of the values and reads the 16-byte block of its
//   byte for each step's 16 tokens, acc += u * c, with sum(u z_v) subtracted
//   at the end. All key and value loads of a wave are issued at the start of
//   their pass.
// The four waves' states are merged through LDS; the chunk's (max, sum,
// output) go to the workspace for part 2.
constexpr int kMaxSteps = 8;  // 16-token steps per wave (C <= 512)

typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4t __attribute__((ext_vector_type(4)));

// Codes of one 32-bit word (8 channels of bytes j..j+3) as four FP16 pairs of
// exact integers 0..15, channel order.
__device__ __forceinline__ u32x4 codes8_to_f16(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    u32x4 out;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        // bytes [lo_b, 0, hi_b, 0] | 0x6400 in each half = 1024 + code
        const uint32_t sel = (uint32_t)b | (0x0Cu << 8) | ((uint32_t)(4 + b) << 16) | (0x0Cu << 24);
        const uint32_t p = __builtin_amdgcn_perm(hi, lo, sel) | 0x64006400u;
        const half2v hv = __builtin_bit_cast(half2v, p) - half2v{(_Float16)1024.0f, (_Float16)1024.0f};
        out[b] = __builtin_bit_cast(uint32_t, hv);
    }
    return out;
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

template <int G>
__global__ __launch_bounds__(kAttnWaves * 64) void k_kv4_attn_chunk(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ lambda,
    const uint8_t* __restrict__ kq, const uint16_t* __restrict__ ks, const uint8_t* __restrict__ kz,
    const uint8_t* __restrict__ vq, const uint16_t* __restrict__ vs, const uint8_t* __restrict__ vz,
    const int32_t* __restrict__ lens, int H, int Tcap, int C, int nchunks,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
    __shared__ float sc_lds[kAttnWaves][G][16 * kMaxSteps];  // scores, then p * s_v
    __shared__ float qs_lds[kAttnWaves][16];
    __shared__ float mrg_m[kAttnWaves][G], mrg_l[kAttnWaves][G], mrg_z[kAttnWaves][G];
    __shared__ float mrg_o[kAttnWaves][G][kD];

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int chunk = blockIdx.x % nchunks;
    const int bh = blockIdx.x / nchunks;  // b * H + h
    const int h = bh % H, b = bh / H;
    const int Hq = H * G;
    const int len = min(max(lens[b], 0), Tcap);
    const int c0 = chunk * C;
    // Part 2 reads a chunk's record only when the chunk starts before len.
    if (c0 >= len) return;

    const size_t rowbase = (size_t)bh * Tcap;
    const int wstart = c0 + wave * (C / kAttnWaves);
    const int wend = min(wstart + C / kAttnWaves, len);
    const int nsteps = wend > wstart ? (wend - wstart + 15) / 16 : 0;
    const int r16 = lane % 16, jg = lane / 16;

    // ---- keys of every step in flight first
    u32x4 kb[kMaxSteps];
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s) {
        if (s < nsteps) {
            const int t = min(wstart + 16 * s + r16, wend - 1);  // masked tokens read a valid row
            kb[s] = *reinterpret_cast<const u32x4*>(kq + (rowbase + t) * 64 + 16 * jg);
        }
    }

    // ---- A operands: query g = r16 (zeros for r16 >= G), channels 32 jg + 8f + 0..7,
    // q' = f16(q * lambda) from an FP32 product (the barrier keeps the backend
    // from forming one mixed-precision multiply that rounds once)
    half8v qa[4];
    float qpart = 0.0f;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (r16 < G) {
            const int ch = 32 * jg + 8 * f;
            const u32x4 qw = *reinterpret_cast<const u32x4*>(q + ((size_t)b * Hq + h * G + r16) * kD + ch);
            const u32x4 lw = *reinterpret_cast<const u32x4*>(lambda + (size_t)h * kD + ch);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float pa = h2f(qw[e] & 0xFFFFu) * h2f(lw[e] & 0xFFFFu);
                float pb = h2f(qw[e] >> 16) * h2f(lw[e] >> 16);
                asm("" : "+v"(pa), "+v"(pb));
                const uint16_t a = f2h(pa), c = f2h(pb);
                w[e] = (uint32_t)a | ((uint32_t)c << 16);
                qpart += h2f(a) + h2f(c);
            }
        }
        qa[f] = __builtin_bit_cast(half8v, w);
    }
    // sum(q') of query r16: add the four lanes of the row (jg = 0..3)
    qpart += __shfl_xor(qpart, 16, kWave);
    qpart += __shfl_xor(qpart, 32, kWave);
    if (lane < 16) qs_lds[wave][lane] = qpart;
    __builtin_amdgcn_wave_barrier();
    float qsum[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) qsum[v] = qs_lds[wave][4 * jg + v];

    // ---- pass 1: scores. Output lane l holds rows (queries) 4 jg + v, column
    // (token) r16 of the step.
    const float inv_sqrt_d = 0.08838834764831845f;  // 1 / sqrt(128)
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s) {
        if (s < nsteps) {
            float4t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int f = 0; f < 4; ++f)
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    qa[f], __builtin_bit_cast(half8v, codes8_to_f16(kb[s][f])), d, 0, 0, 0);
            const int t = wstart + 16 * s + r16;
            const bool valid = t < wend;
            const int tt = valid ? t : wstart;
            const float sk = h2f(ks[rowbase + tt]);
            const float zk = (float)kz[rowbase + tt];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int g = 4 * jg + v;
                if (g < G) {
                    const float sv = valid ? (sk * (d[v] - zk * qsum[v])) * inv_sqrt_d : -INFINITY;
                    sc_lds[wave][g][16 * s + r16] = sv;
                    mx[v] = fmaxf(mx[v], sv);
                }
            }
        }
    }
    // chunk maximum of each query: the 16 lanes of a row group hold its tokens
    float m[G];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        float x = mx[v];
        x = fmaxf(x, __shfl_xor(x, 1, kWave));
        x = fmaxf(x, __shfl_xor(x, 2, kWave));
        x = fmaxf(x, __shfl_xor(x, 4, kWave));
        x = fmaxf(x, __shfl_xor(x, 8, kWave));
        mx[v] = x;
    }
    if (r16 == 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
            if (4 * jg + v < G) mrg_m[wave][4 * jg + v] = mx[v];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = mrg_m[wave][g];

    // ---- values of every step in flight
    u32x4 vb[kMaxSteps];
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s)
        if (s < nsteps)
            vb[s] = *reinterpret_cast<const u32x4*>(
                vq + ((size_t)bh * (Tcap / 16) + (wstart / 16 + s)) * 1024 + (size_t)lane * 16);

    // ---- pass 2a: u = exp(s - m) * s_v in place; the lane's shares of
    // sum(p) and sum(u z_v)
    const int ntok = 16 * nsteps;
    float l[G], zs[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        l[g] = 0.0f;
        zs[g] = 0.0f;
        for (int i = lane; i < ntok; i += kWave) {
            const int t = wstart + i;
            const float sv = sc_lds[wave][g][i];
            float u = 0.0f;
            if (t < wend) {
                const float p = __expf(sv - m[g]);
                u = p * h2f(vs[rowbase + t]);
                l[g] += p;
                zs[g] += u * (float)vz[rowbase + t];
            }
            sc_lds[wave][g][i] = u;
        }
    }
    __builtin_amdgcn_wave_barrier();

    // ---- pass 2b: values
    float acc[G][2];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g][0] = acc[g][1] = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxSteps; ++s) {
        if (s < nsteps) {
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                const uint32_t word = vb[s][w4];
                const uint32_t lo = word & 0x0F0F0F0Fu, hi = (word >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * s + 4 * w4 + e;
                    const float vlo = (float)((lo >> (8 * e)) & 0xFFu);
                    const float vhi = (float)((hi >> (8 * e)) & 0xFFu);
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const float u = sc_lds[wave][g][i];
                        acc[g][0] += u * vlo;
                        acc[g][1] += u * vhi;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        l[g] = wave_sum_f(l[g]);
        zs[g] = wave_sum_f(zs[g]);
    }

    // ---- merge the waves' states; a wave without tokens has l = 0
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (lane == 0) {
            mrg_m[wave][g] = nsteps > 0 ? m[g] : -INFINITY;
            mrg_l[wave][g] = l[g];
            mrg_z[wave][g] = zs[g];
        }
        mrg_o[wave][g][2 * lane] = acc[g][0];
        mrg_o[wave][g][2 * lane + 1] = acc[g][1];
    }
    __syncthreads();
    // wave w finishes query heads g = w, w + 4, ...
    for (int g = wave; g < G; g += kAttnWaves) {
        float M = -INFINITY;
        for (int w = 0; w < kAttnWaves; ++w)
            if (mrg_l[w][g] > 0.0f) M = fmaxf(M, mrg_m[w][g]);
        float L = 0.0f, Z = 0.0f, o0 = 0.0f, o1 = 0.0f;
        for (int w = 0; w < kAttnWaves; ++w) {
            const float e = mrg_l[w][g] > 0.0f ? __expf(mrg_m[w][g] - M) : 0.0f;
            L += e * mrg_l[w][g];
            Z += e * mrg_z[w][g];
            o0 += e * mrg_o[w][g][2 * lane];
            o1 += e * mrg_o[w][g][2 * lane + 1];
        }
        const size_t rec = ((size_t)b * Hq + h * G + g) * nchunks + chunk;
        part_o[rec * kD + 2 * lane] = o0 - Z;
        part_o[rec * kD + 2 * lane + 1] = o1 - Z;
        if (lane == 0) {
            part_ml[rec * 2] = M;
            part_ml[rec * 2 + 1] = L;
        }
    }
}

// Part 2: one wave per (b, query head): combine the chunks that start before
// len[b]; o = sum_c e^(M_c - M) O_c / sum_c e^(M_c - M) L_c, rounded to FP16
// (a sequence of length 0 gives zeros).
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
    float M = -INFINITY;
    for (int c = 0; c < used; ++c) M = fmaxf(M, part_ml[(w * nchunks + c) * 2]);
    float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int c = 0; c < used; ++c) {
        const size_t rec = (size_t)w * nchunks + c;
        const float e = __expf(part_ml[rec * 2] - M);
        L += e * part_ml[rec * 2 + 1];
        o0 += e * part_o[rec * kD + 2 * lane];
        o1 += e * part_o[rec * kD + 2 * lane + 1];
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    reinterpret_cast<uint32_t*>(o + (size_t)w * kD)[lane] =
        (uint32_t)f2h(o0 * inv) | ((uint32_t)f2h(o1 * inv) << 16);
}

unsigned blocks_of(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

void launch_kv4_smooth_scales(const uint16_t* k, int64_t T, int64_t H, uint16_t* lambda,
                              hipStream_t stream) {
    hipLaunchKernelGGL(k_kv4_smooth_scales, dim3(blocks_of(H * kD, kKvThreads)), dim3(kKvThreads), 0,
                       stream, k, (int)T, (int)H, lambda);
}

void launch_kv4_append(const uint16_t* k, const uint16_t* v, const uint16_t* lambda, int64_t B,
                       int64_t T, int64_t H, int64_t Tcap, int64_t t0, uint8_t* kq, uint16_t* ks,
                       uint8_t* kz, uint8_t* vq, uint16_t* vs, uint8_t* vz, hipStream_t stream) {
    const int64_t vecs = B * T * H;
    hipLaunchKernelGGL(k_kv4_append, dim3(blocks_of(vecs, kKvThreads / kWave)), dim3(kKvThreads), 0,
                       stream, k, v, lambda, (int)B, (int)T, (int)H, (int)Tcap, (int)t0, kq, ks, kz,
                       vq, vs, vz);
}

// Chunk length: the smallest of 64, 128, 256, 512 tokens (at least 16 per
// wave) that keeps the number of chunks per sequence at or below 64 and still
// gives at least 1024 workgroups when that is possible.
int64_t kv4_chunk(int64_t B, int64_t H, int64_t Tcap) {
    int64_t C = 64;
    while (C < 512 && (B * H * ((Tcap + 2 * C - 1) / (2 * C)) >= 1024 || (Tcap + C - 1) / C > 64))
        C *= 2;
    return C;
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
                       part_ml)
    if (G == 1) QOQ_ATTN(1);
    else if (G == 2) QOQ_ATTN(2);
    else if (G == 4) QOQ_ATTN(4);
    else QOQ_ATTN(8);
#undef QOQ_ATTN
    hipLaunchKernelGGL(k_kv4_attn_combine, dim3(blocks_of(B * Hq, kKvThreads / kWave)),
                       dim3(kKvThreads), 0, stream, part_o, part_ml, lens, (int)B, (int)Hq, (int)Tcap,
                       (int)C, (int)n, o);
}

}  // namespace qoq
