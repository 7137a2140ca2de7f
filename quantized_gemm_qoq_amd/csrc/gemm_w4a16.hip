// gemm_w4a16.hip -- the W4A16 sibling: FP16 activations against the same QoQ
// 4-bit weights, on the gfx950 FP16 matrix cores with FP32 accumulation.
//
//   acc[m,n] = sum_k x[m,k] * W8^[n,k]         (fp32, W8^ = (q - z) * s_g)
//   y[m,n]   = f16(acc * s_c[n])
//
// This is the format the pages contrast with W4A8: weights stay 4-bit in
// memory and are dequantized to FP16 inside the main loop, activations stay
// FP16, and the products run on the FP16 matrix units ("QServe Guide: W4A8KV4
// Quantization for LLM Serving", "The Problem" item 1; "QServe: Low Bit Width
// Does Not Guarantee High Throughput", section 2, the W4A16 failure mode).
// With QoQ weights the integer group scale is applied before the conversion:
// the codes are unpacked to biased bytes (q - z) * s_g + 128 with the same
// packed multiply-add as the W4A8 kernels, then each byte b becomes the FP16
// value 1024 + b by placing it under the exponent byte 0x64, and one packed
// FP16 subtraction of 1152 yields (q - z) * s_g exactly. Per-channel weights use
// the same unpack with s_g = 1 and the channel's zero. The per-channel scale is
// applied once, in the epilogue.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_f16): lane l holds row (A) or
// channel (B) l % 16 and eight k values; one group of 128 inputs is four such
// operations f = 2s + h, where lane l's k values are 64s + 16(l/16) + 8h + 0..7.
// These are the codes of the lane's packed 16-byte weight load (k-step s,
// bytes 8h..8h+7 of its unpacked 16), and 16 contiguous bytes of the row-major
// activation row. The accumulator lane l holds rows 4(l/16) + 0..3 of channel
// l % 16.
#include <algorithm>

#include "qoq_device.hpp"
#include "qoq_launch.hpp"

namespace qoq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kBufferConfig = 0x00020000;  // gfx9 buffer resource word 3: 32-bit dwords
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ float4v mfma_f16(const half8& a, const half8& b, const float4v& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Biased bytes b0..b3 of a word -> two FP16 pairs (b0 - 128, b1 - 128) and
// (b2 - 128, b3 - 128), exactly: 0x64 above a byte b is the FP16 value 1024 + b.
__device__ __forceinline__ uint32_t bytes01_to_f16(uint32_t w) {
    const half2v h = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, w, 0x04010400u));
    return __builtin_bit_cast(uint32_t, h - half2v{(_Float16)1152.0f, (_Float16)1152.0f});
}
__device__ __forceinline__ uint32_t bytes23_to_f16(uint32_t w) {
    const half2v h = __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0x64646464u, w, 0x04030402u));
    return __builtin_bit_cast(uint32_t, h - half2v{(_Float16)1152.0f, (_Float16)1152.0f});
}

// Four codes (one per byte, 0..15) -> four biased bytes (q - z) * s_g + 128,
// with the group word s_g | C << 16 of the W4A8 kernels (C = (128 - z s_g) 257).
__device__ __forceinline__ uint32_t unpack4_biased(uint32_t codes, uint32_t gw) {
    uint32_t r;
    asm("v_pk_mad_u16 %0, %1, %2, %2 op_sel:[0,0,1] op_sel_hi:[1,0,1]"
        : "=v"(r)
        : "v"(codes), "v"(gw));
    return r;
}

// The FP16 B operands of one k-step s (operations f = 2s and 2s + 1) from a
// lane's 16 packed bytes.
template <int S>
__device__ __forceinline__ void b_operands_f16(u32x4 p, uint32_t gw, half8& b0, half8& b1) {
    const uint32_t w0 = S ? p.z : p.x, w1 = S ? p.w : p.y;
    const uint32_t c0 = unpack4_biased(w0 & 0x0F0F0F0Fu, gw);          // i = 0..3
    const uint32_t c1 = unpack4_biased((w0 >> 4) & 0x0F0F0F0Fu, gw);   // i = 4..7
    const uint32_t c2 = unpack4_biased(w1 & 0x0F0F0F0Fu, gw);          // i = 8..11
    const uint32_t c3 = unpack4_biased((w1 >> 4) & 0x0F0F0F0Fu, gw);   // i = 12..15
    b0 = __builtin_bit_cast(half8, u32x4{bytes01_to_f16(c0), bytes23_to_f16(c0),
                                         bytes01_to_f16(c1), bytes23_to_f16(c1)});
    b1 = __builtin_bit_cast(half8, u32x4{bytes01_to_f16(c2), bytes23_to_f16(c2),
                                         bytes01_to_f16(c3), bytes23_to_f16(c3)});
}

// FP16 output f16(acc * s_c); the barrier keeps the multiply and the
// conversion two separate roundings.
__device__ __forceinline__ uint16_t out_f16(float acc, float sc) {
    float v = acc * sc;
    asm("" : "+v"(v));
    return f2h(v);
}

__device__ __forceinline__ void store4(float4v a, int m_first, int n, int M, int N, float sc,
                                       uint16_t* __restrict__ y, float* __restrict__ acc_out) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = m_first + v;
        if (m < M) {
            const size_t o = (size_t)m * N + n;
            if (acc_out) acc_out[o] = a[v];
            y[o] = out_f16(a[v], sc);
        }
    }
}

// Epilogue of one wave's TM x TN accumulator tiles (rows m0 .. m0 + 16 TM - 1,
// channels n0 .. n0 + 16 TN - 1) with the FP16 outputs staged through a
// wave-private LDS region, 32 rows at a time, so that they leave as 16-byte
// row segments (an accumulator lane holds four rows of one channel). The row
// stride is padded by 16 bytes so that the four row groups of a write fall in
// different banks. acc_out, when given, receives the FP32 sums on the way.
template <int TM, int TN>
__device__ __forceinline__ void w16_staged_epilogue(const float4v (&acc)[TM][TN], uint8_t* region,
                                                    int m0, int n0, int M, int N,
                                                    const uint16_t* __restrict__ s_c,
                                                    uint16_t* __restrict__ y,
                                                    float* __restrict__ acc_out) {
    constexpr int kRowBytes = TN * 32;
    constexpr int kStride = kRowBytes + 16;
    constexpr int kPass = 2;  // row tiles per pass
    constexpr int kChunks = kPass * 16 * kRowBytes / 16;
    static_assert(TM % kPass == 0 && kChunks % kWave == 0, "passes must cover the tiles evenly");
    // The lane index taken afresh, so that nothing lane-derived from before
    // the main loop has to stay live through it.
    const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int c = lane % 16, j = lane / 16;
    float sc[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        const int n = n0 + 16 * i + c;
        sc[i] = n < N ? h2f(s_c[n]) : 0.0f;
    }
#pragma unroll
    for (int p = 0; p < TM; p += kPass) {
#pragma unroll
        for (int a = p; a < p + kPass; ++a) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + a * 16 + 4 * j + v;
#pragma unroll
                for (int i = 0; i < TN; ++i) {
                    const int n = n0 + 16 * i + c;
                    if (acc_out && m < M && n < N) acc_out[(size_t)m * N + n] = acc[a][i][v];
                    *reinterpret_cast<uint16_t*>(region + ((a - p) * 16 + 4 * j + v) * kStride +
                                                 (16 * i + c) * 2) = out_f16(acc[a][i][v], sc[i]);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < kChunks / kWave; ++k) {
            const int q = lane + k * kWave;
            const int row = q / (kRowBytes / 16), col = q % (kRowBytes / 16);
            const u32x4 out = *reinterpret_cast<const u32x4*>(region + row * kStride + col * 16);
            const int m = m0 + p * 16 + row, n = n0 + col * 8;
            if (m < M && n < N) *reinterpret_cast<u32x4*>(y + (size_t)m * N + n) = out;
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming kernel (decode, and up to 256 rows on narrow layers): the
// structure of the W4A8 streaming kernel. A
// workgroup of W waves owns NT channel tiles and MB row tiles; wave w takes
// the contiguous groups [G*w/W, G*(w+1)/W). Weights stream through a ring of R
// register sets (16 bytes per lane per tile per group); activations are read
// straight from the row-major FP16 rows (two 32-byte runs per lane per row
// tile per group, rows past M return zeros without a memory request). The
// waves' partial sums meet in LDS and are added in wave order, so the result
// does not depend on timing.
template <bool kG128, int MB, int NT>
__device__ __forceinline__ void w16_load(u32x4 (&bq)[NT], uint32_t (&pq)[NT], u32x4 (&aq)[MB][4],
                                         __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rp,
                                         __amdgpu_buffer_rsrc_t rx, const uint32_t (&b_off)[NT],
                                         const uint32_t (&p_off)[NT], const uint32_t (&a_off)[MB],
                                         int gi, bool valid) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const uint32_t ob = valid ? b_off[i] + (uint32_t)gi * 1024u : kOutOfRange;
        bq[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)ob, 0, 0);
        if (kG128) {
            const uint32_t op = valid ? p_off[i] + (uint32_t)gi * 16u : kOutOfRange;
            pq[i] = __builtin_amdgcn_raw_buffer_load_b8(rp, (int)op, 0, 0);
        }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const uint32_t oa = (valid && a_off[mb] != kOutOfRange) ? a_off[mb] + (uint32_t)gi * 256u
                                                               : kOutOfRange;
        aq[mb][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)oa, 0, 0);
        aq[mb][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)oa, 16, 0);
        aq[mb][2] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)oa, 128, 0);
        aq[mb][3] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)oa, 144, 0);
    }
}

template <bool kG128, int MB, int NT>
__device__ __forceinline__ void w16_compute(float4v (&acc)[NT][MB], const u32x4 (&bq)[NT],
                                            const uint32_t (&pq)[NT], const u32x4 (&aq)[MB][4],
                                            const uint32_t* lut, const uint32_t (&gw_pc)[NT]) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const uint32_t gw = kG128 ? lut[pq[i] & 0xFFu] : gw_pc[i];
        half8 b[4];
        b_operands_f16<0>(bq[i], gw, b[0], b[1]);
        b_operands_f16<1>(bq[i], gw, b[2], b[3]);
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                acc[i][mb] = mfma_f16(__builtin_bit_cast(half8, aq[mb][f]), b[f], acc[i][mb]);
    }
}

template <bool kG128, int MB, int NT, int R, int W>
__global__ __launch_bounds__(W * 64) void k_w4a16_stream(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ blob,
    const uint16_t* __restrict__ s_c, int M, int N, int K, uint16_t* __restrict__ y,
    float* __restrict__ acc_out) {
    constexpr int kPairs = NT * MB;
    constexpr int kThr = W * 64;
    // red[(w * kPairs + p) * 4 + v][lane]: row v of pair p of wave w.
    __shared__ float red[W * kPairs * 4 * kWave];
    __shared__ uint32_t lut[256];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int G = K / kGroup;
    const int tiles = N / 16;
    const int c = lane % 16, j = lane / 16;
    const int nblk = (tiles + NT - 1) / NT;
    const int mh = blockIdx.x / nblk;
    const int nb = blockIdx.x - mh * nblk;
    const int u0 = mh * MB;

    if (kG128)
        for (int i = threadIdx.x; i < 256; i += kThr) lut[i] = group_word((uint32_t)i);
    __syncthreads();

    const int g0 = G * wave / W;
    const int count = G * (wave + 1) / W - g0;

    const size_t code_bytes = (size_t)N * K / 2;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)x, (short)0, (int)((uint32_t)M * (uint32_t)K * 2u), kBufferConfig);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)blob, (short)0, (int)(uint32_t)code_bytes, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(blob + code_bytes), (short)0, (int)(uint32_t)(kG128 ? N * G : N), kBufferConfig);

    uint32_t b_off[NT], p_off[NT], a_off[MB];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int t = min(nb * NT + i, tiles - 1);
        b_off[i] = ((uint32_t)t * (uint32_t)G + (uint32_t)g0) * 1024u + (uint32_t)lane * 16u;
        p_off[i] = ((uint32_t)t * (uint32_t)G + (uint32_t)g0) * 16u + (uint32_t)c;
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int m = 16 * (u0 + mb) + c;
        a_off[mb] = m < M ? ((uint32_t)m * (uint32_t)K + (uint32_t)g0 * 128u + 16u * j) * 2u
                          : kOutOfRange;
    }
    // Per-channel weights: the unpack with s_g = 1 and the channel's zero (the
    // tiles of a workgroup are handled one at a time, so one word per tile).
    uint32_t gw_pc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int t = min(nb * NT + i, tiles - 1);
        gw_pc[i] = kG128 ? 0u : group_word(blob[code_bytes + 16 * t + c] & 15u);
    }

    float4v acc[NT][MB];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[i][mb] = float4v{0.f, 0.f, 0.f, 0.f};

    u32x4 bq[R][NT];
    uint32_t pq[R][NT];
    u32x4 aq[R][MB][4];
    const int main_count = count / R * R;
#pragma unroll
    for (int r = 0; r < R - 1; ++r)
        w16_load<kG128, MB, NT>(bq[r], pq[r], aq[r], rb, rp, rx, b_off, p_off, a_off, r,
                                r < main_count);
    for (int h = 0; h < main_count; h += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int nxt = h + r + R - 1;
            w16_load<kG128, MB, NT>(bq[(r + R - 1) % R], pq[(r + R - 1) % R], aq[(r + R - 1) % R],
                                    rb, rp, rx, b_off, p_off, a_off, nxt, nxt < main_count);
            w16_compute<kG128, MB, NT>(acc, bq[r], pq[r], aq[r], lut, gw_pc);
        }
    }
    for (int h = main_count; h < count; ++h) {
        w16_load<kG128, MB, NT>(bq[0], pq[0], aq[0], rb, rp, rx, b_off, p_off, a_off, h, true);
        w16_compute<kG128, MB, NT>(acc, bq[0], pq[0], aq[0], lut, gw_pc);
    }

#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[((wave * kPairs + i * MB + mb) * 4 + v) * kWave + lane] = acc[i][mb][v];
    __syncthreads();

    for (int p = wave; p < kPairs; p += W) {
        const int i = p / MB, mb = p % MB;
        const int t = nb * NT + i;
        if (t >= tiles) continue;
        const int n = 16 * t + c;
        float4v a = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < W; ++w)
#pragma unroll
            for (int v = 0; v < 4; ++v) a[v] += red[((w * kPairs + p) * 4 + v) * kWave + lane];
        store4(a, 16 * (u0 + mb) + 4 * j, n, M, N, h2f(s_c[n]), y, acc_out);
    }
}

// ---------------------------------------------------------------------------
// Tiled kernel (any M; the only one for M > 64 or for blobs too large for
// 32-bit buffer offsets). A workgroup of WM x WN waves computes a BM x BN block
// of Y; wave (wm, wn) owns TM x TN 16x16 tiles. Per group of 128 inputs the
// workgroup copies the block's activation rows (BM x 256 bytes, coalesced
// 16-byte loads along each row) into one of two LDS buffers in operand order
// -- slot ((u*4 + f)*64 + 16j + r) holds row 16u + r, inputs 64s + 16j + 8h +
// 0..7 with f = 2s + h -- so that each operand is one conflict-free 16-byte
// LDS read per lane. Weights go straight to registers; the loads for group
// g+1 are issued before the matrix-core work of group g.
template <int N, int kThr>
__device__ __forceinline__ void x_load(u32x4 (&stage)[N], const u32x4* const (&src)[N], int g) {
#pragma unroll
    for (int v = 0; v < N; ++v) stage[v] = src[v][(size_t)g * 16];
}

template <int N>
__device__ __forceinline__ void x_store(u32x4* buf, const u32x4 (&stage)[N], const int (&dst)[N]) {
#pragma unroll
    for (int v = 0; v < N; ++v) buf[dst[v]] = stage[v];
}

template <bool kG128, int TN>
__device__ __forceinline__ void wt_load(u32x4 (&bq)[TN], uint32_t (&pq)[TN],
                                        const u32x4* const (&bptr)[TN],
                                        const uint8_t* const (&pptr)[TN], int g) {
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        bq[i] = bptr[i][(size_t)g * kWave];
        if (kG128) pq[i] = pptr[i][(size_t)g * 16];
    }
}

template <bool kG128, int TM, int TN>
__device__ __forceinline__ void w16_tile_compute(float4v (&acc)[TM][TN], const u32x4* lw,
                                                 const u32x4 (&bq)[TN], const uint32_t (&pq)[TN],
                                                 const uint32_t* lut, const uint32_t (&gw_pc)[TN]) {
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        const uint32_t gw = kG128 ? lut[pq[i] & 0xFFu] : gw_pc[i];
        half8 b[4];
        b_operands_f16<0>(bq[i], gw, b[0], b[1]);
        b_operands_f16<1>(bq[i], gw, b[2], b[3]);
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int a = 0; a < TM; ++a)
                acc[a][i] = mfma_f16(__builtin_bit_cast(half8, lw[(a * 4 + f) * 64]), b[f], acc[a][i]);
    }
}

template <bool kG128, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64, 2) void k_w4a16_tile(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ blob,
    const uint16_t* __restrict__ s_c, int M, int N, int K, uint16_t* __restrict__ y,
    float* __restrict__ acc_out) {
    constexpr int kThr = WM * WN * 64;
    constexpr int TM = BM / WM / 16;
    constexpr int TN = BN / WN / 16;
    constexpr int kAVec = BM * 16;            // 16-byte vectors of A per group (BM rows x 256 B)
    constexpr int kAPerThr = kAVec / kThr;
    static_assert(kAVec % kThr == 0, "A staging must divide evenly");
    __shared__ u32x4 lds_a0[kAVec];
    __shared__ u32x4 lds_a1[kAVec];
    __shared__ uint32_t lut[256];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wave / WN, wn = wave % WN;
    const int c = lane % 16;
    const int G = K / kGroup;
    const int tiles = N / 16;
    const int grid_m = (M + BM - 1) / BM, grid_n = (N + BN - 1) / BN;

    // Block renumbering: contiguous range per XCD, then groups of 4 block rows.
    int pid = blockIdx.x;
    const int nblocks = grid_m * grid_n;
    if (nblocks % 8 == 0) pid = (pid % 8) * (nblocks / 8) + pid / 8;
    constexpr int kGroupM = 4;
    const int per_group = kGroupM * grid_n;
    const int first_m = (pid / per_group) * kGroupM;
    const int gsz = min(grid_m - first_m, kGroupM);
    const int bm = first_m + (pid % per_group) % gsz;
    const int bn = (pid % per_group) / gsz;

    if (kG128)
        for (int i = threadIdx.x; i < 256; i += kThr) lut[i] = group_word((uint32_t)i);

    // A staging: vector idx = threadIdx.x + v * kThr is chunk e = idx % 16 (8
    // inputs) of block row idx / 16; rows past M are clamped to M - 1 (their
    // outputs are never stored).
    const u32x4* xsrc[kAPerThr];
    int a_dst[kAPerThr];
#pragma unroll
    for (int v = 0; v < kAPerThr; ++v) {
        const int idx = threadIdx.x + v * kThr;
        const int row = idx / 16, e = idx % 16;
        const int m = min(bm * BM + row, M - 1);
        xsrc[v] = reinterpret_cast<const u32x4*>(x + (size_t)m * K) + e;
        const int s = e / 8, jj = (e % 8) / 2, h = e % 2;
        a_dst[v] = ((row / 16) * 4 + 2 * s + h) * 64 + 16 * jj + row % 16;
    }

    const size_t code_bytes = (size_t)N * K / 2;
    const u32x4* bptr[TN];
    const uint8_t* pptr[TN];
    uint32_t gw_pc[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        const int t = min(bn * (BN / 16) + wn * TN + i, tiles - 1);
        bptr[i] = reinterpret_cast<const u32x4*>(blob) + (size_t)t * G * kWave + lane;
        pptr[i] = blob + code_bytes + (size_t)t * G * 16 + c;
        gw_pc[i] = kG128 ? 0u : group_word(blob[code_bytes + 16 * (size_t)t + c] & 15u);
    }

    float4v acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = float4v{0.f, 0.f, 0.f, 0.f};

    u32x4 stage[kAPerThr];
    u32x4 b0q[TN], b1q[TN];
    uint32_t p0q[TN], p1q[TN];
    const u32x4* lw0 = lds_a0 + (size_t)(wm * TM) * 4 * 64 + lane;
    const u32x4* lw1 = lds_a1 + (size_t)(wm * TM) * 4 * 64 + lane;

    x_load<kAPerThr, kThr>(stage, xsrc, 0);
    x_store(lds_a0, stage, a_dst);
    x_load<kAPerThr, kThr>(stage, xsrc, min(1, G - 1));
    wt_load<kG128, TN>(b0q, p0q, bptr, pptr, 0);
    __syncthreads();

    // The same two-step loop as the W4A8 tiled kernel (fixed buffer and
    // register names, unconditional halves, an odd count ends with one step).
    int h = 0;
    for (; h + 1 < G; h += 2) {
        x_store(lds_a1, stage, a_dst);
        x_load<kAPerThr, kThr>(stage, xsrc, min(h + 2, G - 1));
        wt_load<kG128, TN>(b1q, p1q, bptr, pptr, h + 1);
        __builtin_amdgcn_sched_barrier(0);
        w16_tile_compute<kG128, TM, TN>(acc, lw0, b0q, p0q, lut, gw_pc);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        x_store(lds_a0, stage, a_dst);
        x_load<kAPerThr, kThr>(stage, xsrc, min(h + 3, G - 1));
        wt_load<kG128, TN>(b0q, p0q, bptr, pptr, min(h + 2, G - 1));
        __builtin_amdgcn_sched_barrier(0);
        w16_tile_compute<kG128, TM, TN>(acc, lw1, b1q, p1q, lut, gw_pc);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    }
    if (h < G) w16_tile_compute<kG128, TM, TN>(acc, lw0, b0q, p0q, lut, gw_pc);

    // Epilogue through LDS (the activation buffers, free once every wave is
    // past its last group; half the waves in each).
    constexpr int kRegion = 2 * 16 * (TN * 32 + 16);
    static_assert(WM * WN / 2 * kRegion <= kAVec * 16, "epilogue regions must fit the buffers");
    __syncthreads();
    uint8_t* region = reinterpret_cast<uint8_t*>(wave < WM * WN / 2 ? lds_a0 : lds_a1) +
                      (wave % (WM * WN / 2)) * kRegion;
    w16_staged_epilogue<TM, TN>(acc, region, bm * BM + wm * TM * 16, (bn * (BN / 16) + wn * TN) * 16, M,
                                N, s_c, y, acc_out);
}

// ---------------------------------------------------------------------------
template <bool kG128, int MB, int NT, int R = 2, int W = 8>
void launch_w16_stream(int64_t M, int64_t N, int64_t K, const uint16_t* x, const uint8_t* blob,
                       const uint16_t* s_c, uint16_t* y, float* acc_out, hipStream_t stream) {
    const int64_t tiles = N / 16, U = (M + 15) / 16;
    const unsigned blocks = (unsigned)(((tiles + NT - 1) / NT) * ((U + MB - 1) / MB));
    hipLaunchKernelGGL((k_w4a16_stream<kG128, MB, NT, R, W>), dim3(blocks), dim3(W * 64), 0,
                       stream, x, blob, s_c, (int)M, (int)N, (int)K, y, acc_out);
}

template <bool kG128, int BN, int WN>
void launch_w16_tile(int64_t M, int64_t N, int64_t K, const uint16_t* x, const uint8_t* blob,
                     const uint16_t* s_c, uint16_t* y, float* acc_out, hipStream_t stream) {
    const unsigned blocks = (unsigned)(((M + 127) / 128) * ((N + BN - 1) / BN));
    hipLaunchKernelGGL((k_w4a16_tile<kG128, 128, BN, 2, WN>), dim3(blocks), dim3(2 * WN * 64), 0,
                       stream, x, blob, s_c, (int)M, (int)N, (int)K, y, acc_out);
}

template <bool kG128>
void launch_w16(int64_t M, int64_t N, int64_t K, const uint16_t* x, const uint8_t* blob,
                const uint16_t* s_c, uint16_t* y, float* acc_out, hipStream_t stream) {
    const int64_t tiles = N / 16;
    // The streaming kernel forms 32-bit byte offsets into the codes and the rows.
    const bool fits = N * K / 2 < (int64_t(1) << 31) && N * (K / kGroup) < (int64_t(1) << 31);
    if (M <= 64 && fits) {
        // Measured on MI355X over the Llama-3-8B and Qwen1.5-72B decode layers
        // (one load set in flight per wave beat a two-deep ring everywhere):
        //   >= 1024 channel tiles: four tiles and four waves per workgroup
        //     (enough workgroups to keep every compute unit streaming);
        //   fewer tiles: 17..64 rows take three tiles per workgroup (the
        //     activation rows are re-read once per workgroup, so wider
        //     workgroups read them fewer times), up to 16 rows two;
        //   33..64 rows: two row tiles and four waves per workgroup; up to 32
        //     rows one row tile, with 16 waves when K has at most 64 groups
        //     (more waves, fewer groups each) and 8 otherwise.
        const int64_t G = K / kGroup;
        auto go = [&](auto launcher) { launcher(M, N, K, x, blob, s_c, y, acc_out, stream); };
        if (tiles >= 1024) {
            if (M <= 32) go(launch_w16_stream<kG128, 1, 4, 1, 4>);
            else go(launch_w16_stream<kG128, 2, 4, 1, 4>);
        } else if (M > 32) {
            go(launch_w16_stream<kG128, 2, 3, 1, 4>);
        } else if (M > 16) {
            if (G <= 64) go(launch_w16_stream<kG128, 1, 3, 1, 16>);
            else go(launch_w16_stream<kG128, 1, 3, 1, 8>);
        } else {
            if (G <= 64) go(launch_w16_stream<kG128, 1, 2, 1, 16>);
            else go(launch_w16_stream<kG128, 1, 2, 1, 8>);
        }
        return;
    }
    // 65..256 rows: the streaming kernel with 64-row workgroups while the
    // tiled kernel would have fewer than 128 workgroups (it then leaves most
    // compute units idle); the tiled kernel otherwise.
    const int64_t tile_blocks = ((M + 127) / 128) * ((N + 255) / 256);
    if (M <= 256 && fits && tile_blocks < 128) {
        launch_w16_stream<kG128, 4, 4, 1, 4>(M, N, K, x, blob, s_c, y, acc_out, stream);
        return;
    }
    launch_w16_tile<kG128, 256, 4>(M, N, K, x, blob, s_c, y, acc_out, stream);
}

}  // namespace

void launch_gemm_w4a16(int mode, const uint16_t* x, const uint8_t* blob, const uint16_t* s_c,
                       int64_t M, int64_t N, int64_t K, uint16_t* y, float* acc_out,
                       hipStream_t stream) {
    if (mode == 0)
        launch_w16<true>(M, N, K, x, blob, s_c, y, acc_out, stream);
    else
        launch_w16<false>(M, N, K, x, blob, s_c, y, acc_out, stream);
}

}  // namespace qoq
