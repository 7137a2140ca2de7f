// gemm.hip -- W4A8 GEMM (and its W8A8 sibling) on the gfx950 INT8 matrix
// cores.
//
//   acc[m,n] = sum_k xq[m,k] * W8^[n,k]   (exact INT32)
//   y[m,n]   = f16((f32(acc) * s_x[m]) * s_c[n])
//
// W8^ is unpacked in registers from the packed UINT4 codes: g128 mode by
// multiplying with the group's integer scale and subtracting the precomputed
// zero-point compensation ("QServe: Low Bit Width Does Not Guarantee High
// Throughput", section 4, the paragraph on the [-119,119] margin); per-channel
// mode feeds the codes themselves and subtracts z[n] * rowsum[m] in the
// epilogue. The rescale by the per-token and per-channel scales happens once,
// after the integer sum ("QServe Guide: W4A8KV4 Quantization for LLM Serving",
// Deep Dive part 1). The W8A8 sibling (the same page, "The Problem" item 2)
// stores W8^ itself, per-channel symmetric INT8, in the same operand order.
//
// Matrix-core mapping (v_mfma_i32_16x16x64_i8): A = activations (16 rows m),
// B = weights (16 channels n). For both operands lane l holds row/channel
// l % 16 and bytes 16*(l/16) .. +15 of the 64-wide k slice; the accumulator
// lane l holds rows 4*(l/16) + 0..3 of channel l % 16.
#include <algorithm>
#include <cmath>

#include "qoq_device.hpp"
#include "qoq_launch.hpp"

namespace qoq {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

// Weight formats of the packed blob (every kernel below is instantiated per
// format):
//   kFmtG128 UINT4 codes + one parameter byte per (channel, group): unpacked
//            to (q - z) * s_g in registers;
//   kFmtPC   UINT4 codes + one zero byte per channel: the codes feed the
//            matrix cores and z[n] * rowsum[m] is subtracted in the epilogue;
//   kFmtW8   INT8 weights in the operand order (no unpack, no parameters).
enum : int { kFmtG128 = 0, kFmtPC = 1, kFmtW8 = 2 };
template <int F>
struct Fmt {
    static constexpr bool kG128 = F == kFmtG128;
    static constexpr bool kZp = F == kFmtPC;          // zero-point in the epilogue
    static constexpr int kVec = F == kFmtW8 ? 2 : 1;  // 16-byte vectors per lane per group
};

// Bytes of the weight codes (the parameters, if any, follow them).
__host__ __device__ __forceinline__ size_t code_bytes_of(int fmt, int64_t N, int64_t K) {
    return fmt == kFmtW8 ? (size_t)N * K : (size_t)N * K / 2;
}

// One k-step (KS = 0 or 1) MFMA B operand of a lane from its loaded weight
// vectors: INT8 weights are the operand; UINT4 codes are unpacked.
template <int F, int KS>
__device__ __forceinline__ int32x4 b_operand(const u32x4 (&p)[Fmt<F>::kVec], uint32_t gw) {
    if constexpr (F == kFmtW8)
        return __builtin_bit_cast(int32x4, p[KS]);
    else
        return unpack_half<F == kFmtG128, KS>(p[0], gw);
}

// FP16 output of one accumulator: (f32(acc) * s_x) * s_c, each product rounded
// to fp32, then the result rounded to FP16.
__device__ __forceinline__ uint16_t output_value(int r, float sx, float sc) {
    float v = ((float)r * sx) * sc;
    // Without this barrier the backend folds the last multiply and the
    // conversion into one mixed-precision FMA that rounds only once.
    asm("" : "+v"(v));
    return f2h(v);
}

// Two outputs of one row, (f32(r)·sx)·sc each, rounded to FP16 and packed
// (low half: r0) by one conversion instruction.
__device__ __forceinline__ uint32_t output_pair(int r0, int r1, float sx, float sc0, float sc1) {
    float v0 = ((float)r0 * sx) * sc0;
    float v1 = ((float)r1 * sx) * sc1;
    asm("" : "+v"(v0));
    asm("" : "+v"(v1));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){v0, v1}, f16x2));
}

// Epilogue for one lane's four accumulator rows of one channel.
template <int F>
__device__ __forceinline__ void store_outputs(int32x4 a, int m_first, int n, int M, int N,
                                              const uint16_t* __restrict__ s_x,
                                              const int32_t* __restrict__ rowsum, float sc,
                                              int zpc, uint16_t* __restrict__ y,
                                              int32_t* __restrict__ acc_out) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int m = m_first + v;
        if (m < M) {
            int r = a[v];
            if (Fmt<F>::kZp) r -= zpc * rowsum[m];
            const size_t o = (size_t)m * N + n;
            if (acc_out) acc_out[o] = r;
            y[o] = output_value(r, h2f(s_x[m]), sc);
        }
    }
}

// ---------------------------------------------------------------------------
// Reference kernel: each wave owns one 16-channel tile and 64 rows, and streams
// the whole K. Used where no tuned kernel applies.
template <int F>
__global__ __launch_bounds__(kThreads) void k_gemm_simple(
    const int8_t* __restrict__ xq, const uint16_t* __restrict__ s_x,
    const int32_t* __restrict__ rowsum, const uint8_t* __restrict__ blob,
    const uint16_t* __restrict__ s_c, int M, int N, int K, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_out) {
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int t = blockIdx.x * kWavesPerBlock + wave;
    if (t * 16 >= N) return;
    const int m0 = blockIdx.y * 64;
    const int G = K / kGroup;
    const int U = (M + 15) / 16;  // activation tiles of 16 rows
    const int c = lane % 16;
    const int j = lane / 16;
    const int n = t * 16 + c;
    constexpr int kV = Fmt<F>::kVec;
    constexpr bool kG128 = Fmt<F>::kG128;
    const u32x4* tiles = reinterpret_cast<const u32x4*>(blob) + (size_t)t * G * kWave * kV + lane;
    const uint8_t* params = blob + code_bytes_of(F, N, K);
    const int32x4* act = reinterpret_cast<const int32x4*>(xq) + lane;

    int32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = int32x4{0, 0, 0, 0};

    for (int g = 0; g < G; ++g) {
        u32x4 p[kV];
#pragma unroll
        for (int v = 0; v < kV; ++v) p[v] = tiles[((size_t)g * kV + v) * kWave];
        const uint32_t gw = kG128 ? group_word(params[((size_t)t * G + g) * 16 + c]) : 0u;
        const int32x4 b0 = b_operand<F, 0>(p, gw);
        const int32x4 b1 = b_operand<F, 1>(p, gw);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int u = m0 / 16 + mb;
            if (u < U) {
                const int32x4* src = act + ((size_t)g * U + u) * 128;
                acc[mb] = mfma16x16x64(src[0], b0, acc[mb]);
                acc[mb] = mfma16x16x64(src[64], b1, acc[mb]);
            }
        }
    }

    const float sc = h2f(s_c[n]);
    const int zpc = Fmt<F>::kZp ? (int)params[n] : 0;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
        store_outputs<F>(acc[mb], m0 + 16 * mb + 4 * j, n, M, N, s_x, rowsum, sc, zpc, y,
                         acc_out);
}

// ---------------------------------------------------------------------------
// Tiled kernel (M > 64): matrix-core bound.
//
// A workgroup of WM x WN waves computes a BM x BN block of Y; wave (wm, wn)
// owns TM x TN 16x16 tiles. Per k-step (one group of 128 inputs):
//   - the block's activations for the group are one contiguous run of BM/16
//     packed 2 KB tiles; the workgroup copies them into one of two LDS buffers
//     with coalesced 16-byte loads, and each wave reads its A operands back
//     with one conflict-free 16-byte LDS read per lane (lane order is memory
//     order in the packed layout);
//   - each wave loads its TN packed weight tiles straight into registers (one
//     16-byte load per lane per tile) and unpacks them there;
//   - the loads for step g+1 are issued before the matrix-core work of step g,
//     and one barrier per step swaps the LDS buffers.
// Blocks are renumbered so that each XCD (blocks are dealt to the 8 XCDs
// round-robin) works through a contiguous, grouped part of the block grid and
// its L2 sees the same activation rows and weight columns many times.
// Per-step pieces of the tiled kernel, force-inlined with arrays passed by
// reference so that every operand stays in registers.
template <int N>
__device__ __forceinline__ void tile_load_a(u32x4 (&stage)[N], const u32x4* __restrict__ act,
                                            const int (&a_src)[N], size_t aoff) {
#pragma unroll
    for (int v = 0; v < N; ++v) stage[v] = act[aoff + a_src[v]];
}

template <int N, int kThr>
__device__ __forceinline__ void tile_store_a(u32x4* buf, const u32x4 (&stage)[N]) {
#pragma unroll
    for (int v = 0; v < N; ++v) buf[threadIdx.x + v * kThr] = stage[v];
}

template <int F, int TN>
__device__ __forceinline__ void tile_load_b(u32x4 (&bq)[TN][Fmt<F>::kVec], uint32_t (&pq)[TN],
                                            const u32x4* const (&bptr)[TN],
                                            const uint8_t* const (&pptr)[TN], int g) {
    constexpr int kV = Fmt<F>::kVec;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
        for (int v = 0; v < kV; ++v) bq[i][v] = bptr[i][((size_t)g * kV + v) * kWave];
        if (Fmt<F>::kG128) pq[i] = pptr[i][(size_t)g * 16];
    }
}

// One k-step: unpack this wave's TN weight tiles, read its TM activation
// tiles from LDS (lw: the wave's first tile, lane offset applied) and issue
// TM x TN x 2 matrix-core operations.
template <int F, int TM, int TN>
__device__ __forceinline__ void tile_compute(int32x4 (&acc)[TM][TN], const u32x4* lw,
                                             const u32x4 (&bq)[TN][Fmt<F>::kVec],
                                             const uint32_t (&pq)[TN]) {
    int32x4 b[TN][2];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        if constexpr (F == kFmtW8) {
            b[i][0] = __builtin_bit_cast(int32x4, bq[i][0]);
            b[i][1] = __builtin_bit_cast(int32x4, bq[i][1]);
        } else {
            GroupConst gc{0u, 0u};
            if (Fmt<F>::kG128) gc = group_const(pq[i]);
            unpack_lane<Fmt<F>::kG128>(bq[i][0], gc, b[i][0], b[i][1]);
        }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int a = 0; a < TM; ++a) {
            const int32x4 af = __builtin_bit_cast(int32x4, lw[a * 128 + ks * 64]);
#pragma unroll
            for (int i = 0; i < TN; ++i) acc[a][i] = mfma16x16x64(af, b[i][ks], acc[a][i]);
        }
    }
}

template <int F, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64, 2) void k_gemm_tile(
    const int8_t* __restrict__ xq, const uint16_t* __restrict__ s_x,
    const int32_t* __restrict__ rowsum, const uint8_t* __restrict__ blob,
    const uint16_t* __restrict__ s_c, int M, int N, int K, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_out, int S, int32_t* __restrict__ part) {
    constexpr int kThr = WM * WN * 64;
    constexpr int TM = BM / WM / 16;
    constexpr int TN = BN / WN / 16;
    constexpr int kAVec = BM * 128 / 16;       // 16-byte vectors of A per group
    constexpr int kAPerThr = kAVec / kThr;     // per thread
    static_assert(kAVec % kThr == 0, "A staging must divide evenly");
    // Two separately declared buffers, each named by fixed code (no run-time
    // buffer index).
    __shared__ u32x4 lds_a0[kAVec];
    __shared__ u32x4 lds_a1[kAVec];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wave / WN, wn = wave % WN;
    const int c = lane % 16, j = lane / 16;
    const int G = K / kGroup;
    const int U = (M + 15) / 16;
    const int tiles = N / 16;
    const int grid_m = (M + BM - 1) / BM, grid_n = (N + BN - 1) / BN;

    // With S > 1 the grid holds S copies of the block grid, copy s taking the
    // groups [G*s/S, G*(s+1)/S) and writing its INT32 partial sums to part[s].
    const int nblocks = grid_m * grid_n;
    const int split = blockIdx.x / nblocks;
    const int g0 = (int)((int64_t)G * split / S);
    const int Gc = (int)((int64_t)G * (split + 1) / S) - g0;  // >= 1: the plan keeps S <= G

    // Block renumbering: contiguous range per XCD, then groups of 4 block rows.
    int pid = blockIdx.x - split * nblocks;
    if (nblocks % 8 == 0) pid = (pid % 8) * (nblocks / 8) + pid / 8;
    constexpr int kGroupM = 4;
    const int per_group = kGroupM * grid_n;
    const int first_m = (pid / per_group) * kGroupM;
    const int gsz = min(grid_m - first_m, kGroupM);
    const int bm = first_m + (pid % per_group) % gsz;
    const int bn = (pid % per_group) / gsz;

    // A staging: vector i of the block's run goes to LDS slot i; thread t
    // moves vectors t, t + kThr, ...
    const int u0 = bm * (BM / 16);
    int a_src[kAPerThr];
#pragma unroll
    for (int v = 0; v < kAPerThr; ++v) {
        const int idx = threadIdx.x + v * kThr;
        const int u = min(u0 + idx / 128, U - 1);      // clamp past the last row tile
        a_src[v] = u * 128 + idx % 128;
    }
    const u32x4* act = reinterpret_cast<const u32x4*>(xq);
    const size_t a_stride = (size_t)U * 128;  // vectors per group

    // Weight tiles of this wave (clamped for the ragged n tail).
    constexpr int kV = Fmt<F>::kVec;
    const u32x4* bptr[TN];
    const uint8_t* pptr[TN];
    const uint8_t* params = blob + code_bytes_of(F, N, K);
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        const int t = min(bn * (BN / 16) + wn * TN + i, tiles - 1);
        bptr[i] = reinterpret_cast<const u32x4*>(blob) + (size_t)t * G * kWave * kV + lane;
        pptr[i] = params + (size_t)t * G * 16 + c;
    }

    int32x4 acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = int32x4{0, 0, 0, 0};

    u32x4 stage[kAPerThr];
    u32x4 b0q[TN][kV], b1q[TN][kV];
    uint32_t p0q[TN], p1q[TN];
    const u32x4* lw0 = lds_a0 + (size_t)(wm * TM) * 128 + lane;
    const u32x4* lw1 = lds_a1 + (size_t)(wm * TM) * 128 + lane;

    // Prologue: group 0 in buffer 0, group 1 in flight to the staging
    // registers, weights of group 0 in flight.
    tile_load_a(stage, act, a_src, (size_t)g0 * a_stride);
    tile_store_a<kAPerThr, kThr>(lds_a0, stage);
    tile_load_a(stage, act, a_src, (size_t)(g0 + min(1, Gc - 1)) * a_stride);
    tile_load_b<F, TN>(b0q, p0q, bptr, pptr, g0);
    __syncthreads();

    // Step h: publish the staged activations of group h+1 into the idle
    // buffer, issue the loads of group h+2 (activations) and h+1 (weights),
    // then run step h on the other buffer. Each load is first used a full step
    // later, so it is neither sunk to its use nor waited for early. Two steps
    // per iteration give each access a fixed buffer and register set; both
    // halves are unconditional (a branch around the second half would let the
    // compiler sink the first half's weight loads into it), and an odd group
    // count finishes with one more step on buffer 0. Group indices of the
    // look-ahead loads are clamped at the end (those loads are never used).
    int h = 0;
    for (; h + 1 < Gc; h += 2) {
        tile_store_a<kAPerThr, kThr>(lds_a1, stage);
        tile_load_a(stage, act, a_src, (size_t)(g0 + min(h + 2, Gc - 1)) * a_stride);
        tile_load_b<F, TN>(b1q, p1q, bptr, pptr, g0 + h + 1);
        __builtin_amdgcn_sched_barrier(0);
        tile_compute<F, TM, TN>(acc, lw0, b0q, p0q);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        tile_store_a<kAPerThr, kThr>(lds_a0, stage);
        tile_load_a(stage, act, a_src, (size_t)(g0 + min(h + 3, Gc - 1)) * a_stride);
        tile_load_b<F, TN>(b0q, p0q, bptr, pptr, g0 + min(h + 2, Gc - 1));
        __builtin_amdgcn_sched_barrier(0);
        tile_compute<F, TM, TN>(acc, lw1, b1q, p1q);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    }
    if (h < Gc) tile_compute<F, TM, TN>(acc, lw0, b0q, p0q);

    // Epilogue (with S > 1: the raw partial sums; the reduction kernel adds
    // them and applies the zero-point compensation and the rescale once).
    const uint8_t* pc_z = params;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        const int t = bn * (BN / 16) + wn * TN + i;
        if (t >= tiles) continue;
        const int n = 16 * t + c;
#pragma unroll
        for (int a = 0; a < TM; ++a) {
            const int m_first = bm * BM + (wm * TM + a) * 16 + 4 * j;
            if (part) {
                int32_t* dst = part + (size_t)split * M * N;
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (m_first + v < M) dst[(size_t)(m_first + v) * N + n] = acc[a][i][v];
            } else {
                store_outputs<F>(acc[a][i], m_first, n, M, N, s_x, rowsum, h2f(s_c[n]),
                                 Fmt<F>::kZp ? (int)pc_z[n] : 0, y, acc_out);
            }
        }
    }
}

// Split-K reduction: adds the S partial sums of each output (INT32 addition is
// exact and order-free), applies the per-channel zero-point compensation and
// the one-time rescale. Each thread handles four consecutive channels of one
// row (N is a multiple of 16).
template <int F>
__global__ __launch_bounds__(kThreads) void k_splitk_reduce(
    const int32_t* __restrict__ part, int S, const uint16_t* __restrict__ s_x,
    const int32_t* __restrict__ rowsum, const uint8_t* __restrict__ pc_z,
    const uint16_t* __restrict__ s_c, int M, int N, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_out) {
    const int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t total = (int64_t)M * N;
    if (q * 4 >= total) return;
    const int m = (int)(q * 4 / N), n0 = (int)(q * 4 % N);
    int32x4 r = reinterpret_cast<const int32x4*>(part)[q];
    for (int s2 = 1; s2 < S; ++s2) r += reinterpret_cast<const int32x4*>(part + (size_t)s2 * total)[q];
    const float sx = h2f(s_x[m]);
    uint16_t out[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int n = n0 + v;
        int rr = r[v];
        if (Fmt<F>::kZp) rr -= (int)pc_z[n] * rowsum[m];
        if (acc_out) acc_out[(size_t)m * N + n] = rr;
        out[v] = output_value(rr, sx, h2f(s_c[n]));
    }
    reinterpret_cast<uint2*>(y)[q] = make_uint2(out[0] | ((uint32_t)out[1] << 16),
                                                out[2] | ((uint32_t)out[3] << 16));
}

// Epilogue of one wave's TM x TN accumulator tiles (rows m0 .. m0 + 16 TM - 1,
// channels n0 .. n0 + 16 TN - 1) with the FP16 outputs staged through a
// wave-private LDS region, 32 rows at a time: each output is written to LDS
// as it is computed (an accumulator lane holds four rows of one channel), then
// the rows are stored as 16-byte segments, so each row of the strip leaves in
// whole 32 TN-byte runs instead of 2-byte pieces. The row stride is padded by
// 16 bytes so that the four row groups of a write fall in different banks.
// acc_out, when given, receives the INT32 sums element by element.
template <int F, int TM, int TN>
__device__ __forceinline__ void staged_epilogue(const int32x4 (&acc)[TM][TN], uint8_t* region,
                                                int m0, int n0, int M, int N,
                                                const uint16_t* __restrict__ s_x,
                                                const int32_t* __restrict__ rowsum,
                                                const uint16_t* __restrict__ s_c,
                                                const uint8_t* __restrict__ pc_z,
                                                uint16_t* __restrict__ y,
                                                int32_t* __restrict__ acc_out) {
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
    int zpc[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        const int n = n0 + 16 * i + c;
        sc[i] = n < N ? h2f(s_c[n]) : 0.0f;
        zpc[i] = Fmt<F>::kZp && n < N ? (int)pc_z[n] : 0;
    }
#pragma unroll
    for (int p = 0; p < TM; p += kPass) {
#pragma unroll
        for (int a = p; a < p + kPass; ++a) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int m = m0 + a * 16 + 4 * j + v;
                const float sx = m < M ? h2f(s_x[m]) : 0.0f;
                const int rs = Fmt<F>::kZp && m < M ? rowsum[m] : 0;
#pragma unroll
                for (int i = 0; i < TN; ++i) {
                    int r = acc[a][i][v];
                    if (Fmt<F>::kZp) r -= zpc[i] * rs;
                    const int n = n0 + 16 * i + c;
                    if (acc_out && m < M && n < N) acc_out[(size_t)m * N + n] = r;
                    *reinterpret_cast<uint16_t*>(region + ((a - p) * 16 + 4 * j + v) * kStride +
                                                 (16 * i + c) * 2) = output_value(r, sx, sc[i]);
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

// The INT32 partial sums of one wave's TM x TN accumulator tiles, staged
// through a wave-private LDS region one row tile (16 rows) at a time and
// stored as 16-byte row segments of dst (an [M, N] slice of the workspace).
template <int TM, int TN>
__device__ __forceinline__ void staged_partials(const int32x4 (&acc)[TM][TN], uint8_t* region,
                                                int m0, int n0, int M, int N,
                                                int32_t* __restrict__ dst) {
    constexpr int kRowBytes = TN * 64;
    constexpr int kChunks = 16 * kRowBytes / 16;
    static_assert(kChunks % kWave == 0, "a row tile must split evenly over the lanes");
    const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int c = lane % 16, j = lane / 16;
#pragma unroll
    for (int a = 0; a < TM; ++a) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int i = 0; i < TN; ++i)
                *reinterpret_cast<int32_t*>(region + (4 * j + v) * kRowBytes + (16 * i + c) * 4) = acc[a][i][v];
#pragma unroll
        for (int k = 0; k < kChunks / kWave; ++k) {
            const int q = lane + k * kWave;
            const int row = q / (kRowBytes / 16), col = q % (kRowBytes / 16);
            const int32x4 out = *reinterpret_cast<const int32x4*>(region + row * kRowBytes + col * 16);
            const int m = m0 + a * 16 + row, n = n0 + col * 4;
            if (m < M && n < N) *reinterpret_cast<int32x4*>(dst + (size_t)m * N + n) = out;
        }
    }
}

// ---------------------------------------------------------------------------
// Wide-wave tiled kernel (M > 64). The waves of a workgroup sit side by side
// in N and each one spans all BM rows of the block (TM = BM/16 row tiles, TN
// channel tiles), so each weight tile is loaded and unpacked by exactly one
// wave and feeds TM x 2 matrix-core operations per group: the unpack work per
// operation falls with BM, which is what keeps the vector ALU off the critical
// path at the gfx950 INT8 matrix-core rate. With BM = 256 the accumulators take
// 256 registers per lane (one wave per SIMD, accumulators in the AccVGPRs).
//   - Activations: one contiguous run of BM/16 packed 2 KB tiles per group,
//     staged through registers into one of two LDS buffers.
//   - Weights: one 16-byte buffer load per lane per tile straight into
//     registers; group parameter bytes map to the packed-multiply constants
//     through a 256-entry LDS table.
//   - Every address is a per-lane 32-bit offset fixed at the start plus a
//     wave-uniform per-group offset (buffer loads), so the loop does no
//     address arithmetic.
// The plan selects this kernel only when every byte offset fits in 32 bits.
constexpr int kBufferConfig = 0x00020000;  // gfx9 buffer resource word 3: 32-bit dwords

template <int N>
__device__ __forceinline__ void wide_load_a(u32x4 (&stage)[N], __amdgpu_buffer_rsrc_t ra,
                                            const uint32_t (&a_off)[N], uint32_t soff) {
#pragma unroll
    for (int v = 0; v < N; ++v)
        stage[v] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)a_off[v], (int)soff, 0);
}

template <int F, int TN>
__device__ __forceinline__ void wide_load_b(u32x4 (&bq)[TN][Fmt<F>::kVec], uint32_t (&pq)[TN],
                                            __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rp,
                                            const uint32_t (&b_off)[TN],
                                            const uint32_t (&p_off)[TN], int g) {
    constexpr int kV = Fmt<F>::kVec;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
        for (int v = 0; v < kV; ++v)
            bq[i][v] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)b_off[i], (g * kV + v) * 1024, 0);
        if (Fmt<F>::kG128) pq[i] = __builtin_amdgcn_raw_buffer_load_b8(rp, (int)p_off[i], g * 16, 0);
    }
}

// One group on one wave: unpack the TN weight tiles (both k-steps) and run the
// TM x TN x 2 matrix-core operations, reading each activation tile from LDS
// just ahead of its use. The group pattern at the end asks the scheduler to
// interleave the k-step-1 unpack and the LDS reads with the k-step-0
// matrix-core operations.
template <int F, int TM, int TN>
__device__ __forceinline__ void wide_compute(int32x4 (&acc)[TM][TN], const u32x4* lw,
                                             const u32x4 (&bq)[TN][Fmt<F>::kVec],
                                             const uint32_t (&pq)[TN], const uint32_t* lut) {
    constexpr bool kG128 = Fmt<F>::kG128;
    uint32_t gw[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i) gw[i] = kG128 ? lut[pq[i] & 0xFFu] : 0u;
    int32x4 b0[TN], b1[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i) b0[i] = b_operand<F, 0>(bq[i], gw[i]);
#pragma unroll
    for (int i = 0; i < TN; ++i) b1[i] = b_operand<F, 1>(bq[i], gw[i]);
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        const int32x4 af = __builtin_bit_cast(int32x4, lw[a * 128]);
#pragma unroll
        for (int i = 0; i < TN; ++i) acc[a][i] = mfma16x16x64(af, b0[i], acc[a][i]);
    }
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        const int32x4 af = __builtin_bit_cast(int32x4, lw[a * 128 + 64]);
#pragma unroll
        for (int i = 0; i < TN; ++i) acc[a][i] = mfma16x16x64(af, b1[i], acc[a][i]);
    }
    // Scheduling pattern (masks: 0x2 VALU, 0x8 MFMA, 0x100 LDS read). INT8
    // weights need no unpack: only the LDS reads are interleaved.
    constexpr int kUnpackHalf = (F == kFmtG128 ? 14 : F == kFmtPC ? 6 : 0) * TN;
    constexpr int kValuPerRow = (kUnpackHalf + TM - 1) / TM;
    if (kG128) {
        __builtin_amdgcn_sched_group_barrier(0x002, TN, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, TN, 0);
    }
    if (kUnpackHalf > 0) __builtin_amdgcn_sched_group_barrier(0x002, kUnpackHalf, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
        if (kValuPerRow > 0) __builtin_amdgcn_sched_group_barrier(0x002, kValuPerRow, 0);
    }
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
    }
}

template <int F, int BM, int BN, int WN>
__global__ __launch_bounds__(WN * 64, 2) void k_gemm_wide(
    const int8_t* __restrict__ xq, const uint16_t* __restrict__ s_x,
    const int32_t* __restrict__ rowsum, const uint8_t* __restrict__ blob,
    const uint16_t* __restrict__ s_c, int M, int N, int K, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_out, int group_m) {
    constexpr int kThr = WN * 64;
    constexpr int TM = BM / 16;
    constexpr int TN = BN / WN / 16;
    constexpr int kAVec = BM * 128 / 16;   // 16-byte vectors of A per group
    constexpr int kAPerThr = kAVec / kThr;
    static_assert(kAVec % kThr == 0, "A staging must divide evenly");
    __shared__ u32x4 lds_a0[kAVec];
    __shared__ u32x4 lds_a1[kAVec];
    __shared__ uint32_t lut[256];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c = lane % 16;
    const int G = K / kGroup;
    const int U = (M + 15) / 16;
    const int tiles = N / 16;
    const int grid_m = (M + BM - 1) / BM, grid_n = (N + BN - 1) / BN;

    // Block renumbering: contiguous range per XCD, then groups of group_m block
    // rows.
    int pid = blockIdx.x;
    const int nblocks = grid_m * grid_n;
    if (nblocks % 8 == 0) pid = (pid % 8) * (nblocks / 8) + pid / 8;
    const int per_group = group_m * grid_n;
    const int first_m = (pid / per_group) * group_m;
    const int gsz = min(grid_m - first_m, group_m);
    const int bm = first_m + (pid % per_group) % gsz;
    const int bn = (pid % per_group) / gsz;

    constexpr bool kG128 = Fmt<F>::kG128;
    constexpr int kV = Fmt<F>::kVec;
    if (kG128)
        for (int i = threadIdx.x; i < 256; i += kThr) lut[i] = group_word((uint32_t)i);

    const size_t code_bytes = code_bytes_of(F, N, K);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)xq, (short)0, (int)((uint32_t)G * (uint32_t)U * 2048u), kBufferConfig);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)blob, (short)0, (int)(uint32_t)code_bytes, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(blob + code_bytes), (short)0, (int)(uint32_t)(kG128 ? N * G : N), kBufferConfig);

    // Activation vector idx = threadIdx.x + v * kThr of the block's run goes to
    // LDS slot idx (row tiles past the last one are clamped; their rows are
    // never stored).
    const int u0 = bm * (BM / 16);
    uint32_t a_off[kAPerThr];
#pragma unroll
    for (int v = 0; v < kAPerThr; ++v) {
        const int idx = threadIdx.x + v * kThr;
        const int u = min(u0 + idx / 128, U - 1);
        a_off[v] = (uint32_t)(u * 128 + idx % 128) * 16u;
    }
    const uint32_t a_step = (uint32_t)U * 2048u;  // bytes per group

    // Weight tiles of this wave (clamped for the ragged n tail).
    uint32_t b_off[TN], p_off[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
        const int t = min(bn * (BN / 16) + wave * TN + i, tiles - 1);
        b_off[i] = ((uint32_t)t * (uint32_t)G * 64u * kV + (uint32_t)lane) * 16u;
        p_off[i] = (uint32_t)t * (uint32_t)G * 16u + (uint32_t)c;
    }

    int32x4 acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = int32x4{0, 0, 0, 0};

    u32x4 stage[kAPerThr];
    u32x4 b0q[TN][kV], b1q[TN][kV];
    uint32_t p0q[TN], p1q[TN];
    const u32x4* lw0 = lds_a0 + lane;
    const u32x4* lw1 = lds_a1 + lane;

    // Prologue: group 0 in buffer 0, group 1 in flight to the staging
    // registers, weights of group 0 in flight.
    wide_load_a(stage, ra, a_off, 0u);
    tile_store_a<kAPerThr, kThr>(lds_a0, stage);
    wide_load_a(stage, ra, a_off, (uint32_t)min(1, G - 1) * a_step);
    wide_load_b<F, TN>(b0q, p0q, rb, rp, b_off, p_off, 0);
    __syncthreads();

    // Step h: issue the weight loads of group h+1, run group h, then publish
    // the staged activations of group h+1 into the idle buffer and issue the
    // activation loads of group h+2. The wait for the staged activations thus
    // falls after the step's matrix-core operations are issued, and every load
    // has a whole step to arrive. Two steps per iteration give each buffer and
    // register set a fixed name; both halves are unconditional (a branch would
    // let the compiler sink loads to their use), and an odd group count ends
    // with one more step. Look-ahead group indices are clamped at the end.
    int h = 0;
    for (; h + 1 < G; h += 2) {
        wide_load_b<F, TN>(b1q, p1q, rb, rp, b_off, p_off, h + 1);
        __builtin_amdgcn_sched_barrier(0);
        wide_compute<F, TM, TN>(acc, lw0, b0q, p0q, lut);
        __builtin_amdgcn_sched_barrier(0);
        tile_store_a<kAPerThr, kThr>(lds_a1, stage);
        wide_load_a(stage, ra, a_off, (uint32_t)min(h + 2, G - 1) * a_step);
        __syncthreads();
        wide_load_b<F, TN>(b0q, p0q, rb, rp, b_off, p_off, min(h + 2, G - 1));
        __builtin_amdgcn_sched_barrier(0);
        wide_compute<F, TM, TN>(acc, lw1, b1q, p1q, lut);
        __builtin_amdgcn_sched_barrier(0);
        tile_store_a<kAPerThr, kThr>(lds_a0, stage);
        wide_load_a(stage, ra, a_off, (uint32_t)min(h + 3, G - 1) * a_step);
        __syncthreads();
    }
    if (h < G) wide_compute<F, TM, TN>(acc, lw0, b0q, p0q, lut);

    // Epilogue through LDS (the activation buffers, free once every wave is
    // past its last group).
    static_assert(WN == 4 && 2 * 2 * 16 * (TN * 32 + 16) <= kAVec * 16,
                  "two epilogue regions must fit each activation buffer");
    __syncthreads();
    uint8_t* region = reinterpret_cast<uint8_t*>(wave < 2 ? lds_a0 : lds_a1) +
                      (wave % 2) * (2 * 16 * (TN * 32 + 16));
    staged_epilogue<F, TM, TN>(acc, region, bm * BM, (bn * (BN / 16) + wave * TN) * 16, M, N, s_x,
                               rowsum, s_c, blob + code_bytes, y, acc_out);
}

// ---------------------------------------------------------------------------
// LDS-pipelined kernel (M > 64). A workgroup of kW waves owns a BM x BN block
// (one 8-wave workgroup of 128 x 256, or two 4-wave workgroups of 128 x 128,
// per compute unit); wave (wm, wn) computes BM/WM rows x BN/WN channels (TM
// row tiles x TN channel tiles), so every weight tile is unpacked by WM
// waves. Both operands reach LDS by direct buffer-to-LDS loads (no staging
// registers), three groups deep: the loads of group g+2 are issued at the
// start of step g into the buffer that step g-1 has just finished reading, and
// step g waits only for its own group's loads (the load counter is in order,
// so the wait leaves the next group's loads in flight), then one barrier
// publishes the group to all waves. The three buffers are separate arrays
// named by fixed code (three steps per loop iteration), so that the compiler
// can tell the loads into one buffer from the reads of another. Small grids split K over S
// copies of the block grid; each copy writes its exact INT32 partial sums and
// the split-K reduction kernel finishes them.
template <int F, int TM, int TN>
__device__ __forceinline__ void lds_compute(int32x4 (&acc)[TM][TN], const u32x4* la,
                                            const u32x4* lb, const uint8_t* lp) {
    constexpr bool kG128 = Fmt<F>::kG128;
    constexpr int kV = Fmt<F>::kVec;
    u32x4 bq[TN][kV];
    uint32_t gw[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
        for (int v = 0; v < kV; ++v) bq[i][v] = lb[(i * kV + v) * 64];
        gw[i] = kG128 ? group_word(lp[i * 16]) : 0u;
    }
    int32x4 b0[TN], b1[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i) b0[i] = b_operand<F, 0>(bq[i], gw[i]);
#pragma unroll
    for (int i = 0; i < TN; ++i) b1[i] = b_operand<F, 1>(bq[i], gw[i]);
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        const int32x4 af = __builtin_bit_cast(int32x4, la[a * 128]);
#pragma unroll
        for (int i = 0; i < TN; ++i) acc[a][i] = mfma16x16x64(af, b0[i], acc[a][i]);
    }
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        const int32x4 af = __builtin_bit_cast(int32x4, la[a * 128 + 64]);
#pragma unroll
        for (int i = 0; i < TN; ++i) acc[a][i] = mfma16x16x64(af, b1[i], acc[a][i]);
    }
    // Scheduling pattern (masks: 0x2 VALU, 0x8 MFMA, 0x100 LDS read): the
    // weight reads first, the k-step-0 unpack, then the k-step-1 unpack spread
    // over the k-step-0 matrix-core operations.
    constexpr int kUnpackHalf = (F == kFmtG128 ? 14 : F == kFmtPC ? 6 : 0) * TN;
    constexpr int kGroupWord = kG128 ? 7 * TN : 0;
    constexpr int kValuPerRow = (kUnpackHalf + TM - 1) / TM;
    __builtin_amdgcn_sched_group_barrier(0x100, TN * (kV + (kG128 ? 1 : 0)), 0);
    if (kUnpackHalf > 0) __builtin_amdgcn_sched_group_barrier(0x002, kGroupWord + kUnpackHalf, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
        if (kValuPerRow > 0) __builtin_amdgcn_sched_group_barrier(0x002, kValuPerRow, 0);
    }
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, TN, 0);
    }
}

#define QOQ_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

template <int F, int BM, int WM, int BN, int kW>
__global__ __launch_bounds__(kW * 64, 8 / kW) void k_gemm_lds(
    const int8_t* __restrict__ xq, const uint16_t* __restrict__ s_x,
    const int32_t* __restrict__ rowsum, const uint8_t* __restrict__ blob,
    const uint16_t* __restrict__ s_c, int M, int N, int K, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_out, int group_m, int S, int32_t* __restrict__ part) {
    constexpr int kThr = kW * 64;
    constexpr int WN = kW / WM;
    constexpr int TM = BM / 16 / WM, TN = BN / WN / 16;
    constexpr bool kG128 = Fmt<F>::kG128;
    constexpr int kV = Fmt<F>::kVec;
    constexpr int kAVec = BM * 128 / 16;         // 16-byte vectors of A per group
    constexpr int kBVec = (BN / 16) * 64 * kV;   // of B
    constexpr int kPVec = kG128 ? 16 : 0;        // 256 parameter bytes
    constexpr int kStageVec = kAVec + kBVec + kPVec;
    constexpr int kADma = kAVec / kThr;          // loads per wave per group
    constexpr int kBDma = kBVec / kThr;
    static_assert(kAVec % kThr == 0 && kBVec % kThr == 0, "loads must divide evenly");
    static_assert(3 * kStageVec * 16 * (8 / kW) <= 160 * 1024,
                  "three stages of every resident workgroup must fit the LDS");
    // Wait for all but the next group's loads (wave 0's parameter load of the
    // next group may be waited for too), and for this wave's LDS reads.
    constexpr int kD = kADma + kBDma;
    static_assert(kD < 64, "the load counter holds 6 bits");
    constexpr int kWaitStep = (kD & 15) | ((kD >> 4) << 14) | (7 << 4);  // vmcnt(kD) lgkmcnt(0)
    constexpr int kWaitAll = (7 << 4);                                   // vmcnt(0) lgkmcnt(0)
    __shared__ u32x4 st0[kStageVec];
    __shared__ u32x4 st1[kStageVec];
    __shared__ u32x4 st2[kStageVec];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wave / WN, wn = wave % WN;
    const int c = lane % 16;
    const int G = K / kGroup;
    const int U = (M + 15) / 16;
    const int tiles = N / 16;
    const int grid_m = (M + BM - 1) / BM, grid_n = (N + BN - 1) / BN;

    // With S > 1 the grid holds S copies of the block grid, copy s taking the
    // groups [G*s/S, G*(s+1)/S) and writing its INT32 partial sums to part[s].
    const int nblocks = grid_m * grid_n;
    const int split = blockIdx.x / nblocks;
    const int g0 = (int)((int64_t)G * split / S);
    const int Gc = (int)((int64_t)G * (split + 1) / S) - g0;  // >= 1: the plan keeps S <= G

    // Block renumbering: contiguous range per XCD, then groups of group_m
    // block rows.
    int pid = blockIdx.x - split * nblocks;
    if (nblocks % 8 == 0) pid = (pid % 8) * (nblocks / 8) + pid / 8;
    const int per_group = group_m * grid_n;
    const int first_m = (pid / per_group) * group_m;
    const int gsz = min(grid_m - first_m, group_m);
    const int bm = first_m + (pid % per_group) % gsz;
    const int bn = (pid % per_group) / gsz;

    const size_t code_bytes = code_bytes_of(F, N, K);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)xq, (short)0, (int)((uint32_t)G * (uint32_t)U * 2048u), kBufferConfig);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)blob, (short)0, (int)(uint32_t)code_bytes, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(blob + code_bytes), (short)0, (int)(uint32_t)(kG128 ? N * G : N), kBufferConfig);

    // Load v of this wave moves 16-byte vectors (v * 8 + wave) * 64 + lane of
    // the group's A run (BM/16 packed 2 KB row tiles, clamped past the last
    // one) and of its B run (16 channel tiles of kV KB, clamped past the last
    // one) to the same LDS vector index. Wave 0 also moves the 256 parameter
    // bytes, 4 per lane (tile lane/4, channels 4*(lane%4) .. +3).
    const int u0 = bm * (BM / 16);
    uint32_t a_off[kADma], b_off[kBDma];
#pragma unroll
    for (int v = 0; v < kADma; ++v) {
        const int idx = (v * kW + wave) * 64 + lane;
        const int u = min(u0 + idx / 128, U - 1);
        a_off[v] = (uint32_t)(u * 128 + idx % 128) * 16u;
    }
#pragma unroll
    for (int v = 0; v < kBDma; ++v) {
        const int idx = (v * kW + wave) * 64 + lane;
        const int t = min(bn * (BN / 16) + idx / (64 * kV), tiles - 1);
        b_off[v] = ((uint32_t)t * (uint32_t)G * 64u * kV + (uint32_t)(idx % (64 * kV))) * 16u;
    }
    const uint32_t p_off =
        (uint32_t)min(bn * (BN / 16) + lane / 4, tiles - 1) * (uint32_t)G * 16u + 4u * (lane % 4);
    const uint32_t a_step = (uint32_t)U * 2048u;  // bytes per group

    auto issue = [&](u32x4* st, int g) {
#pragma unroll
        for (int v = 0; v < kADma; ++v)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, QOQ_LDS_PTR(st + (v * kW + wave) * 64), 16,
                                                     (int)a_off[v], (int)((uint32_t)g * a_step), 0, 0);
#pragma unroll
        for (int v = 0; v < kBDma; ++v)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, QOQ_LDS_PTR(st + kAVec + (v * kW + wave) * 64),
                                                     16, (int)b_off[v], g * kV * 1024, 0, 0);
        if (kG128 && wave == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rp, QOQ_LDS_PTR(st + kAVec + kBVec), 4, (int)p_off,
                                                     g * 16, 0, 0);
    };

    int32x4 acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = int32x4{0, 0, 0, 0};

    const int la = (wm * TM) * 128 + lane;
    const int lb = kAVec + (wn * TN) * 64 * kV + lane;
    const int lp = (kAVec + kBVec) * 16 + (wn * TN) * 16 + c;  // byte index

    // Step g: wait for group g, publish it, refill the buffer step g-1 read
    // with group g+2 (clamped at the end: those loads are never read), run g.
    auto step = [&](const u32x4* cur, u32x4* refill, int g) {
        __builtin_amdgcn_s_waitcnt(kWaitStep);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(refill, g0 + min(g + 2, Gc - 1));
        __builtin_amdgcn_sched_barrier(0);
        lds_compute<F, TM, TN>(acc, cur + la, cur + lb, reinterpret_cast<const uint8_t*>(cur) + lp);
        __builtin_amdgcn_sched_barrier(0);
    };

    issue(st0, g0);
    issue(st1, g0 + min(1, Gc - 1));
    int h = 0;
    for (; h + 2 < Gc; h += 3) {
        step(st0, st2, h);
        step(st1, st0, h + 1);
        step(st2, st1, h + 2);
    }
    if (h < Gc) step(st0, st2, h);
    if (h + 1 < Gc) step(st1, st0, h + 1);
    // No load may still be writing this workgroup's LDS when it exits.
    __builtin_amdgcn_s_waitcnt(kWaitAll);

    // Epilogue through LDS (buffers 0 and 1, half the waves in each, free once
    // every wave's loads have landed and every wave is past its last group):
    // with S > 1 the raw partial sums (the reduction kernel adds them and
    // applies the zero-point compensation and the rescale once), else the
    // outputs.
    static_assert((kW / 2) * 2 * 16 * (TN * 32 + 16) <= kStageVec * 16 &&
                      (kW / 2) * 16 * TN * 64 <= kStageVec * 16,
                  "epilogue regions must fit two buffers");
    __syncthreads();
    uint8_t* half = reinterpret_cast<uint8_t*>(wave < kW / 2 ? st0 : st1);
    const int slot = wave % (kW / 2);
    const int m0 = bm * BM + wm * TM * 16, n0 = (bn * (BN / 16) + wn * TN) * 16;
    if (part)
        staged_partials<TM, TN>(acc, half + slot * (16 * TN * 64), m0, n0, M, N, part + (size_t)split * M * N);
    else
        staged_epilogue<F, TM, TN>(acc, half + slot * (2 * 16 * (TN * 32 + 16)), m0, n0, M, N, s_x, rowsum,
                                   s_c, blob + code_bytes, y, acc_out);
}
#undef QOQ_LDS_PTR

// ---------------------------------------------------------------------------
// Large-block persistent kernel (many 256 x 256 blocks). One 4-wave workgroup
// per CU, one wave per SIMD; wave w computes all 256 rows of the block for 64
// channels (16 x 4 accumulator tiles = all 256 AccVGPRs), so each weight tile
// is unpacked once per 16 matrix-core operations (half the unpack per
// operation of the 128-row waves) and a block moves 48 KB from L2 per group
// for 65536 outputs instead of 32 KB for 32768.
//   - Operands: A by direct buffer-to-LDS loads into four 32 KB stages; B (and
//     the g128 parameter bytes) straight into four named register sets. The
//     loads of group g+3 are issued during group g, so three groups are in
//     flight behind the one being computed.
//   - The weights are the first matrix-core operand, so an accumulator lane
//     holds four consecutive channels of one row (c[n][m] = sum_k w[n,k]
//     x[m,k]); the epilogue stores them as one 8-byte piece per (row tile,
//     channel tile) without an LDS round trip.
//   - Each k-step (64 of a group's 128 inputs) is 16 sub-blocks fenced against
//     the scheduler: the LDS read of activation fragment a+3 (the last three
//     read the next k-step's first fragments), one load of a later group, the
//     four operations of fragment a, and one register of the next k-step's B
//     operands. One barrier per group, between its k-steps, publishes group
//     g+1 and frees the stage of group g-1.
//   - Persistent: with more blocks than CUs, each workgroup walks the blocks of
//     its XCD's contiguous share of the raster, and the pipeline runs through
//     block boundaries (the next block's first groups load during the
//     epilogue). The group count must be a multiple of four (the named stages).
//   - The matrix-core operations are inline asm on accumulators tied to their
//     AccVGPRs: with the builtin, blocks that hold two operations on one
//     accumulator make the register allocator move accumulators through VGPRs.
//     No wait states precede them: every VGPR they read is written by a VALU
//     at least two instructions earlier (B operands are built one k-step ahead,
//     activation fragments come from LDS reads), which a CPU test checks on
//     the generated assembly. A wait state after a VALU is costly here: the
//     s_nop waits for the VALU, so the operation after it issues late. 16 wait
//     states separate the last operation from the epilogue's AccVGPR reads (the
//     compiler inserts 8 for a VALU read of a 16x16x64 result).
//   - The B unpack is spread one VALU instruction per matrix-core operation
//     (a VALU beside an operation in flight is free; several in a row are
//     not); the g128 steps are asm so that the compiler's inline-asm hazard
//     padding does not put an s_nop after a VALU.
__device__ __forceinline__ void mfma_tied(int32x4& c, int32x4 x, int32x4 w) {
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(w), "v"(x));
}

// One k-step of a wave: 16 sub-blocks (see above), each of four fenced
// phases (one matrix-core operation each). af holds activation fragments
// 0..2 of this k-step on entry and of the next one on exit; bcur this k-step's
// B operands on entry and the next one's (built from bsrc with gwsrc, k-step
// KSN) on exit: register R of tile t is built in sub-block 4t + R, one step
// per phase. hook(a, phase) adds work to phase `phase` of sub-block a.
template <int F, int KSN, typename Hook>
__device__ __forceinline__ void big_kstep(int32x4 (&acc)[16][4], u32x4 (&af)[4], int32x4 (&bcur)[4],
                                          const u32x4* lcur, const u32x4* lnext,
                                          const u32x4 (&bsrc)[4][Fmt<F>::kVec], const uint32_t (&gwsrc)[4],
                                          Hook&& hook) {
    int32x4 bn[4];
#pragma unroll
    for (int a = 0; a < 16; ++a) {
        const int t = a / 4, R = a % 4;
        const int na = a + 3;
        af[na % 4] = na < 16 ? lcur[na * 128] : lnext[(na - 16) * 128];
        hook(a, 0);
        const int32x4 xa = __builtin_bit_cast(int32x4, af[a % 4]);
        uint32_t x;
        if constexpr (F == kFmtW8) {
            x = bsrc[t][KSN][R];
        } else {
            const uint32_t w = R < 2 ? (KSN ? bsrc[t][0].z : bsrc[t][0].x) : (KSN ? bsrc[t][0].w : bsrc[t][0].y);
            x = (R & 1) ? (w >> 4) : (w & 0x0F0F0F0Fu);
        }
        // the pins keep each step in its phase (earlier passes would
        // otherwise sink the unpack to the end of the k-step)
        asm volatile("" : "+v"(x));
        mfma_tied(acc[a][0], xa, bcur[0]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (F != kFmtW8) {
            if (R & 1) x &= 0x0F0F0F0Fu;
            asm volatile("" : "+v"(x));
        }
        hook(a, 1);
        mfma_tied(acc[a][1], xa, bcur[1]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (F == kFmtG128)  // q * s + (128 - z s) per byte (see unpack4_g128w)
            asm volatile("v_pk_mad_u16 %0, %0, %1, %1 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "+v"(x) : "v"(gwsrc[t]));
        hook(a, 2);
        mfma_tied(acc[a][2], xa, bcur[2]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (F == kFmtG128) asm volatile("v_xor_b32 %0, 0x80808080, %0" : "+v"(x));
        hook(a, 3);
        mfma_tied(acc[a][3], xa, bcur[3]);
        bn[t][R] = (int)x;
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) bcur[i] = bn[i];
}

#define QOQ_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

template <int F, bool kAccOut>
__global__ __launch_bounds__(256, 1) void k_gemm_big(
    const int8_t* __restrict__ xq, const uint16_t* __restrict__ s_x,
    const int32_t* __restrict__ rowsum, const uint8_t* __restrict__ blob,
    const uint16_t* __restrict__ s_c, int M, int N, int K, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_out, int group_m) {
    constexpr int NS = 4, BM = 256, BN = 256, kW = 4, TN = 4;
    constexpr bool kG128 = Fmt<F>::kG128;
    constexpr bool kZp = Fmt<F>::kZp;
    constexpr int kV = Fmt<F>::kVec;
    constexpr int kAVec = BM * 128 / 16;  // 16-byte vectors of A per group (32 KB)
    constexpr int kADma = kAVec / (kW * 64);
    constexpr int kD = kADma + 4 * kV + (kG128 ? 4 : 0);  // loads per wave per group
    static_assert(2 * kD < 64, "the load counter holds 6 bits");
    constexpr int kWaitMid = (kD & 15) | ((kD >> 4) << 14) | (7 << 4);              // vmcnt(kD) lgkmcnt(0)
    constexpr int kWaitPro = ((2 * kD) & 15) | (((2 * kD) >> 4) << 14) | (7 << 4);  // vmcnt(2 kD) lgkmcnt(0)
    constexpr int kWaitAll = (7 << 4);
    __shared__ u32x4 st0[kAVec];
    __shared__ u32x4 st1[kAVec];
    __shared__ u32x4 st2[kAVec];
    __shared__ u32x4 st3[kAVec];
    __shared__ u32x4 ep[kW * 512];  // 8 KB per wave: the epilogue's scales
    auto stage = [&](auto jc) __attribute__((always_inline)) -> u32x4* {
        constexpr int J = decltype(jc)::value % NS;
        if constexpr (J == 0) return st0;
        else if constexpr (J == 1) return st1;
        else if constexpr (J == 2) return st2;
        else return st3;
    };

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c = lane % 16;
    const int G = K / kGroup;
    const int U = (M + 15) / 16;
    const int tiles = N / 16;
    const int grid_m = (M + BM - 1) / BM, grid_n = (N + BN - 1) / BN;
    const int T = grid_m * grid_n;

    // The blocks of this workgroup. With more blocks than workgroups, XCD x
    // owns the contiguous range [xT/8, (x+1)T/8) of the raster (workgroups are
    // dealt to the XCDs round-robin) and deals it to its workgroups in turn;
    // otherwise each workgroup takes one block.
    int t_first, t_step, n_my;
    if (T > (int)gridDim.x) {
        const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8, slots = gridDim.x / 8;
        const int lo = xcd * T / 8, hi = (xcd + 1) * T / 8;
        t_first = lo + slot;
        t_step = slots;
        n_my = t_first < hi ? (hi - t_first + slots - 1) / slots : 0;
    } else {
        int pid = blockIdx.x;
        if (T % 8 == 0) pid = (pid % 8) * (T / 8) + pid / 8;
        t_first = pid;
        t_step = 0;
        n_my = 1;
    }
    // Raster: groups of group_m block rows, column by column.
    auto block_of = [&](int k, int& bm, int& bn) __attribute__((always_inline)) {
        const int t = t_first + k * t_step;
        const int per_group = group_m * grid_n;
        const int first_m = (t / per_group) * group_m;
        const int gsz = min(grid_m - first_m, group_m);
        bm = first_m + (t % per_group) % gsz;
        bn = (t % per_group) / gsz;
    };

    const size_t code_bytes = code_bytes_of(F, N, K);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)xq, (short)0, (int)((uint32_t)G * (uint32_t)U * 2048u), kBufferConfig);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)blob, (short)0, (int)(uint32_t)code_bytes, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(blob + code_bytes), (short)0, (int)(uint32_t)(kG128 ? N * G : N), kBufferConfig);
    const __amdgpu_buffer_rsrc_t rsx = __builtin_amdgcn_make_buffer_rsrc((void*)s_x, (short)0, 2 * M, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)rowsum, (short)0, kZp ? 4 * M : 0, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc((void*)s_c, (short)0, 2 * N, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rz =
        __builtin_amdgcn_make_buffer_rsrc((void*)(blob + code_bytes), (short)0, kZp ? N : 0, kBufferConfig);
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc((void*)y, (short)0, (int)((uint32_t)M * (uint32_t)N * 2u), kBufferConfig);

    // Load offsets: a per-lane constant part and a per-block scalar part. DMA
    // load v of this wave moves vector (4v + wave) * 64 + lane of the group's
    // A run, i.e. row tile u0 + (4v + wave) / 2 (clamped) and half (4v + wave)
    // % 2; row tiles past the last are clamped and their rows never stored.
    const uint32_t va = (uint32_t)(((wave & 1) * 64 + lane) * 16);
    const uint32_t vb = (uint32_t)lane * 16u;
    // g128 parameter bytes arrive as the aligned dword that holds the lane's
    // byte (a byte load's narrowed loop copies would wait on recent loads)
    const uint32_t vp = (uint32_t)(c & ~3), psh = 8u * (uint32_t)(c & 3);
    const uint32_t a_step = (uint32_t)U * 2048u;
    uint32_t oa[kADma], ob[4], op[4];
    auto load_offsets = [&](int k) __attribute__((always_inline)) {
        int bm, bn;
        block_of(k, bm, bn);
        const int u0 = bm * (BM / 16);
#pragma unroll
        for (int v = 0; v < kADma; ++v) oa[v] = (uint32_t)min(u0 + ((v * kW + wave) >> 1), U - 1) * 2048u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t t = (uint32_t)min(bn * (BN / 16) + wave * TN + i, tiles - 1);
            ob[i] = t * (uint32_t)G * 64u * kV * 16u;
            op[i] = t * (uint32_t)G * 16u;
        }
    };
    uint32_t sa[kADma], sb[4], sp[4];  // scalar offsets of the next refill
    auto refill_offsets = [&](int gl) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < kADma; ++v) sa[v] = oa[v] + (uint32_t)gl * a_step;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sb[i] = ob[i] + (uint32_t)gl * (uint32_t)kV * 1024u;
            sp[i] = op[i] + (uint32_t)gl * 16u;
        }
    };

    u32x4 bq[NS][4][kV];
    uint32_t pq[NS][4];
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) pq[j][i] = 0;
    // Load a (0..15) of a group into stage st / register set j: for g128 the 4
    // parameter dwords first (the oldest loads of the group, so that the word
    // computation one group ahead waits on them alone), then 8 DMA loads of A,
    // then the 4 (8 for INT8 weights) B loads.
    auto load_one = [&](u32x4* st, int j, int a) __attribute__((always_inline)) {
        const int ap = kG128 ? a - 4 : a;
        if (kG128 && a < 4) {
            pq[j][a] = __builtin_amdgcn_raw_buffer_load_b32(rp, (int)vp, (int)sp[a], 0);
        } else if (ap < kADma) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, QOQ_LDS_PTR(st + (ap * kW + wave) * 64), 16, (int)va,
                                                     (int)sa[ap], 0, 0);
        } else if (ap < kADma + 4) {
            const int i = ap - kADma;
#pragma unroll
            for (int v = 0; v < kV; ++v)
                bq[j][i][v] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)vb, (int)(sb[i] + v * 1024u), 0);
        }
    };

    int32x4 acc[16][TN];
#pragma unroll
    for (int a = 0; a < 16; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = int32x4{0, 0, 0, 0};

    uint32_t gw[4], gwn[4], gts[4], gte[4];
    u32x4 af[4];
    int32x4 bcur[4];
    int kl = 0;  // block of the load stream
    // Epilogue scales of the block being computed: s_x and rowsum of 4 of its
    // rows, s_c and zero of 4 consecutive channels per channel tile.
    uint32_t sxw0 = 0, sxw1 = 0, zw[TN];
    uint2 scw[TN];
    u32x4 rsv = {0, 0, 0, 0};
    int m0 = 0, n0 = 0;
    uint8_t* rows = reinterpret_cast<uint8_t*>(ep) + wave * 8192;  // 256 s_x, 256 rowsum, 64 s_c, 64 z

    // Group g (of the block being computed) in stage/set J, g+1 in J+1; the
    // loads of stream position g+3 (the next block's groups when g+3 >= G)
    // refill J-1, which every wave finished with before this group's barrier.
    auto group = [&](auto jc, int g) __attribute__((always_inline)) {
        constexpr int J = decltype(jc)::value % NS;
        constexpr int JN = (J + 1) % NS, JR = (J + NS - 1) % NS;
        const u32x4* cur = stage(std::integral_constant<int, J>{});
        const u32x4* nxt = stage(std::integral_constant<int, JN>{});
        u32x4* ref = stage(std::integral_constant<int, JR>{});
        // k-step 0 hooks: the next group's g128 words, one step per phase in
        // sub-blocks 4t+1 and 4t+2 (the value of group_word: s | ((0x8080 -
        // 257 z s) << 16) with s = hi + 1, z = lo of the byte); the scalar
        // offsets of this group's refill (moving the load stream to the next
        // block when it gets there); this block's epilogue scales in its
        // first group.
        auto hook0 = [&](int a, int ph) __attribute__((always_inline)) {
            if constexpr (kG128) {
                const int t = a / 4;
                if (a % 4 == 1 && (ph == 0 || ph == 2)) {
                    gts[t] = ph == 0 ? __builtin_amdgcn_ubfe(pq[JN][t], psh + 4, 4) : gts[t] + 1u;
                    asm volatile("" : "+v"(gts[t]));
                }
                if ((a % 4 == 1 && (ph == 1 || ph == 3)) || (a % 4 == 2 && ph < 2)) {
                    if (a % 4 == 1) gte[t] = ph == 1 ? __builtin_amdgcn_ubfe(pq[JN][t], psh, 4) : __umul24(gte[t], gts[t]);
                    else gte[t] = ph == 0 ? (gte[t] << 8) + gte[t] : 0x8080u - gte[t];
                    asm volatile("" : "+v"(gte[t]));
                }
                if (a % 4 == 2 && ph == 2) {
                    gwn[t] = (gte[t] << 16) | gts[t];
                    asm volatile("" : "+v"(gwn[t]));
                }
            }
            if (a == 5 && ph == 0) {
                int gl = g + 3;
                if (gl >= G) {
                    gl -= G;
                    if (gl == 0 && kl + 1 < n_my) load_offsets(++kl);
                }
                refill_offsets(gl);
#pragma unroll
                for (int v = 0; v < kADma; ++v) asm volatile("" : "+s"(sa[v]));
#pragma unroll
                for (int i = 0; i < 4; ++i) asm volatile("" : "+s"(sb[i]), "+s"(sp[i]));
            }
            if (a == 9 && ph == 0 && g == 0) {
                sxw0 = __builtin_amdgcn_raw_buffer_load_b32(rsx, (m0 + 4 * lane) * 2, 0, 0);
                sxw1 = __builtin_amdgcn_raw_buffer_load_b32(rsx, (m0 + 4 * lane) * 2 + 4, 0, 0);
                if (kZp) rsv = __builtin_amdgcn_raw_buffer_load_b128(rrs, (m0 + 4 * lane) * 4, 0, 0);
#pragma unroll
                for (int i = 0; i < TN; ++i) {
                    const int nq = n0 + 16 * i + 4 * (lane / 16);
                    const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(rsc, nq * 2, 0, 0);
                    scw[i] = make_uint2(v2[0], v2[1]);
                    zw[i] = kZp ? __builtin_amdgcn_raw_buffer_load_b32(rz, nq, 0, 0) : 0u;
                }
            }
        };
        big_kstep<F, 1>(acc, af, bcur, cur + lane, cur + lane + 64, bq[J], gw, hook0);
        __builtin_amdgcn_s_waitcnt(kWaitMid);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        auto issue_one = [&](int a, int ph) __attribute__((always_inline)) {
            if (ph == 0) load_one(ref, JR, a);
        };
        big_kstep<F, 0>(acc, af, bcur, cur + lane + 64, nxt + lane, bq[JN], gwn, issue_one);
#pragma unroll
        for (int i = 0; i < 4; ++i) gw[i] = gwn[i];
    };

    // Prologue: groups 0..2 of the first block in flight, wait for group 0.
    // (Without blocks, return before any load; with blocks, the block loop
    // needs no guard, which would otherwise pull the prologue's B loads past
    // its DMA loads and leave the wait counts at the group loop's head
    // assuming the wrong order.)
    if (n_my == 0) return;
    __builtin_assume(n_my > 0);
    load_offsets(0);
#pragma unroll
    for (int j = 0; j < NS - 1; ++j) {
        u32x4* st = j == 0 ? st0 : j == 1 ? st1 : st2;
        refill_offsets(j);
#pragma unroll
        for (int a = 0; a < 16; ++a) load_one(st, j, a);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitPro);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) gw[i] = kG128 ? group_word(__builtin_amdgcn_ubfe(pq[0][i], psh, 8)) : 0u;
    af[0] = st0[lane];
    af[1] = st0[lane + 128];
    af[2] = st0[lane + 256];
#pragma unroll
    for (int i = 0; i < 4; ++i) bcur[i] = b_operand<F, 0>(bq[0][i], gw[i]);

    const int jq = lane / 16;
    for (int k = 0; k < n_my; ++k) {
        int bm, bn;
        block_of(k, bm, bn);
        m0 = bm * BM;
        n0 = (bn * (BN / 16) + wave * TN) * 16;
        // G is a positive multiple of NS (the plan's condition), so the loop
        // runs at least once: without a zero-trip path to the epilogue the
        // accumulators are zeroed once per block and reach the epilogue in
        // the registers the loop left them in.
        int h = 0;
        do {
            group(std::integral_constant<int, 0>{}, h);
            group(std::integral_constant<int, 1>{}, h + 1);
            group(std::integral_constant<int, 2>{}, h + 2);
            group(std::integral_constant<int, 3>{}, h + 3);
            // The register allocator may place AccVGPR copies on this loop's
            // edges, and it does not know that the asm above wrote them: give
            // every such copy the wait states a matrix-core result needs.
            asm volatile("s_nop 7\n\ts_nop 7");
            h += NS;
        } while (h < G);
        // Epilogue. 16 wait states after the last matrix-core operation, and
        // every accumulator passed through an empty asm so that no read moves
        // above them. Lane (c, jq) holds rows m0 + 16a + c, channels n0 + 16i +
        // 4jq .. +3. The scales go through the wave's LDS region. Two lane
        // swaps per register turn the four-channel pieces of a tile pair into
        // eight consecutive channels per lane, so each (row tile, tile pair)
        // leaves as one 16-byte store per lane (16 rows x 64 bytes; 8-byte
        // stores of 16 rows x 32 bytes drained at about 4 TB/s, these at 6.5).
        // Stores outside the output get an out-of-range offset (no branches).
        asm volatile("s_nop 7\n\ts_nop 7");
#pragma unroll
        for (int a = 0; a < 16; ++a)
#pragma unroll
            for (int b = 0; b < TN; ++b) asm volatile("" : "+a"(acc[a][b]));
        *reinterpret_cast<uint2*>(rows + lane * 8) = make_uint2(sxw0, sxw1);
        if (kZp) *reinterpret_cast<u32x4*>(rows + 512 + lane * 16) = rsv;
#pragma unroll
        for (int i = 0; i < TN; ++i) {
            *reinterpret_cast<uint2*>(rows + 1536 + (16 * i + 4 * jq) * 2) = scw[i];
            if (kZp) *reinterpret_cast<uint32_t*>(rows + 1664 + 16 * i + 4 * jq) = zw[i];
        }
        if constexpr (kAccOut) {
            const __amdgpu_buffer_rsrc_t racc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)acc_out, (short)0, (int)((uint32_t)M * (uint32_t)N * 4u), kBufferConfig);
#pragma unroll
            for (int a = 0; a < 16; ++a) {
                const int m = m0 + 16 * a + c;
                const int rs = kZp ? *reinterpret_cast<const int*>(rows + 512 + (16 * a + c) * 4) : 0;
#pragma unroll
                for (int i = 0; i < TN; ++i) {
                    const int n = n0 + 16 * i + 4 * jq;
                    const uint32_t zz = kZp ? *reinterpret_cast<const uint32_t*>(rows + 1664 + 16 * i + 4 * jq) : 0u;
                    u32x4 r;
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        r[v] = (uint32_t)(acc[a][i][v] - (kZp ? (int)((zz >> (8 * v)) & 0xFFu) * rs : 0));
                    const uint32_t off = (m < M && n < N) ? ((uint32_t)m * (uint32_t)N + (uint32_t)n) * 4u : 0x80000000u;
                    __builtin_amdgcn_raw_buffer_store_b128(r, racc, (int)off, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // The lane's 4 TN channel scales as fp32, once per block (converting
        // them per row tile was a sixth of the epilogue's instructions).
        float scf[TN][4];
#pragma unroll
        for (int i = 0; i < TN; ++i) {
            const uint2 scq = *reinterpret_cast<const uint2*>(rows + 1536 + (16 * i + 4 * jq) * 2);
#pragma unroll
            for (int v = 0; v < 4; ++v) scf[i][v] = h2f(((v < 2 ? scq.x : scq.y) >> (16 * (v & 1))) & 0xFFFFu);
        }
#pragma unroll
        for (int a = 0; a < 16; ++a) {
            const int m = m0 + 16 * a + c;
            const float sx = h2f(*reinterpret_cast<const uint16_t*>(rows + (16 * a + c) * 2));
            const int rs = kZp ? *reinterpret_cast<const int*>(rows + 512 + (16 * a + c) * 4) : 0;
            uint32_t d[TN][2];  // FP16 pairs: channels 4jq, 4jq+1 and 4jq+2, 4jq+3 of tile i
#pragma unroll
            for (int i = 0; i < TN; ++i) {
                const uint32_t zz = kZp ? *reinterpret_cast<const uint32_t*>(rows + 1664 + 16 * i + 4 * jq) : 0u;
                int r[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    r[v] = acc[a][i][v];
                    if (kZp) r[v] -= (int)((zz >> (8 * v)) & 0xFFu) * rs;
                }
                d[i][0] = output_pair(r[0], r[1], sx, scf[i][0], scf[i][1]);
                d[i][1] = output_pair(r[2], r[3], sx, scf[i][2], scf[i][3]);
            }
#pragma unroll
            for (int p = 0; p < TN; p += 2) {
                // Rows of 16 lanes (jq) hold quads 0..3 of tiles p (X) and p+1
                // (Y). The 32-lane swap gives [Xq0 Xq1 Yq0 Yq1] / [Xq2 Xq3 Yq2
                // Yq3], the 16-lane swap [Xq0 Xq2 Yq0 Yq2] / [Xq1 Xq3 Yq1 Yq3]:
                // row jq then holds channels 8jq .. 8jq+7 of the pair.
                u32x4 o;
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const auto h32 = __builtin_amdgcn_permlane32_swap(d[p][k], d[p + 1][k], false, false);
                    const auto h16 = __builtin_amdgcn_permlane16_swap(h32[0], h32[1], false, false);
                    o[k] = h16[0];
                    o[2 + k] = h16[1];
                }
                const int n = n0 + 16 * p + 8 * jq;
                const uint32_t off = (m < M && n < N) ? ((uint32_t)m * (uint32_t)N + (uint32_t)n) * 2u : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b128(o, ry, (int)off, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int a = 0; a < 16; ++a)
#pragma unroll
            for (int b = 0; b < TN; ++b) acc[a][b] = int32x4{0, 0, 0, 0};
    }
    // No load may still be writing this workgroup's LDS when it exits.
    __builtin_amdgcn_s_waitcnt(kWaitAll);
}
#undef QOQ_LDS_PTR

// ---------------------------------------------------------------------------
// Pipelined decode kernel (M <= 64): weight streaming at HBM rate.
//
// A workgroup of W waves owns NT 16-channel tiles and the whole K; wave w takes
// the contiguous groups [G*w/W, G*(w+1)/W) and keeps all 16*MB rows and its NT
// tiles in registers, so an activation fragment is reused NT times and a
// weight fragment MB times. The loads run R groups ahead through a ring of R
// register sets: the loop body is unrolled R times so that every set has a
// fixed name, every load and every matrix-core step is unconditional (a load
// guarded by a branch would be sunk to its use by the compiler), and every
// wait on the in-order load counter is static. A prefetch past the wave's last
// group gets an out-of-range buffer offset: the load returns zeros without a
// memory request and is never consumed. Groups left over when the count is not
// a multiple of R run one at a time after the pipelined part. The waves' sums
// are added with LDS integer atomics (exact and order-free), then each wave
// runs the epilogue for a share of the (tile, row block) pairs.
constexpr uint32_t kOutOfRange = 0x80000000u;

template <int F, int MB, int NT, int PL>
__device__ __forceinline__ void stream_load(u32x4 (&bq)[NT][Fmt<F>::kVec], uint32_t (&pq)[NT],
                                            int32x4 (&aq)[MB][2], __amdgpu_buffer_rsrc_t rb,
                                            __amdgpu_buffer_rsrc_t rp, __amdgpu_buffer_rsrc_t ra,
                                            const uint32_t (&b_off)[NT],
                                            const uint32_t (&p_off)[NT],
                                            const uint32_t (&a_off)[MB], int gi, bool valid,
                                            uint32_t a_step) {
    constexpr int kV = Fmt<F>::kVec;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const uint32_t ob = valid ? b_off[i] + (uint32_t)gi * (1024u * kV) : kOutOfRange;
        bq[i][0] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)ob, 0, 0);
        if constexpr (kV == 2) bq[i][1] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)ob, 1024, 0);
        if (Fmt<F>::kG128 && PL == 0) {
            const uint32_t op = valid ? p_off[i] + (uint32_t)gi * 16u : kOutOfRange;
            pq[i] = __builtin_amdgcn_raw_buffer_load_b8(rp, (int)op, 0, 0);
        }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const uint32_t oa = valid ? a_off[mb] + (uint32_t)gi * a_step : kOutOfRange;
        aq[mb][0] = __builtin_bit_cast(int32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)oa, 0, 0));
        aq[mb][1] =
            __builtin_bit_cast(int32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)oa, 1024, 0));
    }
}

// The parameter byte of tile i and group h of a wave (h counted from the
// wave's first group) from the wave's parameter dwords pd: dword d = (h NT +
// i) 4 + q of the wave's run sits in lane d % 64 of pd[d / 64] and holds
// channels 4q .. 4q + 3, so lane c takes it from lane (h NT + i) 4 + c / 4
// with one cross-lane read (ds_bpermute, no memory access).
template <int PL, int NT>
__device__ __forceinline__ uint32_t param_byte(const uint32_t (&pd)[PL], int i, int h, int c) {
    const int base = (h * NT + i) * 4;  // wave-uniform, a multiple of 4
    const int blk = base >> 6;
    uint32_t w = pd[0];
#pragma unroll
    for (int k = 1; k < PL; ++k) w = blk == k ? pd[k] : w;
    const int src = (base & 63) + (c >> 2);
    const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)w);
    return (v >> ((c & 3) * 8)) & 0xFFu;
}

template <int F, int MB, int NT, int PL>
__device__ __forceinline__ void stream_compute(int32x4 (&acc)[NT][MB],
                                               const u32x4 (&bq)[NT][Fmt<F>::kVec],
                                               const uint32_t (&pq)[NT],
                                               const int32x4 (&aq)[MB][2],
                                               const uint32_t (&pd)[PL > 0 ? PL : 1], int h, int c) {
    // the group word from the parameter byte in a few integer operations (a
    // table in LDS would need a barrier before the first group)
    uint32_t gw[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        if constexpr (Fmt<F>::kG128 && PL > 0)
            gw[i] = group_word(param_byte<PL, NT>(pd, i, h, c));
        else
            gw[i] = Fmt<F>::kG128 ? group_word(pq[i] & 0xFFu) : 0u;
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int32x4 b0 = b_operand<F, 0>(bq[i], gw[i]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[i][mb] = mfma16x16x64(aq[mb][0], b0, acc[i][mb]);
        const int32x4 b1 = b_operand<F, 1>(bq[i], gw[i]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[i][mb] = mfma16x16x64(aq[mb][1], b1, acc[i][mb]);
    }
}

template <int F, int MB, int NT, int R, int W, int PL>
__global__ __launch_bounds__(W * 64) void k_gemm_stream(
    const int8_t* __restrict__ xq, const uint16_t* __restrict__ s_x,
    const int32_t* __restrict__ rowsum, const uint8_t* __restrict__ blob,
    const uint16_t* __restrict__ s_c, int M, int N, int K, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_out) {
    constexpr int kPairs = NT * MB;
    constexpr int kThr = W * 64;
    // The waves' partial tiles are summed through LDS: each wave writes its
    // own slice and the epilogue adds the slices in wave order when they fit
    // in 96 KB (then nothing needs zeroing and no barrier precedes the first
    // loads); otherwise the waves add into one zeroed copy.
    // red[(s * kPairs + p) * 64 + lane]: the four accumulator rows of pair p
    // held by a lane, one 16-byte LDS access per lane and pair, slice s.
    constexpr bool kSlices = W * kPairs * kWave * 16 <= 96 * 1024;
    __shared__ int32x4 red[(kSlices ? W : 1) * kPairs * kWave];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int G = K / kGroup;
    const int tiles = N / 16;
    const int U = (M + 15) / 16;
    const int c = lane % 16, j = lane / 16;
    // Block b covers channel tiles [NT*nb, NT*nb + NT) and row tiles
    // [MB*mh, MB*mh + MB), with b = mh * nblk + nb: the row halves of one
    // channel band run on the same XCD (blocks are dealt to the XCDs
    // round-robin), so its weights come from HBM once.
    const int nblk = (tiles + NT - 1) / NT;
    const int mh = blockIdx.x / nblk;
    const int nb = blockIdx.x - mh * nblk;
    const int u0 = mh * MB;

    constexpr bool kG128 = Fmt<F>::kG128;
    constexpr int kV = Fmt<F>::kVec;
    const int g0 = G * wave / W;
    const int count = G * (wave + 1) / W - g0;

    const size_t code_bytes = code_bytes_of(F, N, K);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)xq, (short)0, (int)((uint32_t)G * (uint32_t)U * 2048u), kBufferConfig);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)blob, (short)0, (int)(uint32_t)code_bytes, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(blob + code_bytes), (short)0, (int)(uint32_t)(kG128 ? N * G : N), kBufferConfig);

    // Per-lane byte offsets of this wave's first group; out-of-range tiles and
    // row blocks are clamped (their results are never stored).
    uint32_t b_off[NT], p_off[NT], a_off[MB];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int t = min(nb * NT + i, tiles - 1);
        b_off[i] = ((uint32_t)t * (uint32_t)G + (uint32_t)g0) * (1024u * kV) + (uint32_t)lane * 16u;
        p_off[i] = ((uint32_t)t * (uint32_t)G + (uint32_t)g0) * 16u + (uint32_t)c;
    }
    const uint32_t a_step = (uint32_t)U * 2048u;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        a_off[mb] = (uint32_t)g0 * a_step + (uint32_t)min(u0 + mb, U - 1) * 2048u + (uint32_t)lane * 16u;

    int32x4 acc[NT][MB];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[i][mb] = int32x4{0, 0, 0, 0};

    u32x4 bq[R][NT][kV];
    uint32_t pq[R][NT];
    int32x4 aq[R][MB][2];
    const int main_count = count / R * R;
    // The ring's first loads go out before anything else: the epilogue's
    // scale loads (and the LDS set-up, if any) then overlap their latency.
#pragma unroll
    for (int r = 0; r < R - 1; ++r)
        stream_load<F, MB, NT, PL>(bq[r], pq[r], aq[r], rb, rp, ra, b_off, p_off, a_off, r,
                                   r < main_count, a_step);
    // g128 parameters: with PL > 0 the wave's NT x count parameter bytes
    // arrive as 4 bytes per lane per load (dword d = (h NT + i) 4 + q holds
    // channels 4q .. 4q + 3 of group g0 + h of tile i), PL loads in all
    // instead of one 1-byte load per tile and group; param_byte() hands each
    // lane its byte. Dwords past the wave's groups get an out-of-range offset
    // (no memory request).
    uint32_t pd[PL > 0 ? PL : 1];
    if constexpr (kG128 && PL > 0) {
        uint32_t off[PL];
#pragma unroll
        for (int L = 0; L < PL; ++L) {
            const int d = 64 * L + lane;
            const int hh = d / (4 * NT), i = (d >> 2) % NT;
            const int t = min(nb * NT + i, tiles - 1);
            off[L] = hh < count ? ((uint32_t)t * (uint32_t)G + (uint32_t)(g0 + hh)) * 16u + 4u * (uint32_t)(d & 3)
                                : kOutOfRange;
        }
        // all offsets first, then the loads back to back (interleaving them
        // made the compiler reuse a load's destination as a temporary, which
        // costs a wait for that load)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int L = 0; L < PL; ++L) pd[L] = __builtin_amdgcn_raw_buffer_load_b32(rp, (int)off[L], 0, 0);
    }
    // Operands of this wave's epilogue pairs (p = wave + e W), read now (after
    // the first weight loads, and kept as raw bits until the epilogue, so that
    // nothing waits for them early) so that the stores at the end wait on no
    // global load.
    __builtin_amdgcn_sched_barrier(0);
    constexpr int kEp = (kPairs + W - 1) / W;
    uint32_t ep_sc[kEp], ep_sx[kEp][4];
    int ep_z[kEp], ep_rs[kEp][4];
#pragma unroll
    for (int e = 0; e < kEp; ++e) {
        const int p = wave + e * W;
        const int t = min(nb * NT + min(p, kPairs - 1) / MB, tiles - 1);
        const int n = 16 * t + c;
        const int mrow = 16 * (u0 + min(p, kPairs - 1) % MB) + 4 * j;
        ep_sc[e] = s_c[n];
        ep_z[e] = Fmt<F>::kZp ? (int)blob[code_bytes + n] : 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = min(mrow + v, M - 1);
            ep_sx[e][v] = s_x[m];
            ep_rs[e][v] = Fmt<F>::kZp ? rowsum[m] : 0;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!kSlices) {
        for (int i = threadIdx.x; i < kPairs * kWave; i += kThr) red[i] = int32x4{0, 0, 0, 0};
        __syncthreads();
    }
    for (int h = 0; h < main_count; h += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int nxt = h + r + R - 1;
            stream_load<F, MB, NT, PL>(bq[(r + R - 1) % R], pq[(r + R - 1) % R],
                                       aq[(r + R - 1) % R], rb, rp, ra, b_off, p_off, a_off, nxt,
                                       nxt < main_count, a_step);
            // the look-ahead loads leave before this group's unpack, which
            // would otherwise be scheduled first and wait for every load
            __builtin_amdgcn_sched_barrier(0);
            stream_compute<F, MB, NT, PL>(acc, bq[r], pq[r], aq[r], pd, h + r, c);
        }
    }
    for (int h = main_count; h < count; ++h) {
        stream_load<F, MB, NT, PL>(bq[0], pq[0], aq[0], rb, rp, ra, b_off, p_off, a_off, h, true,
                                   a_step);
        stream_compute<F, MB, NT, PL>(acc, bq[0], pq[0], aq[0], pd, h, c);
    }

    // Sum the waves' partial tiles in LDS.
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int idx = (i * MB + mb) * kWave + lane;
            if (kSlices) {
                red[wave * kPairs * kWave + idx] = acc[i][mb];
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v) atomicAdd(reinterpret_cast<int*>(red + idx) + v, acc[i][mb][v]);
            }
        }
    __syncthreads();

#pragma unroll
    for (int e = 0; e < kEp; ++e) {
        const int p = wave + e * W;
        if (p >= kPairs) break;
        const int i = p / MB, mb = p % MB;
        const int t = nb * NT + i;
        if (t >= tiles) continue;
        const int n = 16 * t + c;
        const int m_first = 16 * (u0 + mb) + 4 * j;
        // all slices' reads issued together, then added in wave order
        int32x4 r4;
        if (kSlices) {
            int32x4 part[W];
#pragma unroll
            for (int w2 = 0; w2 < W; ++w2) part[w2] = red[(w2 * kPairs + p) * kWave + lane];
            r4 = part[0];
#pragma unroll
            for (int w2 = 1; w2 < W; ++w2) r4 += part[w2];
        } else {
            r4 = red[p * kWave + lane];
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int m = m_first + v;
            if (m < M) {
                int r = r4[v];
                if (Fmt<F>::kZp) r -= ep_z[e] * ep_rs[e][v];
                const size_t o = (size_t)m * N + n;
                if (acc_out) acc_out[o] = r;
                y[o] = output_value(r, h2f(ep_sx[e][v]), h2f(ep_sc[e]));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Plans.

constexpr int kCUs = 256;

enum Kind { kSimple = 0, kTile = 2, kWide = 3, kStream = 4, kLds = 5, kBig = 6 };

struct Plan {
    int kind = kSimple;
    int mb = 0, nt = 0, r = 2, w = 8;  // stream kernel: row tiles, channel tiles, ring depth, waves,
    int mgrid = 1;                     //   workgroups along M
    int pl = 0;                        //   and g128 parameter loads per wave (0: one per tile and group)
    int bn = 256;                      // 16-row-wave tiled and LDS-pipelined kernels: 128 x bn blocks
    int s = 1;                         //   and its K splits (partial sums in the workspace)
    int64_t ws_bytes = 0;
    int group_m = 4;                   // wide and LDS-pipelined kernels: block rows per XCD raster group
    int64_t nblk = 0;
};

// The buffer-load kernels form 32-bit byte offsets, and mark prefetches past
// the end with offset 2^31: every real offset must stay below that.
bool fits_buffer_offsets(int fmt, int64_t M, int64_t N, int64_t K) {
    const int64_t G = K / kGroup, U = (M + 15) / 16;
    return G * U * 2048 < (int64_t(1) << 31) &&
           (int64_t)code_bytes_of(fmt, N, K) < (int64_t(1) << 31) && N * G < (int64_t(1) << 31);
}

// Measured on MI355X over the Llama-3-8B and Qwen1.5-72B layers:
//   M <= 64: the streaming kernel; three 16-channel tiles per workgroup once
//     that still leaves two workgroups per compute unit, else two; for 16 rows
//     a two-deep ring and 8 waves, for 17..32 rows 16 waves that each load one
//     group at a time (the activation bytes then dominate, and more waves with
//     fewer groups each beat a deeper ring, which would not fit the registers
//     of 16 waves); for 33..64 rows two 32-row workgroups per band of three
//     channel tiles.
//   64 < M <= 256, K <= 16384, 4-bit weights, when 64-row workgroups over
//     bands of four channel tiles make between 3/4 and one round of the
//     compute units: the streaming kernel with 8 waves that each load one
//     group at a time (Qwen1.5-72B o_proj at M = 128 22-25% faster and
//     Llama-3-8B down at M = 256 16% faster than the split LDS-pipelined
//     plan, with no partial sums; with more workgroups (qkv and gate_up) the
//     activation re-reads made it 10-60% slower, and at K = 24576 it tied);
//   M > 64 otherwise, counting 128 x 256 blocks (nb128):
//     nb128 <= 256: the LDS-pipelined kernel with 128-row blocks, one 8-wave
//       workgroup per compute unit; below 128 blocks, with a workspace, split
//       over K into min(8, 256 / nb128) ranges (the split sums are added by
//       the reduction kernel); without one, M >= 512 runs unsplit and
//       M < 512 takes the 16-row-wave tiled kernel; for 4-bit weights with
//       M < 512 and K <= 16384, 128 x 128 blocks of two 4-wave workgroups
//       per compute unit instead, split in powers of two;
//     nb128 > 256, M >= 512: the wide-wave tiled kernel, two 4-wave
//       workgroups of 128 x 256 per compute unit (256-row blocks of the
//       LDS-pipelined kernel were 3-15% slower on the Llama-3-8B o_proj at
//       M = 4096 and the Qwen1.5-72B qkv at M = 1024, and 2-3% faster on the
//       Qwen1.5-72B gate_up at M = 1024); M < 512: the LDS-pipelined kernel
//       with 128-row blocks;
//     at least one round of 256 x 256 blocks (whole or not), with the group
//       count a multiple of 4: the large-block persistent kernel (against
//       the wide kernel: Llama-3-8B gate_up at M = 4096 15% faster in g128;
//       Qwen1.5-72B qkv at M = 1024, 1.5 rounds, 11%). Below one round it
//       would leave CUs idle.
// Shapes whose offsets do not fit the buffer-load kernels take the reference
// kernel (M <= 64) or the 16-row-wave tiled kernel, split over K (M > 64).
// Workgroups of the streaming kernel with 64-row blocks and bands of four
// channel tiles.
int64_t stream64_grid(int64_t M, int64_t N) { return ((M + 63) / 64) * ((N / 16 + 3) / 4); }

Plan plan_gemm(int fmt, int64_t M, int64_t N, int64_t K, bool have_ws) {
    Plan p;
    const int64_t tiles = N / 16;
    const bool fits = fits_buffer_offsets(fmt, M, N, K);
    const int64_t nb128 = ((M + 127) / 128) * ((N + 255) / 256);  // 128 x 256 blocks
    if (M <= 64) {
        if (fits) {
            p.kind = kStream;
            p.nt = (tiles + 2) / 3 >= 2 * kCUs ? 3 : 2;
            if (M <= 16) {
                // g128 keeps 8 waves (two groups in flight each), whose
                // parameter bytes fit two 4-byte lane loads; the other formats
                // stream with 4 waves, four groups in flight each
                p.mb = 1;
                p.r = fmt == kFmtG128 ? 2 : 4;
                p.w = fmt == kFmtG128 ? 8 : 4;
            } else if (M <= 32) {
                p.mb = 2;
                p.r = 1;
                p.w = 16;
            } else {
                // Two workgroups along M (32 rows each) per band of three
                // channel tiles: every compute unit gets work, and each one
                // re-reads half the activations.
                p.mb = 2;
                p.nt = 3;
                p.r = 1;
                p.w = 2 * ((tiles + 2) / 3) <= kCUs ? 16 : 8;
            }
        }
    } else if (fits && M <= 256 && K <= 16384 && fmt != kFmtW8 &&
               4 * stream64_grid(M, N) >= 3 * kCUs && stream64_grid(M, N) <= kCUs) {
        // 64-row workgroups of the streaming kernel over bands of four
        // channel tiles, when they make between 3/4 and one round
        p.kind = kStream;
        p.mb = 4;
        p.nt = 4;
        p.r = 1;
        p.w = 8;
    } else if (fits && (M >= 512 || nb128 >= kCUs / 2 || have_ws)) {
        // 128 x 256 blocks that fill at most one round of the compute units
        // run as one 8-wave workgroup per CU (two waves per SIMD even then),
        // split over K (at least two groups per split, at most 8 splits) until
        // they fill about one round; with more blocks, the wide kernel's two
        // 4-wave workgroups per CU.
        p.kind = nb128 > kCUs && M >= 512 ? kWide : kLds;
        // At least one round of 256 x 256 blocks with the group count a
        // multiple of four: the large-block persistent kernel (also with a
        // partial last round: Qwen1.5-72B qkv at M = 1024, 1.5 rounds, ran
        // 11% faster on it than on the wide kernel).
        const int64_t nb256 = ((M + 255) / 256) * ((N + 255) / 256);
        if (nb256 >= kCUs && (K / kGroup) % 4 == 0 && M * N * 2 < (int64_t(1) << 31)) {
            p.kind = kBig;
            p.group_m = 8;
        }
        if (p.kind == kLds && M < 512 && K <= 16384 && fmt != kFmtW8) {
            // Below 512 rows, 4-bit weights, K <= 16384: 128 x 128 blocks, two
            // 4-wave workgroups per CU, split over K in the smallest power of
            // two (at most 8, at least two groups per split) that gives one
            // round of workgroups. Against 128 x 256 blocks of 8 waves this
            // halves the split count and so the partial-sum traffic (Qwen1.5-
            // 72B o_proj at M = 128: 6-12% faster, Llama-3-8B gate_up and down
            // at M = 256: 5-8%); with longer K (Qwen1.5-72B down, K = 24576)
            // the partial sums weigh less and 8-wave blocks were 2-10% faster.
            p.bn = 128;
            const int64_t nb = ((M + 127) / 128) * ((N + 127) / 128);
            while (p.s < 8 && nb * p.s < kCUs && 2 * p.s <= K / kGroup / 2) p.s *= 2;
        } else if (p.kind == kLds && nb128 < kCUs / 2) {
            p.s = (int)std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(8, kCUs / nb128), K / kGroup / 2));
        }
    } else {
        p.kind = kTile;
        const int64_t gm128 = (M + 127) / 128, gn256 = (N + 255) / 256, gn128 = (N + 127) / 128;
        // 128 x 256 blocks once they alone cover the compute units, else
        // 128 x 128; if even those are fewer than the compute units, split K
        // (at least two groups per split) until they cover them. The partial
        // sums then cost 8 * S * M * N bytes of traffic, small next to the
        // GEMM for these shapes.
        p.bn = gm128 * gn256 >= kCUs ? 256 : 128;
        const int64_t nblk = gm128 * (p.bn == 256 ? gn256 : gn128);
        if (nblk < kCUs)
            p.s = (int)std::min<int64_t>(std::min<int64_t>(8, (kCUs + nblk - 1) / nblk), K / kGroup / 2);
        if (p.s < 1) p.s = 1;
    }
    if (p.kind == kStream) {
        const int64_t U = (M + 15) / 16;
        p.mgrid = (int)((U + p.mb - 1) / p.mb);
        p.nblk = (tiles + p.nt - 1) / p.nt;
        // g128: a wave's NT x (groups per wave) parameter bytes in 4-byte lane
        // loads, 64 lanes per load, when that takes at most 2 loads (a third
        // load made the compiler wait for all of them before the first group)
        const int64_t per_wave = (K / kGroup + p.w - 1) / p.w;
        const int64_t loads = (p.nt * per_wave + 15) / 16;
        p.pl = fmt != kFmtG128 || loads > 2 ? 0 : (int)loads;
    }
    if (p.kind != kTile && p.kind != kLds) p.s = 1;
    p.ws_bytes = p.s > 1 ? (int64_t)p.s * M * N * 4 : 0;
    if (!have_ws) p.s = 1;
    return p;
}

struct GemmArgs {
    int32_t* part;  // split-K partial sums (workspace), or null
    const int8_t* xq;
    const uint16_t* s_x;
    const int32_t* rowsum;
    const uint8_t* blob;
    const uint16_t* s_c;
    int M, N, K;
    uint16_t* y;
    int32_t* acc_out;
    hipStream_t stream;
    int group_m;
};

template <int F, int MB, int NT, int R, int W, int PL>
void launch_stream_t(const Plan& p, const GemmArgs& a) {
    hipLaunchKernelGGL((k_gemm_stream<F, MB, NT, R, W, PL>), dim3((unsigned)(p.nblk * p.mgrid)),
                       dim3(W * 64), 0, a.stream, a.xq, a.s_x, a.rowsum, a.blob, a.s_c, a.M, a.N, a.K,
                       a.y, a.acc_out);
}

template <int F, int MB, int NT, int R, int W>
void launch_stream_pl(const Plan& p, const GemmArgs& a) {
    if constexpr (F == kFmtG128) {
        if (p.pl == 1) { launch_stream_t<F, MB, NT, R, W, 1>(p, a); return; }
        if (p.pl == 2) { launch_stream_t<F, MB, NT, R, W, 2>(p, a); return; }
    }
    launch_stream_t<F, MB, NT, R, W, 0>(p, a);
}

template <int F, int MB, int NT>
void launch_stream_rw(const Plan& p, const GemmArgs& a) {
    if (p.r == 1) launch_stream_pl<F, MB, NT, 1, 16>(p, a);
    else if (p.r == 4) launch_stream_pl<F, MB, NT, 4, 4>(p, a);
    else launch_stream_pl<F, MB, NT, 2, 8>(p, a);
}

template <int F, int MB>
void launch_stream_nt(const Plan& p, const GemmArgs& a) {
    if (p.nt == 3) launch_stream_rw<F, MB, 3>(p, a);
    else launch_stream_rw<F, MB, 2>(p, a);
}

template <int F>
void launch_stream(const Plan& p, const GemmArgs& a) {
    if constexpr (F != kFmtW8) {
        if (p.mb == 4) {
            launch_stream_pl<F, 4, 4, 1, 8>(p, a);
            return;
        }
    }
    if (p.mb == 1) launch_stream_nt<F, 1>(p, a);
    else launch_stream_nt<F, 2>(p, a);
}

template <int F, int BM, int BN, int WM, int WN>
void launch_tile_t(const Plan& p, const GemmArgs& a) {
    const unsigned blocks = (unsigned)(((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * p.s);
    int32_t* part = p.s > 1 ? a.part : nullptr;
    hipLaunchKernelGGL((k_gemm_tile<F, BM, BN, WM, WN>), dim3(blocks), dim3(WM * WN * 64), 0,
                       a.stream, a.xq, a.s_x, a.rowsum, a.blob, a.s_c, a.M, a.N, a.K, a.y,
                       a.acc_out, p.s, part);
    if (part) {
        const int64_t quads = (int64_t)a.M * a.N / 4;
        hipLaunchKernelGGL(k_splitk_reduce<F>, dim3((unsigned)((quads + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, a.stream, part, p.s, a.s_x, a.rowsum,
                           a.blob + code_bytes_of(F, a.N, a.K), a.s_c, a.M, a.N, a.y, a.acc_out);
    }
}

template <int F, int BM, int BN, int WN>
void launch_wide_t(const GemmArgs& a) {
    const unsigned blocks = (unsigned)(((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN));
    hipLaunchKernelGGL((k_gemm_wide<F, BM, BN, WN>), dim3(blocks), dim3(WN * 64), 0, a.stream,
                       a.xq, a.s_x, a.rowsum, a.blob, a.s_c, a.M, a.N, a.K, a.y, a.acc_out,
                       a.group_m);
}

template <int F, int BM, int WM, int BN = 256, int kW = 8>
void launch_lds_t(const Plan& p, const GemmArgs& a) {
    const unsigned blocks = (unsigned)(((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * p.s);
    int32_t* part = p.s > 1 ? a.part : nullptr;
    hipLaunchKernelGGL((k_gemm_lds<F, BM, WM, BN, kW>), dim3(blocks), dim3(kW * 64), 0, a.stream, a.xq, a.s_x,
                       a.rowsum, a.blob, a.s_c, a.M, a.N, a.K, a.y, a.acc_out, a.group_m, p.s, part);
    if (part) {
        const int64_t quads = (int64_t)a.M * a.N / 4;
        hipLaunchKernelGGL(k_splitk_reduce<F>, dim3((unsigned)((quads + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, a.stream, part, p.s, a.s_x, a.rowsum,
                           a.blob + code_bytes_of(F, a.N, a.K), a.s_c, a.M, a.N, a.y, a.acc_out);
    }
}

template <int F>
void launch_big(const GemmArgs& a) {
    const int64_t T = (int64_t)((a.M + 255) / 256) * ((a.N + 255) / 256);
    const unsigned blocks = (unsigned)std::min<int64_t>(T, kCUs);
    if (a.acc_out)
        hipLaunchKernelGGL((k_gemm_big<F, true>), dim3(blocks), dim3(256), 0, a.stream, a.xq, a.s_x, a.rowsum,
                           a.blob, a.s_c, a.M, a.N, a.K, a.y, a.acc_out, a.group_m);
    else
        hipLaunchKernelGGL((k_gemm_big<F, false>), dim3(blocks), dim3(256), 0, a.stream, a.xq, a.s_x, a.rowsum,
                           a.blob, a.s_c, a.M, a.N, a.K, a.y, a.acc_out, a.group_m);
}

template <int F>
void launch_simple(const GemmArgs& a) {
    const dim3 grid((unsigned)((a.N / 16 + 3) / 4), (unsigned)((a.M + 63) / 64));
    hipLaunchKernelGGL(k_gemm_simple<F>, grid, dim3(kThreads), 0, a.stream, a.xq, a.s_x,
                       a.rowsum, a.blob, a.s_c, a.M, a.N, a.K, a.y, a.acc_out);
}

template <int F>
void launch_plan(const Plan& p, const GemmArgs& a) {
    switch (p.kind) {
        case kStream:
            launch_stream<F>(p, a);
            break;
        case kWide:
            launch_wide_t<F, 128, 256, 4>(a);
            break;
        case kBig:
            // the INT32 sums' buffer offsets must fit too; else the wide kernel
            if (a.acc_out && (int64_t)a.M * a.N * 4 >= (int64_t(1) << 31)) {
                const GemmArgs w{a.part, a.xq, a.s_x, a.rowsum, a.blob, a.s_c, a.M, a.N, a.K, a.y, a.acc_out,
                                 a.stream, 4};
                launch_wide_t<F, 128, 256, 4>(w);
            } else {
                launch_big<F>(a);
            }
            break;
        case kLds:
            if constexpr (F != kFmtW8) {
                // 128 x 128 blocks: 128 x 32 waves for g128 (each weight tile
                // unpacked once), 64 x 64 waves for per-channel codes (no
                // unpack to repeat, half the activation reads from LDS)
                if (p.bn == 128) {
                    if (F == kFmtPC) launch_lds_t<F, 128, 2, 128, 4>(p, a);
                    else launch_lds_t<F, 128, 1, 128, 4>(p, a);
                    break;
                }
            }
            launch_lds_t<F, 128, 1>(p, a);
            break;
        case kTile:
            if (p.bn == 256) launch_tile_t<F, 128, 256, 2, 4>(p, a);
            else launch_tile_t<F, 128, 128, 2, 2>(p, a);
            break;
        default:
            launch_simple<F>(a);
            break;
    }
}

}  // namespace

int64_t gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K) {
    return plan_gemm(fmt, M, N, K, true).ws_bytes;
}

void launch_gemm(int fmt, const int8_t* xq, const uint16_t* s_x, const int32_t* rowsum,
                 const uint8_t* blob, const uint16_t* s_c, int64_t M, int64_t N, int64_t K,
                 uint16_t* y, int32_t* acc_out, void* ws, hipStream_t stream) {
    const Plan p = plan_gemm(fmt, M, N, K, ws != nullptr);
    const GemmArgs a{static_cast<int32_t*>(ws), xq, s_x, rowsum, blob, s_c, (int)M, (int)N, (int)K,
                     y, acc_out, stream, p.group_m};
    if (fmt == kFmtG128)
        launch_plan<kFmtG128>(p, a);
    else if (fmt == kFmtPC)
        launch_plan<kFmtPC>(p, a);
    else
        launch_plan<kFmtW8>(p, a);
}

}  // namespace qoq
