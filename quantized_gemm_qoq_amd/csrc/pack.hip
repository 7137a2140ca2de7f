// pack.hip -- offline reorder of UINT4 codes (and of the INT8 weights of the
// W8A8 sibling) into the gfx950 MFMA operand order, and its inverse.
//
// The pages' procedure reorders the W4 packs offline so that the fragments the
// matrix units consume next to each other need no extra address arithmetic
// ("QServe: Low Bit Width Does Not Guarantee High Throughput", section 4,
// evaluation pseudocode step 5). Here the unit of reorder is one 16-byte load
// per lane: a tile of 16 output channels x 128 inputs (one group) is 64 lanes x
// 16 bytes, and lane l's bytes are exactly the 32 codes that the two MFMA
// 16x16x64 k-steps of that group pair with activation bytes
// 64s + 16(l/16) + 0..15 of channel l % 16. The layout is written out in
// qoq.h (qoq_packed_bytes).
#include "qoq_device.hpp"
#include "qoq_launch.hpp"

namespace qoq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t nib_merge(uint32_t lo_bytes, uint32_t hi_bytes) {
    return (lo_bytes & 0x0F0F0F0Fu) | ((hi_bytes & 0x0F0F0F0Fu) << 4);
}

// One thread per (tile, lane): reads the lane's two runs of 16 codes (k-steps
// 0 and 1) and writes its 16 packed bytes.
__global__ __launch_bounds__(kThreads) void k_pack_codes(const uint8_t* __restrict__ q, int64_t N,
                                                         int K, uint8_t* __restrict__ blob) {
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int G = K / kGroup;
    const int64_t total = (N / 16) * G * kWave;
    if (tid >= total) return;
    const int lane = (int)(tid % kWave);
    const int64_t tg = tid / kWave;
    const int64_t t = tg / G;
    const int g = (int)(tg % G);
    const int64_t n = 16 * t + (lane % 16);
    const int j = lane / 16;
    const uint8_t* src = q + n * K + g * kGroup + 16 * j;
    const uint4 s0 = *reinterpret_cast<const uint4*>(src);
    const uint4 s1 = *reinterpret_cast<const uint4*>(src + 64);
    uint4 o;
    o.x = nib_merge(s0.x, s0.y);
    o.y = nib_merge(s0.z, s0.w);
    o.z = nib_merge(s1.x, s1.y);
    o.w = nib_merge(s1.z, s1.w);
    reinterpret_cast<uint4*>(blob)[tid] = o;  // tile (t, g) starts at (t*G + g) * 64 lanes
}

__global__ __launch_bounds__(kThreads) void k_unpack_codes(const uint8_t* __restrict__ blob,
                                                           int64_t N, int K,
                                                           uint8_t* __restrict__ q) {
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int G = K / kGroup;
    const int64_t total = (N / 16) * G * kWave;
    if (tid >= total) return;
    const int lane = (int)(tid % kWave);
    const int64_t tg = tid / kWave;
    const int64_t t = tg / G;
    const int g = (int)(tg % G);
    const int64_t n = 16 * t + (lane % 16);
    const int j = lane / 16;
    const uint4 p = reinterpret_cast<const uint4*>(blob)[tid];
    uint4 s0, s1;
    s0.x = p.x & 0x0F0F0F0Fu; s0.y = (p.x >> 4) & 0x0F0F0F0Fu;
    s0.z = p.y & 0x0F0F0F0Fu; s0.w = (p.y >> 4) & 0x0F0F0F0Fu;
    s1.x = p.z & 0x0F0F0F0Fu; s1.y = (p.z >> 4) & 0x0F0F0F0Fu;
    s1.z = p.w & 0x0F0F0F0Fu; s1.w = (p.w >> 4) & 0x0F0F0F0Fu;
    uint8_t* dst = q + n * K + g * kGroup + 16 * j;
    *reinterpret_cast<uint4*>(dst) = s0;
    *reinterpret_cast<uint4*>(dst + 64) = s1;
}

// g128 parameters: 16 bytes per (tile t, group g) at (t * G + g) * 16, byte c
// of which is ((s_g - 1) << 4) | z of channel 16 t + c. One thread per byte.
__global__ __launch_bounds__(kThreads) void k_pack_params_g128(const uint8_t* __restrict__ s_g,
                                                               const uint8_t* __restrict__ z,
                                                               int64_t N, int G,
                                                               uint8_t* __restrict__ params) {
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (tid >= N * G) return;
    const int64_t t = tid / (16 * (int64_t)G);
    const int64_t rem = tid % (16 * (int64_t)G);
    const int64_t g = rem / 16, n = 16 * t + rem % 16;
    params[tid] = (uint8_t)(((s_g[n * G + g] - 1) << 4) | (z[n * G + g] & 15));
}

__global__ __launch_bounds__(kThreads) void k_unpack_params_g128(const uint8_t* __restrict__ params,
                                                                 int64_t N, int G,
                                                                 uint8_t* __restrict__ s_g,
                                                                 uint8_t* __restrict__ z) {
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (tid >= N * G) return;
    const int64_t n = tid / G;
    const int64_t g = tid % G;
    const uint8_t b = params[((n / 16) * G + g) * 16 + n % 16];
    s_g[tid] = (uint8_t)((b >> 4) + 1);
    z[tid] = (uint8_t)(b & 15);
}

__global__ __launch_bounds__(kThreads) void k_copy_bytes(const uint8_t* __restrict__ src, int64_t n,
                                                         uint8_t* __restrict__ dst) {
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (tid < n) dst[tid] = src[tid];
}

// INT8 weights: one thread per 16-byte slot of the blob. Slot index
// (((t * G + g) * 2 + s) * 4 + j) * 16 + c holds inputs 128g + 64s + 16j + 0..15
// of channel 16t + c, which is the B operand of lane 16j + c for k-step s.
__global__ __launch_bounds__(kThreads) void k_pack_w8(const int8_t* __restrict__ q, int64_t N,
                                                      int K, uint8_t* __restrict__ blob) {
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int G = K / kGroup;
    if (tid >= N * K / 16) return;
    const int c = (int)(tid % 16);
    const int j = (int)((tid / 16) % 4);
    const int s = (int)((tid / 64) % 2);
    const int64_t tg = tid / 128;
    const int64_t t = tg / G;
    const int g = (int)(tg % G);
    const int8_t* src = q + (16 * t + c) * K + g * kGroup + 64 * s + 16 * j;
    reinterpret_cast<uint4*>(blob)[tid] = *reinterpret_cast<const uint4*>(src);
}

unsigned blocks_for(int64_t threads) { return (unsigned)((threads + kThreads - 1) / kThreads); }

}  // namespace

int64_t packed_bytes(int mode, int64_t N, int64_t K) {
    const int64_t codes = N * K / 2;
    if (mode == 0) return codes + N * (K / kGroup);
    return codes + N;
}

void launch_pack(int mode, const uint8_t* q, const uint8_t* s_g, const uint8_t* z, int64_t N,
                 int64_t K, uint8_t* blob, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    const int64_t lanes = (N / 16) * G * kWave;
    hipLaunchKernelGGL(k_pack_codes, dim3(blocks_for(lanes)), dim3(kThreads), 0, stream, q, N,
                       (int)K, blob);
    uint8_t* params = blob + N * K / 2;
    if (mode == 0) {
        hipLaunchKernelGGL(k_pack_params_g128, dim3(blocks_for(N * G)), dim3(kThreads), 0, stream,
                           s_g, z, N, G, params);
    } else {
        hipLaunchKernelGGL(k_copy_bytes, dim3(blocks_for(N)), dim3(kThreads), 0, stream, z, N,
                           params);
    }
}

void launch_unpack(int mode, const uint8_t* blob, int64_t N, int64_t K, uint8_t* q, uint8_t* s_g,
                   uint8_t* z, hipStream_t stream) {
    const int G = (int)(K / kGroup);
    const int64_t lanes = (N / 16) * G * kWave;
    hipLaunchKernelGGL(k_unpack_codes, dim3(blocks_for(lanes)), dim3(kThreads), 0, stream, blob, N,
                       (int)K, q);
    const uint8_t* params = blob + N * K / 2;
    if (mode == 0) {
        hipLaunchKernelGGL(k_unpack_params_g128, dim3(blocks_for(N * G)), dim3(kThreads), 0, stream,
                           params, N, G, s_g, z);
    } else {
        hipLaunchKernelGGL(k_copy_bytes, dim3(blocks_for(N)), dim3(kThreads), 0, stream, params, N,
                           z);
    }
}

void launch_pack_w8(const int8_t* q, int64_t N, int64_t K, uint8_t* blob, hipStream_t stream) {
    hipLaunchKernelGGL(k_pack_w8, dim3(blocks_for(N * K / 16)), dim3(kThreads), 0, stream, q, N,
                       (int)K, blob);
}

}  // namespace qoq
