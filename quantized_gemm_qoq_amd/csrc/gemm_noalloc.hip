// gemm_noalloc.hip -- qoq_w4a8_gemm_noalloc: the W4A8 GEMM for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops
// that forbid hipMalloc). Its split-K partial sums live in a file-scope device
// array, `scratch`, instead of a caller workspace; everything else is
// qoq_w4a8_gemm's.
//
// Host code never passes `scratch` itself to a kernel (in host code the name is
// a stand-in, not a device address): the first call on each device looks up
// that device's copy with hipGetSymbolAddress, with the device current, and
// keeps the address for later calls.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "qoq.h"

namespace {

static __device__ __align__(256) uint8_t scratch[QOQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // address of each device's `scratch`, once looked up

// The device the call's kernels run on: the stream's, or the current one for
// the null stream.
bool call_device(hipStream_t stream, int* dev) {
    if (stream) return hipStreamGetDevice(stream, dev) == hipSuccess;
    return hipGetDevice(dev) == hipSuccess;
}

// This device's copy of `scratch`, looked up once with the device current.
void* device_scratch(int dev) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev]) return g_scratch_ptr[dev];
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t rc = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (rc != hipSuccess || !p) {
        (void)hipGetLastError();
        return nullptr;
    }
    g_scratch_ptr[dev] = p;
    return p;
}

}  // namespace

extern "C" {

qoq_status qoq_w4a8_gemm_noalloc(int mode, const int8_t* xq, const uint16_t* s_x,
                                 const int32_t* rowsum, const void* blob, const uint16_t* s_c,
                                 int64_t M, int64_t N, int64_t K, uint16_t* y, int32_t* acc_out,
                                 void* stream) {
    const int64_t need = qoq_gemm_workspace_bytes(mode, M, N, K);
    if (need < 0) return mode == QOQ_MODE_G128 || mode == QOQ_MODE_PER_CHANNEL ? QOQ_ERR_SHAPE : QOQ_ERR_MODE;
    if (need > QOQ_NOALLOC_SCRATCH_BYTES) return QOQ_ERR_WORKSPACE;
    if (M == 0 || N == 0)  // the empty call: nothing to look up or launch
        return qoq_w4a8_gemm(mode, xq, s_x, rowsum, blob, s_c, M, N, K, y, acc_out, nullptr, 0, stream);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    int dev = -1;
    if (!call_device(st, &dev) || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return QOQ_ERR_HIP;
    }
    void* ws = device_scratch(dev);
    if (!ws) return QOQ_ERR_HIP;
    return qoq_w4a8_gemm(mode, xq, s_x, rowsum, blob, s_c, M, N, K, y, acc_out, ws,
                         QOQ_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
