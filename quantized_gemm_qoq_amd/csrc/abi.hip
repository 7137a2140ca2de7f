// abi.hip -- the C ABI of libqoq (declared and documented in include/qoq.h):
// argument validation, then one enqueue on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qoq.h"
#include "qoq_launch.hpp"

#include <cmath>

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_mode(int mode) { return mode == QOQ_MODE_G128 || mode == QOQ_MODE_PER_CHANNEL; }

bool valid_k(int64_t K) { return K >= QOQ_GROUP && K <= QOQ_MAX_K && K % QOQ_GROUP == 0; }

// Clears any stale runtime error, runs the enqueue, then reports whether the
// launches were accepted.
template <typename F>
qoq_status launch_checked(F&& f) {
    (void)hipGetLastError();
    f();
    return hipGetLastError() == hipSuccess ? QOQ_OK : QOQ_ERR_HIP;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int qoq_abi_version(void) { return QOQ_ABI_VERSION; }

const char* qoq_status_str(int status) {
    switch (status) {
        case QOQ_OK: return "ok";
        case QOQ_ERR_NULL: return "a required pointer is NULL";
        case QOQ_ERR_SHAPE: return "shape outside the supported limits";
        case QOQ_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case QOQ_ERR_MODE: return "unknown quantization mode";
        case QOQ_ERR_HIP: return "HIP runtime error at launch";
        case QOQ_ERR_WORKSPACE: return "workspace smaller than the call needs";
        case QOQ_ERR_HEADER: return "checkpoint header does not describe the expected blob";
        default: return "unknown status";
    }
}

qoq_status qoq_quantize_weights(int mode, const uint16_t* w, int64_t N, int64_t K, uint8_t* q,
                                uint16_t* s_c, uint8_t* s_g, uint8_t* z, void* stream) {
    if (!valid_mode(mode)) return QOQ_ERR_MODE;
    if (N < 0 || N % 16 || !valid_k(K)) return QOQ_ERR_SHAPE;
    if (N == 0) return QOQ_OK;
    if (!w || !q || !s_c || !z) return QOQ_ERR_NULL;
    if (mode == QOQ_MODE_G128 && !s_g) return QOQ_ERR_NULL;
    if (!aligned16(w) || !aligned16(q) || !aligned16(s_c) || !aligned16(z) ||
        (mode == QOQ_MODE_G128 && !aligned16(s_g)))
        return QOQ_ERR_ALIGN;
    return launch_checked([&] {
        qoq::launch_quantize_weights(mode, w, N, K, q, s_c, s_g, z, as_stream(stream));
    });
}

int64_t qoq_packed_bytes(int mode, int64_t N, int64_t K) {
    if (!valid_mode(mode) || N < 16 || N % 16 || !valid_k(K)) return -1;
    return qoq::packed_bytes(mode, N, K);
}

qoq_status qoq_pack_weights(int mode, const uint8_t* q, const uint8_t* s_g, const uint8_t* z,
                            int64_t N, int64_t K, void* blob, void* stream) {
    if (!valid_mode(mode)) return QOQ_ERR_MODE;
    if (N < 16 || N % 16 || !valid_k(K)) return QOQ_ERR_SHAPE;
    if (!q || !z || !blob) return QOQ_ERR_NULL;
    if (mode == QOQ_MODE_G128 && !s_g) return QOQ_ERR_NULL;
    if (!aligned16(q) || !aligned16(z) || !aligned16(blob) ||
        (mode == QOQ_MODE_G128 && !aligned16(s_g)))
        return QOQ_ERR_ALIGN;
    return launch_checked([&] {
        qoq::launch_pack(mode, q, s_g, z, N, K, static_cast<uint8_t*>(blob), as_stream(stream));
    });
}

qoq_status qoq_unpack_weights(int mode, const void* blob, int64_t N, int64_t K, uint8_t* q,
                              uint8_t* s_g, uint8_t* z, void* stream) {
    if (!valid_mode(mode)) return QOQ_ERR_MODE;
    if (N < 16 || N % 16 || !valid_k(K)) return QOQ_ERR_SHAPE;
    if (!blob || !q || !z) return QOQ_ERR_NULL;
    if (mode == QOQ_MODE_G128 && !s_g) return QOQ_ERR_NULL;
    if (!aligned16(blob) || !aligned16(q) || !aligned16(z) ||
        (mode == QOQ_MODE_G128 && !aligned16(s_g)))
        return QOQ_ERR_ALIGN;
    return launch_checked([&] {
        qoq::launch_unpack(mode, static_cast<const uint8_t*>(blob), N, K, q, s_g, z,
                           as_stream(stream));
    });
}

int64_t qoq_act_bytes(int64_t M, int64_t K) {
    if (M < 0 || M > INT32_MAX - 15 || !valid_k(K)) return -1;
    return (M + 15) / 16 * 16 * K;
}

qoq_status qoq_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, uint16_t* s_x,
                            int32_t* rowsum, void* stream) {
    if (M < 0 || M > INT32_MAX - 15 || !valid_k(K)) return QOQ_ERR_SHAPE;
    if (M == 0) return QOQ_OK;
    if (!x || !xq || !s_x) return QOQ_ERR_NULL;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(s_x) || (rowsum && !aligned16(rowsum)))
        return QOQ_ERR_ALIGN;
    return launch_checked(
        [&] { qoq::launch_quantize_act(x, M, K, xq, s_x, rowsum, as_stream(stream)); });
}

int64_t qoq_gemm_workspace_bytes(int mode, int64_t M, int64_t N, int64_t K) {
    if (!valid_mode(mode) || M < 0 || M > INT32_MAX || N < 0 || N % 16 || N > INT32_MAX ||
        !valid_k(K))
        return -1;
    if (M == 0 || N == 0) return 0;
    return qoq::gemm_workspace_bytes(mode, M, N, K);
}

qoq_status qoq_w4a8_gemm(int mode, const int8_t* xq, const uint16_t* s_x, const int32_t* rowsum,
                         const void* blob, const uint16_t* s_c, int64_t M, int64_t N, int64_t K,
                         uint16_t* y, int32_t* acc_out, void* workspace, int64_t workspace_bytes,
                         void* stream) {
    if (!valid_mode(mode)) return QOQ_ERR_MODE;
    if (M < 0 || M > INT32_MAX - 15 || N < 0 || N % 16 || N > INT32_MAX || !valid_k(K))
        return QOQ_ERR_SHAPE;
    if (M == 0 || N == 0) return QOQ_OK;
    if (!xq || !s_x || !blob || !s_c || !y) return QOQ_ERR_NULL;
    if (mode == QOQ_MODE_PER_CHANNEL && !rowsum) return QOQ_ERR_NULL;
    if (!aligned16(xq) || !aligned16(s_x) || !aligned16(blob) || !aligned16(s_c) ||
        !aligned16(y) || (rowsum && !aligned16(rowsum)) || (acc_out && !aligned16(acc_out)) ||
        (workspace && !aligned16(workspace)))
        return QOQ_ERR_ALIGN;
    if (workspace && workspace_bytes < qoq::gemm_workspace_bytes(mode, M, N, K))
        return QOQ_ERR_WORKSPACE;
    return launch_checked([&] {
        qoq::launch_gemm(mode, xq, s_x, rowsum, static_cast<const uint8_t*>(blob), s_c, M, N, K, y,
                         acc_out, workspace, as_stream(stream));
    });
}

int64_t qoq_w8a8_packed_bytes(int64_t N, int64_t K) {
    if (N < 16 || N % 16 || !valid_k(K)) return -1;
    return N * K;
}

qoq_status qoq_w8a8_quantize_weights(const uint16_t* w, int64_t N, int64_t K, int8_t* q,
                                     uint16_t* s_c, void* stream) {
    if (N < 0 || N % 16 || !valid_k(K)) return QOQ_ERR_SHAPE;
    if (N == 0) return QOQ_OK;
    if (!w || !q || !s_c) return QOQ_ERR_NULL;
    if (!aligned16(w) || !aligned16(q) || !aligned16(s_c)) return QOQ_ERR_ALIGN;
    return launch_checked(
        [&] { qoq::launch_quantize_weights_w8(w, N, K, q, s_c, as_stream(stream)); });
}

qoq_status qoq_w8a8_pack_weights(const int8_t* q, int64_t N, int64_t K, void* blob, void* stream) {
    if (N < 16 || N % 16 || !valid_k(K)) return QOQ_ERR_SHAPE;
    if (!q || !blob) return QOQ_ERR_NULL;
    if (!aligned16(q) || !aligned16(blob)) return QOQ_ERR_ALIGN;
    return launch_checked(
        [&] { qoq::launch_pack_w8(q, N, K, static_cast<uint8_t*>(blob), as_stream(stream)); });
}

int64_t qoq_w8a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || M > INT32_MAX || N < 0 || N % 16 || N > INT32_MAX || !valid_k(K)) return -1;
    if (M == 0 || N == 0) return 0;
    return qoq::gemm_workspace_bytes(qoq::kGemmFmtW8, M, N, K);
}

qoq_status qoq_w8a8_gemm(const int8_t* xq, const uint16_t* s_x, const void* blob,
                         const uint16_t* s_c, int64_t M, int64_t N, int64_t K, uint16_t* y,
                         int32_t* acc_out, void* workspace, int64_t workspace_bytes, void* stream) {
    if (M < 0 || M > INT32_MAX - 15 || N < 0 || N % 16 || N > INT32_MAX || !valid_k(K))
        return QOQ_ERR_SHAPE;
    if (M == 0 || N == 0) return QOQ_OK;
    if (!xq || !s_x || !blob || !s_c || !y) return QOQ_ERR_NULL;
    if (!aligned16(xq) || !aligned16(s_x) || !aligned16(blob) || !aligned16(s_c) ||
        !aligned16(y) || (acc_out && !aligned16(acc_out)) || (workspace && !aligned16(workspace)))
        return QOQ_ERR_ALIGN;
    if (workspace && workspace_bytes < qoq::gemm_workspace_bytes(qoq::kGemmFmtW8, M, N, K))
        return QOQ_ERR_WORKSPACE;
    return launch_checked([&] {
        qoq::launch_gemm(qoq::kGemmFmtW8, xq, s_x, nullptr, static_cast<const uint8_t*>(blob), s_c,
                         M, N, K, y, acc_out, workspace, as_stream(stream));
    });
}

qoq_status qoq_silu_mul_quantize_act(const uint16_t* gate_up, int64_t M, int64_t I, int8_t* xq,
                                     uint16_t* s_x, int32_t* rowsum, uint16_t* h, void* stream) {
    if (M < 0 || M > INT32_MAX - 15 || !valid_k(I)) return QOQ_ERR_SHAPE;
    if (M == 0) return QOQ_OK;
    if (!gate_up || !xq || !s_x) return QOQ_ERR_NULL;
    if (!aligned16(gate_up) || !aligned16(xq) || !aligned16(s_x) || (rowsum && !aligned16(rowsum)) ||
        (h && !aligned16(h)))
        return QOQ_ERR_ALIGN;
    return launch_checked([&] {
        qoq::launch_silu_mul_quantize_act(gate_up, M, I, xq, s_x, rowsum, h, as_stream(stream));
    });
}

int64_t qoq_silu_mul_workspace_bytes(int64_t M, int64_t I) {
    if (M < 0 || M > INT32_MAX - 15 || !valid_k(I)) return -1;
    return qoq::silu_mul_workspace_bytes(M, I);
}

qoq_status qoq_silu_mul_quantize_act_ws(const uint16_t* gate_up, int64_t M, int64_t I, int8_t* xq,
                                        uint16_t* s_x, int32_t* rowsum, uint16_t* h,
                                        void* workspace, int64_t workspace_bytes, void* stream) {
    if (M < 0 || M > INT32_MAX - 15 || !valid_k(I)) return QOQ_ERR_SHAPE;
    if (M == 0) return QOQ_OK;
    if (!gate_up || !xq || !s_x) return QOQ_ERR_NULL;
    if (!aligned16(gate_up) || !aligned16(xq) || !aligned16(s_x) || (rowsum && !aligned16(rowsum)) ||
        (h && !aligned16(h)) || (workspace && !aligned16(workspace)))
        return QOQ_ERR_ALIGN;
    const int64_t need = qoq::silu_mul_workspace_bytes(M, I);
    if (workspace && workspace_bytes < need) return QOQ_ERR_WORKSPACE;
    return launch_checked([&] {
        qoq::launch_silu_mul_quantize_act_ws(gate_up, M, I, xq, s_x, rowsum, h, need > 0 ? workspace : nullptr,
                                             as_stream(stream));
    });
}

qoq_status qoq_rmsnorm_quantize_act(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M,
                                   int64_t K, int8_t* xq, uint16_t* s_x, int32_t* rowsum,
                                   uint16_t* y, void* stream) {
    if (M < 0 || M > INT32_MAX - 15 || !valid_k(K) || K > QOQ_RMSNORM_MAX_K) return QOQ_ERR_SHAPE;
    if (!(eps > 0.0f) || !std::isfinite(eps)) return QOQ_ERR_SHAPE;
    if (M == 0) return QOQ_OK;
    if (!x || !gamma || !xq || !s_x) return QOQ_ERR_NULL;
    if (!aligned16(x) || !aligned16(gamma) || !aligned16(xq) || !aligned16(s_x) ||
        (rowsum && !aligned16(rowsum)) || (y && !aligned16(y)))
        return QOQ_ERR_ALIGN;
    return launch_checked([&] {
        qoq::launch_rmsnorm_quantize_act(x, gamma, eps, M, K, xq, s_x, rowsum, y, as_stream(stream));
    });
}

namespace {
bool valid_kv_shape(int64_t B, int64_t H, int64_t d, int64_t Tcap) {
    return B >= 0 && B <= INT32_MAX && H >= 1 && H <= 1024 && d == 128 && Tcap >= 16 &&
           Tcap % 16 == 0 && Tcap <= (int64_t(1) << 24);
}
}  // namespace

qoq_status qoq_kv4_smooth_scales(const uint16_t* k, int64_t T, int64_t H, int64_t d,
                                 uint16_t* lambda, void* stream) {
    if (T < 0 || T > INT32_MAX || H < 1 || H > 1024 || d != 128) return QOQ_ERR_SHAPE;
    if (!lambda || (T > 0 && !k)) return QOQ_ERR_NULL;
    if ((k && !aligned16(k)) || !aligned16(lambda)) return QOQ_ERR_ALIGN;
    return launch_checked([&] { qoq::launch_kv4_smooth_scales(k, T, H, lambda, as_stream(stream)); });
}

qoq_status qoq_kv4_append(const uint16_t* k, const uint16_t* v, const uint16_t* lambda,
                          int64_t B, int64_t T, int64_t H, int64_t d, int64_t Tcap, int64_t t0,
                          uint8_t* kq, uint16_t* ks, uint8_t* kz, uint8_t* vq, uint16_t* vs,
                          uint8_t* vz, void* stream) {
    if (!valid_kv_shape(B, H, d, Tcap) || T < 0 || t0 < 0 || t0 + T > Tcap ||
        B * T * H > INT32_MAX)
        return QOQ_ERR_SHAPE;
    if (B == 0 || T == 0) return QOQ_OK;
    if (!k || !v || !lambda || !kq || !ks || !kz || !vq || !vs || !vz) return QOQ_ERR_NULL;
    if (!aligned16(k) || !aligned16(v) || !aligned16(lambda) || !aligned16(kq) || !aligned16(ks) ||
        !aligned16(kz) || !aligned16(vq) || !aligned16(vs) || !aligned16(vz))
        return QOQ_ERR_ALIGN;
    return launch_checked([&] {
        qoq::launch_kv4_append(k, v, lambda, B, T, H, Tcap, t0, kq, ks, kz, vq, vs, vz,
                               as_stream(stream));
    });
}

int64_t qoq_kv4_attention_workspace_bytes(int64_t B, int64_t Hq, int64_t H, int64_t d,
                                          int64_t Tcap) {
    if (!valid_kv_shape(B, H, d, Tcap) || Hq < H || Hq % H || Hq / H > 8 || (Hq / H) & (Hq / H - 1))
        return -1;
    return qoq::kv4_workspace_bytes(B, Hq, H, Tcap);
}

qoq_status qoq_kv4_decode_attention(const uint16_t* q, const uint16_t* lambda, const uint8_t* kq,
                                    const uint16_t* ks, const uint8_t* kz, const uint8_t* vq,
                                    const uint16_t* vs, const uint8_t* vz, const int32_t* lens,
                                    int64_t B, int64_t Hq, int64_t H, int64_t d, int64_t Tcap,
                                    uint16_t* o, void* workspace, int64_t workspace_bytes,
                                    void* stream) {
    const int64_t need = qoq_kv4_attention_workspace_bytes(B, Hq, H, d, Tcap);
    if (need < 0) return QOQ_ERR_SHAPE;
    if (B == 0) return QOQ_OK;
    if (!q || !lambda || !kq || !ks || !kz || !vq || !vs || !vz || !lens || !o || !workspace)
        return QOQ_ERR_NULL;
    if (!aligned16(q) || !aligned16(lambda) || !aligned16(kq) || !aligned16(ks) || !aligned16(kz) ||
        !aligned16(vq) || !aligned16(vs) || !aligned16(vz) || !aligned16(lens) || !aligned16(o) ||
        !aligned16(workspace))
        return QOQ_ERR_ALIGN;
    if (workspace_bytes < need) return QOQ_ERR_WORKSPACE;
    return launch_checked([&] {
        qoq::launch_kv4_decode_attention(q, lambda, kq, ks, kz, vq, vs, vz, lens, B, Hq, H, Tcap, o,
                                         workspace, as_stream(stream));
    });
}

qoq_status qoq_w4a16_gemm(int mode, const uint16_t* x, const void* blob, const uint16_t* s_c,
                          int64_t M, int64_t N, int64_t K, uint16_t* y, float* acc_out,
                          void* stream) {
    if (!valid_mode(mode)) return QOQ_ERR_MODE;
    if (M < 0 || M > INT32_MAX || N < 0 || N % 16 || N > INT32_MAX || !valid_k(K))
        return QOQ_ERR_SHAPE;
    if (M == 0 || N == 0) return QOQ_OK;
    if (!x || !blob || !s_c || !y) return QOQ_ERR_NULL;
    if (!aligned16(x) || !aligned16(blob) || !aligned16(s_c) || !aligned16(y) ||
        (acc_out && !aligned16(acc_out)))
        return QOQ_ERR_ALIGN;
    return launch_checked([&] {
        qoq::launch_gemm_w4a16(mode, x, static_cast<const uint8_t*>(blob), s_c, M, N, K, y, acc_out,
                               as_stream(stream));
    });
}

namespace {
int64_t blob_bytes_of(int format, int64_t N, int64_t K) {
    if (format == QOQ_FORMAT_W8A8) return qoq_w8a8_packed_bytes(N, K);
    return qoq_packed_bytes(format, N, K);
}
}  // namespace

static_assert(sizeof(qoq_blob_header) == 64, "the checkpoint header is 64 bytes");

qoq_status qoq_blob_header_init(int format, int64_t N, int64_t K, qoq_blob_header* h) {
    if (!h) return QOQ_ERR_NULL;
    if (!valid_mode(format) && format != QOQ_FORMAT_W8A8) return QOQ_ERR_MODE;
    const int64_t bytes = blob_bytes_of(format, N, K);
    if (bytes < 0) return QOQ_ERR_SHAPE;
    qoq_blob_header t{};
    t.magic = QOQ_BLOB_MAGIC;
    t.abi_version = QOQ_ABI_VERSION;
    t.format = (uint32_t)format;
    t.group = QOQ_GROUP;
    t.n = N;
    t.k = K;
    t.blob_bytes = bytes;
    t.scale_bytes = 2 * N;
    *h = t;
    return QOQ_OK;
}

qoq_status qoq_blob_header_check(const qoq_blob_header* h, int format, int64_t N, int64_t K) {
    if (!h) return QOQ_ERR_NULL;
    qoq_blob_header want;
    const qoq_status st = qoq_blob_header_init(format, N, K, &want);
    if (st != QOQ_OK) return st;
    bool same = h->magic == want.magic && h->abi_version == want.abi_version &&
                h->format == want.format && h->group == want.group && h->n == want.n &&
                h->k == want.k && h->blob_bytes == want.blob_bytes &&
                h->scale_bytes == want.scale_bytes;
    for (int i = 0; i < 16; ++i) same = same && h->reserved[i] == 0;
    return same ? QOQ_OK : QOQ_ERR_HEADER;
}

}  // extern "C"
