// qoq_launch.hpp -- host-side launchers of the libqoq kernels. Arguments are
// validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qoq {

void launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, uint16_t* s_x,
                         int32_t* rowsum, hipStream_t stream);

void launch_quantize_weights(int mode, const uint16_t* w, int64_t N, int64_t K, uint8_t* q,
                             uint16_t* s_c, uint8_t* s_g, uint8_t* z, hipStream_t stream);

int64_t packed_bytes(int mode, int64_t N, int64_t K);

void launch_pack(int mode, const uint8_t* q, const uint8_t* s_g, const uint8_t* z, int64_t N,
                 int64_t K, uint8_t* blob, hipStream_t stream);

void launch_unpack(int mode, const uint8_t* blob, int64_t N, int64_t K, uint8_t* q, uint8_t* s_g,
                   uint8_t* z, hipStream_t stream);

// Fused producer of the down projection's input: h = f16(SiLU(gate) * up)
// from gate_up [M, 2I], then the per-token quantization of launch_quantize_act
// (same outputs); h [M, I] is written when not null.
void launch_rmsnorm_quantize_act(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M,
                                 int64_t K, int8_t* xq, uint16_t* s_x, int32_t* rowsum,
                                 uint16_t* y, hipStream_t stream);
int64_t silu_mul_workspace_bytes(int64_t M, int64_t I);
void launch_silu_mul_quantize_act_ws(const uint16_t* gate_up, int64_t M, int64_t I, int8_t* xq,
                                     uint16_t* s_x, int32_t* rowsum, uint16_t* h, void* ws,
                                     hipStream_t stream);
void launch_silu_mul_quantize_act(const uint16_t* gate_up, int64_t M, int64_t I, int8_t* xq,
                                  uint16_t* s_x, int32_t* rowsum, uint16_t* h,
                                  hipStream_t stream);

// INT8 weights of the W8A8 sibling: per-channel symmetric quantization, and
// the reorder into the operand order (N * K bytes).
void launch_quantize_weights_w8(const uint16_t* w, int64_t N, int64_t K, int8_t* q, uint16_t* s_c,
                                hipStream_t stream);
void launch_pack_w8(const int8_t* q, int64_t N, int64_t K, uint8_t* blob, hipStream_t stream);

// Weight format of a GEMM call: 0 g128 UINT4, 1 per-channel UINT4, 2 INT8.
constexpr int kGemmFmtW8 = 2;

// Workspace bytes the GEMM plan for this shape uses when given one (0: none).
int64_t gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K);

// ws: null (a plan without split K is used) or gemm_workspace_bytes() bytes
// of device memory for split-K partial sums (no initialisation needed).
void launch_gemm(int fmt, const int8_t* xq, const uint16_t* s_x, const int32_t* rowsum,
                 const uint8_t* blob, const uint16_t* s_c, int64_t M, int64_t N, int64_t K,
                 uint16_t* y, int32_t* acc_out, void* ws, hipStream_t stream);

// W4A16 sibling: FP16 activations x [M,K] (row-major) against the W4 blob of
// qoq_pack_weights (either mode); acc_out (fp32 [M,N], may be null) receives
// the accumulators before the per-channel scale.
void launch_gemm_w4a16(int mode, const uint16_t* x, const uint8_t* blob, const uint16_t* s_c,
                       int64_t M, int64_t N, int64_t K, uint16_t* y, float* acc_out,
                       hipStream_t stream);

// KV4 decode attention with SmoothAttention (head dimension 128).
void launch_kv4_smooth_scales(const uint16_t* k, int64_t T, int64_t H, uint16_t* lambda,
                              hipStream_t stream);
void launch_kv4_append(const uint16_t* k, const uint16_t* v, const uint16_t* lambda, int64_t B,
                       int64_t T, int64_t H, int64_t Tcap, int64_t t0, uint8_t* kq, uint16_t* ks,
                       uint8_t* kz, uint8_t* vq, uint16_t* vs, uint8_t* vz, hipStream_t stream);
int64_t kv4_chunk(int64_t B, int64_t H, int64_t Tcap);
int64_t kv4_workspace_bytes(int64_t B, int64_t Hq, int64_t H, int64_t Tcap);
void launch_kv4_decode_attention(const uint16_t* q, const uint16_t* lambda, const uint8_t* kq,
                                 const uint16_t* ks, const uint8_t* kz, const uint8_t* vq,
                                 const uint16_t* vs, const uint8_t* vz, const int32_t* lens,
                                 int64_t B, int64_t Hq, int64_t H, int64_t Tcap, uint16_t* o,
                                 void* ws, hipStream_t stream);

}  // namespace qoq
