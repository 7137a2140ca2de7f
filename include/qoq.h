/*
 * qoq.h -- C ABI of libqoq, a QoQ W4A8 GEMM (QServe, arXiv 2405.04532) and
 * its W8A8 and W4A16 siblings for AMD Instinct MI355X (gfx950).
 *
 *   Y[M,N] = X[M,K] * W[N,K]^T
 *
 * X is FP16, quantized per token to INT8; W is held as UINT4 codes under
 * progressive group quantization (per-channel INT8 in the protective range
 * [-119,119], then groups of 128 with an integer scale and a UINT4 zero) or
 * under plain per-channel UINT4; the GEMM unpacks the codes to INT8 in
 * registers, accumulates INT8 x INT8 products in INT32 on the matrix cores and
 * rescales once per output in FP32 before writing FP16.
 *
 * Passages defining each operation (page title, then section):
 *   [EN]    "QServe: Low Bit Width Does Not Guarantee High Throughput", section 4
 *           "Formalization and procedure": stage-1 and stage-2 equations and the
 *           paragraph on the [-119,119] overflow margin, the integer scale and the
 *           precomputed zero-point compensation; evaluation pseudocode steps 2, 4,
 *           5 and 6 (progressive quantization, per-channel vs g128 choice, offline
 *           pack reorder, register unpack feeding INT8 GEMM).
 *   [SUM]   "QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
 *           Serving" (research.elamur.ai), "Key points": FP16 per-channel scales,
 *           range [-119,119], then group INT4; multiply first, subtract after.
 *   [GUIDE] "QServe Guide: W4A8KV4 Quantization for LLM Serving", "Deep Dive" part 1
 *           (per-token INT8 activations; one rescale by the two scales) and
 *           "High-Throughput Native INT8 Tensor Core GEMMs" (INT32 accumulators).
 *   [WIKI]  "QoQ / QServe — Quantification W4A8KV4", example configuration:
 *           weight group size 128.
 *   [W8A8]  "QServe Guide: W4A8KV4 Quantization for LLM Serving", "The Problem"
 *           item 2 (weights and activations both INT8 on the INT8 matrix
 *           units) and "Deep Dive" part 1 (per-channel symmetric weight
 *           scaling, here at 8 bits); "QServe: Low Bit Width Does Not Guarantee
 *           High Throughput", section 3, judgment A (W8A8 suits large batches,
 *           the format W4A8 is compared against).
 *   [W4A16] "QServe Guide: W4A8KV4 Quantization for LLM Serving", "The Problem"
 *           item 1 (4-bit weights dequantized to FP16 in the main loop, FP16
 *           activations, FP16 matrix units); "QServe: Low Bit Width Does Not
 *           Guarantee High Throughput", section 2 (the W4A16 failure mode and
 *           its small-batch roofline advantage).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, allocated and owned by the
 *     caller. The library never allocates, frees or keeps them past the call.
 *   - FP16 values are passed as raw binary16 bits (uint16_t); no HIP or PyTorch
 *     header is needed to include this file.
 *   - Every call validates its arguments on the host first. On a validation
 *     error it returns a non-zero qoq_status, launches nothing and writes
 *     nothing. Otherwise it enqueues its kernels on `stream` (a hipStream_t; NULL
 *     is the default stream) and returns without synchronizing; a launch failure
 *     is reported as QOQ_ERR_HIP. Faults inside a kernel surface at the caller's
 *     next synchronization.
 *   - Shapes: K is a multiple of 128 with 128 <= K <= 132096 (so that every
 *     INT32 accumulator is exact: 132096 * 128 * 127 < 2^31); N is a multiple
 *     of 16; M >= 0. M == 0 or N == 0 is an empty call that returns QOQ_OK.
 *   - Every pointer is 16-byte aligned (QOQ_ERR_ALIGN otherwise).
 *   - Inputs must be finite; results for NaN or infinite inputs are unspecified.
 *   - Rounding: every "round" is round-half-to-even; scales are computed in IEEE
 *     fp32 (correctly rounded division) and stored as FP16 (round to nearest
 *     even), and the stored FP16 scale is the one used to quantize.
 *   - There is no global mutable state, except in qoq_w4a8_gemm_noalloc (its
 *     fixed scratch array): calls on different streams or threads are
 *     independent.
 */
#ifndef QOQ_H_
#define QOQ_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QOQ_ABI_VERSION 6
#define QOQ_GROUP 128
#define QOQ_MAX_K 132096
#define QOQ_RMSNORM_MAX_K 32768 /* row length of qoq_rmsnorm_quantize_act */

typedef enum {
    QOQ_MODE_G128 = 0,        /* progressive: INT8 [-119,119] per channel, then g128 UINT4 */
    QOQ_MODE_PER_CHANNEL = 1  /* UINT4 per output channel, zero-point in the epilogue */
} qoq_mode;

typedef enum {
    QOQ_OK = 0,
    QOQ_ERR_NULL = 1,   /* a required pointer is NULL */
    QOQ_ERR_SHAPE = 2,  /* M, N or K outside the limits above */
    QOQ_ERR_ALIGN = 3,  /* a pointer is not 16-byte aligned */
    QOQ_ERR_MODE = 4,   /* mode is neither QOQ_MODE_G128 nor QOQ_MODE_PER_CHANNEL */
    QOQ_ERR_HIP = 5,    /* the HIP runtime reported an error at launch */
    QOQ_ERR_WORKSPACE = 6, /* workspace given but smaller than the *_workspace_bytes() value */
    QOQ_ERR_HEADER = 7     /* a checkpoint header that does not describe the expected blob */
} qoq_status;

/* QOQ_ABI_VERSION of the loaded library. */
int qoq_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* qoq_status_str(int status);

/*
 * Weight quantization, offline ([EN] section 4, both equations; [SUM]).
 *
 *   w   [N,K] FP16 row-major, output channel n is row n (the nn.Linear layout).
 *   q   [N,K] uint8, one UINT4 code (0..15) per byte.
 *   s_c [N]   FP16 per-channel scale.
 *   QOQ_MODE_G128, with G = K/128:
 *     s_c[n] = f16(max_k |w[n,k]| / 119)
 *     w8     = clip(round(w / s_c), -119, 119)               (stage 1)
 *     per group g: mn = min(0, min w8), mx = max(0, max w8)
 *     s_g[n,g] = max(1, ceil((mx - mn)/15))  (uint8, 1..16)  (stage 2)
 *     z[n,g]   = round(-mn / s_g)            (uint8, 0..15)
 *     q        = clip(round(w8 / s_g) + z, 0, 15)
 *     so that (q - z) * s_g lies in [-127, 127] and W^ = s_c * s_g * (q - z).
 *     s_g and z are [N,G] row-major.
 *   QOQ_MODE_PER_CHANNEL (s_g must be NULL):
 *     mn = min(0, min_k w), mx = max(0, max_k w), s_c = f16((mx - mn)/15),
 *     z[n] = clip(round(-mn/s_c), 0, 15), q = clip(round(w/s_c) + z, 0, 15);
 *     W^ = s_c * (q - z). z is [N].
 *   A scale that is 0 (all-zero row, or one that rounds to 0 in FP16) gives
 *   q = 0 and z = 0 for that row.
 */
qoq_status qoq_quantize_weights(int mode, const uint16_t* w, int64_t N, int64_t K,
                                uint8_t* q, uint16_t* s_c, uint8_t* s_g, uint8_t* z,
                                void* stream);

/*
 * Size in bytes of the packed weight blob, or -1 for an unsupported shape or
 * mode. The blob is laid out for the gfx950 INT8 MFMA operand ([EN] pseudocode
 * step 5: the codes are reordered offline so that the main loop does no
 * address arithmetic beyond one 16-byte load per lane):
 *
 *   Codes: N*K/2 bytes at offset 0, in tiles of 16 output channels x 128 input
 *   channels (one group), 1024 bytes each. Tile (t, g) = channels 16t..16t+15,
 *   inputs 128g..128g+127, starts at byte (t*G + g)*1024. Write the position of
 *   input k inside its group as k % 128 = 64*s + 16*j + i (s in 0..1, j in
 *   0..3, i in 0..15) and c = n % 16. Then the code of (n, k) lives in
 *     lane  = 16*j + c                 (the tile is 64 lanes x 16 bytes)
 *     kappa = 16*s + i                 (the lane's code index, 0..31)
 *     byte  = 16*lane + 4*(kappa/8) + (kappa % 4)
 *     the low nibble when kappa % 8 < 4, else the high nibble.
 *   So one 16-byte load by lane l brings, for channel c = l % 16, the 32 codes
 *   that the MFMA k-steps s = 0 and 1 pair with activation bytes
 *   128g + 64s + 16(l/16) + (0..15); (word & 0x0F0F0F0F) and
 *   ((word >> 4) & 0x0F0F0F0F) of each 32-bit word give four codes in k order.
 *
 *   Parameters at offset N*K/2:
 *     QOQ_MODE_G128: N*G bytes, 16 per (tile t, group g) at (t*G + g)*16, so
 *       that the 16 channels of a tile's group sit in one 16-byte run; byte c
 *       of the run is ((s_g[16t+c,g] - 1) << 4) | z[16t+c,g].
 *     QOQ_MODE_PER_CHANNEL: N bytes, z[n].
 */
int64_t qoq_packed_bytes(int mode, int64_t N, int64_t K);

/* Pack canonical codes (q [N,K], s_g [N,G] or NULL, z) into `blob`
 * (qoq_packed_bytes(mode, N, K) bytes). Needs N >= 16. */
qoq_status qoq_pack_weights(int mode, const uint8_t* q, const uint8_t* s_g, const uint8_t* z,
                            int64_t N, int64_t K, void* blob, void* stream);

/* Inverse of qoq_pack_weights, for inspection and tests. */
qoq_status qoq_unpack_weights(int mode, const void* blob, int64_t N, int64_t K,
                              uint8_t* q, uint8_t* s_g, uint8_t* z, void* stream);

/*
 * Per-token INT8 activation quantization, every call ([GUIDE] Deep Dive part 1).
 *
 *   x      [M,K] FP16 row-major.
 *   s_x[m] = f16(max_k |x[m,k]| / 127)                   (FP16, [M])
 *   xq     = clamp(round(x / s_x), -128, 127)            (int8, packed, below)
 *   rowsum[m] = sum_k xq[m,k]  (int32, [M]; may be NULL; required later by the
 *             per-channel GEMM's zero-point compensation)
 *   A scale of 0 gives xq = 0 for that row.
 *
 * xq is written in the order the gfx950 INT8 MFMA consumes its A operand, so
 * that every operand load of the GEMM is one coalesced 1 KB read (the same
 * idea as the offline weight reorder, applied to the per-call activations).
 * qoq_act_bytes(M, K) bytes, Mp = roundup(M, 16) rows (rows M..Mp-1 are 0):
 *   tile (g, u) = rows 16u..16u+15, inputs 128g..128g+127, 2048 bytes at
 *   offset (g * Mp/16 + u) * 2048; with k % 128 = 64*s + 16*j + i and
 *   r = m % 16, the byte of (m, k) is at 1024*s + 16*(16*j + r) + i.
 */
int64_t qoq_act_bytes(int64_t M, int64_t K);

qoq_status qoq_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* xq,
                            uint16_t* s_x, int32_t* rowsum, void* stream);

/*
 * Workspace bytes that qoq_w4a8_gemm uses for this shape when it is given a
 * workspace (0 if its plan needs none), or -1 for an unsupported shape or
 * mode. For M > 64 with too few output blocks to cover the compute units, the
 * plan splits K into S ranges whose exact INT32 partial sums (S*M*N*4 bytes)
 * are added by a second kernel; without a workspace the unsplit plan runs.
 */
int64_t qoq_gemm_workspace_bytes(int mode, int64_t M, int64_t N, int64_t K);

/*
 * W4A8 GEMM with the FP16 epilogue ([EN] section 4 and pseudocode step 6;
 * [GUIDE] "INT32 accumulators" and the one-time rescale).
 *
 *   xq packed INT8 activations from qoq_quantize_act, s_x [M] FP16, rowsum
 *   [M] int32 (required in per-channel mode, ignored in g128 mode), blob from
 *   qoq_pack_weights, s_c [N] FP16.
 *   acc[m,n] = sum_k xq[m,k] * (q[n,k] - z) * s_g     (g128; exact INT32)
 *            = sum_k xq[m,k] * (q[n,k] - z[n])        (per-channel; computed as
 *              sum_k xq*q - z[n]*rowsum[m], exact)
 *   y[m,n]   = f16( (f32(acc) * f32(s_x[m])) * f32(s_c[n]) )  (FP16 [M,N])
 *   acc_out  [M,N] int32 receives acc when not NULL (for inspection).
 *
 *   workspace: NULL, or device memory of workspace_bytes bytes, used for
 *   split-K partial sums (no initialisation needed; its contents are
 *   overwritten). A workspace smaller than qoq_gemm_workspace_bytes(mode, M,
 *   N, K) gives QOQ_ERR_WORKSPACE. Calls that overlap in time (e.g. on
 *   different streams) must not share a workspace.
 */
qoq_status qoq_w4a8_gemm(int mode, const int8_t* xq, const uint16_t* s_x, const int32_t* rowsum,
                         const void* blob, const uint16_t* s_c, int64_t M, int64_t N, int64_t K,
                         uint16_t* y, int32_t* acc_out, void* workspace, int64_t workspace_bytes,
                         void* stream);

/*
 * W4A8 GEMM that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, serving loops and harnesses that
 * forbid hipMalloc. The same computation, arguments and errors as
 * qoq_w4a8_gemm, without the workspace arguments: the split-K partial sums go
 * to a fixed device array of QOQ_NOALLOC_SCRATCH_BYTES (32 MiB) inside the
 * library, one per GPU, held from the library's load until the process ends.
 * That is the most any plan needs (a split plan keeps its split count times
 * its 128 x 256 output blocks at most 256, so at most 256 x 128 x 256 x 4
 * bytes); a shape whose plan needed more would return QOQ_ERR_WORKSPACE and
 * launch nothing. Every call on a GPU
 * uses that GPU's one array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and must not be issued;
 * no contents are carried from one call to the next. The first call on each
 * GPU looks up the array's address (hipGetSymbolAddress) and keeps it, the one
 * piece of global state of this entry point.
 */
#define QOQ_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
qoq_status qoq_w4a8_gemm_noalloc(int mode, const int8_t* xq, const uint16_t* s_x,
                                 const int32_t* rowsum, const void* blob, const uint16_t* s_c,
                                 int64_t M, int64_t N, int64_t K, uint16_t* y, int32_t* acc_out,
                                 void* stream);

/*
 * ---- W8A8 sibling ([W8A8]) ------------------------------------------------
 * The same per-token INT8 activations (qoq_quantize_act) against INT8 weights,
 * for comparing the formats on one harness: twice the weight bytes of W4A8,
 * no unpack in the main loop.
 *
 * Weight quantization, offline:
 *   w   [N,K] FP16 row-major; q [N,K] int8 row-major; s_c [N] FP16.
 *   s_c[n] = f16(max_k |w[n,k]| / 127)
 *   q      = clamp(round(w / s_c), -128, 127)   (|w / s_c| <= 127 * (1 + 2^-11)
 *            rounds to at most 127, so the codes are symmetric in practice)
 *   A scale of 0 gives q = 0 for that row. Shapes as for qoq_quantize_weights.
 */
qoq_status qoq_w8a8_quantize_weights(const uint16_t* w, int64_t N, int64_t K, int8_t* q,
                                     uint16_t* s_c, void* stream);

/*
 * Size of the packed INT8 weights (N*K bytes), or -1 for an unsupported shape.
 * Tiles of 16 output channels x 128 inputs, 2048 bytes each; tile (t, g) starts
 * at byte (t*G + g)*2048. With c = n % 16 and k % 128 = 64*s + 16*j + i, the
 * byte of (n, k) is at 1024*s + 16*(16*j + c) + i within its tile -- the order
 * of the packed activations with the channel in place of the row, so that one
 * 1 KB coalesced read gives every lane of a wave its MFMA B operand for one
 * k-step.
 */
int64_t qoq_w8a8_packed_bytes(int64_t N, int64_t K);

/* Pack row-major INT8 weights q [N,K] into `blob` (qoq_w8a8_packed_bytes(N, K)
 * bytes). Needs N >= 16. */
qoq_status qoq_w8a8_pack_weights(const int8_t* q, int64_t N, int64_t K, void* blob,
                                 void* stream);

/* Workspace bytes of qoq_w8a8_gemm's plan for this shape (0: none), or -1 for
 * an unsupported shape; the same split-K rule as qoq_gemm_workspace_bytes. */
int64_t qoq_w8a8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * W8A8 GEMM with the FP16 epilogue.
 *   xq, s_x from qoq_quantize_act (rowsum is not needed), blob from
 *   qoq_w8a8_pack_weights, s_c [N] FP16 from qoq_w8a8_quantize_weights.
 *   acc[m,n] = sum_k xq[m,k] * q[n,k]                            (exact INT32)
 *   y[m,n]   = f16( (f32(acc) * f32(s_x[m])) * f32(s_c[n]) )     (FP16 [M,N])
 *   acc_out, workspace and errors as for qoq_w4a8_gemm (the workspace bound is
 *   qoq_w8a8_gemm_workspace_bytes).
 */
qoq_status qoq_w8a8_gemm(const int8_t* xq, const uint16_t* s_x, const void* blob,
                         const uint16_t* s_c, int64_t M, int64_t N, int64_t K, uint16_t* y,
                         int32_t* acc_out, void* workspace, int64_t workspace_bytes,
                         void* stream);

/*
 * ---- Fused producer of the down projection's input -------------------------
 * ([GUIDE] "High-Throughput Native INT8 Tensor Core GEMMs": the GEMM writes
 * FP16 back for the operators that follow; Deep Dive part 1: every INT8 GEMM
 * input is quantized per token.) In the MLP the down projection's input is
 * SiLU(gate) * up of the gate_up GEMM's FP16 output; this call produces it and
 * quantizes it in one pass over the gate_up rows:
 *   gate_up [M, 2I] FP16 row-major: gate = columns 0..I-1, up = columns I..2I-1
 *   h[m,k]  = f16( (g / (1 + exp(-g))) * u )   g = gate, u = up, each step one
 *             IEEE fp32 operation, with exp(x) defined as: +inf for x > 88,
 *             0 for x < -86, else n = rint(x * log2(e)),
 *             r = (x - n * 0.693145751953125) - n * (ln 2 - 0.693145751953125),
 *             p = the degree-7 Taylor polynomial of e^r in Horner form
 *             (coefficients 1/k! rounded to fp32), exp = p * 2^n
 *             (Cody and Waite's reduction; within 1.2 fp32 ulps of e^x)
 *   then xq, s_x, rowsum exactly as qoq_quantize_act(h, M, I, ...).
 *   h [M, I] FP16 receives h when not NULL. I follows the K rules.
 */
qoq_status qoq_silu_mul_quantize_act(const uint16_t* gate_up, int64_t M, int64_t I, int8_t* xq,
                                     uint16_t* s_x, int32_t* rowsum, uint16_t* h, void* stream);

/*
 * The same call for few rows: with a workspace of
 * qoq_silu_mul_workspace_bytes(M, I) bytes (device memory, 16-byte aligned,
 * no initialisation needed), each row is shared by several workgroups in two
 * passes (the largest |h| of each share, then the codes, the row sum gathered
 * in a per-row 64-bit tally in the workspace), so that rows use more than one
 * compute unit. The size is 0 where the one-pass kernels are as fast (more
 * than 32 rows, or I < 12288). The outputs are those of
 * qoq_silu_mul_quantize_act bit for bit. A NULL workspace (or a size 0 one)
 * runs the one-pass kernels; a workspace smaller than needed gives
 * QOQ_ERR_WORKSPACE. Calls that overlap in time must not share a workspace.
 * qoq_silu_mul_workspace_bytes returns -1 for an unsupported shape.
 */
int64_t qoq_silu_mul_workspace_bytes(int64_t M, int64_t I);
qoq_status qoq_silu_mul_quantize_act_ws(const uint16_t* gate_up, int64_t M, int64_t I, int8_t* xq,
                                        uint16_t* s_x, int32_t* rowsum, uint16_t* h,
                                        void* workspace, int64_t workspace_bytes, void* stream);

/*
 * qoq_rmsnorm_quantize_act: the other producer of a GEMM input. ([GUIDE]
 * "High-Throughput Native INT8 Tensor Core GEMMs": the GEMM's FP16 output goes
 * on to the next layer norm; Deep Dive part 1: the GEMM input is quantized per
 * token.) The pages do not write the norm out; this is the RMSNorm of the
 * models they serve, made exact so that the codes are unique:
 *   x [M, K] FP16 row-major, gamma [K] FP16, eps > 0 (finite fp32)
 *   S    = sum_k x[m,k]^2, exactly (every FP16 square is a multiple of 2^-48)
 *   ms   = f32( f64(S) / K )            S rounded to fp64, fp64 division
 *   r    = 1 / sqrt(ms + eps)           fp32 add, square root, division
 *   y[m,k] = f16( (x[m,k] * r) * gamma[k] )   two fp32 products
 *   then xq, s_x, rowsum exactly as qoq_quantize_act(y, M, K, ...), every
 *   rounding to nearest even. y [M, K] FP16 receives y when not NULL.
 *   K follows the K rules and is at most QOQ_RMSNORM_MAX_K; x, gamma finite,
 *   with |gamma| small enough that y stays finite (|y| <= |gamma| sqrt(K)).
 *   eps <= 0, infinite or NaN gives QOQ_ERR_SHAPE.
 */
qoq_status qoq_rmsnorm_quantize_act(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M,
                                   int64_t K, int8_t* xq, uint16_t* s_x, int32_t* rowsum,
                                   uint16_t* y, void* stream);

/*
 * ---- KV4 decode attention with SmoothAttention -----------------------------
 * ([EN] section 4, the SmoothAttention paragraph; [GUIDE] part 3, SmoothAttention
 * and the 4-bit KV cache; [EN] section 3, judgment C: KV4 needs the attention
 * kernel's support, FP16 QK/SV.) Head dimension d = 128; H KV heads, Hq query
 * heads with Hq / H in {1, 2, 4, 8} (grouped-query attention: query head hq uses
 * KV head hq / (Hq / H)).
 *
 * qoq_kv4_smooth_scales: calibration keys k [T][H][128] FP16 ->
 *   lambda[h][j] = f16(sqrt(max_t |k[t][h][j]|))  (alpha = 0.5), 1 where the
 *   maximum is 0. Keys are cached as K / lambda; queries are multiplied by
 *   lambda, which leaves every q . k unchanged.
 *
 * qoq_kv4_append: quantize T new tokens k, v [B][T][H][128] FP16 into positions
 *   t0 .. t0+T-1 of the cache (t0 + T <= Tcap, Tcap a multiple of 16). For each
 *   (b, t, h) vector x = k / lambda (fp32 division) or x = v:
 *     mn = min(0, min x), mx = max(0, max x), s = f16((mx - mn) / 15),
 *     z = clip(round(-mn / s), 0, 15), c = clip(round(x / s) + z, 0, 15)
 *     (s = 0 gives c = z = 0), the per-channel W4 formulas applied per vector.
 *   Cache layout (all caller-allocated, device memory):
 *     kq [B][H][Tcap][64] bytes: byte j of a token holds channel 2j (low nibble)
 *                         and 2j + 1 (high nibble);
 *     vq [B][H][Tcap/16][64][16] bytes: blocks of 16 tokens; byte (blk, j, i) is
 *                         byte j of token 16*blk + i, nibbles as for kq;
 *     ks, vs [B][H][Tcap] FP16 scales; kz, vz [B][H][Tcap] uint8 zeros.
 *
 * qoq_kv4_decode_attention: one query token per sequence, q [B][Hq][128] FP16,
 *   lens [B] int32 device array of cached lengths (values are clamped to
 *   [0, Tcap]; a length of 0 gives a zero output). With q' = f16(q * lambda)
 *   (fp32 product) and k^ = s (c - z), v^ likewise:
 *     score_t = (q' . k^_t) / sqrt(128), p = softmax over t < len,
 *     o[b][hq] = f16(sum_t p_t v^_t)           o [B][Hq][128] FP16
 *   computed with FP16 products and FP32 sums in an order of the kernel's
 *   own (the result is not bit-specified; it is within the rounding of
 *   those operations of the exact value). Query heads per KV head: 1, 2, 4
 *   or 8. workspace: device memory of at least
 *   qoq_kv4_attention_workspace_bytes() bytes (per-chunk partial results; no
 *   initialisation needed); calls that overlap in time must not share one.
 */
qoq_status qoq_kv4_smooth_scales(const uint16_t* k, int64_t T, int64_t H, int64_t d,
                                 uint16_t* lambda, void* stream);

qoq_status qoq_kv4_append(const uint16_t* k, const uint16_t* v, const uint16_t* lambda,
                          int64_t B, int64_t T, int64_t H, int64_t d, int64_t Tcap, int64_t t0,
                          uint8_t* kq, uint16_t* ks, uint8_t* kz, uint8_t* vq, uint16_t* vs,
                          uint8_t* vz, void* stream);

/* -1 for an unsupported shape. */
int64_t qoq_kv4_attention_workspace_bytes(int64_t B, int64_t Hq, int64_t H, int64_t d,
                                          int64_t Tcap);

qoq_status qoq_kv4_decode_attention(const uint16_t* q, const uint16_t* lambda, const uint8_t* kq,
                                    const uint16_t* ks, const uint8_t* kz, const uint8_t* vq,
                                    const uint16_t* vs, const uint8_t* vz, const int32_t* lens,
                                    int64_t B, int64_t Hq, int64_t H, int64_t d, int64_t Tcap,
                                    uint16_t* o, void* workspace, int64_t workspace_bytes,
                                    void* stream);

/*
 * ---- W4A16 sibling ([W4A16]) ----------------------------------------------
 * FP16 activations against the same QoQ 4-bit weights (the blob and s_c of
 * qoq_quantize_weights / qoq_pack_weights, either mode), so that it differs
 * from qoq_w4a8_gemm only in the activation precision. The codes are
 * dequantized to FP16 in the main loop and multiplied on the FP16 matrix cores
 * with FP32 accumulation:
 *   x   [M,K] FP16 row-major (not quantized).
 *   acc[m,n] = sum_k x[m,k] * W8^[n,k]   in FP32, W8^ = (q - z) * s_g (g128) or
 *              q - z (per-channel), each product exact; the order of the FP32
 *              additions is the kernel's and is not specified, so acc lies
 *              within (K - 1) * 2^-24 * sum_k |x * W8^| of the exact sum.
 *   y[m,n]   = f16(f32(acc) * f32(s_c[n]))               (FP16 [M,N])
 *   acc_out  [M,N] float receives acc when not NULL (for inspection).
 * No workspace. Errors as for qoq_w4a8_gemm.
 */
qoq_status qoq_w4a16_gemm(int mode, const uint16_t* x, const void* blob, const uint16_t* s_c,
                          int64_t M, int64_t N, int64_t K, uint16_t* y, float* acc_out,
                          void* stream);

/*
 * ---- Checkpoint header ------------------------------------------------------
 * [EN] section 4, evaluation pseudocode, output: the quantized (W4A8KV4)
 * checkpoint. A packed weight matrix is stored as this 64-byte header, then the
 * blob of the pack call (blob_bytes bytes), then the FP16 per-channel scales
 * s_c (scale_bytes = 2 N bytes). The header is host memory: the GEMMs take
 * device pointers and never read it; a loader checks it with
 * qoq_blob_header_check before it copies the blob to the device, so that a
 * checkpoint written by a library with another blob layout, for another
 * format, group size or shape, is refused instead of being misread.
 * Little-endian fields, no padding.
 */
#define QOQ_BLOB_MAGIC 0x314B5051u /* the bytes "QPK1" */
#define QOQ_FORMAT_W8A8 2          /* format code of the W8A8 sibling's blob */

typedef struct {
    uint32_t magic;       /* QOQ_BLOB_MAGIC */
    uint32_t abi_version; /* QOQ_ABI_VERSION of the library that packed the blob */
    uint32_t format;      /* QOQ_MODE_G128, QOQ_MODE_PER_CHANNEL or QOQ_FORMAT_W8A8 */
    uint32_t group;       /* QOQ_GROUP */
    int64_t n;            /* output channels N */
    int64_t k;            /* input channels K */
    int64_t blob_bytes;   /* qoq_packed_bytes(format, N, K) or qoq_w8a8_packed_bytes(N, K) */
    int64_t scale_bytes;  /* 2 * N */
    uint8_t reserved[16]; /* zero */
} qoq_blob_header;

/* Fills *h for a blob of this format and shape (host memory). QOQ_ERR_NULL
 * for a NULL h, QOQ_ERR_MODE for an unknown format, QOQ_ERR_SHAPE for a shape
 * the pack calls reject; *h is written only on QOQ_OK. */
qoq_status qoq_blob_header_init(int format, int64_t N, int64_t K, qoq_blob_header* h);

/* QOQ_OK if *h is exactly what qoq_blob_header_init(format, N, K) writes;
 * QOQ_ERR_HEADER if any field differs (magic, ABI version, format, group,
 * shape, byte counts or a non-zero reserved byte); QOQ_ERR_NULL, QOQ_ERR_MODE
 * or QOQ_ERR_SHAPE as for qoq_blob_header_init. Reads nothing but *h. */
qoq_status qoq_blob_header_check(const qoq_blob_header* h, int format, int64_t N, int64_t K);

#ifdef __cplusplus
}
#endif

#endif /* QOQ_H_ */
