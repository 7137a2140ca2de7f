/*
 * qoq_oracle.c -- plain, slow, obviously correct CPU oracle for the QoQ W4A8
 * GEMM path (QServe, arXiv 2405.04532).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this library. It shares no source, header, table or
 * helper with the GPU library; the two are written independently from the same
 * description of the method and of the packed layout.
 *
 * Sources (page title, then the part of it that is followed):
 *   [EN]  "QServe: Low Bit Width Does Not Guarantee High Throughput"
 *         (English edition of the tabzhangjx.github.io blog post), section 4
 *         "Formalization and procedure": the stage-1 equation (per-channel INT8
 *         in the protective range [-119,119] with scale s_c = max|W_c|/119), the
 *         stage-2 equation (group UINT4 codes q = clip(round(W8/s_cg) + z, 0, 15)
 *         and reconstruction W^ = s_c * s_cg * (q - z)), and the paragraph after
 *         it (integer scale, multiply then subtract a precomputed zero-point
 *         compensation, no FP16 dequantisation in the main loop).
 *   [ZH]  "QServe：低比特不等于高吞吐" (the same post in Chinese), section 4:
 *         the same two equations.
 *   [SUM] "QServe: W4A8KV4 Quantization and System Co-design for Efficient LLM
 *         Serving" (research.elamur.ai summary), "Key points": per-channel FP16
 *         scales, protective range [-119,119], then group INT4; multiply first,
 *         subtract afterward.
 *   [GUIDE] "QServe Guide: W4A8KV4 Quantization for LLM Serving" (aifetchly),
 *         "Deep Dive" part 1: per-token symmetric INT8 activations,
 *         X8 = clamp(round(X / dX), -128, 127) with dX = max|X| / 127, and the
 *         output rescale Y = (sum_k X8 * W8) * (dX * dW) applied once; "High-
 *         Throughput Native INT8 Tensor Core GEMMs": INT32 accumulation.
 *         (That page's signed-INT4 weight format contradicts the other pages
 *         and is not used.)
 *   [WIKI] "QoQ / QServe — Quantification W4A8KV4" (brain.gartu.xyz), example
 *         configuration: weight group size 128.
 *
 * Readings where the pages are silent (numbered as in the rest of the
 * repository):
 *   R1  every "round" is round-half-to-even;
 *   R2  scales are computed in IEEE fp32 (one rounding per operation), stored as
 *       FP16 (round to nearest even), and the stored FP16 value is the one used
 *       to quantize;
 *   R3  group scale s_cg = max(1, ceil((mx - mn) / 15)), an integer;
 *   R4  group zero z = round(-mn / s_cg), exact rational rounding;
 *   R5  the group range always spans zero: mn = min(0, min W8), mx = max(0, max W8);
 *   R6  a group is 128 consecutive input channels (K) of one output channel;
 *   R7  per-channel mode: asymmetric UINT4 directly from FP16 with an FP16
 *       scale s_c = (mx - mn)/15 and a UINT4 zero, the zero-point handled in
 *       the epilogue;
 *   R8  a zero scale (all-zero row, or a scale that rounds to 0 in FP16) gives
 *       codes 0 and zero 0 (or Xq = 0);
 *   R9  the GEMM accumulator is the exact integer sum; per-channel mode's
 *       accumulator is sum_k Xq * (q - z);
 *   R10 the output is acc * s_x * s_c; here it is computed in fp64, where it is
 *       exact (31 + 11 + 11 significant bits <= 53);
 *   R13 the W8A8 sibling quantizes weights per output channel, symmetric, with
 *       scale max|W|/127 and the activations' clamp [-128, 127];
 *   R14 the W4A16 sibling keeps the activations in FP16 and reads the same QoQ
 *       4-bit weights, so that it differs from W4A8 only in the activation
 *       precision;
 *   R15 the fused producer of the down projection's input rounds
 *       SiLU(gate) * up to FP16 before quantizing it, with the exponential
 *       defined step by step below (orc_exp_f32);
 *   R16 KV4 attention: SmoothAttention scales per (KV head, channel) from
 *       calibration keys, FP16 queries multiplied by them, one asymmetric
 *       UINT4 range per (token, head) vector for keys and values.
 *   R17 the RMSNorm producer of a GEMM input: the exact sum of squares,
 *       each later step one IEEE operation (orc_rmsnorm below).
 *
 * Inputs must be finite FP16 (passed as raw binary16 bits).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_SHAPE 1
#define ORC_ERR_OVERFLOW 2
#define ORC_ERR_MODE 3

#define ORC_MODE_G128 0
#define ORC_MODE_PER_CHANNEL 1

#define GROUP 128

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16, written out from the format's definition.             */
/* ------------------------------------------------------------------------ */

/* Exact value of a binary16 bit pattern. */
double orc_f16_to_f64(uint16_t h) {
    int sign = h >> 15;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Widening to fp32 is exact: every binary16 value is a binary32 value. */
static float f16_to_f32(uint16_t h) { return (float)orc_f16_to_f64(h); }

/* binary32 -> binary16, round to nearest, ties to even. */
uint16_t orc_f32_to_f16(float f) {
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f)) return sign | 0x7e00;
    if (isinf(f)) return sign | 0x7c00;
    double a = fabs((double)f);
    if (a < ldexp(1.0, -14)) {
        /* Subnormal range: the grid spacing is 2^-24. A result of 1024 units is
         * the smallest normal number, whose encoding is the same integer. */
        double r = nearbyint(a * ldexp(1.0, 24));
        return sign | (uint16_t)r;
    }
    int e;
    (void)frexp(a, &e); /* a in [2^(e-1), 2^e) */
    int E = e - 1;      /* unbiased exponent */
    double r = nearbyint(ldexp(a, 10 - E)); /* 11-bit significand, RNE */
    if (r == 2048.0) {
        r = 1024.0;
        E += 1;
    }
    if (E > 15) return sign | 0x7c00; /* overflow rounds to infinity */
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)(r - 1024.0);
}

/* ------------------------------------------------------------------------ */
/* Small exact helpers.                                                      */
/* ------------------------------------------------------------------------ */

/* Round-half-to-even of the rational a / b, b > 0 (reading R1). */
static int64_t rne_div(int64_t a, int64_t b) {
    int64_t u = a < 0 ? -a : a;
    int64_t t = u / b, r = u % b;
    if (2 * r > b || (2 * r == b && (t & 1))) t += 1;
    return a < 0 ? -t : t;
}

static int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

/* Round-half-to-even of a finite float, as an integer (reading R1). */
static int64_t rne_f32(float v) { return (int64_t)rintf(v); }

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Activations: per-token symmetric INT8 ([GUIDE] Deep Dive part 1).         */
/*   s_x[m]  = f16( max_k |X[m,k]| / 127 )          (fp32 division, R2)       */
/*   Xq[m,k] = clamp( round(X[m,k] / s_x[m]), -128, 127 )                    */
/*   rowsum[m] = sum_k Xq[m,k]   (needed by per-channel mode's epilogue)     */
/* ------------------------------------------------------------------------ */
int orc_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* xq,
                     uint16_t* s_x, int32_t* rowsum) {
    if (M < 0 || K < 1) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = x + m * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(f16_to_f32(row[k]));
            if (a > amax) amax = a;
        }
        uint16_t s = orc_f32_to_f16(amax / 127.0f);
        float sf = f16_to_f32(s);
        int64_t sum = 0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t v = 0;
            if (sf != 0.0f) v = clamp64(rne_f32(f16_to_f32(row[k]) / sf), -128, 127);
            xq[m * K + k] = (int8_t)v;
            sum += v;
        }
        s_x[m] = s;
        if (rowsum) rowsum[m] = (int32_t)sum;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Weights, progressive group quantization ([EN]/[ZH] section 4, [SUM]).     */
/* Stage 1 (per output channel n):                                           */
/*   s_c[n]   = f16( max_k |W[n,k]| / 119 )                                  */
/*   W8[n,k]  = clip( round(W[n,k] / s_c[n]), -119, 119 )                    */
/* Stage 2 (per group g of 128 consecutive k, R3-R6):                        */
/*   mn = min(0, min W8), mx = max(0, max W8)                                */
/*   s_g = max(1, ceil((mx - mn) / 15));  z = round(-mn / s_g)               */
/*   q   = clip( round(W8 / s_g) + z, 0, 15 )                                */
/* w8 (optional, may be NULL) receives the stage-1 INT8 values.              */
/* ------------------------------------------------------------------------ */
int orc_quantize_weights_g128(const uint16_t* w, int64_t N, int64_t K, uint16_t* s_c,
                              uint8_t* q, uint8_t* s_g, uint8_t* z, int8_t* w8) {
    if (N < 0 || K < GROUP || K % GROUP) return ORC_ERR_SHAPE;
    const int64_t G = K / GROUP;
#pragma omp parallel
    {
        int64_t* row8 = (int64_t*)malloc((size_t)K * sizeof(int64_t));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            const uint16_t* row = w + n * K;
            float amax = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                float a = fabsf(f16_to_f32(row[k]));
                if (a > amax) amax = a;
            }
            uint16_t sc = orc_f32_to_f16(amax / 119.0f);
            float scf = f16_to_f32(sc);
            s_c[n] = sc;
            for (int64_t k = 0; k < K; ++k) {
                row8[k] = 0;
                if (scf != 0.0f) row8[k] = clamp64(rne_f32(f16_to_f32(row[k]) / scf), -119, 119);
                if (w8) w8[n * K + k] = (int8_t)row8[k];
            }
            for (int64_t g = 0; g < G; ++g) {
                const int64_t* grp = row8 + g * GROUP;
                int64_t mn = 0, mx = 0;
                for (int i = 0; i < GROUP; ++i) {
                    if (grp[i] < mn) mn = grp[i];
                    if (grp[i] > mx) mx = grp[i];
                }
                int64_t sg = (mx - mn + 14) / 15; /* integer ceiling */
                if (sg < 1) sg = 1;
                int64_t zz = rne_div(-mn, sg);
                s_g[n * G + g] = (uint8_t)sg;
                z[n * G + g] = (uint8_t)zz;
                for (int i = 0; i < GROUP; ++i)
                    q[n * K + g * GROUP + i] = (uint8_t)clamp64(rne_div(grp[i], sg) + zz, 0, 15);
            }
        }
        free(row8);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Weights, per-channel W4 (reading R7).                                     */
/*   mn = min(0, min_k W), mx = max(0, max_k W)                              */
/*   s_c = f16( (mx - mn) / 15 );  z = clip( round(-mn / s_c), 0, 15 )       */
/*   q   = clip( round(W / s_c) + z, 0, 15 )                                 */
/* ------------------------------------------------------------------------ */
int orc_quantize_weights_pc(const uint16_t* w, int64_t N, int64_t K, uint16_t* s_c,
                            uint8_t* q, uint8_t* z) {
    if (N < 0 || K < 1) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint16_t* row = w + n * K;
        float mn = 0.0f, mx = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = f16_to_f32(row[k]);
            if (v < mn) mn = v;
            if (v > mx) mx = v;
        }
        uint16_t sc = orc_f32_to_f16((mx - mn) / 15.0f);
        float scf = f16_to_f32(sc);
        s_c[n] = sc;
        int64_t zz = 0;
        if (scf != 0.0f) zz = clamp64(rne_f32(-mn / scf), 0, 15);
        z[n] = (uint8_t)zz;
        for (int64_t k = 0; k < K; ++k) {
            int64_t v = 0;
            if (scf != 0.0f) v = clamp64(rne_f32(f16_to_f32(row[k]) / scf) + zz, 0, 15);
            q[n * K + k] = (uint8_t)v;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Reconstruction ([EN] section 4, stage-2 equation): W^ = s_c * s_g * (q - z) */
/* (per-channel mode: W^ = s_c * (q - z)). Exact in fp64.                    */
/* ------------------------------------------------------------------------ */
int orc_dequantize_weights(int mode, const uint16_t* s_c, const uint8_t* q, const uint8_t* s_g,
                           const uint8_t* z, int64_t N, int64_t K, double* w_hat) {
    if (mode != ORC_MODE_G128 && mode != ORC_MODE_PER_CHANNEL) return ORC_ERR_MODE;
    if (mode == ORC_MODE_G128 && (K < GROUP || K % GROUP)) return ORC_ERR_SHAPE;
    const int64_t G = K / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double sc = orc_f16_to_f64(s_c[n]);
        for (int64_t k = 0; k < K; ++k) {
            double v;
            if (mode == ORC_MODE_G128)
                v = sc * (double)s_g[n * G + k / GROUP] *
                    (double)((int)q[n * K + k] - (int)z[n * G + k / GROUP]);
            else
                v = sc * (double)((int)q[n * K + k] - (int)z[n]);
            w_hat[n * K + k] = v;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Packed layout (the gfx950 MFMA operand order; the GPU packer implements   */
/* the same written specification independently).                          */
/*                                                                          */
/* Codes: one 1024-byte tile per (t, g), t = n / 16, g = k / 128, at byte    */
/* offset (t * G + g) * 1024. Within a tile, with c = n % 16 and the offset  */
/* kk = k % 128 written as kk = 64 s + 16 j + i (s in 0..1, j in 0..3,       */
/* i in 0..15):                                                              */
/*   lane  = 16 j + c                (64 lanes x 16 bytes)                   */
/*   kappa = 16 s + i                (0..31, the lane's code index)          */
/*   byte  = 16 lane + 4 (kappa / 8) + (kappa % 4)                           */
/*   nibble: low if (kappa % 8) < 4, else high.                              */
/* Parameters follow the codes (offset N * K / 2):                           */
/*   g128: 16 bytes per (t, g) at (t * G + g) * 16, byte c of which is       */
/*         ((s_g - 1) << 4) | z of channel 16 t + c in group g;              */
/*   per-channel: N bytes, byte n is z[n].                                   */
/* ------------------------------------------------------------------------ */
int64_t orc_packed_bytes(int mode, int64_t N, int64_t K) {
    if (K < GROUP || K % GROUP || N < 16 || N % 16) return -1;
    int64_t codes = N * K / 2;
    if (mode == ORC_MODE_G128) return codes + N * (K / GROUP);
    if (mode == ORC_MODE_PER_CHANNEL) return codes + N;
    return -1;
}

int orc_pack(int mode, const uint8_t* q, const uint8_t* s_g, const uint8_t* z, int64_t N,
             int64_t K, uint8_t* blob) {
    int64_t total = orc_packed_bytes(mode, N, K);
    if (total < 0) return ORC_ERR_SHAPE;
    memset(blob, 0, (size_t)total);
    const int64_t G = K / GROUP;
    for (int64_t n = 0; n < N; ++n) {
        int64_t t = n / 16, c = n % 16;
        for (int64_t k = 0; k < K; ++k) {
            int64_t g = k / GROUP, kk = k % GROUP;
            int64_t s = kk / 64, j = (kk % 64) / 16, i = kk % 16;
            int64_t lane = 16 * j + c;
            int64_t kappa = 16 * s + i;
            int64_t off = (t * G + g) * 1024 + 16 * lane + 4 * (kappa / 8) + (kappa % 4);
            int shift = (kappa % 8) < 4 ? 0 : 4;
            blob[off] |= (uint8_t)((q[n * K + k] & 15) << shift);
        }
    }
    uint8_t* params = blob + N * K / 2;
    if (mode == ORC_MODE_G128) {
        for (int64_t n = 0; n < N; ++n)
            for (int64_t g = 0; g < G; ++g)
                params[((n / 16) * G + g) * 16 + n % 16] =
                    (uint8_t)(((s_g[n * G + g] - 1) << 4) | (z[n * G + g] & 15));
    } else {
        for (int64_t n = 0; n < N; ++n) params[n] = z[n];
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Packed activations (the GPU quantizer's output order; written here from    */
/* the same written specification, independently of the GPU code).          */
/* Mp = roundup(M, 16) rows; rows M..Mp-1 are zero. Tile (g, u) = rows        */
/* 16u..16u+15, inputs 128g..128g+127, 2048 bytes at (g * Mp/16 + u) * 2048. */
/* With k % 128 = 64 s + 16 j + i and r = m % 16, the byte of (m, k) is at    */
/* 1024 s + 16 (16 j + r) + i within the tile.                               */
/* ------------------------------------------------------------------------ */
int64_t orc_act_bytes(int64_t M, int64_t K) {
    if (M < 0 || K < GROUP || K % GROUP) return -1;
    return (M + 15) / 16 * 16 * K;
}

int orc_pack_act(const int8_t* xq, int64_t M, int64_t K, int8_t* out) {
    int64_t total = orc_act_bytes(M, K);
    if (total < 0) return ORC_ERR_SHAPE;
    memset(out, 0, (size_t)total);
    const int64_t U = (M + 15) / 16;
    for (int64_t m = 0; m < M; ++m) {
        const int64_t u = m / 16, r = m % 16;
        for (int64_t k = 0; k < K; ++k) {
            const int64_t g = k / GROUP, kk = k % GROUP;
            const int64_t s = kk / 64, j = (kk % 64) / 16, i = kk % 16;
            out[(g * U + u) * 2048 + 1024 * s + 16 * (16 * j + r) + i] = xq[m * K + k];
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* GEMM: INT8 x INT8 with an exact integer accumulator ([GUIDE] "INT32       */
/* accumulators"; [EN] section 4: the weight operand is the INT8 value       */
/* W8^ = (q - z) * s_g of the stage-2 equation).                             */
/*   g128:        acc[m,n] = sum_k Xq[m,k] * (q[n,k] - z[n,g]) * s_g[n,g]     */
/*   per-channel: acc[m,n] = sum_k Xq[m,k] * (q[n,k] - z[n])                 */
/* The sum is taken in int64; a value outside int32 is an error.            */
/* ------------------------------------------------------------------------ */
static void weight_row_int(int mode, const uint8_t* q, const uint8_t* s_g, const uint8_t* z,
                           int64_t n, int64_t K, int64_t* out) {
    const int64_t G = K / GROUP;
    for (int64_t k = 0; k < K; ++k) {
        if (mode == ORC_MODE_G128)
            out[k] = ((int64_t)q[n * K + k] - z[n * G + k / GROUP]) * s_g[n * G + k / GROUP];
        else
            out[k] = (int64_t)q[n * K + k] - z[n];
    }
}

int orc_gemm(int mode, const int8_t* xq, const uint8_t* q, const uint8_t* s_g, const uint8_t* z,
             int64_t M, int64_t N, int64_t K, int32_t* acc) {
    if (mode != ORC_MODE_G128 && mode != ORC_MODE_PER_CHANNEL) return ORC_ERR_MODE;
    if (M < 0 || N < 0 || K < 1 || (mode == ORC_MODE_G128 && K % GROUP)) return ORC_ERR_SHAPE;
    int overflow = 0;
#pragma omp parallel
    {
        int64_t* wrow = (int64_t*)malloc((size_t)K * sizeof(int64_t));
#pragma omp for schedule(static) reduction(| : overflow)
        for (int64_t n = 0; n < N; ++n) {
            weight_row_int(mode, q, s_g, z, n, K, wrow);
            for (int64_t m = 0; m < M; ++m) {
                const int8_t* xr = xq + m * K;
                int64_t s = 0;
                for (int64_t k = 0; k < K; ++k) s += (int64_t)xr[k] * wrow[k];
                if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
                acc[m * N + n] = (int32_t)s;
            }
        }
        free(wrow);
    }
    return overflow ? ORC_ERR_OVERFLOW : ORC_OK;
}

/* The same accumulator at P chosen (m, n) points, for shapes too large to
 * contract whole on the host. */
int orc_gemm_points(int mode, const int8_t* xq, const uint8_t* q, const uint8_t* s_g,
                    const uint8_t* z, int64_t M, int64_t N, int64_t K, int64_t P,
                    const int64_t* ms, const int64_t* ns, int32_t* acc) {
    if (mode != ORC_MODE_G128 && mode != ORC_MODE_PER_CHANNEL) return ORC_ERR_MODE;
    if (K < 1 || (mode == ORC_MODE_G128 && K % GROUP)) return ORC_ERR_SHAPE;
    for (int64_t p = 0; p < P; ++p)
        if (ms[p] < 0 || ms[p] >= M || ns[p] < 0 || ns[p] >= N) return ORC_ERR_SHAPE;
    const int64_t G = K / GROUP;
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t p = 0; p < P; ++p) {
        int64_t m = ms[p], n = ns[p];
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t wv = mode == ORC_MODE_G128
                             ? ((int64_t)q[n * K + k] - z[n * G + k / GROUP]) * s_g[n * G + k / GROUP]
                             : (int64_t)q[n * K + k] - z[n];
            s += (int64_t)xq[m * K + k] * wv;
        }
        if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
        acc[p] = (int32_t)s;
    }
    return overflow ? ORC_ERR_OVERFLOW : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Epilogue ([GUIDE] Deep Dive part 1: the rescale by the activation scale    */
/* and the weight scale, applied once): Y[m,n] = acc[m,n] * s_x[m] * s_c[n]. */
/* Computed in fp64, where it is exact (R10); not rounded to FP16.           */
/* ------------------------------------------------------------------------ */
int orc_epilogue(const int32_t* acc, const uint16_t* s_x, const uint16_t* s_c, int64_t M,
                 int64_t N, double* y) {
    if (M < 0 || N < 0) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = (double)acc[m * N + n] * orc_f16_to_f64(s_x[m]) * orc_f16_to_f64(s_c[n]);
    return ORC_OK;
}

int orc_epilogue_points(const int32_t* acc, const uint16_t* s_x, const uint16_t* s_c, int64_t P,
                        const int64_t* ms, const int64_t* ns, double* y) {
    for (int64_t p = 0; p < P; ++p)
        y[p] = (double)acc[p] * orc_f16_to_f64(s_x[ms[p]]) * orc_f16_to_f64(s_c[ns[p]]);
    return ORC_OK;
}

/* Array forms of the binary16 conversions, for tests over many values. */
void orc_f32_to_f16_array(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_f16(in[i]);
}

void orc_f16_to_f64_array(const uint16_t* in, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f64(in[i]);
}

/* ------------------------------------------------------------------------ */
/* W8A8 sibling ("QServe Guide: W4A8KV4 Quantization for LLM Serving", "The  */
/* Problem" item 2: weights and activations both INT8 on the INT8 matrix     */
/* units; weight scaling per output channel and symmetric as in "Deep Dive"  */
/* part 1, with the 8-bit bound 127 in place of the 4-bit bound 7: reading  */
/* R13 above).                                                              */
/*   s_c[n] = f16( max_k |W[n,k]| / 127 )          (fp32 division, R2)        */
/*   q[n,k] = clamp( round(W[n,k] / s_c[n]), -128, 127 )   (R8: q = 0 if s_c = 0) */
/* |W / s_c| <= 127 * (1 + 2^-11) rounds to at most 127, so -128 never       */
/* occurs and the weights are symmetric in practice.                        */
/* ------------------------------------------------------------------------ */
int orc_quantize_weights_w8(const uint16_t* w, int64_t N, int64_t K, uint16_t* s_c, int8_t* q) {
    if (N < 0 || K < 1) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint16_t* row = w + n * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(f16_to_f32(row[k]));
            if (a > amax) amax = a;
        }
        uint16_t sc = orc_f32_to_f16(amax / 127.0f);
        float scf = f16_to_f32(sc);
        s_c[n] = sc;
        for (int64_t k = 0; k < K; ++k) {
            int64_t v = 0;
            if (scf != 0.0f) v = clamp64(rne_f32(f16_to_f32(row[k]) / scf), -128, 127);
            q[n * K + k] = (int8_t)v;
        }
    }
    return ORC_OK;
}

/* Packed INT8 weights: one 2048-byte tile per (t, g), t = n / 16, g = k / 128,
 * at byte offset (t * G + g) * 2048. With c = n % 16 and k % 128 = 64 s +
 * 16 j + i (s in 0..1, j in 0..3, i in 0..15), the byte of (n, k) sits at
 * 1024 s + 16 (16 j + c) + i within the tile: the same order as the packed
 * activations, with the channel in place of the row. */
int64_t orc_w8_packed_bytes(int64_t N, int64_t K) {
    if (K < GROUP || K % GROUP || N < 16 || N % 16) return -1;
    return N * K;
}

int orc_pack_w8(const int8_t* q, int64_t N, int64_t K, uint8_t* blob) {
    if (orc_w8_packed_bytes(N, K) < 0) return ORC_ERR_SHAPE;
    const int64_t G = K / GROUP;
    for (int64_t n = 0; n < N; ++n) {
        const int64_t t = n / 16, c = n % 16;
        for (int64_t k = 0; k < K; ++k) {
            const int64_t g = k / GROUP, kk = k % GROUP;
            const int64_t s = kk / 64, j = (kk % 64) / 16, i = kk % 16;
            blob[(t * G + g) * 2048 + 1024 * s + 16 * (16 * j + c) + i] = (uint8_t)q[n * K + k];
        }
    }
    return ORC_OK;
}

/* acc[m,n] = sum_k Xq[m,k] * q[n,k], exact in int64; a value outside int32 is
 * an error. The output is the same one-time rescale as for W4A8
 * (orc_epilogue): Y = acc * s_x[m] * s_c[n]. */
int orc_gemm_w8(const int8_t* xq, const int8_t* q, int64_t M, int64_t N, int64_t K, int32_t* acc) {
    if (M < 0 || N < 0 || K < 1) return ORC_ERR_SHAPE;
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t n = 0; n < N; ++n) {
        const int8_t* wr = q + n * K;
        for (int64_t m = 0; m < M; ++m) {
            const int8_t* xr = xq + m * K;
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int64_t)xr[k] * wr[k];
            if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
            acc[m * N + n] = (int32_t)s;
        }
    }
    return overflow ? ORC_ERR_OVERFLOW : ORC_OK;
}

int orc_gemm_w8_points(const int8_t* xq, const int8_t* q, int64_t M, int64_t N, int64_t K,
                       int64_t P, const int64_t* ms, const int64_t* ns, int32_t* acc) {
    if (K < 1) return ORC_ERR_SHAPE;
    for (int64_t p = 0; p < P; ++p)
        if (ms[p] < 0 || ms[p] >= M || ns[p] < 0 || ns[p] >= N) return ORC_ERR_SHAPE;
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t p = 0; p < P; ++p) {
        const int8_t* xr = xq + ms[p] * K;
        const int8_t* wr = q + ns[p] * K;
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k) s += (int64_t)xr[k] * wr[k];
        if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
        acc[p] = (int32_t)s;
    }
    return overflow ? ORC_ERR_OVERFLOW : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* W4A16 sibling ("QServe Guide: W4A8KV4 Quantization for LLM Serving", "The */
/* Problem" item 1: 4-bit weights dequantized in the main loop, activations  */
/* kept in FP16, FP16 matrix units; "QServe: Low Bit Width Does Not          */
/* Guarantee High Throughput", section 2, the W4A16 failure mode). Reading   */
/* R14: the weights are the same QoQ 4-bit weights as W4A8 (either mode),    */
/* so that the two formats differ only in the activation precision:          */
/*   Y[m,n] = sum_k X[m,k] * W^[n,k],  W^ = s_c * s_g * (q - z)              */
/*          = s_c[n] * sum_k X[m,k] * W8^[n,k]                               */
/* The inner sum is taken in fp64 over the integer weights W8^ (every term   */
/* X * W8^ is exact in fp64, and so is the final product by s_c up to one    */
/* rounding); absum[m,n] = s_c[n] * sum_k |X[m,k] * W8^[n,k]| is returned     */
/* for the error bound of an fp32 accumulation (absum may be NULL).          */
/* ------------------------------------------------------------------------ */
int orc_gemm_w4a16(int mode, const uint16_t* x, const uint16_t* s_c, const uint8_t* q,
                   const uint8_t* s_g, const uint8_t* z, int64_t M, int64_t N, int64_t K,
                   double* y, double* absum) {
    if (mode != ORC_MODE_G128 && mode != ORC_MODE_PER_CHANNEL) return ORC_ERR_MODE;
    if (M < 0 || N < 0 || K < 1 || (mode == ORC_MODE_G128 && K % GROUP)) return ORC_ERR_SHAPE;
#pragma omp parallel
    {
        int64_t* wrow = (int64_t*)malloc((size_t)K * sizeof(int64_t));
        double* xrow = (double*)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            weight_row_int(mode, q, s_g, z, n, K, wrow);
            const double sc = orc_f16_to_f64(s_c[n]);
            for (int64_t m = 0; m < M; ++m) {
                for (int64_t k = 0; k < K; ++k) xrow[k] = orc_f16_to_f64(x[m * K + k]);
                double s = 0.0, a = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const double t = xrow[k] * (double)wrow[k];
                    s += t;
                    a += fabs(t);
                }
                y[m * N + n] = s * sc;
                if (absum) absum[m * N + n] = a * sc;
            }
        }
        free(wrow);
        free(xrow);
    }
    return ORC_OK;
}

/* The same at P chosen (m, n) points. */
int orc_gemm_w4a16_points(int mode, const uint16_t* x, const uint16_t* s_c, const uint8_t* q,
                          const uint8_t* s_g, const uint8_t* z, int64_t M, int64_t N, int64_t K,
                          int64_t P, const int64_t* ms, const int64_t* ns, double* y,
                          double* absum) {
    if (mode != ORC_MODE_G128 && mode != ORC_MODE_PER_CHANNEL) return ORC_ERR_MODE;
    if (K < 1 || (mode == ORC_MODE_G128 && K % GROUP)) return ORC_ERR_SHAPE;
    for (int64_t p = 0; p < P; ++p)
        if (ms[p] < 0 || ms[p] >= M || ns[p] < 0 || ns[p] >= N) return ORC_ERR_SHAPE;
    const int64_t G = K / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < P; ++p) {
        const int64_t m = ms[p], n = ns[p];
        double s = 0.0, a = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const int64_t wv =
                mode == ORC_MODE_G128
                    ? ((int64_t)q[n * K + k] - z[n * G + k / GROUP]) * s_g[n * G + k / GROUP]
                    : (int64_t)q[n * K + k] - z[n];
            const double t = orc_f16_to_f64(x[m * K + k]) * (double)wv;
            s += t;
            a += fabs(t);
        }
        const double sc = orc_f16_to_f64(s_c[n]);
        y[p] = s * sc;
        if (absum) absum[p] = a * sc;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Fused producer of the down projection's input (reading R15): the MLP's   */
/* h = SiLU(gate) * up, rounded to FP16, then the per-token INT8            */
/* quantization of orc_quantize_act. The pages quantize the activations     */
/* that feed each INT8 GEMM per token ("QServe Guide: W4A8KV4 Quantization  */
/* for LLM Serving", Deep Dive part 1); the input of the down projection is */
/* the product of the gate and up projections of the same MLP, whose        */
/* outputs are one fused [M, 2I] matrix here (gate in columns 0..I-1, up in */
/* columns I..2I-1).                                                        */
/*                                                                          */
/* The exponential is defined here, step by step, so that the GPU computes  */
/* the same FP32 value (the quantized codes depend on it): Cody and Waite's */
/* range reduction x = n ln2 + r with ln2 split in two parts (the first     */
/* with trailing zero bits, so that n * ln2_hi is exact), then exp(r) by    */
/* its Taylor polynomial of degree 7 in Horner form, then the scaling by    */
/* 2^n. Every step is one IEEE fp32 operation (no fused multiply-add):      */
/*   x > 88  -> +inf;  x < -86 -> 0   (keeps 2^n and the result normal)     */
/*   n = rint(x * log2(e))                                                  */
/*   r = (x - n * ln2_hi) - n * ln2_lo                                      */
/*   p = (((((((1/7! r + 1/6!) r + 1/5!) r + 1/4!) r + 1/3!) r + 1/2) r + 1) r + 1 */
/*   exp(x) = p * 2^n                                                       */
/* The constants are the fp32 roundings of the stated real numbers.          */
/* ------------------------------------------------------------------------ */
#define ORC_LN2_HI 0.693145751953125f /* ln 2 to 16 significant bits (exact in fp32) */

float orc_exp_f32(float x) {
    if (x > 88.0f) return INFINITY;
    if (x < -86.0f) return 0.0f;
    const float log2e = (float)1.4426950408889634;   /* 1 / ln 2 */
    const float ln2_lo = (float)(0.6931471805599453 - 0.693145751953125);
    const float n = rintf(x * log2e);
    const float r = (x - n * ORC_LN2_HI) - n * ln2_lo;
    float p = (float)(1.0 / 5040.0);
    p = p * r + (float)(1.0 / 720.0);
    p = p * r + (float)(1.0 / 120.0);
    p = p * r + (float)(1.0 / 24.0);
    p = p * r + (float)(1.0 / 6.0);
    p = p * r + 0.5f;
    p = p * r + 1.0f;
    p = p * r + 1.0f;
    /* 2^n as an fp32 bit pattern (n in [-124, 127] after the clamps) */
    const int32_t ni = (int32_t)n;
    const uint32_t bits = (uint32_t)(ni + 127) << 23;
    float scale;
    memcpy(&scale, &bits, sizeof scale);
    return p * scale;
}

void orc_exp_f32_array(const float* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_exp_f32(in[i]);
}

/* h[m,k] = f16( (g / (1 + exp(-g))) * u ), g = gate_up[m, k], u = gate_up[m, I + k],
 * every operation in IEEE fp32 (reading R15). */
int orc_silu_mul(const uint16_t* gate_up, int64_t M, int64_t I, uint16_t* h) {
    if (M < 0 || I < 1) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = gate_up + m * 2 * I;
        for (int64_t k = 0; k < I; ++k) {
            const float g = f16_to_f32(row[k]);
            const float u = f16_to_f32(row[I + k]);
            const float t = 1.0f + orc_exp_f32(-g);
            const float s = g / t;
            h[m * I + k] = orc_f32_to_f16(s * u);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* KV4 decode attention with SmoothAttention (reading R16).                 */
/*                                                                          */
/* SmoothAttention ("QServe: Low Bit Width Does Not Guarantee High          */
/* Throughput", section 4, the SmoothAttention paragraph; "QServe Guide",   */
/* part 3): a per-channel scale lambda_j moves key outliers into the        */
/* queries, K'_j = K_j / lambda_j and Q'_j = Q_j * lambda_j, which leaves    */
/* Q K^T unchanged; lambda_j = max_t |K_{t,j}|^alpha with alpha = 0.5,       */
/* estimated on calibration keys. Here per (KV head, channel):              */
/*   lambda[h,j] = f16( sqrt( max_t |K[t,h,j]| ) )   (1 if the maximum is 0)  */
/* KV4: every token's key (after smoothing) and value vector of one head is   */
/* quantized to asymmetric UINT4 over its d channels, with an FP16 scale and */
/* a UINT4 zero (the per-channel W4 formulas of reading R7, one range per    */
/* (token, head)):                                                          */
/*   x = K[t,h,:] / lambda[h,:]  (fp32 division)   or   x = V[t,h,:]         */
/*   mn = min(0, min x), mx = max(0, max x), s = f16((mx - mn) / 15)          */
/*   z = clip(round(-mn / s), 0, 15), q = clip(round(x / s) + z, 0, 15)      */
/*   (s = 0: q = z = 0)                                                     */
/* Layouts: keys and values in [B][T][H][d] FP16; caches [B][H][Tcap][d]     */
/* codes (one per byte here; the GPU packs two per byte), scales and zeros   */
/* [B][H][Tcap].                                                            */
/* ------------------------------------------------------------------------ */
int orc_kv4_smooth_scales(const uint16_t* k, int64_t T, int64_t H, int64_t d, uint16_t* lambda) {
    if (T < 0 || H < 1 || d < 1) return ORC_ERR_SHAPE;
    for (int64_t h = 0; h < H; ++h)
        for (int64_t j = 0; j < d; ++j) {
            float mx = 0.0f;
            for (int64_t t = 0; t < T; ++t) {
                const float a = fabsf(f16_to_f32(k[(t * H + h) * d + j]));
                if (a > mx) mx = a;
            }
            lambda[h * d + j] = mx > 0.0f ? orc_f32_to_f16(sqrtf(mx)) : orc_f32_to_f16(1.0f);
        }
    return ORC_OK;
}

/* One (token, head) vector -> codes, FP16 scale, zero. */
static void kv4_quant_vec(const float* x, int64_t d, uint8_t* q, uint16_t* s_out, uint8_t* z_out) {
    float mn = 0.0f, mx = 0.0f;
    for (int64_t j = 0; j < d; ++j) {
        if (x[j] < mn) mn = x[j];
        if (x[j] > mx) mx = x[j];
    }
    const uint16_t sb = orc_f32_to_f16((mx - mn) / 15.0f);
    const float sf = f16_to_f32(sb);
    int64_t zz = 0;
    if (sf != 0.0f) zz = clamp64(rne_f32(-mn / sf), 0, 15);
    for (int64_t j = 0; j < d; ++j)
        q[j] = (uint8_t)(sf != 0.0f ? clamp64(rne_f32(x[j] / sf) + zz, 0, 15) : 0);
    *s_out = sb;
    *z_out = (uint8_t)zz;
}

int orc_kv4_quantize(const uint16_t* k, const uint16_t* v, const uint16_t* lambda, int64_t B,
                     int64_t T, int64_t H, int64_t d, int64_t Tcap, uint8_t* kq, uint16_t* ks,
                     uint8_t* kz, uint8_t* vq, uint16_t* vs, uint8_t* vz) {
    if (B < 0 || T < 0 || H < 1 || d < 1 || Tcap < T) return ORC_ERR_SHAPE;
#pragma omp parallel
    {
        float* x = (float*)malloc((size_t)d * sizeof(float));
#pragma omp for schedule(static) collapse(2)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t t = 0; t < T; ++t) {
                    const int64_t src = ((b * T + t) * H + h) * d;
                    const int64_t row = (b * H + h) * Tcap + t;
                    for (int64_t j = 0; j < d; ++j)
                        x[j] = f16_to_f32(k[src + j]) / f16_to_f32(lambda[h * d + j]);
                    kv4_quant_vec(x, d, kq + row * d, ks + row, kz + row);
                    for (int64_t j = 0; j < d; ++j) x[j] = f16_to_f32(v[src + j]);
                    kv4_quant_vec(x, d, vq + row * d, vs + row, vz + row);
                }
        free(x);
    }
    return ORC_OK;
}

/* Decode attention of one query token per sequence, in fp64 from the cache:
 *   q'[j]   = f16( q[b,hq,j] * lambda[h,j] )   (h = hq / (Hq / H), FP16 queries)
 *   k^[t,j] = s_t * (q_t,j - z_t)   (exact), the same for v^
 *   score_t = sum_j q'[j] k^[t,j] / sqrt(d),  p = softmax(score over t < len[b])
 *   o[b,hq,:] = sum_t p_t v^[t,:]        (fp64, not rounded) */
int orc_kv4_decode_attention(const uint16_t* q, const uint16_t* lambda, const uint8_t* kq,
                             const uint16_t* ks, const uint8_t* kz, const uint8_t* vq,
                             const uint16_t* vs, const uint8_t* vz, const int32_t* lens,
                             int64_t B, int64_t Hq, int64_t H, int64_t d, int64_t Tcap,
                             double* o) {
    if (B < 0 || H < 1 || Hq < H || Hq % H || d < 1) return ORC_ERR_SHAPE;
    for (int64_t b = 0; b < B; ++b)
        if (lens[b] < 1 || lens[b] > Tcap) return ORC_ERR_SHAPE;
    const int64_t group = Hq / H;
#pragma omp parallel
    {
        double* qs = (double*)malloc((size_t)d * sizeof(double));
        double* sc = (double*)malloc((size_t)Tcap * sizeof(double));
#pragma omp for schedule(static) collapse(2)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t hq = 0; hq < Hq; ++hq) {
                const int64_t h = hq / group;
                for (int64_t j = 0; j < d; ++j)
                    qs[j] = orc_f16_to_f64(orc_f32_to_f16(f16_to_f32(q[(b * Hq + hq) * d + j]) *
                                                          f16_to_f32(lambda[h * d + j])));
                const int64_t L = lens[b];
                double mx = -INFINITY;
                for (int64_t t = 0; t < L; ++t) {
                    const int64_t row = (b * H + h) * Tcap + t;
                    const double s = orc_f16_to_f64(ks[row]);
                    double acc = 0.0;
                    for (int64_t j = 0; j < d; ++j)
                        acc += qs[j] * (s * ((double)kq[row * d + j] - (double)kz[row]));
                    sc[t] = acc / sqrt((double)d);
                    if (sc[t] > mx) mx = sc[t];
                }
                double den = 0.0;
                for (int64_t t = 0; t < L; ++t) {
                    sc[t] = exp(sc[t] - mx);
                    den += sc[t];
                }
                for (int64_t j = 0; j < d; ++j) {
                    double acc = 0.0;
                    for (int64_t t = 0; t < L; ++t) {
                        const int64_t row = (b * H + h) * Tcap + t;
                        acc += sc[t] * (orc_f16_to_f64(vs[row]) *
                                        ((double)vq[row * d + j] - (double)vz[row]));
                    }
                    o[(b * Hq + hq) * d + j] = acc / den;
                }
            }
        free(qs);
        free(sc);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm producer of a GEMM input (reading R17). The GEMM's FP16 outputs  */
/* feed the next layer's norm, whose output is quantized per token to INT8  */
/* for the next GEMM ("QServe Guide: W4A8KV4 Quantization for LLM Serving", */
/* "High-Throughput Native INT8 Tensor Core GEMMs" and "Deep Dive" part 1). */
/* The pages do not give the norm; the models they serve use RMSNorm,       */
/*   y_k = x_k / sqrt(mean_k(x_k^2) + eps) * gamma_k,                        */
/* made exact here so that the INT8 codes downstream are unique:           */
/*   S  = sum_k x_k^2, exactly (each FP16 x_k = M 2^(e - 24) squares to an   */
/*        integer multiple of 2^-48; the sum is kept in 128 bits)           */
/*   ms = f32( f64(S) / K )      S rounded to fp64, fp64 division, to fp32  */
/*   r  = 1 / sqrt(ms + eps)     fp32 add, fp32 sqrt, fp32 division         */
/*   y_k = f16( (x_k * r) * gamma_k )   two fp32 products, then FP16        */
/* with every rounding to nearest even. r is returned per row when r_out is */
/* not NULL. eps > 0.                                                       */
/* ------------------------------------------------------------------------ */
int orc_rmsnorm(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M, int64_t K,
                uint16_t* y, float* r_out) {
    if (M < 0 || K < 1 || !(eps > 0.0f) || isinf(eps)) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* row = x + m * K;
        unsigned __int128 S = 0;  /* in units of 2^-48 */
        for (int64_t k = 0; k < K; ++k) {
            const unsigned e = (row[k] >> 10) & 31u, f = row[k] & 1023u;
            const uint64_t mant = e ? (1024u | f) : f;   /* |x| = mant * 2^(max(e,1) - 25) */
            const unsigned shift = 2u * (e ? e - 1u : 0u); /* x^2 = mant^2 * 2^(shift - 48) */
            S += (unsigned __int128)(mant * mant) << shift;
        }
        const double s64 = (double)S * 0x1p-48;
        const float ms = (float)(s64 / (double)K);
        const float v = ms + eps;
        const float r = 1.0f / sqrtf(v);
        if (r_out) r_out[m] = r;
        for (int64_t k = 0; k < K; ++k) {
            const float t = f16_to_f32(row[k]) * r;
            y[m * K + k] = orc_f32_to_f16(t * f16_to_f32(gamma[k]));
        }
    }
    return ORC_OK;
}
