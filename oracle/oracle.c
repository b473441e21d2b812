/*
 * Scalar CPU oracle for the BitNet b1.58 BitLinear layer.  TEST
 * INFRASTRUCTURE ONLY: see oracle.h for who may load it, the method's source
 * (transformers "BitNet" page, sections "Model details" and "BitNetConfig")
 * and the packed format.
 *
 * Build: gcc -O2 -fno-tree-vectorize -ffp-contract=off -fPIC -shared
 * (x86-64 SSE arithmetic: binary32 operations are correctly rounded and no
 * multiply-add is fused).  Built twice from this one file: without OpenMP
 * (liboracle.so, one core; the pragmas below are then inert) and with
 * -fopenmp (liboracle_mt.so).  The pragmas only split the outermost loop of a
 * step over threads (tokens, or tokens x output rows): every element is still
 * computed by the same inner loop in the same order, so both builds give
 * identical results.  Sums whose order spans the split loop (the absmean)
 * stay serial.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* "Model details" / Quantization: weights are scaled by their absmean.
 * The page does not fix the granularity; one scale per weight tensor. */
float orc_absmean_scale(const float* W, int64_t N, int64_t K) {
    double total = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double row = 0.0;
        for (int64_t k = 0; k < K; ++k) row += fabs((double)W[n * K + k]);
        total += row;
    }
    float mean = (float)(total / (double)(N * K));
    /* floor keeps the divide below finite for an all-zero tensor */
    if (!(mean >= 1e-5f)) mean = 1e-5f;
    return mean;
}

/* "Model details" / Quantization: ternary {-1, 0, +1} from W / absmean,
 * rounded to the nearest integer (ties to even) and clipped. */
void orc_ternarize(const float* W, int64_t N, int64_t K, float gamma, int8_t* q) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N * K; ++i) {
        float t = W[i] / gamma;
        float r = rintf(t);
        if (r > 1.0f) r = 1.0f;
        if (r < -1.0f) r = -1.0f;
        q[i] = (int8_t)r;
    }
}

/* Byte holding weight (n, k) and the bit offset of its code (layout in
 * oracle.h): rows in tiles of 16 (the last tile has R = N - 16t rows); in a
 * tile, the 16-byte chunk c = k / 64 of tile row r sits at 16 (c R + r);
 * inside a chunk, weight 16d + 4j + b sits in byte 4d + b at bit 2j. */
static int64_t packed_offset(int64_t n, int64_t k, int64_t N, int64_t K) {
    const int64_t t = n / 16, r = n % 16;
    const int64_t R = N - 16 * t < 16 ? N - 16 * t : 16;
    const int64_t c = k / 64, kk = k % 64;
    return 16 * t * (K / 4) + 16 * (c * R + r) + 4 * (kk / 16) + (kk % 4);
}
static int packed_shift(int64_t k) { return (int)(2 * ((k / 4) % 4)); }

int orc_pack(const int8_t* q, int64_t N, int64_t K, uint8_t* packed) {
    if (K % 64 != 0) return -1;
    memset(packed, 0, (size_t)(N * (K / 4)));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int v = q[n * K + k];
            if (v < -1 || v > 1) return -1;
            unsigned code = (unsigned)(v + 1);
            packed[packed_offset(n, k, N, K)] |= (uint8_t)(code << packed_shift(k));
        }
    }
    return 0;
}

int orc_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* q) {
    if (K % 64 != 0) return -1;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            unsigned code = (packed[packed_offset(n, k, N, K)] >> packed_shift(k)) & 3u;
            if (code == 3u) return -1;
            q[n * K + k] = (int8_t)((int)code - 1);
        }
    }
    return 0;
}

/* The plain 2-bit form of ternary weights: row-major, four consecutive
 * weights per byte, weight k of row n in byte n*(K/4) + k/4 at bits
 * 2*(k%4) (lowest first), code q + 1.  The page names packed 1.58-bit
 * weights ("Model variants") without a layout; this is the form a caller
 * outside this library is most likely to hold. */
int orc_pack_canonical(const int8_t* q, int64_t N, int64_t K, uint8_t* bytes) {
    if (K % 4 != 0) return -1;
    memset(bytes, 0, (size_t)(N * (K / 4)));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            int v = q[n * K + k];
            if (v < -1 || v > 1) return -1;
            bytes[n * (K / 4) + k / 4] |= (uint8_t)((unsigned)(v + 1) << (2 * (k % 4)));
        }
    }
    return 0;
}

int orc_unpack_canonical(const uint8_t* bytes, int64_t N, int64_t K, int8_t* q) {
    if (K % 4 != 0) return -1;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            unsigned code = (bytes[n * (K / 4) + k / 4] >> (2 * (k % 4))) & 3u;
            if (code == 3u) return -1;
            q[n * K + k] = (int8_t)((int)code - 1);
        }
    }
    return 0;
}

/* "Model details" / Quantization: activations to 8-bit integers by absmax,
 * one scale per token.  Range [-127, 127] so that the largest entry of every
 * token maps to exactly +-127. */
void orc_quant_act(const float* X, int64_t M, int64_t K,
                   int8_t* xq, float* gamma_x, int32_t* rowsum) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const float* x = X + m * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(x[k]);
            if (a > amax) amax = a;
        }
        float g = amax;
        if (!(g >= 1e-5f)) g = 1e-5f;
        float s = 127.0f / g;
        int32_t sum = 0;
        for (int64_t k = 0; k < K; ++k) {
            float r = rintf(x[k] * s);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            xq[m * K + k] = (int8_t)r;
            sum += (int32_t)r;
        }
        gamma_x[m] = g;
        if (rowsum) rowsum[m] = sum;
    }
}

/* "Model details": subln normalisation, no bias in normalisation layers;
 * "BitNetConfig": rms_norm_eps.  Root-mean-square normalisation with a gain. */
void orc_rmsnorm(const float* V, int64_t M, int64_t K, const float* gain,
                 float eps, float* Z) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const float* v = V + m * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) ss += (double)v[k] * (double)v[k];
        double ms = ss / (double)K;
        float r = (float)(1.0 / sqrt(ms + (double)eps));
        for (int64_t k = 0; k < K; ++k) {
            float t = v[k] * r;
            Z[m * K + k] = gain ? t * gain[k] : t;
        }
    }
}

/* W1.58A8 contraction: int8 activations times ternary weights, int32 sum. */
void orc_int_matmul(const int8_t* xq, int64_t M, int64_t K,
                    const int8_t* q, int64_t N, int32_t* acc) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int32_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int32_t)xq[m * K + k] * (int32_t)q[n * K + k];
            acc[m * N + n] = s;
        }
    }
}

/* Undo both scales: x ~ xq * gamma_x / 127 and w ~ q * gamma_w. */
void orc_dequant(const int32_t* acc, int64_t M, int64_t N,
                 const float* gamma_x, float gamma_w, float* Y) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float d = (gamma_x[m] * gamma_w) / 127.0f;
        for (int64_t n = 0; n < N; ++n) Y[m * N + n] = (float)acc[m * N + n] * d;
    }
}

/* "Model details": squared ReLU activation in the feed-forward layers. */
void orc_relu2(float* Y, int64_t count) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        float r = Y[i] > 0.0f ? Y[i] : 0.0f;
        Y[i] = r * r;
    }
}

void orc_add(float* H, const float* Y, int64_t count) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) H[i] = H[i] + Y[i];
}

void orc_ffn_layer(float* H, int64_t M, int64_t Hd, int64_t F,
                   const float* pre_gain, float pre_eps,
                   const int8_t* q_up, float gamma_up,
                   const float* sub_gain, float sub_eps,
                   const int8_t* q_down, float gamma_down,
                   int residual,
                   float* y1_out, int8_t* xq2_out, float* g2_out) {
    float* u = (float*)malloc(sizeof(float) * (size_t)(M * Hd));
    int8_t* xq1 = (int8_t*)malloc((size_t)(M * Hd));
    float* g1 = (float*)malloc(sizeof(float) * (size_t)M);
    int32_t* acc1 = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M * F));
    float* y1 = (float*)malloc(sizeof(float) * (size_t)(M * F));
    float* z = (float*)malloc(sizeof(float) * (size_t)(M * F));
    int8_t* xq2 = (int8_t*)malloc((size_t)(M * F));
    float* g2 = (float*)malloc(sizeof(float) * (size_t)M);
    int32_t* acc2 = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M * Hd));
    float* y2 = (float*)malloc(sizeof(float) * (size_t)(M * Hd));

    if (pre_gain) orc_rmsnorm(H, M, Hd, pre_gain, pre_eps, u);
    else memcpy(u, H, sizeof(float) * (size_t)(M * Hd));
    orc_quant_act(u, M, Hd, xq1, g1, NULL);
    orc_int_matmul(xq1, M, Hd, q_up, F, acc1);
    orc_dequant(acc1, M, F, g1, gamma_up, y1);
    orc_relu2(y1, M * F);
    orc_rmsnorm(y1, M, F, sub_gain, sub_eps, z);
    orc_quant_act(z, M, F, xq2, g2, NULL);
    orc_int_matmul(xq2, M, F, q_down, Hd, acc2);
    orc_dequant(acc2, M, Hd, g2, gamma_down, y2);
    if (residual) orc_add(H, y2, M * Hd);
    else memcpy(H, y2, sizeof(float) * (size_t)(M * Hd));

    if (y1_out) memcpy(y1_out, y1, sizeof(float) * (size_t)(M * F));
    if (xq2_out) memcpy(xq2_out, xq2, (size_t)(M * F));
    if (g2_out) memcpy(g2_out, g2, sizeof(float) * (size_t)M);

    free(u); free(xq1); free(g1); free(acc1); free(y1);
    free(z); free(xq2); free(g2); free(acc2); free(y2);
}

/* Gating product of the gated FFN: elementwise, binary32. */
void orc_mul(float* a, const float* b, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) a[i] = a[i] * b[i];
}

/* Gated FFN block ("Model details" / Architecture: squared ReLU in the
 * feed-forward layers; "BitNetConfig": hidden_act relu2).  The gate and up
 * projections read the same quantised input; ReLU^2 is applied to the gate
 * output and the result multiplies the up output, element by element. */
void orc_ffn_layer_gated(float* H, int64_t M, int64_t Hd, int64_t F,
                         const float* pre_gain, float pre_eps,
                         const int8_t* q_gate, float gamma_gate,
                         const int8_t* q_up, float gamma_up,
                         const float* sub_gain, float sub_eps,
                         const int8_t* q_down, float gamma_down,
                         int residual,
                         float* y1_out, int8_t* xq2_out, float* g2_out) {
    float* u = (float*)malloc(sizeof(float) * (size_t)(M * Hd));
    int8_t* xq1 = (int8_t*)malloc((size_t)(M * Hd));
    float* g1 = (float*)malloc(sizeof(float) * (size_t)M);
    int32_t* acc = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M * F));
    float* yg = (float*)malloc(sizeof(float) * (size_t)(M * F));
    float* yu = (float*)malloc(sizeof(float) * (size_t)(M * F));
    float* z = (float*)malloc(sizeof(float) * (size_t)(M * F));
    int8_t* xq2 = (int8_t*)malloc((size_t)(M * F));
    float* g2 = (float*)malloc(sizeof(float) * (size_t)M);
    int32_t* acc2 = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M * Hd));
    float* y2 = (float*)malloc(sizeof(float) * (size_t)(M * Hd));

    if (pre_gain) orc_rmsnorm(H, M, Hd, pre_gain, pre_eps, u);
    else memcpy(u, H, sizeof(float) * (size_t)(M * Hd));
    orc_quant_act(u, M, Hd, xq1, g1, NULL);
    orc_int_matmul(xq1, M, Hd, q_gate, F, acc);
    orc_dequant(acc, M, F, g1, gamma_gate, yg);
    orc_relu2(yg, M * F);
    orc_int_matmul(xq1, M, Hd, q_up, F, acc);
    orc_dequant(acc, M, F, g1, gamma_up, yu);
    orc_mul(yg, yu, M * F);                     /* h = ReLU^2(gate) * up */
    orc_rmsnorm(yg, M, F, sub_gain, sub_eps, z);
    orc_quant_act(z, M, F, xq2, g2, NULL);
    orc_int_matmul(xq2, M, F, q_down, Hd, acc2);
    orc_dequant(acc2, M, Hd, g2, gamma_down, y2);
    if (residual) orc_add(H, y2, M * Hd);
    else memcpy(H, y2, sizeof(float) * (size_t)(M * Hd));

    if (y1_out) memcpy(y1_out, yg, sizeof(float) * (size_t)(M * F));
    if (xq2_out) memcpy(xq2_out, xq2, (size_t)(M * F));
    if (g2_out) memcpy(g2_out, g2, sizeof(float) * (size_t)M);

    free(u); free(xq1); free(g1); free(acc); free(yg); free(yu);
    free(z); free(xq2); free(g2); free(acc2); free(y2);
}
