/*
 * Scalar CPU oracle for the BitNet b1.58 BitLinear layer (W1.58A8).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the
 * package entry module and the CPU-baseline leg of the benchmark may load
 * this code.  The product (the HIP library and its Python binding) never
 * calls it and shares no code, header, table or constant with it.
 *
 * Source of the method: the Hugging Face transformers documentation page
 * "BitNet", section "Model details":
 *   - Architecture: BitLinear layers replace the linear layers; squared ReLU
 *     in the feed-forward layers; subln normalisation; no bias terms in the
 *     linear or normalisation layers.
 *   - Quantization: 1.58-bit weights and 8-bit activations (W1.58A8); the
 *     weights are mapped to ternary {-1, 0, +1} with absmean quantisation,
 *     the activations to 8-bit integers with per-token absmax quantisation.
 * Section "BitNetConfig" supplies rms_norm_eps = 1e-05, hidden_size 2560,
 * intermediate_size 6912, num_hidden_layers 30, hidden_act "relu2".
 *
 * Arithmetic: IEEE binary32 with round-to-nearest-even, no FMA contraction;
 * accumulations the page leaves open are done in binary64 (see each
 * function).  Every function is a plain loop nest: no blocking, no fusion.
 *
 * Packed weight format (the page names "packed 1.58-bit weights" in section
 * "Model variants" but gives no layout; this is the reading used here):
 *   code = q + 1 in {0, 1, 2}, two bits per weight, N*K/4 bytes, no padding.
 *   A row's weights come in chunks of 64 (16 bytes); chunk c holds weights
 *   64c .. 64c+63, and weight 64c + 16d + 4j + b (d, j, b in 0..3) sits in
 *   byte 4d + b of the chunk at bits 2j..2j+1 (so the chunk's 32-bit word d
 *   holds 16 consecutive weights).  Rows are grouped in tiles of 16: tile t
 *   holds rows 16t .. 16t+R-1 (R = 16, or N - 16t for the last tile) and
 *   starts at byte 16t * K/4; inside it, chunk c of tile row r is at byte
 *   16 (c R + r).  K must be a multiple of 64.
 */
#ifndef BITNET_ORACLE_H
#define BITNET_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* absmean weight scale: mean of |W| over the whole [N][K] tensor, summed in
 * binary64 (row by row, k ascending, rows in order), rounded once to binary32,
 * floored at 1e-5. */
float orc_absmean_scale(const float* W, int64_t N, int64_t K);

/* q[n][k] = clamp(rint(W[n][k] / gamma), -1, +1), one binary32 divide. */
void orc_ternarize(const float* W, int64_t N, int64_t K, float gamma, int8_t* q);

/* 2-bit encoding of ternary q (layout above).  Returns 0, or -1 when K is not
 * a multiple of 64 or a value lies outside {-1, 0, 1}. */
int orc_pack(const int8_t* q, int64_t N, int64_t K, uint8_t* packed);

/* Inverse of orc_pack.  Returns 0, or -1 on a bad K or on code 3. */
int orc_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* q);

/* Plain row-major 2-bit form: code q + 1 of weight k of row n in byte
 * n*(K/4) + k/4 at bits 2*(k%4) (four consecutive weights per byte, the
 * lowest first).  K must be a multiple of 4.  Returns 0, or -1 on a bad K,
 * a non-ternary value (pack) or code 3 (unpack). */
int orc_pack_canonical(const int8_t* q, int64_t N, int64_t K, uint8_t* bytes);
int orc_unpack_canonical(const uint8_t* bytes, int64_t N, int64_t K, int8_t* q);

/* Threads of the OpenMP build (liboracle_mt.so): sets the count when n > 0
 * and returns the count in force; the one-core build returns 1. */
int orc_set_threads(int n);

/* Per-token absmax quantisation of X[M][K]:
 *   gamma_x[m] = max(max_k |X[m][k]|, 1e-5)
 *   s          = 127 / gamma_x[m]                (binary32 divide)
 *   xq[m][k]   = clamp(rint(X[m][k] * s), -127, 127)
 *   rowsum[m]  = sum_k xq[m][k]                  (rowsum may be NULL) */
void orc_quant_act(const float* X, int64_t M, int64_t K,
                   int8_t* xq, float* gamma_x, int32_t* rowsum);

/* RMSNorm with gain and no bias, per row of V[M][K]:
 *   ms = sum_k (double)v^2 / K ;  r = (float)(1 / sqrt(ms + (double)eps))
 *   Z[m][k] = (V[m][k] * r) * gain[k]   (gain NULL means all ones) */
void orc_rmsnorm(const float* V, int64_t M, int64_t K, const float* gain,
                 float eps, float* Z);

/* Exact integer contraction acc[m][n] = sum_k xq[m][k] * q[n][k]. */
void orc_int_matmul(const int8_t* xq, int64_t M, int64_t K,
                    const int8_t* q, int64_t N, int32_t* acc);

/* Dequantisation: d_m = (gamma_x[m] * gamma_w) / 127 ; Y[m][n] = acc * d_m. */
void orc_dequant(const int32_t* acc, int64_t M, int64_t N,
                 const float* gamma_x, float gamma_w, float* Y);

/* Squared ReLU in place: y <- (y > 0 ? y : 0)^2. */
void orc_relu2(float* Y, int64_t count);

/* Residual add in place: H <- H + Y. */
void orc_add(float* H, const float* Y, int64_t count);

/* One BitNet feed-forward block over hidden rows H[M][Hd] (in/out):
 *   u   = pre_gain ? RMSNorm(H; pre_gain) : H
 *   xq1 = absmax-quant(u);  y1 = dequant(xq1 . q_up^T);  y1 = relu2(y1)
 *   z   = RMSNorm(y1; sub_gain)
 *   xq2 = absmax-quant(z);  y2 = dequant(xq2 . q_down^T)
 *   H   = residual ? H + y2 : y2
 * q_up is ternary [F][Hd], q_down is ternary [Hd][F].  The weight scales are
 * the absmean gammas.  Optional intermediate outputs may be NULL:
 *   y1_out [M][F] (after relu2), xq2_out [M][F], g2_out [M]. */
void orc_ffn_layer(float* H, int64_t M, int64_t Hd, int64_t F,
                   const float* pre_gain, float pre_eps,
                   const int8_t* q_up, float gamma_up,
                   const float* sub_gain, float sub_eps,
                   const int8_t* q_down, float gamma_down,
                   int residual,
                   float* y1_out, int8_t* xq2_out, float* g2_out);

/* a[i] = a[i] * b[i] in binary32 (the gating product). */
void orc_mul(float* a, const float* b, int64_t n);

/* Gated BitNet FFN block: as orc_ffn_layer, but the up projection's output
 * is multiplied elementwise by ReLU^2 of a gate projection of the same
 * quantised input,
 *   y_gate = dequant(xq1 . q_gate^T), y_up = dequant(xq1 . q_up^T)
 *   h = ReLU^2(y_gate) * y_up            (binary32, one rounding each)
 * then subln RMSNorm of h, quantisation and the down projection as in the
 * ungated block.  q_gate is ternary [F][Hd].  y1_out, if not NULL, receives h. */
void orc_ffn_layer_gated(float* H, int64_t M, int64_t Hd, int64_t F,
                         const float* pre_gain, float pre_eps,
                         const int8_t* q_gate, float gamma_gate,
                         const int8_t* q_up, float gamma_up,
                         const float* sub_gain, float sub_eps,
                         const int8_t* q_down, float gamma_down,
                         int residual,
                         float* y1_out, int8_t* xq2_out, float* g2_out);

#ifdef __cplusplus
}
#endif
#endif
