/*
 * bitlinear.h -- C ABI of the MI355X (gfx950) BitLinear W1.58A8 library.
 *
 * The layer is the one described on the transformers "BitNet" documentation
 * page, section "Model details":
 *   - Quantization: 1.58-bit weights and 8-bit activations (W1.58A8); weights
 *     are made ternary {-1, 0, +1} by absmean quantisation, activations become
 *     8-bit integers by per-token absmax quantisation.
 *   - Architecture: BitLinear layers, squared ReLU (ReLU^2) in the feed-forward
 *     layers, subln normalisation, no bias in linear or normalisation layers.
 * Section "BitNetConfig" gives rms_norm_eps = 1e-05 and the model shapes
 * (hidden 2560, intermediate 6912, 30 layers); section "Model variants" names
 * packed 1.58-bit weights for deployment without giving a layout.
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers.  Every array argument is a DEVICE pointer (hipMalloc'd or from a
 * framework allocator) unless marked "host".  The caller owns all memory; no
 * call allocates device memory.  Scratch comes from a caller-supplied
 * workspace whose size the matching *_workspace_bytes() query returns.
 *
 * Layouts.  No padding; all row-major except the packed weights:
 *   W       fp32 [N][K]     latent weights, out x in (y = x . W^T)
 *   packed  u8   N*K/4      2-bit codes c = q + 1 (code 3 never occurs),
 *                           stored as [N][K/4] bytes but grouped by tiles
 *                           of 16 rows, not by row.  A row's weights come in
 *                           16-byte chunks of 64: chunk c holds weights
 *                           64c .. 64c+63, weight 64c + 16d + 4j + b (d, j,
 *                           b in 0..3) in byte 4d + b at bits 2j..2j+1, so
 *                           the chunk's little-endian 32-bit word d holds 16
 *                           consecutive weights.  Tile t holds rows 16t ..
 *                           16t+R-1 (R = 16, or N - 16t for the last tile)
 *                           and starts at byte 16t * K/4; inside it, chunk c
 *                           of tile row r is at byte 16 (c R + r).  A
 *                           matrix whose N is a multiple of 16 is therefore
 *                           the concatenation of its tiles' layouts.
 *   X       fp32 [M][K]     activations, one row per token
 *   Xq      int8 [M][K]     quantised activations, in [-127, 127]
 *   Y       fp32 [M][N]     outputs
 *
 * Scales.  w_scale is one fp32 per weight tensor (the absmean, gamma_w);
 * x_scale is one fp32 per token (the absmax, gamma_x).  Both are floored at
 * 1e-5.  Dequantisation is y = acc * ((gamma_x * gamma_w) / 127).
 *
 * Shapes.  K must be a positive multiple of 64; N >= 1; M >= 0 (M == 0 is an
 * empty batch: validated, then nothing is launched).  Limits: M*K, M*N and
 * N*K below 2^31.
 *
 * Alignment.  W, X, Xq, packed, Y, acc and residual need 16-byte alignment;
 * scale, rowsum and gain arrays need 4-byte alignment; the workspace needs
 * 256-byte alignment.
 *
 * Streams.  Every call enqueues its kernels on the caller's stream and
 * returns without synchronising.  Results are deterministic: the same inputs
 * give bit-identical outputs on every run (no floating-point atomics).
 *
 * Errors.  Calls return BL_OK (0) or a negative bl_status.  Arguments are
 * validated before anything is launched, so a rejected call has no effect.
 * bitlinear_last_error() returns a thread-local message describing the last
 * failure on the calling thread.  Non-finite inputs are outside the contract
 * and are not checked.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum bl_status {
    BL_OK = 0,
    BL_ERR_NULL = -1,        /* a required pointer is NULL */
    BL_ERR_SHAPE = -2,       /* bad M, N or K (see Shapes) */
    BL_ERR_ALIGN = -3,       /* a pointer is not aligned as required */
    BL_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
    BL_ERR_HIP = -5,         /* HIP runtime reported an error (launch, device) */
    BL_ERR_UNSUPPORTED = -6  /* valid request the library does not implement */
};

/* Static description of a status code (never NULL). */
const char* bitlinear_status_string(int status);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* bitlinear_last_error(void);

/* ABI version of this header, (major << 16) | minor. */
int bitlinear_abi_version(void);
#define BITLINEAR_ABI_VERSION ((1 << 16) | 4)

/* ------------------------------------------------------------------------
 * Weight packing ("Model details" / Quantization: absmean ternary weights).
 *
 *   gamma_w   = max(mean_{n,k} |W[n][k]|, 1e-5)   one scale for the tensor;
 *               the sum runs in binary64 and is rounded once to binary32
 *   q[n][k]   = clamp(rint(W[n][k] / gamma_w), -1, 1)   (ties to even)
 *   packed    = 2-bit codes q + 1 in the layout above
 *
 * W        in   fp32 [N][K]
 * packed   out  u8 [N][K/4]
 * w_scale  out  fp32 [1], gamma_w
 * ws       scratch of bitlinear_pack_workspace_bytes(N, K) bytes
 * Offline step: run once per weight tensor.
 * ---------------------------------------------------------------------- */
size_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K);
int bitlinear_pack_weights(const float* W, int64_t N, int64_t K,
                           uint8_t* packed, float* w_scale,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Packed-layout conversion ("Model variants": packed 1.58-bit weights for
 * deployment; the page gives no byte layout).
 *
 * The plain ("canonical") 2-bit form is row-major [N][K/4] bytes with the
 * code q + 1 of weight k of row n in byte n*(K/4) + k/4 at bits 2*(k%4),
 * four consecutive weights per byte, lowest bits first.  It holds the same
 * numbers as the tile layout above, which is what every other call reads.
 *
 * bitlinear_import_canonical: canonical u8 [N][K/4] (4-byte aligned) ->
 *                             packed u8 [N][K/4] in the tile layout.
 * bitlinear_export_canonical: the inverse (packed 16-byte aligned, canonical
 *                             4-byte aligned).
 * bitlinear_unpack_weights:   packed -> q int8 [N][K] in {-1, 0, 1}
 *                             (16-byte aligned).
 * Both directions are exact and lossless.  Inputs must hold codes 0..2 only;
 * a code 3 is outside the contract (it is carried through, and unpacks to 2).
 * K must be a positive multiple of 64; input and output must not overlap.
 * The weight scale gamma_w is unaffected: keep it beside either form.
 * ---------------------------------------------------------------------- */
int bitlinear_import_canonical(const uint8_t* canonical, int64_t N, int64_t K,
                               uint8_t* packed, hipStream_t stream);
int bitlinear_export_canonical(const uint8_t* packed, int64_t N, int64_t K,
                               uint8_t* canonical, hipStream_t stream);
int bitlinear_unpack_weights(const uint8_t* packed, int64_t N, int64_t K,
                             int8_t* q, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Activation quantisation ("Model details" / Quantization: per-token absmax
 * 8-bit activations), optionally preceded by RMSNorm with a gain and no bias
 * ("Model details" / Architecture; eps from "BitNetConfig").
 *
 * With BL_QUANT_RMSNORM in flags, each row is first normalised:
 *   r = (float)(1 / sqrt(sum_k (double)x^2 / K + (double)norm_eps))
 *   z = (x * r) * gain[k]           (gain NULL means all ones)
 * and then, for each row (z = x without the flag):
 *   gamma_x = max(max_k |z|, 1e-5);  s = 127 / gamma_x
 *   Xq[k]   = clamp(rint(z[k] * s), -127, 127)      (ties to even)
 *   rowsum  = sum_k Xq[k]
 *
 * X         in   fp32 [M][K]
 * norm_gain in   fp32 [K] or NULL (ignored without BL_QUANT_RMSNORM)
 * Xq        out  int8 [M][K]
 * x_scale   out  fp32 [M], gamma_x
 * x_rowsum  out  int32 [M], may be NULL
 * No output may overlap X, the gain or another output (BL_ERR_UNSUPPORTED).
 * ---------------------------------------------------------------------- */
#define BL_QUANT_RMSNORM 0x1u
int bitlinear_quant_act(const float* X, int64_t M, int64_t K, uint32_t flags,
                        const float* norm_gain, float norm_eps,
                        int8_t* Xq, float* x_scale, int32_t* x_rowsum,
                        hipStream_t stream);

/* ------------------------------------------------------------------------
 * BitLinear forward: the W1.58A8 contraction with int32 accumulation and the
 * dequantising epilogue ("Model details" / Quantization), with optional fused
 * squared ReLU, residual add and subln requantisation ("Model details" /
 * Architecture).
 *
 *   acc[m][n] = sum_k Xq[m][k] * q[n][k]                  (exact int32)
 *   y[m][n]   = (float)acc[m][n] * ((x_scale[m] * w_scale) / 127)
 *   BL_EPI_RELU2:       y = max(y, 0)^2
 *   BL_EPI_RESIDUAL:    y = y + residual[m][n]
 *   BL_EPI_MUL:         y = y * mul_by[m][n]   (after ReLU^2; the gating
 *                       product ReLU^2(gate) * up of a gated feed-forward
 *                       block; not together with BL_EPI_RESIDUAL)
 *   BL_EPI_SUBLN_QUANT: out_q, out_q_scale, out_q_rowsum = the
 *                       bitlinear_quant_act of y with BL_QUANT_RMSNORM,
 *                       gain norm_gain (NULL = ones), eps norm_eps.
 *
 * Xq         in  int8 [M][K]
 * x_scale    in  fp32 [M]
 * x_rowsum   in  int32 [M] = sum_k Xq[m][k], or NULL (then computed inside)
 * packed     in  u8 [N][K/4], from bitlinear_pack_weights
 * w_scale    in  fp32 [1]
 * epi        in  host pointer to a bl_epilogue, or NULL for plain dequant
 * Y          out fp32 [M][N]; may be NULL only with BL_EPI_SUBLN_QUANT.
 *                With BL_EPI_RESIDUAL (BL_EPI_MUL), Y may equal residual
 *                (mul_by), in place; any other overlap between an output and
 *                an input or another output is rejected (BL_ERR_UNSUPPORTED).
 * acc_out    out int32 [M][N], the exact accumulators, or NULL
 * ws         scratch of bitlinear_forward_workspace_bytes(M, K, N, flags)
 * ---------------------------------------------------------------------- */
#define BL_EPI_RELU2       0x1u
#define BL_EPI_RESIDUAL    0x2u
#define BL_EPI_SUBLN_QUANT 0x4u
#define BL_EPI_MUL         0x8u

typedef struct bl_epilogue {
    uint32_t flags;          /* BL_EPI_* bits */
    const float* residual;   /* [M][N] for BL_EPI_RESIDUAL */
    const float* norm_gain;  /* [N] or NULL (ones) for BL_EPI_SUBLN_QUANT */
    float norm_eps;          /* RMSNorm eps for BL_EPI_SUBLN_QUANT (1e-5) */
    int8_t* out_q;           /* [M][N] requantised output */
    float* out_q_scale;      /* [M] its absmax scales */
    int32_t* out_q_rowsum;   /* [M] its row sums, or NULL */
    const float* mul_by;     /* [M][N] for BL_EPI_MUL */
} bl_epilogue;

size_t bitlinear_forward_workspace_bytes(int64_t M, int64_t K, int64_t N,
                                         uint32_t epi_flags);
int bitlinear_forward(const int8_t* Xq, const float* x_scale,
                      const int32_t* x_rowsum, int64_t M, int64_t K,
                      const uint8_t* packed, const float* w_scale, int64_t N,
                      const bl_epilogue* epi, float* Y, int32_t* acc_out,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Grouped BitLinear: up to BL_MAX_GROUPS weight matrices of the same K on the
 * same quantised rows, each with its own weight scale, epilogue and outputs
 * ("Model details" / Architecture: the BitLinear layers of a block that read
 * one input, e.g. the attention block's q, k and v projections, whose
 * absmean scales are per tensor; "BitNetConfig": 20 heads, 5 key/value
 * heads).  Results are identical to one bitlinear_forward per matrix; for
 * M <= 64, K <= 8192 and M * N < 2^29 for every matrix the contractions of
 * all matrices stream in one launch.
 *
 * Xq, x_scale, M, K   as in bitlinear_forward
 * x_rowsum   in  int32 [M], required here
 * groups     in  host array of n_groups (1..BL_MAX_GROUPS) bl_group:
 *   packed, w_scale, N   one matrix, as in bitlinear_forward
 *   epi                  its epilogue, as bitlinear_forward's (with
 *                        BL_EPI_SUBLN_QUANT the requantisation of its Y runs
 *                        after the contraction)
 *   Y                    out fp32 [M][N], required
 *   acc_out              out int32 [M][N] or NULL
 * Overlap rules of bitlinear_forward for each matrix, and no output of one
 * matrix may overlap another matrix's inputs or outputs.  No workspace.
 * ---------------------------------------------------------------------- */
#define BL_MAX_GROUPS 4

typedef struct bl_group {
    const uint8_t* packed;   /* [N][K/4] */
    const float* w_scale;    /* [1] */
    int64_t N;
    bl_epilogue epi;         /* flags 0 for plain dequantisation */
    float* Y;                /* [M][N] */
    int32_t* acc_out;        /* [M][N] or NULL */
} bl_group;

int bitlinear_forward_grouped(const int8_t* Xq, const float* x_scale,
                              const int32_t* x_rowsum, int64_t M, int64_t K,
                              const bl_group* groups, int32_t n_groups,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * Fused quantise + BitLinear: bitlinear_quant_act followed by
 * bitlinear_forward, from fp32 activation rows, with the same results as the
 * two calls.  For a few tokens (M <= 4) it is one launch in which every
 * workgroup quantises the rows itself; otherwise the two steps run in turn
 * through the workspace.
 *
 * X           in  fp32 [M][K]
 * quant_flags     BL_QUANT_RMSNORM or 0; norm_gain / norm_eps as in
 *                 bitlinear_quant_act
 * packed, w_scale, N  as in bitlinear_forward
 * epi         in  host pointer or NULL; BL_EPI_RELU2, BL_EPI_RESIDUAL and
 *                 BL_EPI_MUL are accepted here (BL_ERR_UNSUPPORTED otherwise)
 * Y           out fp32 [M][N]; may equal epi->residual or epi->mul_by
 *                 (in place).  Y must not overlap X or norm_gain, nor
 *                 residual / mul_by other than by being equal to it
 *                 (BL_ERR_UNSUPPORTED): for a few tokens every workgroup
 *                 reads all of X while others write Y.
 * ws          scratch of bitlinear_quant_forward_workspace_bytes(M, K, N)
 * ---------------------------------------------------------------------- */
size_t bitlinear_quant_forward_workspace_bytes(int64_t M, int64_t K, int64_t N);
int bitlinear_quant_forward(const float* X, int64_t M, int64_t K, uint32_t quant_flags,
                            const float* norm_gain, float norm_eps,
                            const uint8_t* packed, const float* w_scale, int64_t N,
                            const bl_epilogue* epi, float* Y,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Grouped fused quantise + BitLinear: bitlinear_quant_act followed by
 * bitlinear_forward_grouped on the quantised rows, with the same results
 * bit for bit.  For a few tokens (M <= 8) against many 16-row tiles in all
 * (at least 512, K <= 2560, M * N < 2^29 for every matrix) it is one
 * contraction launch in which every
 * workgroup quantises the rows itself, exactly as the standalone quantiser
 * would; otherwise the rows are quantised into the workspace first.
 *
 * X           in  fp32 [M][K]; quant_flags / norm_gain / norm_eps as in
 *                 bitlinear_quant_act
 * groups      as in bitlinear_forward_grouped; no output may overlap X, the
 *                 gain or the workspace
 * ws          scratch of bitlinear_quant_forward_grouped_workspace_bytes(M, K)
 *             (the quantised rows; its contents afterwards are unspecified)
 * Errors as bitlinear_quant_act and bitlinear_forward_grouped.
 * ---------------------------------------------------------------------- */
size_t bitlinear_quant_forward_grouped_workspace_bytes(int64_t M, int64_t K);
int bitlinear_quant_forward_grouped(const float* X, int64_t M, int64_t K, uint32_t quant_flags,
                                    const float* norm_gain, float norm_eps,
                                    const bl_group* groups, int32_t n_groups,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * BitLinear from latent weights, the forward pass of quantisation-aware
 * training ("Model details" / Quantization: the weights are quantised to
 * ternary by absmean and the activations per token by absmax inside the
 * forward pass; the latent weights stay in high precision):
 *
 *   gamma_w, q = absmean-ternarise(W)          exactly as bitlinear_pack_weights
 *   Y          = BitLinear(X; q, gamma_w)      exactly as bitlinear_quant_forward
 *
 * Y is the dequantised ("fake-quant") product: in real arithmetic
 * Y[m][n] = sum_k (xq[m][k] * gamma_x[m] / 127) * (q[n][k] * gamma_w) (+ epilogue);
 * the integer sum is exact and rounding enters only in the scaling.
 *
 * X           in  fp32 [M][K]; quant_flags / norm_gain / norm_eps as in
 *                 bitlinear_quant_act
 * W           in  latent weights [N][K], fp32 (w_dtype BL_DTYPE_F32) or bf16
 *                 (BL_DTYPE_BF16, widened exactly to fp32); 16-byte aligned
 * epi         in  host pointer or NULL; BL_EPI_RELU2, BL_EPI_RESIDUAL and
 *                 BL_EPI_MUL as in bitlinear_quant_forward
 * Y           out fp32 [M][N] (overlap rules of bitlinear_quant_forward)
 * w_scale     out fp32 [1], gamma_w, or NULL (kept in the workspace)
 * ws          scratch of bitlinear_latent_forward_workspace_bytes(M, K, N):
 *             the packed weights (N*K/4 bytes) and the quantised rows
 * BL_ERR_UNSUPPORTED for another w_dtype; other errors as bitlinear_quant_forward.
 * ---------------------------------------------------------------------- */
#define BL_DTYPE_F32 0u
#define BL_DTYPE_BF16 1u

size_t bitlinear_latent_forward_workspace_bytes(int64_t M, int64_t K, int64_t N);
int bitlinear_latent_forward(const float* X, int64_t M, int64_t K, uint32_t quant_flags,
                             const float* norm_gain, float norm_eps,
                             const void* W, uint32_t w_dtype, int64_t N,
                             const bl_epilogue* epi, float* Y, float* w_scale,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * BitNet feed-forward stack: for each layer in order, on hidden [M][H]
 * ("Model details" / Architecture: BitLinear FFN with ReLU^2 and subln, no
 * bias; "BitNetConfig": hidden 2560, intermediate 6912, 30 layers):
 *
 *   u  = BL_FFN_PRE_NORM ? RMSNorm(hidden; pre_norm_gain) : hidden
 *   xq = absmax-quant(u)
 *   y1 = ReLU^2(BitLinear(xq; up))                          [M][F]
 *        or, for a gated layer (gate != NULL),
 *   y1 = ReLU^2(BitLinear(xq; gate)) * BitLinear(xq; up)    [M][F]
 *   x2 = absmax-quant(RMSNorm(y1; sub_norm_gain))           subln
 *   y2 = BitLinear(x2; down)                                [M][H]
 *   hidden = BL_FFN_RESIDUAL ? hidden + y2 : y2
 *
 * layers     in  host array of n_layers descriptors holding device pointers
 * hidden     in/out fp32 [M][H]
 * norm_eps   eps of both RMSNorms (1e-5)
 * ws         scratch of bitnet_ffn_workspace_bytes(M, H, F); calls that
 *            share one workspace must not overlap in time, and hidden must
 *            not lie in the workspace (BL_ERR_UNSUPPORTED).
 * A gate matrix needs its scale (gate_scale) and has the up matrix's shape.
 * ---------------------------------------------------------------------- */
#define BL_FFN_PRE_NORM 0x1u
#define BL_FFN_RESIDUAL 0x2u
/* BL_FFN_PERSISTENT: one token (M == 1), ungated layers: all layers run in
 * one persistent launch (one workgroup per CU; the phases of a layer hand
 * their rows to each other through device memory, each value carrying its
 * own ready flag, instead of through kernel boundaries, and each phase's
 * weight loads are issued while the previous row is still in flight).
 * Results are bit-identical to the call without the flag.
 * BL_ERR_UNSUPPORTED for M > 1, a gated layer, or a shape without a
 * persistent plan (hidden 2560 / intermediate 6912 has one).  The launch
 * needs every one of its workgroups resident at once: do not run it beside
 * work that holds CUs for as long as it waits (each wait gives up after about
 * a second; the outputs are then not valid). */
#define BL_FFN_PERSISTENT 0x4u

typedef struct bitnet_ffn_layer {
    const float* pre_norm_gain;  /* [H] or NULL (ones) */
    const uint8_t* up;           /* [F][H/4] packed */
    const float* up_scale;       /* [1] */
    const uint8_t* gate;         /* [F][H/4] packed, or NULL (ungated) */
    const float* gate_scale;     /* [1], with gate */
    const float* sub_norm_gain;  /* [F] or NULL (ones) */
    const uint8_t* down;         /* [H][F/4] packed */
    const float* down_scale;     /* [1] */
} bitnet_ffn_layer;

size_t bitnet_ffn_workspace_bytes(int64_t M, int64_t H, int64_t F);
int bitnet_ffn_forward(const bitnet_ffn_layer* layers, int32_t n_layers,
                       float* hidden, int64_t M, int64_t H, int64_t F,
                       uint32_t flags, float norm_eps,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * bitnet_ffn_forward without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and errors as
 * bitnet_ffn_forward, but its scratch is a fixed array inside the library,
 * BITNET_FFN_NOALLOC_MAX_BYTES (64 MiB) on every GPU it runs on (held until
 * the process ends); calls whose bitnet_ffn_workspace_bytes(M, H, F) exceeds
 * it return BL_ERR_WORKSPACE (at H = 2560, F = 6912: M up to 1806 tokens).
 * Allocates nothing: the first call on a device looks the array up
 * (hipGetSymbolAddress), so make one call on each device before capturing a
 * graph.  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (other streams, other threads) race and give wrong
 * results; calls in order on one stream are safe.
 * ---------------------------------------------------------------------- */
#define BITNET_FFN_NOALLOC_MAX_BYTES ((size_t)64 << 20)
int bitnet_ffn_forward_noalloc(const bitnet_ffn_layer* layers, int32_t n_layers,
                               float* hidden, int64_t M, int64_t H, int64_t F,
                               uint32_t flags, float norm_eps, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* BITLINEAR_H */
