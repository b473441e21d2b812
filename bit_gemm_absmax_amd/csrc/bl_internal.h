// Internal declarations shared by the HIP translation units of libbitlinear.
// Not part of the public ABI (include/bitlinear.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bitlinear.h"

namespace bl {

// Fused epilogue description handed to the contraction kernels by value.
// After the dequantisation: optional ReLU^2, then either y + aux (residual)
// or y * aux (the gating product); aux is [M][N] and may alias Y.
struct Epi {
    uint32_t flags;     // kEpi* bits (the subln requantisation is host-side)
    const float* aux;   // [M][N] residual or multiplier, or nullptr
};

constexpr uint32_t kEpiRelu2 = 0x1u;
constexpr uint32_t kEpiResidual = 0x2u;
constexpr uint32_t kEpiMul = 0x4u;

// ---- launchers (return hipError_t of the launch) ----------------------------

// Weight packing: partial binary64 sums of |W| into `partial` (count returned
// by pack_partial_blocks), then ternarise + pack.  W is fp32, or bf16 when
// `bf16` (widened exactly to fp32 before any arithmetic).
int pack_partial_blocks(int64_t count);
hipError_t launch_pack(const void* W, bool bf16, int64_t N, int64_t K, uint8_t* packed, float* w_scale,
                       double* partial, hipStream_t s);

// Between the plain row-major 2-bit form and the tile layout (to_tile: plain
// -> tile), and the tile layout -> int8 q [N][K].  K % 64 == 0.
hipError_t launch_relayout(const uint8_t* in, int64_t N, int64_t K, bool to_tile, uint8_t* out, hipStream_t s);
hipError_t launch_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* q, hipStream_t s);

// Per-row absmax quantisation with optional RMSNorm (gain may be null).
hipError_t launch_quant(const float* X, int64_t M, int64_t K, bool rmsnorm,
                        const float* gain, float eps, int8_t* Xq, float* scale,
                        int32_t* rowsum, hipStream_t s);
bool quant_supported(int64_t K);
// Workgroup size used to quantise a row of length K (256 up to 4096, 512 up
// to 16384, else 1024); every kernel that quantises rows uses this size, so
// all of them reduce in the same order.
int quant_threads(int64_t K);
// float4 per thread that cover a row of length K at quant_threads(K).
int quant_depth(int64_t K);

// rowsum[m] = sum_k Xq[m][k]
hipError_t launch_rowsum(const int8_t* Xq, int64_t M, int64_t K, int32_t* rowsum,
                         hipStream_t s);

// Skinny MFMA contraction for decode / batched decode, M <= 64.
bool gemv_supported(int64_t M, int64_t K, int64_t N);
hipError_t launch_gemv(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                       int64_t K, const uint8_t* packed, const float* ws, int64_t N, Epi epi,
                       float* Y, int32_t* acc_out, hipStream_t s);

// Several matrices of the same K on the same int8 rows in one skinny launch
// (at most gemv_max_groups()), each with its own scale, epilogue and outputs.
struct GroupMat {
    const uint8_t* packed;
    const float* w_scale;
    int64_t N;
    Epi epi;
    float* Y;
    int32_t* acc_out;
};
int gemv_max_groups();
hipError_t launch_gemv_grouped(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                               const GroupMat* groups, int count, hipStream_t s);
// The grouped contraction quantising its fp32 rows itself (bitlinear_quant_act
// then launch_gemv_grouped, in one launch, with the same results): few
// tokens, K whose quantiser runs 256 threads, many tiles.
bool gemv_grouped_quant_supported(int64_t M, int64_t K, const GroupMat* g, int count);
hipError_t launch_gemv_grouped_quant(const float* X, int64_t M, int64_t K, bool rmsnorm, const float* gain, float eps,
                                     const GroupMat* g, int count, hipStream_t s);

// The gated pair ReLU^2(BitLinear(x; gate)) * BitLinear(x; up) in one
// skinny launch (same shapes as launch_gemv).
hipError_t launch_gemv_gated(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                             const uint8_t* up, const float* up_scale, const uint8_t* gate, const float* gate_scale,
                             int64_t N, float* Y, hipStream_t s);

// Compute units of the current device (looked up once per device).
int cu_count();

// int8 MFMA GEMM for any M.
hipError_t launch_gemm(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                       int64_t K, const uint8_t* packed, const float* ws, int64_t N, Epi epi,
                       float* Y, int32_t* acc_out, hipStream_t s);

// Contraction + dequant epilogue, choosing the kernel from M.  rowsum must be valid (not null).
hipError_t launch_contract(const int8_t* Xq, const float* x_scale,
                           const int32_t* rowsum, int64_t M, int64_t K,
                           const uint8_t* packed, const float* w_scale, int64_t N,
                           Epi epi, float* Y, int32_t* acc_out, hipStream_t s);

// Few-token BitLinear from fp32 rows: every workgroup quantises the rows
// itself (optional RMSNorm with gain), then contracts its slice of output
// rows; epilogue ReLU^2, then residual add or gating product (Y may alias aux).
bool decode_supported(int64_t M, int64_t K, int64_t N);
hipError_t launch_decode_bitlinear(const float* X, int64_t M, int64_t K, bool rmsnorm, const float* gain,
                                   float eps, const uint8_t* packed, const float* w_scale, int64_t N,
                                   uint32_t epi, const float* aux, float* Y, hipStream_t s);
// The same for a gated pair: Y = ReLU^2(BitLinear(x; gate)) * BitLinear(x; up),
// both from one in-workgroup quantisation of the rows.
hipError_t launch_decode_gated(const float* X, int64_t M, int64_t K, bool rmsnorm, const float* gain, float eps,
                               const uint8_t* up, const float* up_scale, const uint8_t* gate,
                               const float* gate_scale, int64_t N, float* Y, hipStream_t s);

// The FFN stack for one token in one persistent launch (all layers), for
// hidden H and intermediate F it supports (stack_supported) and up to
// stack_max_layers() layers per launch; ws: stack_ws_bytes() of scratch (layer
// descriptors, arrival counter), y1: F floats.  The layers must be ungated.
bool stack_supported(int64_t H, int64_t F);
size_t stack_ws_bytes();
int stack_max_layers();
hipError_t launch_stack(const bitnet_ffn_layer* layers, int n_layers, float* hidden, int64_t H, int64_t F,
                        bool pre, bool residual, float eps, float* y1, void* ws, hipStream_t s);

}  // namespace bl
