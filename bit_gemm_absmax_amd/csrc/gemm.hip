// Prefill contraction: int8 MFMA GEMM over unpacked ternary weights
// (transformers "BitNet" page, "Model details" / Quantization: W1.58A8; with
// thousands of tokens the product is a dense contraction).
//
// Tiling: a workgroup computes a BM x BN tile of acc with WM x WN waves, each
// owning a (BM/WM) x (BN/WN) sub-tile of 16x16 MFMA fragments
// (v_mfma_i32_16x16x64_i8).  Per k-step of 64:
//   - the int8 activation tile [BM][64] goes HBM -> LDS;
//   - the packed weight tile [BN][16 bytes] goes HBM -> LDS (4x smaller than
//     int8), and each wave expands its own 32-bit words into int8 codes in
//     registers: one shift + mask per 4 weights, producing 16 consecutive k
//     in order, which is exactly a 16-byte MFMA operand.
// The MFMA accumulates codes (q + 1); the epilogue subtracts the token's
// activation row sum, dequantises and applies the fused ReLU^2 / residual.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN* kWave) void k_gemm(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ rowsum, int M, int K, const uint4* __restrict__ Wp,
    const float* __restrict__ w_scale, int N, Epi epi, float* Y,
    int32_t* __restrict__ acc_out) {
    constexpr int NT = WM * WN * kWave;
    constexpr int TM = BM / WM;
    constexpr int TN = BN / WN;
    constexpr int FM = TM / 16;
    constexpr int FN = TN / 16;
    constexpr int APITCH = 80;  // bytes per LDS row of A: 64 + 16 to spread banks
    __shared__ __align__(16) int8_t sA[BM * APITCH];
    __shared__ __align__(16) uint32_t sB[BN * 4];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int wm = wave / WN;
    const int wn = wave % WN;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int C = K / 64;

    v4i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    for (int kc = 0; kc < C; ++kc) {
        for (int i = tid; i < BM * 4; i += NT) {
            const int row = i / 4, c16 = i % 4;
            const int m = m0 + row;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (m < M) v = *reinterpret_cast<const uint4*>(Xq + (int64_t)m * K + kc * 64 + c16 * 16);
            *reinterpret_cast<uint4*>(sA + row * APITCH + c16 * 16) = v;
        }
        for (int i = tid; i < BN; i += NT) {
            const int n = n0 + i;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (n < N) v = Wp[(int64_t)n * C + kc];
            *reinterpret_cast<uint4*>(sB + i * 4) = v;
        }
        __syncthreads();

        v4i a[FM];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int row = wm * TM + fm * 16 + (lane % 16);
            a[fm] = *reinterpret_cast<const v4i*>(sA + row * APITCH + 16 * (lane / 16));
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int col = wn * TN + fn * 16 + (lane % 16);
            const uint32_t w = sB[col * 4 + lane / 16];
            const v4i b = v4i{codes4(w, 0), codes4(w, 1), codes4(w, 2), codes4(w, 3)};
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                acc[fm][fn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[fm], b, acc[fm][fn], 0, 0, 0);
        }
        __syncthreads();
    }

    const float ws = *w_scale;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + wm * TM + fm * 16 + 4 * (lane / 16) + r;
            if (m >= M) continue;
            const int rsum = rowsum[m];
            const float d = (x_scale[m] * ws) / 127.0f;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int n = n0 + wn * TN + fn * 16 + (lane % 16);
                if (n >= N) continue;
                const int av = acc[fm][fn][r] - rsum;
                float y = (float)av * d;
                if (epi.flags & kEpiRelu2) {
                    const float t = y > 0.0f ? y : 0.0f;
                    y = t * t;
                }
                const int64_t o = (int64_t)m * N + n;
                if (epi.flags & kEpiResidual) y = y + epi.residual[o];
                if (Y != nullptr) Y[o] = y;
                if (acc_out != nullptr) acc_out[o] = av;
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                       const uint8_t* packed, const float* ws, int64_t N, Epi epi, float* Y,
                       int32_t* acc_out, hipStream_t s) {
    constexpr int BM = 128, BN = 128;
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    hipLaunchKernelGGL((k_gemm<BM, BN, 2, 2>), grid, dim3(256), 0, s, Xq, xs, rs, (int)M, (int)K,
                       reinterpret_cast<const uint4*>(packed), ws, (int)N, epi, Y, acc_out);
    return hipGetLastError();
}

hipError_t launch_contract(const int8_t* Xq, const float* x_scale, const int32_t* rowsum,
                           int64_t M, int64_t K, const uint8_t* packed, const float* w_scale,
                           int64_t N, Epi epi, float* Y, int32_t* acc_out, hipStream_t s) {
    if (gemv_supported(M, K))
        return launch_gemv(Xq, x_scale, rowsum, M, K, packed, w_scale, N, epi, Y, acc_out, s);
    return launch_gemm(Xq, x_scale, rowsum, M, K, packed, w_scale, N, epi, Y, acc_out, s);
}

}  // namespace bl
