// Decode contraction for a few tokens (M <= 4): a bandwidth-bound GEMV over
// the packed ternary weights (transformers "BitNet" page, "Model details" /
// Quantization: W1.58A8, int8 activations times ternary weights).
//
// Layout of the work: each row of packed weights is K/64 chunks of 16 bytes
// (64 weights).  G lanes share a row; lane g of the group takes chunks
// g, g + G, ...  Every lane first issues all of its 16-byte weight loads
// (coalesced: the G lanes of a row read G consecutive chunks), then the
// workgroup stages the int8 activation rows in LDS while those loads are in
// flight, then each 32-bit weight word is expanded with one shift and one
// mask per 4 weights into int8 codes 0..2 and fed to v_dot4 against four
// activations.  The code offset is removed once per output:
//   sum_k (q+1) * x  -  sum_k x  =  sum_k q * x.
// The G partial sums meet in an xor-butterfly inside the wave; integer sums
// are exact, so the result does not depend on that order.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kGemvThreads = 256;

template <int MT, int NCH>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ rowsum, int K, const uint4* __restrict__ Wp,
    const float* __restrict__ w_scale, int N, int G, Epi epi, float* Y,
    int32_t* __restrict__ acc_out) {
    extern __shared__ uint4 sx[];  // MT rows of K int8
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int rows_per_wave = kWave / G;
    const int n = (blockIdx.x * (kGemvThreads / kWave) + wave) * rows_per_wave + lane / G;
    const int gl = lane % G;
    const int C = K / 64;

    uint4 w[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = gl + i * G;
        w[i] = (n < N && c < C) ? Wp[(int64_t)n * C + c] : make_uint4(0u, 0u, 0u, 0u);
    }

    const uint4* xg = reinterpret_cast<const uint4*>(Xq);
    for (int i = threadIdx.x; i < MT * K / 16; i += kGemvThreads) sx[i] = xg[i];
    __syncthreads();

    int acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0;

#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int c = gl + i * G;
        if (c < C) {
            const uint32_t wd[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int c0 = codes4(wd[d], 0);
                const int c1 = codes4(wd[d], 1);
                const int c2 = codes4(wd[d], 2);
                const int c3 = codes4(wd[d], 3);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const uint4 xv = sx[(m * K + 64 * c + 16 * d) / 16];
                    int a = acc[m];
                    a = __builtin_amdgcn_sdot4(c0, (int)xv.x, a, false);
                    a = __builtin_amdgcn_sdot4(c1, (int)xv.y, a, false);
                    a = __builtin_amdgcn_sdot4(c2, (int)xv.z, a, false);
                    a = __builtin_amdgcn_sdot4(c3, (int)xv.w, a, false);
                    acc[m] = a;
                }
            }
        }
    }

    for (int mask = G / 2; mask >= 1; mask >>= 1) {
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] += __shfl_xor(acc[m], mask, kWave);
    }

    if (n >= N) return;
    const float ws = *w_scale;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if (gl == (m % G)) {
            const int a = acc[m] - rowsum[m];
            const float d = (x_scale[m] * ws) / 127.0f;
            float y = (float)a * d;
            if (epi.flags & kEpiRelu2) {
                const float r = y > 0.0f ? y : 0.0f;
                y = r * r;
            }
            const int64_t o = (int64_t)m * N + n;
            if (epi.flags & kEpiResidual) y = y + epi.residual[o];
            if (Y != nullptr) Y[o] = y;
            if (acc_out != nullptr) acc_out[o] = a;
        }
    }
}

template <int MT>
hipError_t launch_mt(int nch, const int8_t* Xq, const float* xs, const int32_t* rs, int64_t K,
                     const uint8_t* packed, const float* ws, int64_t N, int G, Epi epi, float* Y,
                     int32_t* acc_out, hipStream_t s) {
    const int rows_per_block = (kGemvThreads / kWave) * (kWave / G);
    const unsigned blocks = (unsigned)((N + rows_per_block - 1) / rows_per_block);
    const size_t lds = (size_t)MT * (size_t)K;
#define BL_GCASE(C)                                                                         \
    case C:                                                                                 \
        hipLaunchKernelGGL((k_gemv<MT, C>), dim3(blocks), dim3(kGemvThreads), lds, s, Xq, xs, \
                           rs, (int)K, reinterpret_cast<const uint4*>(packed), ws, (int)N, G, \
                           epi, Y, acc_out);                                                \
        break;
    switch (nch) {
        BL_GCASE(1)
        BL_GCASE(2)
        BL_GCASE(3)
        BL_GCASE(4)
        BL_GCASE(5)
        BL_GCASE(6)
        BL_GCASE(7)
        BL_GCASE(8)
        default:
            return hipErrorInvalidValue;
    }
#undef BL_GCASE
    return hipGetLastError();
}

}  // namespace

// Lanes per row: the smallest power of two that keeps every lane at <= 4
// chunks, capped at a wave; chunks per lane follow.
bool gemv_supported(int64_t M, int64_t K) {
    return M >= 1 && M <= 4 && K <= 32768 && M * K <= 65536;
}

hipError_t launch_gemv(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                       int64_t K, const uint8_t* packed, const float* ws, int64_t N, Epi epi,
                       float* Y, int32_t* acc_out, hipStream_t s) {
    const int64_t C = K / 64;
    int G = 1;
    while (G < 64 && G * 4 < C) G *= 2;
    const int nch = (int)((C + G - 1) / G);
    switch (M) {
        case 1: return launch_mt<1>(nch, Xq, xs, rs, K, packed, ws, N, G, epi, Y, acc_out, s);
        case 2: return launch_mt<2>(nch, Xq, xs, rs, K, packed, ws, N, G, epi, Y, acc_out, s);
        case 3: return launch_mt<3>(nch, Xq, xs, rs, K, packed, ws, N, G, epi, Y, acc_out, s);
        case 4: return launch_mt<4>(nch, Xq, xs, rs, K, packed, ws, N, G, epi, Y, acc_out, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace bl
