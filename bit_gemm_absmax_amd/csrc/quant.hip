// Activation quantiser: per-token absmax int8 quantisation, optionally after
// RMSNorm with a gain and no bias (transformers "BitNet" page, "Model
// details": per-token absmax 8-bit activations, subln normalisation, no bias
// in normalisation layers; "BitNetConfig": rms_norm_eps).
//
// One workgroup per token row (quant_row_* in bl_device.h).
// The row is loaded once into registers (NV float4 per thread, NV the
// smallest that covers the row: unused slots still cost load issue and
// registers), so the row-wide reductions -- sum of squares (binary64),
// max |z| and the int8 row sum -- never re-read HBM.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

template <int NT, int NV>
__global__ __launch_bounds__(NT) void k_quant(const float* __restrict__ X, int K, int rmsnorm,
                                              const float* __restrict__ gain, float eps,
                                              int8_t* __restrict__ Xq, float* __restrict__ scale,
                                              int32_t* __restrict__ rowsum) {
    constexpr int NW = NT / kWave;
    __shared__ double dslot[NW];
    __shared__ float fslot[NW], fslot2[NW];
    __shared__ int islot[NW];
    const int64_t m = blockIdx.x;
    float4 v[NV], gv[NV];
    quant_row_load<NT, NV>(X + m * K, rmsnorm ? gain : nullptr, K, v, gv);
    const float gamma = quant_row_finish<NT, NV>(v, gv, K, rmsnorm != 0, rmsnorm && gain != nullptr, eps,
                                                Xq + m * K, dslot, fslot, fslot2,
                                                rowsum != nullptr ? islot : nullptr);
    if (rowsum != nullptr) __syncthreads();
    if (threadIdx.x == 0) {
        scale[m] = gamma;
        if (rowsum != nullptr) {
            int t = 0;
#pragma unroll
            for (int i = 0; i < NW; ++i) t += islot[i];
            rowsum[m] = t;
        }
    }
}

__global__ __launch_bounds__(256) void k_rowsum(const int8_t* __restrict__ Xq, int K,
                                                int32_t* __restrict__ rowsum) {
    __shared__ int islot[4];
    const int64_t m = blockIdx.x;
    const int* x = reinterpret_cast<const int*>(Xq + m * K);
    int s = 0;
    for (int i = threadIdx.x; i < K / 4; i += 256) s = __builtin_amdgcn_sdot4(x[i], 0x01010101, s, false);
    s = block_sum<4>(s, islot);
    if (threadIdx.x == 0) rowsum[m] = s;
}

}  // namespace

int quant_threads(int64_t K) { return K <= 4096 ? 256 : (K <= 16384 ? 512 : 1024); }

bool quant_supported(int64_t K) { return K >= 4 && K % 4 == 0 && K <= 1024 * 4 * 8; }

namespace {
template <int NT, int NV>
void go_quant(const float* X, int64_t M, int64_t K, bool rmsnorm, const float* gain, float eps, int8_t* Xq,
              float* scale, int32_t* rowsum, hipStream_t s) {
    hipLaunchKernelGGL((k_quant<NT, NV>), dim3((unsigned)M), dim3(NT), 0, s, X, (int)K, rmsnorm ? 1 : 0, gain, eps,
                       Xq, scale, rowsum);
}
template <int NT>
void go_quant_nt(int nv, const float* X, int64_t M, int64_t K, bool rmsnorm, const float* gain, float eps,
                 int8_t* Xq, float* scale, int32_t* rowsum, hipStream_t s) {
    switch (nv) {
        case 1: go_quant<NT, 1>(X, M, K, rmsnorm, gain, eps, Xq, scale, rowsum, s); break;
        case 2: go_quant<NT, 2>(X, M, K, rmsnorm, gain, eps, Xq, scale, rowsum, s); break;
        case 3: go_quant<NT, 3>(X, M, K, rmsnorm, gain, eps, Xq, scale, rowsum, s); break;
        case 4: go_quant<NT, 4>(X, M, K, rmsnorm, gain, eps, Xq, scale, rowsum, s); break;
        case 5: go_quant<NT, 5>(X, M, K, rmsnorm, gain, eps, Xq, scale, rowsum, s); break;
        case 6: go_quant<NT, 6>(X, M, K, rmsnorm, gain, eps, Xq, scale, rowsum, s); break;
        case 7: go_quant<NT, 7>(X, M, K, rmsnorm, gain, eps, Xq, scale, rowsum, s); break;
        default: go_quant<NT, 8>(X, M, K, rmsnorm, gain, eps, Xq, scale, rowsum, s);
    }
}
}  // namespace

int quant_depth(int64_t K) {
    const int64_t per = 4 * (int64_t)quant_threads(K);
    return (int)((K + per - 1) / per);
}

hipError_t launch_quant(const float* X, int64_t M, int64_t K, bool rmsnorm, const float* gain,
                        float eps, int8_t* Xq, float* scale, int32_t* rowsum, hipStream_t s) {
    // The workgroup size follows quant_threads(K), which the fused
    // few-token kernels use too, so both quantise a row to the same values
    // (the depth NV does not change any result: slots past the row are 0).
    const int nv = quant_depth(K);
    switch (quant_threads(K)) {
        case 256: go_quant_nt<256>(nv, X, M, K, rmsnorm, gain, eps, Xq, scale, rowsum, s); break;
        case 512: go_quant_nt<512>(nv, X, M, K, rmsnorm, gain, eps, Xq, scale, rowsum, s); break;
        default: go_quant_nt<1024>(nv, X, M, K, rmsnorm, gain, eps, Xq, scale, rowsum, s);
    }
    return hipGetLastError();
}

hipError_t launch_rowsum(const int8_t* Xq, int64_t M, int64_t K, int32_t* rowsum, hipStream_t s) {
    hipLaunchKernelGGL(k_rowsum, dim3((unsigned)M), dim3(256), 0, s, Xq, (int)K, rowsum);
    return hipGetLastError();
}

}  // namespace bl
