// Activation quantiser: per-token absmax int8 quantisation, optionally after
// RMSNorm with a gain and no bias (transformers "BitNet" page, "Model
// details": per-token absmax 8-bit activations, subln normalisation, no bias
// in normalisation layers; "BitNetConfig": rms_norm_eps).
//
// One workgroup per token row.  The row is loaded once into registers
// (NV float4 per thread), so the three row-wide reductions -- sum of squares
// (binary64), max |z| and the int8 row sum -- never re-read HBM.
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
    __shared__ float fslot[NW];
    __shared__ int islot[NW];
    const int64_t m = blockIdx.x;
    const int n4 = K / 4;
    const float4* x4 = reinterpret_cast<const float4*>(X + m * K);

    float4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = threadIdx.x + i * NT;
        v[i] = idx < n4 ? x4[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    if (rmsnorm) {
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            ss += (double)v[i].x * (double)v[i].x;
            ss += (double)v[i].y * (double)v[i].y;
            ss += (double)v[i].z * (double)v[i].z;
            ss += (double)v[i].w * (double)v[i].w;
        }
        ss = block_sum<NW>(ss, dslot);
        const float r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
        const float4* g4 = reinterpret_cast<const float4*>(gain);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = threadIdx.x + i * NT;
            float4 t = v[i];
            t.x = t.x * r;
            t.y = t.y * r;
            t.z = t.z * r;
            t.w = t.w * r;
            if (gain != nullptr && idx < n4) {
                const float4 g = g4[idx];
                t.x = t.x * g.x;
                t.y = t.y * g.y;
                t.z = t.z * g.z;
                t.w = t.w * g.w;
            }
            v[i] = t;
        }
    }

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        amax = fmaxf(amax, fabsf(v[i].x));
        amax = fmaxf(amax, fabsf(v[i].y));
        amax = fmaxf(amax, fabsf(v[i].z));
        amax = fmaxf(amax, fabsf(v[i].w));
    }
    amax = block_max<NW>(amax, fslot);
    float g = amax;
    if (!(g >= 1e-5f)) g = 1e-5f;
    const float s = 127.0f / g;

    int sum = 0;
    int* q4 = reinterpret_cast<int*>(Xq + m * K);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = threadIdx.x + i * NT;
        if (idx < n4) {
            const float e[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            uint32_t packed = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                float t = rintf(e[b] * s);
                t = t > 127.0f ? 127.0f : t;
                t = t < -127.0f ? -127.0f : t;
                const int qi = (int)t;
                sum += qi;
                packed |= ((uint32_t)qi & 0xFFu) << (8 * b);
            }
            q4[idx] = (int)packed;
        }
    }
    sum = block_sum<NW>(sum, islot);
    if (threadIdx.x == 0) {
        scale[m] = g;
        if (rowsum != nullptr) rowsum[m] = sum;
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

template <int NT>
hipError_t launch_nt(int nv, const float* X, int64_t M, int64_t K, int rms, const float* gain,
                     float eps, int8_t* Xq, float* scale, int32_t* rowsum, hipStream_t s) {
#define BL_QCASE(V)                                                                        \
    case V:                                                                                \
        hipLaunchKernelGGL((k_quant<NT, V>), dim3((unsigned)M), dim3(NT), 0, s, X, (int)K, \
                           rms, gain, eps, Xq, scale, rowsum);                             \
        break;
    switch (nv) {
        BL_QCASE(1)
        BL_QCASE(2)
        BL_QCASE(3)
        BL_QCASE(4)
        BL_QCASE(5)
        BL_QCASE(6)
        BL_QCASE(7)
        BL_QCASE(8)
        default:
            return hipErrorInvalidValue;
    }
#undef BL_QCASE
    return hipGetLastError();
}

}  // namespace

bool quant_supported(int64_t K) { return K >= 4 && K % 4 == 0 && K <= 1024 * 4 * 8; }

hipError_t launch_quant(const float* X, int64_t M, int64_t K, bool rmsnorm, const float* gain,
                        float eps, int8_t* Xq, float* scale, int32_t* rowsum, hipStream_t s) {
    const int64_t n4 = K / 4;
    if (n4 <= 256 * 8) {
        const int nv = (int)((n4 + 255) / 256);
        return launch_nt<256>(nv, X, M, K, rmsnorm ? 1 : 0, gain, eps, Xq, scale, rowsum, s);
    }
    const int nv = (int)((n4 + 1023) / 1024);
    return launch_nt<1024>(nv, X, M, K, rmsnorm ? 1 : 0, gain, eps, Xq, scale, rowsum, s);
}

hipError_t launch_rowsum(const int8_t* Xq, int64_t M, int64_t K, int32_t* rowsum, hipStream_t s) {
    hipLaunchKernelGGL(k_rowsum, dim3((unsigned)M), dim3(256), 0, s, Xq, (int)K, rowsum);
    return hipGetLastError();
}

}  // namespace bl
