// Device-side helpers for the gfx950 kernels: wave64 butterfly reductions and
// fixed-order block reductions.  Every reduction here has an order that
// depends only on the launch shape, so results are run-to-run identical.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

constexpr int kWave = 64;

// xor-butterfly: every lane ends with the same value, and because each step
// adds the same two operands on both partner lanes, the result is the same
// on every lane even for floating point.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

// Block reductions over NW waves through a small LDS array; the final sum
// runs over the waves in index order.  All threads get the result.  The
// caller must pass distinct `slot` arrays for back-to-back reductions or
// separate them with a barrier (these helpers end with one).
template <int NW>
__device__ __forceinline__ double block_sum(double v, double* slot) {
    v = wave_sum(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) slot[w] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < NW; ++i) t += slot[i];
    __syncthreads();
    return t;
}
template <int NW>
__device__ __forceinline__ int block_sum(int v, int* slot) {
    v = wave_sum(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) slot[w] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) t += slot[i];
    __syncthreads();
    return t;
}
template <int NW>
__device__ __forceinline__ float block_max(float v, float* slot) {
    v = wave_max(v);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) slot[w] = v;
    __syncthreads();
    float t = slot[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) t = fmaxf(t, slot[i]);
    __syncthreads();
    return t;
}

// Sum (binary64) and max (binary32) in one pass: one LDS round, one barrier.
template <int NW>
__device__ __forceinline__ void block_sum_max(double& v, float& mx, double* dslot, float* fslot) {
    v = wave_sum(v);
    mx = wave_max(mx);
    const int w = threadIdx.x / kWave;
    if ((threadIdx.x % kWave) == 0) {
        dslot[w] = v;
        fslot[w] = mx;
    }
    __syncthreads();
    double t = 0.0;
    float m = fslot[0];
#pragma unroll
    for (int i = 0; i < NW; ++i) t += dslot[i];
#pragma unroll
    for (int i = 1; i < NW; ++i) m = fmaxf(m, fslot[i]);
    __syncthreads();
    v = t;
    mx = m;
}

// The 2-bit weight word: 16 codes, weight 4j + b of the group in byte b at
// bits 2j..2j+1.  Shifting by 2j and masking leaves, in byte b, the code of
// weight 4j + b: four consecutive weights as four int8 values 0..2, in the
// same order as four consecutive int8 activations.
__device__ __forceinline__ int codes4(uint32_t w, int j) {
    return (int)((w >> (2 * j)) & 0x03030303u);
}

// The same four weights as signed int8 q = code - 1: adding 0x7F to a byte
// holding 0..2 cannot carry (0x7F..0x81), and flipping bit 7 then maps
// 0x7F, 0x80, 0x81 to 0xFF, 0x00, 0x01, i.e. -1, 0, +1.
__device__ __forceinline__ int signed4(uint32_t w, int j) {
    return (int)((((w >> (2 * j)) & 0x03030303u) + 0x7F7F7F7Fu) ^ 0x80808080u);
}

// One token row of the activation quantiser, run by a whole workgroup of NT
// threads: optional RMSNorm (binary64 sum of squares, r rounded once to
// binary32, z = (x * r) * gain), then absmax int8 quantisation.  Thread t
// owns float4 indices t + NT*i (i < NV), so K <= 4 * NT * NV.  Every kernel
// uses these functions with the same NT for a given K, so the reduction
// order (per-thread in i, then the wave butterfly, then the waves in index
// order) and hence every result is the same in every kernel.  Without a
// gain, max|x| is reduced together with the sum of squares: rounding is
// monotonic, so max_k |fl(x_k * r)| equals fl(max_k |x_k| * r), the same
// value a second pass would give.
//
// quant_row_load issues the row's loads (so a caller can put them ahead of
// other traffic); quant_row_finish does the arithmetic and writes xq (global
// memory or LDS), returning gamma and, if asked, the int8 row sum to all
// threads.
struct QuantRow {
    float gamma;
    int rowsum;
};

template <int NT, int NV>
__device__ __forceinline__ void quant_row_load(const float* __restrict__ x, int K, float4 (&v)[NV]) {
    const int n4 = K / 4;
    const float4* x4 = reinterpret_cast<const float4*>(x);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int idx = threadIdx.x + i * NT;
        v[i] = idx < n4 ? x4[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

template <int NT, int NV>
__device__ __forceinline__ QuantRow quant_row_finish(float4 (&v)[NV], int K, bool rmsnorm,
                                                     const float* __restrict__ gain, float eps, int8_t* xq,
                                                     double* dslot, float* fslot, int* islot,
                                                     bool want_rowsum) {
    constexpr int NW = NT / kWave;
    const int n4 = K / 4;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        amax = fmaxf(amax, fabsf(v[i].x));
        amax = fmaxf(amax, fabsf(v[i].y));
        amax = fmaxf(amax, fabsf(v[i].z));
        amax = fmaxf(amax, fabsf(v[i].w));
    }
    float g;
    if (rmsnorm) {
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            ss += (double)v[i].x * (double)v[i].x;
            ss += (double)v[i].y * (double)v[i].y;
            ss += (double)v[i].z * (double)v[i].z;
            ss += (double)v[i].w * (double)v[i].w;
        }
        block_sum_max<NW>(ss, amax, dslot, fslot);
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
                const float4 gg = g4[idx];
                t.x = t.x * gg.x;
                t.y = t.y * gg.y;
                t.z = t.z * gg.z;
                t.w = t.w * gg.w;
            }
            v[i] = t;
        }
        if (gain != nullptr) {
            amax = 0.0f;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                amax = fmaxf(amax, fabsf(v[i].x));
                amax = fmaxf(amax, fabsf(v[i].y));
                amax = fmaxf(amax, fabsf(v[i].z));
                amax = fmaxf(amax, fabsf(v[i].w));
            }
            g = block_max<NW>(amax, fslot);
        } else {
            g = amax * r;
        }
    } else {
        g = block_max<NW>(amax, fslot);
    }
    if (!(g >= 1e-5f)) g = 1e-5f;
    const float s = 127.0f / g;
    int sum = 0;
    int* q4 = reinterpret_cast<int*>(xq);
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
    if (want_rowsum) sum = block_sum<NW>(sum, islot);
    return QuantRow{g, sum};
}

}  // namespace bl
