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

// The 2-bit weight word: 16 codes, weight 4j + b of the group in byte b at
// bits 2j..2j+1.  Shifting by 2j and masking leaves, in byte b, the code of
// weight 4j + b: four consecutive weights as four int8 values 0..2, in the
// same order as four consecutive int8 activations.
__device__ __forceinline__ int codes4(uint32_t w, int j) {
    return (int)((w >> (2 * j)) & 0x03030303u);
}

}  // namespace bl
