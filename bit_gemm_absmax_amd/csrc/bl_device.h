// Device-side helpers for the gfx950 kernels: wave64 butterfly reductions and
// fixed-order block reductions.  Every reduction here has an order that
// depends only on the launch shape, so results are run-to-run identical.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

constexpr int kWave = 64;

// Raw buffer access.  A load whose byte offset is at or past the
// descriptor's size returns zero in hardware, so bounds-checked loads need no
// branch: every load issues unconditionally, and the in-order vmcnt counter
// lets a kernel wait for an early load while later ones are still in flight
// (a load under a divergent branch makes the compiler wait for everything).
// Dword 3 = 0x00020000 selects 32-bit data format, which raw loads need to
// be valid on gfx9-family parts.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOob = 0x80000000u;  // an offset past every descriptor used here

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Non-temporal (nt) load, for data read once and streamed (the batched
// kernel's packed weights): a plain streaming read kernel measured about
// 6.2 TB/s with default loads and 7.1 TB/s with nt ones.  The M <= 4 decode
// launches keep default loads: nt made the K = 6912 one 0.15 us slower.
__device__ __forceinline__ uint4 buf_load16_nt(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}
__device__ __forceinline__ float4 buf_load16f(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load4f(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ int buf_load4i(Rsrc r, uint32_t off) {
    return (int)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

// s_waitcnt on the vector-memory counter only: at most N loads in flight,
// LDS counter left at its maximum; gfx9 encoding: vmcnt bits [3:0] and
// [15:14], expcnt [6:4], lgkmcnt [11:8].  Loads complete in issue order, so
// this also waits for every load issued before the last N.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// LDS destination of a direct buffer->LDS load (the base goes in M0; lane i
// of the wave writes its 16 bytes at base + 16 i).
typedef __attribute__((address_space(3))) void* lds_ptr;

// One 16-byte-per-lane direct buffer->LDS load.  A plain (non-template)
// function, so the builtin's operands are never template-dependent: clang's
// host pass, which checks them against the host target's limits (sizes 1, 2
// or 4), would otherwise drop the calling template as a substitution failure.
__device__ __forceinline__ void dma16(Rsrc r, lds_ptr dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}

// Wave reductions.  Within each row of 16 lanes, four DPP steps pair lane i
// with i^1, i^2 (quad permutes), 7-i (half mirror) and 15-i (mirror); after
// the first two steps the four lanes of a quad agree, so each step combines
// two equal groups and every lane computes the same two operands (in either
// order: + and max are commutative), hence the same value.  The four row
// values are then read into scalars and combined as (r0 + r1) + (r2 + r3).
// The order depends only on lane numbers, so results are run-to-run
// identical and the same in every kernel that calls these.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, dpp<CTRL>(__builtin_bit_cast(int, v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)dpp<CTRL>((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)dpp<CTRL>((int)(uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int lane_read(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float lane_read(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ double lane_read(double v, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
    v = v + dpp<kDppXor1>(v);
    v = v + dpp<kDppXor2>(v);
    v = v + dpp<kDppHalfMirror>(v);
    v = v + dpp<kDppMirror>(v);
    return (lane_read(v, 0) + lane_read(v, 16)) + (lane_read(v, 32) + lane_read(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    v = fmaxf(v, dpp<kDppMirror>(v));
    return fmaxf(fmaxf(lane_read(v, 0), lane_read(v, 16)), fmaxf(lane_read(v, 32), lane_read(v, 48)));
}

// Block reductions over NW waves through a small LDS array; the final
// combine runs over the waves in index order, and all threads get the
// result.  One barrier each and none at the end: a slot array may be used
// again only after a further barrier (distinct arrays for back-to-back
// reductions).
template <int NW>
__device__ __forceinline__ double block_sum(double v, double* slot) {
    v = wave_sum(v);
    if ((threadIdx.x % kWave) == 0) slot[threadIdx.x / kWave] = v;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < NW; ++i) t += slot[i];
    return t;
}
template <int NW>
__device__ __forceinline__ int block_sum(int v, int* slot) {
    v = wave_sum(v);
    if ((threadIdx.x % kWave) == 0) slot[threadIdx.x / kWave] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) t += slot[i];
    return t;
}
template <int NW>
__device__ __forceinline__ float block_max(float v, float* slot) {
    v = wave_max(v);
    if ((threadIdx.x % kWave) == 0) slot[threadIdx.x / kWave] = v;
    __syncthreads();
    float t = slot[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) t = fmaxf(t, slot[i]);
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

// Four elements quantised at scale s, q = clamp(rint(x * s), -127, 127), as
// four int8 in one word (element b in byte b).  Each q is formed as the byte
// of q + 128 in 1..255 (an exact float, med3 being the clamp, converted and
// inserted in one instruction); flipping bit 7 then turns the biased byte
// into the two's-complement int8 q.
__device__ __forceinline__ uint32_t quant4(float4 v, float s) {
    const float e[4] = {v.x, v.y, v.z, v.w};
    uint32_t packed = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const float t = __builtin_amdgcn_fmed3f(rintf(e[b] * s), -127.0f, 127.0f);
        packed = __builtin_amdgcn_cvt_pk_u8_f32(t + 128.0f, b, packed);
    }
    return packed ^ 0x80808080u;
}

// One token row of the activation quantiser, run by a whole workgroup of NT
// threads: optional RMSNorm (binary64 sum of squares, r rounded once to
// binary32, z = (x * r) * gain), then absmax int8 quantisation.  Thread t
// owns float4 indices t + NT*i (i < NV), so K <= 4 * NT * NV; slots past the
// row hold zeros, which change no sum or max, so any NV that covers the row
// gives the same results.  Every kernel uses these functions with the same
// NT for a given K, so the reduction order (per-thread in i, then the wave
// reduction, then the waves in index order) and hence every result is the
// same in every kernel.  Without a gain, max|x| is reduced together with the
// sum of squares: rounding is monotonic, so max_k |fl(x_k * r)| equals
// fl(max_k |x_k| * r), the same value a second pass would give.
//
// quant_row_load issues the row's loads, and the gain's (zeros when there is
// none), so a caller can put them ahead of other traffic; quant_row_finish
// does the arithmetic, writes xq (global memory or LDS) and returns gamma to
// all threads.
//
// VT < NT: a workgroup of NT threads reproduces the VT-thread quantiser
// exactly: threads t < VT own float4 t + VT*i as a VT-thread workgroup's
// would, threads from VT on load and store nothing and reduce zeros, and the
// block reductions then add those waves' +0.0 (or take their max with 0)
// after the real ones, which changes no bit.  AUX is the load's cache policy
// (0: default).  With rs_slot, lane 0 of each wave also writes the wave's
// share of the int8 row sum to rs_slot[wave]: the caller adds the NT/64
// entries after its next barrier.  Slot arrays follow block_sum's rule.
template <int NT, int NV, int VT = NT, int AUX = 0>
__device__ __forceinline__ void quant_row_load_x(const float* x, int K, float4 (&v)[NV]) {
    const Rsrc rx = make_rsrc(x, (uint32_t)K * 4u);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const uint32_t off = (VT == NT || (int)threadIdx.x < VT) ? (uint32_t)(threadIdx.x + i * VT) * 16u : kOob;
        v[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, AUX));
    }
}
template <int NT, int NV, int VT = NT>
__device__ __forceinline__ void quant_row_load(const float* x, const float* gain, int K, float4 (&v)[NV],
                                               float4 (&gv)[NV]) {
    quant_row_load_x<NT, NV, VT>(x, K, v);
    const Rsrc rg = make_rsrc(gain, gain != nullptr ? (uint32_t)K * 4u : 0u);
#pragma unroll
    for (int i = 0; i < NV; ++i)
        gv[i] = buf_load16f(rg, (VT == NT || (int)threadIdx.x < VT) ? (uint32_t)(threadIdx.x + i * VT) * 16u : kOob);
}

template <int NT, int NV, int VT = NT>
__device__ __forceinline__ float quant_row_finish(float4 (&v)[NV], const float4 (&gv)[NV], int K, bool rmsnorm,
                                                  bool has_gain, float eps, int8_t* xq, double* dslot,
                                                  float* fslot, float* fslot2, int* rs_slot) {
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
        // x * x of a binary32 x is exact in binary64, so the fused multiply-add
        // rounds once, exactly as the separate add of the product would
        double ss = 0.0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            ss = __builtin_fma((double)v[i].x, (double)v[i].x, ss);
            ss = __builtin_fma((double)v[i].y, (double)v[i].y, ss);
            ss = __builtin_fma((double)v[i].z, (double)v[i].z, ss);
            ss = __builtin_fma((double)v[i].w, (double)v[i].w, ss);
        }
        block_sum_max<NW>(ss, amax, dslot, fslot);
        const float r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float4 t = v[i];
            t.x = t.x * r;
            t.y = t.y * r;
            t.z = t.z * r;
            t.w = t.w * r;
            if (has_gain) {
                t.x = t.x * gv[i].x;
                t.y = t.y * gv[i].y;
                t.z = t.z * gv[i].z;
                t.w = t.w * gv[i].w;
            }
            v[i] = t;
        }
        if (has_gain) {
            amax = 0.0f;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                amax = fmaxf(amax, fabsf(v[i].x));
                amax = fmaxf(amax, fabsf(v[i].y));
                amax = fmaxf(amax, fabsf(v[i].z));
                amax = fmaxf(amax, fabsf(v[i].w));
            }
            g = block_max<NW>(amax, fslot2);
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
        const int idx = (VT == NT || (int)threadIdx.x < VT) ? threadIdx.x + i * VT : n4;  // n4: stores nothing
        const uint32_t packed = quant4(v[i], s);
        sum = __builtin_amdgcn_sdot4((int)packed, 0x01010101, sum, false);  // slots past the row hold 0
        if (idx < n4) q4[idx] = (int)packed;
    }
    if (rs_slot != nullptr) {
        sum = wave_sum(sum);
        if ((threadIdx.x % kWave) == 0) rs_slot[threadIdx.x / kWave] = sum;
    }
    return g;
}

}  // namespace bl
