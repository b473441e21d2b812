// Weight packer: absmean ternarisation and 2-bit packing of latent fp32 or
// bf16 weights (transformers "BitNet" page, "Model details" / Quantization:
// ternary {-1, 0, +1} weights by absmean quantisation; "Model variants":
// packed 1.58-bit weights for deployment).
//
// Two launches, both streaming W once from HBM:
//   1. k_absmean_partial: each block sums |W| in binary64 over a grid-stride
//      slice and writes one partial.
//   2. k_ternary_pack: every block re-reduces the partials in the same fixed
//      order (a few KB from L2, identical result in every block), forms
//      gamma_w = max((float)(sum / (N*K)), 1e-5), and turns each group of 16
//      weights into one 32-bit word of 2-bit codes, stored at its place in
//      the packed layout: rows in tiles of 16 (the last tile has the rows
//      left), each tile chunk-major, so 16 rows' 16-byte chunks c sit side by
//      side and a wave's weight loads (one row per adjacent lane) read whole
//      lines.
// The partial count depends only on N*K, so the binary64 summation order,
// and hence gamma_w, is the same on every run.
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxPartials = 1024;

// Latent weight element types: load4(W, i) returns weights 4i..4i+3 as fp32.
// A bf16 value is the upper half of the fp32 with the same bits, so widening
// is exact and both types go through the same arithmetic.
struct InF32 {
    static __device__ __forceinline__ float4 load4(const void* W, int64_t i) {
        return reinterpret_cast<const float4*>(W)[i];
    }
};
struct InBF16 {
    static __device__ __forceinline__ float4 load4(const void* W, int64_t i) {
        const uint2 u = reinterpret_cast<const uint2*>(W)[i];  // little-endian: element 2j in the low half
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    }
};

template <typename In>
__global__ __launch_bounds__(kThreads) void k_absmean_partial(const void* __restrict__ W, int64_t n4,
                                                              double* __restrict__ partial) {
    __shared__ double slot[kThreads / kWave];
    double s = 0.0;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
        const float4 v = In::load4(W, i);
        s += fabs((double)v.x);
        s += fabs((double)v.y);
        s += fabs((double)v.z);
        s += fabs((double)v.w);
    }
    s = block_sum<kThreads / kWave>(s, slot);
    if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

// code = clamp(rint(w / gamma), -1, 1) + 1 (binary32 quotient, ties to
// even), computed without the divide.  rint of the rounded quotient |w|/gamma
// is nonzero exactly when that quotient exceeds 0.5, i.e. when |w|/gamma lies
// above the midpoint 0.5 + 2^-25 between 0.5 and the next binary32 (at the
// midpoint the tie goes to 0.5, whose significand is even): 2|w| > gamma
// (1 + 2^-24).  For binary32 gamma = m 2^e (2^23 <= m < 2^24) the next
// binary32 above gamma is gamma (1 + 1/m) > gamma (1 + 2^-24), and 2|w| is an
// exact binary32, so that holds exactly when 2|w| > gamma.  The clip then
// leaves the sign of w.
__device__ __forceinline__ uint32_t ternary_code(float w, float gamma) {
    return 2.0f * fabsf(w) > gamma ? (w > 0.0f ? 2u : 0u) : 1u;
}

template <typename In>
__global__ __launch_bounds__(kThreads) void k_ternary_pack(const void* __restrict__ W,
                                                           int64_t nwords, int64_t N, int64_t K,
                                                           const double* __restrict__ partial,
                                                           int nparts, double count,
                                                           uint32_t* __restrict__ packed,
                                                           float* __restrict__ w_scale) {
    __shared__ double slot[kThreads / kWave];
    double s = 0.0;
    for (int i = threadIdx.x; i < nparts; i += kThreads) s += partial[i];
    s = block_sum<kThreads / kWave>(s, slot);
    float gamma = (float)(s / count);
    if (!(gamma >= 1e-5f)) gamma = 1e-5f;
    if (blockIdx.x == 0 && threadIdx.x == 0) *w_scale = gamma;

    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t w = (int64_t)blockIdx.x * kThreads + threadIdx.x; w < nwords; w += stride) {
        float4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = In::load4(W, 4 * w + j);
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // float4 j holds weights 4j + b (b = 0..3) of the group: byte b, bits 2j.
            word |= ternary_code(v[j].x, gamma) << (2 * j);
            word |= ternary_code(v[j].y, gamma) << (8 + 2 * j);
            word |= ternary_code(v[j].z, gamma) << (16 + 2 * j);
            word |= ternary_code(v[j].w, gamma) << (24 + 2 * j);
        }
        // word w is group g of row n: chunk c = g / 4, word d = g % 4 of it;
        // tile t = n / 16 (R rows) starts at word t * K, chunk c of tile row
        // r at word 4 (c R + r)
        const int64_t gpr = K / 16;
        const int64_t n = w / gpr, g = w % gpr;
        const int64_t t = n / 16;
        const int64_t R = N - 16 * t < 16 ? N - 16 * t : 16;
        packed[t * K + 4 * ((g / 4) * R + (n % 16)) + (g % 4)] = word;
    }
}

// The plain row-major 2-bit form (weight k of row n in byte n K/4 + k/4 at
// bits 2 (k % 4)) and this library's tile-grouped layout hold the same 32-bit
// words of 16 consecutive weights, in different places and with the 2-bit
// fields transposed: in the plain word, byte j field b is weight 4j + b; in
// the tile word, byte b field j is.  The transpose is its own inverse, so one
// kernel converts either way (TO_TILE picks which index is read).
__device__ __forceinline__ uint32_t transpose_fields(uint32_t w) {
    uint32_t t = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) t |= ((w >> (8 * j + 2 * b)) & 3u) << (8 * b + 2 * j);
    return t;
}

// Word index of group g (16 weights) of row n in the tile layout.
__device__ __forceinline__ int64_t tile_word(int64_t n, int64_t g, int64_t N, int64_t K) {
    const int64_t t = n / 16;
    const int64_t R = N - 16 * t < 16 ? N - 16 * t : 16;
    return t * K + 4 * ((g / 4) * R + (n % 16)) + (g % 4);
}

template <bool TO_TILE>
__global__ __launch_bounds__(kThreads) void k_relayout(const uint32_t* __restrict__ in, int64_t nwords, int64_t N,
                                                       int64_t K, uint32_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t gpr = K / 16;
    for (int64_t w = (int64_t)blockIdx.x * kThreads + threadIdx.x; w < nwords; w += stride) {
        const int64_t tw = tile_word(w / gpr, w % gpr, N, K);
        if (TO_TILE) out[tw] = transpose_fields(in[w]);
        else out[w] = transpose_fields(in[tw]);
    }
}

// Tile layout -> int8 q [N][K]: the tile word of group g of row n gives the
// 16 weights 16g .. 16g + 15 of the row, four consecutive ones per field
// shift (signed4), stored as one 16-byte write.
__global__ __launch_bounds__(kThreads) void k_unpack(const uint32_t* __restrict__ packed, int64_t nwords, int64_t N,
                                                     int64_t K, int4* __restrict__ q) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const int64_t gpr = K / 16;
    for (int64_t w = (int64_t)blockIdx.x * kThreads + threadIdx.x; w < nwords; w += stride) {
        const uint32_t v = packed[tile_word(w / gpr, w % gpr, N, K)];
        q[w] = make_int4(signed4(v, 0), signed4(v, 1), signed4(v, 2), signed4(v, 3));
    }
}

}  // namespace

int pack_partial_blocks(int64_t count) {
    const int64_t per_block = (int64_t)kThreads * 4 * 16;  // 16 float4 per thread
    int64_t g = (count + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > kMaxPartials) g = kMaxPartials;
    return (int)g;
}

namespace {
template <typename In>
hipError_t go_pack(const void* W, int64_t N, int64_t K, uint8_t* packed, float* w_scale, double* partial,
                   hipStream_t s) {
    const int64_t count = N * K;
    const int g = pack_partial_blocks(count);
    hipLaunchKernelGGL(k_absmean_partial<In>, dim3(g), dim3(kThreads), 0, s, W, count / 4, partial);
    const int64_t nwords = count / 16;
    int64_t blocks = (nwords + kThreads - 1) / kThreads;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(k_ternary_pack<In>, dim3((unsigned)blocks), dim3(kThreads), 0, s, W, nwords, N, K,
                       partial, g, (double)count, reinterpret_cast<uint32_t*>(packed), w_scale);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_pack(const void* W, bool bf16, int64_t N, int64_t K, uint8_t* packed, float* w_scale,
                       double* partial, hipStream_t s) {
    return bf16 ? go_pack<InBF16>(W, N, K, packed, w_scale, partial, s)
                : go_pack<InF32>(W, N, K, packed, w_scale, partial, s);
}

namespace {
unsigned word_blocks(int64_t nwords) {
    int64_t blocks = (nwords + kThreads - 1) / kThreads;
    return (unsigned)(blocks > 8192 ? 8192 : blocks < 1 ? 1 : blocks);
}
}  // namespace

hipError_t launch_relayout(const uint8_t* in, int64_t N, int64_t K, bool to_tile, uint8_t* out, hipStream_t s) {
    const int64_t nwords = N * K / 16;
    const uint32_t* i = reinterpret_cast<const uint32_t*>(in);
    uint32_t* o = reinterpret_cast<uint32_t*>(out);
    if (to_tile)
        hipLaunchKernelGGL(k_relayout<true>, dim3(word_blocks(nwords)), dim3(kThreads), 0, s, i, nwords, N, K, o);
    else
        hipLaunchKernelGGL(k_relayout<false>, dim3(word_blocks(nwords)), dim3(kThreads), 0, s, i, nwords, N, K, o);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* q, hipStream_t s) {
    const int64_t nwords = N * K / 16;
    hipLaunchKernelGGL(k_unpack, dim3(word_blocks(nwords)), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint32_t*>(packed), nwords, N, K, reinterpret_cast<int4*>(q));
    return hipGetLastError();
}

}  // namespace bl
