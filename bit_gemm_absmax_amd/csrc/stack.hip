// The whole BitNet feed-forward stack for one token in a single persistent
// launch (transformers "BitNet" page, "Model details" / Architecture: BitLinear
// layers with squared ReLU and subln, no bias; "BitNetConfig": 30 layers,
// hidden 2560, intermediate 6912).
//
// One workgroup per CU stays resident for all layers.  Each layer is two
// phases:
//   up:   every workgroup with up tiles quantises hidden (RMSNorm with the
//         pre-norm gain, then absmax) into its LDS, contracts its 16-row
//         tiles of the up matrix and publishes ReLU^2 of the dequantised
//         outputs (y1);
//   down: every workgroup with a down tile quantises all of y1 (subln
//         RMSNorm, then absmax) into its LDS, contracts its 16-row tile of the
//         down matrix and adds the result to its 16 values of hidden, which
//         it keeps in registers for the whole launch and publishes.
// Every row quantisation is the one the two-launch path runs (quant_row_*
// with the same thread-to-element map and reduction order: the 2560-wide row
// as a 256-thread workgroup would, the 6912-wide one with all 512 threads),
// so the results are bit-identical to it.
//
// There is no grid-wide barrier: every published value carries its own
// ready flag, written with it in one store, and a reader polls the values it
// needs until all flags say "this layer".  A y1 value is never negative, so
// its sign bit carries the flag (the layer's parity); a hidden value is
// stored as a 64-bit pair with the layer number.  One flag bit is enough for
// y1 and stale layer numbers cannot be mistaken for hidden ones, because
// nothing can be published twice ahead of a reader: a workgroup that writes
// y1 of layer l + 1 has read all of hidden after layer l, which every down
// workgroup wrote only after reading all of y1 of layer l, and the same
// holds for hidden the other way round.  (Only workgroups that publish in
// the next phase read in this one.)  The prep kernel sets every flag to
// "stale" before the launch.  Published data crosses XCDs, whose L2s are not
// coherent with each other: it is stored write-through and read past the L2
// (system-coherent cache policy on those accesses only).
//
// The weights a workgroup needs in the next phase do not depend on the
// activations, so their loads are issued in the current phase, right after
// the first loads of the row it quantises: they land while it quantises,
// contracts and waits for the next row.  Every poll is bounded: past its
// limit the workgroup records the failure and leaves, and the others leave
// when they see the record, so the launch always ends (its outputs are then
// not valid).
#include "bitlinear.h"
#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

constexpr int kSW = 8;                 // waves per workgroup
constexpr int kST = kSW * kWave;       // 512 threads
constexpr int kCoh = 1 | 16;           // sc0 sc1: system-coherent load / write-through store
constexpr uint32_t kSpinLimit = 1u << 20;  // polls per row (each a memory round trip): about a second
constexpr uint32_t kSign = 0x80000000u;

__device__ __forceinline__ float load_coh4(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCoh));
}
__device__ __forceinline__ void store_coh4(uint32_t v, Rsrc r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kCoh);
}
__device__ __forceinline__ uint4 load_coh16(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoh));
}
__device__ __forceinline__ uint2 load_coh8(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCoh));
}
__device__ __forceinline__ void store_coh8(uint2 v, Rsrc r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u, v), r, off, 0, kCoh);
}

// One more poll of a row: false once this thread has polled kSpinLimit times
// (the failure is then recorded) or another workgroup has failed.
__device__ __forceinline__ bool poll_again(uint32_t& spins, uint32_t* failed) {
    if (++spins > kSpinLimit) {
        __hip_atomic_store(failed, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return false;
    }
    if ((spins & 255u) == 0u && __hip_atomic_load(failed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)
        return false;
    __builtin_amdgcn_s_sleep(1);
    // the polled words change under this thread: the compiler must reload
    // them on every round (the raw buffer loads are otherwise free to hoist)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return true;
}

// Hidden after layer `gen - 1` as published pairs {bits, gen}, read into v in
// the VT-thread quantiser's element map.  issue: the first loads; settle:
// polls until every pair of this thread carries `gen`.  64-bit accesses,
// each of which is single-copy atomic.
template <int NV, int VT>
struct HiddenRow {
    uint2 e[NV][4];
    __device__ __forceinline__ bool valid(int i, int K) const {
        return (int)threadIdx.x < VT && (int)threadIdx.x + i * VT < K / 4;
    }
    __device__ __forceinline__ void load(Rsrc r, int i, int K) {
        const uint32_t base = valid(i, K) ? (uint32_t)(threadIdx.x + i * VT) * 32u : kOob;
#pragma unroll
        for (int k = 0; k < 4; ++k) e[i][k] = load_coh8(r, base == kOob ? kOob : base + 8u * k);
    }
    __device__ __forceinline__ void issue(Rsrc r, int K) {
#pragma unroll
        for (int i = 0; i < NV; ++i) load(r, i, K);
    }
    __device__ __forceinline__ bool settle(Rsrc r, int K, uint32_t gen, uint32_t* failed, float4 (&v)[NV]) {
        uint32_t spins = 0;
        bool good = true;
        for (;;) {
            bool all = true;
#pragma unroll
            for (int i = 0; i < NV; ++i)
                all = all && (!valid(i, K) || (e[i][0].y == gen && e[i][1].y == gen && e[i][2].y == gen &&
                                                e[i][3].y == gen));
            if (all) break;
            if (!poll_again(spins, failed)) {
                good = false;
                break;
            }
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (valid(i, K) && !(e[i][0].y == gen && e[i][1].y == gen && e[i][2].y == gen && e[i][3].y == gen))
                    load(r, i, K);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i)
            v[i] = float4{__builtin_bit_cast(float, e[i][0].x), __builtin_bit_cast(float, e[i][1].x),
                          __builtin_bit_cast(float, e[i][2].x), __builtin_bit_cast(float, e[i][3].x)};
        return good;
    }
};

// y1 of layer l as published words (value bits, sign bit = l & 1), read into
// v in the VT-thread quantiser's element map; as HiddenRow.
template <int NV, int VT>
struct Y1Row {
    uint4 e[NV];
    __device__ __forceinline__ bool valid(int i, int K) const {
        return (int)threadIdx.x < VT && (int)threadIdx.x + i * VT < K / 4;
    }
    __device__ __forceinline__ void load(Rsrc r, int i, int K) {
        e[i] = load_coh16(r, valid(i, K) ? (uint32_t)(threadIdx.x + i * VT) * 16u : kOob);
    }
    __device__ __forceinline__ void issue(Rsrc r, int K) {
#pragma unroll
        for (int i = 0; i < NV; ++i) load(r, i, K);
    }
    static __device__ __forceinline__ bool ready(uint4 w, uint32_t flag) {
        return (((w.x ^ flag) | (w.y ^ flag) | (w.z ^ flag) | (w.w ^ flag)) & kSign) == 0u;
    }
    __device__ __forceinline__ bool settle(Rsrc r, int K, uint32_t flag, uint32_t* failed, float4 (&v)[NV]) {
        uint32_t spins = 0;
        bool good = true;
        for (;;) {
            bool all = true;
#pragma unroll
            for (int i = 0; i < NV; ++i) all = all && (!valid(i, K) || ready(e[i], flag));
            if (all) break;
            if (!poll_again(spins, failed)) {
                good = false;
                break;
            }
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if (valid(i, K) && !ready(e[i], flag)) load(r, i, K);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i)
            v[i] = float4{__builtin_bit_cast(float, e[i].x & ~kSign), __builtin_bit_cast(float, e[i].y & ~kSign),
                          __builtin_bit_cast(float, e[i].z & ~kSign), __builtin_bit_cast(float, e[i].w & ~kSign)};
        return good;
    }
};

// Weights of one 16-row tile for this lane: wave w takes chunk quads
// w, w + 8, ... of the row; lane (fr, fg) loads chunk 4 s + fg of tile row fr
// (tile layout: chunk c of row r at byte 16 (c R + r) of the tile).  A tile
// past the matrix or a chunk past the row reads zeros.
template <int Q>
__device__ __forceinline__ void load_tile(const uint8_t* W, int tile, int N, int K, uint4 (&w)[Q]) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int fr = lane & 15, fg = lane >> 4;
    const int C = K / 64, nq = (C + 3) / 4;
    const int r0 = tile * 16;
    const int rows = __builtin_amdgcn_readfirstlane(N - r0 < 0 ? 0 : (N - r0 < 16 ? N - r0 : 16));
    const Rsrc rw = make_rsrc(W + (int64_t)(rows > 0 ? r0 : 0) * (K / 4), (uint32_t)rows * (uint32_t)(K / 4));
#pragma unroll
    for (int i = 0; i < Q; ++i) {
        const int s = wave + i * kSW;
        const int c = 4 * s + fg;
        w[i] = buf_load16(rw, (s < nq && c < C) ? (uint32_t)(c * rows + fr) * 16u : kOob);
    }
}

// The gain of one row in the VT-thread quantiser's element map (plain loads;
// zeros without a gain).
template <int NV, int VT>
__device__ __forceinline__ void load_gain(const float* gain, int K, float4 (&gv)[NV]) {
    const Rsrc rg = make_rsrc(gain, gain != nullptr ? (uint32_t)K * 4u : 0u);
#pragma unroll
    for (int i = 0; i < NV; ++i)
        gv[i] = buf_load16f(rg, (int)threadIdx.x < VT ? (uint32_t)(threadIdx.x + i * VT) * 16u : kOob);
}

// Contract T tiles against the quantised row xq (LDS) in one pass; the wave
// partials meet in red[T][kSW][16] and thread 16 j + n (n < 16) returns the
// exact sum of column n of tile j.
template <int Q, int T>
__device__ __forceinline__ int contract_tiles(const uint4 (&w)[T][Q], const int8_t* xq, int K, int* red) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int fr = lane & 15, fg = lane >> 4;
    const int C = K / 64, nq = (C + 3) / 4;
    v4i acc[T];
#pragma unroll
    for (int j = 0; j < T; ++j) acc[j] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < Q; ++i) {
        const int s = wave + i * kSW;
        if (s < nq) {
            const int c = 4 * s + fg;
            const int koff = c < C ? 64 * c : 0;  // a chunk past the row has zero weights
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                // token row 0 in every A row (rows past the one token are don't-care)
                const v4i a = *reinterpret_cast<const v4i*>(xq + koff + 16 * d);
#pragma unroll
                for (int j = 0; j < T; ++j) {
                    const uint32_t wd = d == 0 ? w[j][i].x : d == 1 ? w[j][i].y : d == 2 ? w[j][i].z : w[j][i].w;
                    const v4i b = v4i{codes4(wd, 0), codes4(wd, 1), codes4(wd, 2), codes4(wd, 3)};
                    acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[j], 0, 0, 0);
                }
            }
        }
    }
    // acc[j][0] of lanes fg = 0 is token 0, column fr of tile j
    if (fg == 0) {
#pragma unroll
        for (int j = 0; j < T; ++j) red[(j * kSW + wave) * 16 + fr] = acc[j][0];
    }
    __syncthreads();
    int sum = 0;
    if ((int)threadIdx.x < 16 * T) {
        const int j = threadIdx.x / 16, n = threadIdx.x % 16;
#pragma unroll
        for (int q = 0; q < kSW; ++q) sum += red[(j * kSW + q) * 16 + n];
    }
    __syncthreads();  // red is reused by the next contraction
    return sum;
}

// A plain load of one float from device memory, as a global (not flat)
// access: a flat access in flight makes every later wait for vector loads a
// wait for all of them, which would stall the weight loads issued ahead.
__device__ __forceinline__ float load_global(const float* p) {
    return *(const __attribute__((address_space(1))) float*)p;
}

// NVH / NVF: float4 per thread of the hidden / intermediate row in the
// quantiser's map for 256 / VF threads; QU / QD: chunk quads per lane of an
// up / down tile; UT: up tiles per workgroup (tiles g, g + nwg, ...).
template <int NVH, int NVF, int VF, int QU, int QD, int UT>
__global__ __launch_bounds__(kST) void k_stack(const bitnet_ffn_layer* __restrict__ layers, int n_layers,
                                               float* hidden, int H, int F, int pre, int residual, float eps,
                                               uint32_t* y1x, uint2* hx, uint32_t* failed) {
    extern __shared__ __align__(16) int8_t lds[];  // [xq: max(H, F) bytes] [red: UT x kSW x 16 ints]
    __shared__ double dslot[kSW];
    __shared__ float fslot[kSW], fslot2[kSW];
    __shared__ int islot[kSW];
    __shared__ int bad;  // a poll of this workgroup failed
    int* red = reinterpret_cast<int*>(lds + (H > F ? H : F));
    const int nwg = (int)gridDim.x;
    const int g = blockIdx.x;
    const bool has_up = g * 16 < F;  // the host launches at least H / 16 workgroups
    const bool has_dn = g * 16 < H;
    const Rsrc rh = make_rsrc(hidden, (uint32_t)H * 4u);
    const Rsrc rhx = make_rsrc(hx, (uint32_t)H * 8u);
    const Rsrc ry = make_rsrc(y1x, (uint32_t)F * 4u);
    if (threadIdx.x == 0) bad = 0;  // read only after the quantiser's barriers

    // this workgroup's 16 values of hidden, thread n < 16 holding row 16 g + n
    const int hn = g * 16 + (int)threadIdx.x;
    const bool mine = has_dn && threadIdx.x < 16 && hn < H;
    float h_own = load_coh4(rh, mine ? (uint32_t)hn * 4u : kOob);

    uint4 wu[UT][QU];
#pragma unroll
    for (int j = 0; j < UT; ++j) load_tile<QU>(layers[0].up, g + j * nwg, F, H, wu[j]);

    for (int l = 0; l < n_layers; ++l) {
        const bool last = l + 1 == n_layers;
        const uint8_t* down_w = layers[l].down;
        // on the last layer the up tiles past the matrix: loads that read nothing
        const uint8_t* up_next = layers[last ? l : l + 1].up;
        const int up_t0 = last ? F / 16 : g;
        const float* pre_gain = pre ? layers[l].pre_norm_gain : nullptr;
        const float* sub_gain = layers[l].sub_norm_gain;
        const float up_scale = load_global(layers[l].up_scale);
        const float down_scale = load_global(layers[l].down_scale);

        // ---- up (the down tile's weights go out right after the row's
        // first loads: vector loads complete in issue order, so they must not
        // go before what is needed first)
        uint4 wd[1][QD];
        if (has_up) {
            float4 v[NVH], gv[NVH];
            HiddenRow<NVH, 256> row;
            if (l == 0) quant_row_load_x<kST, NVH, 256, kCoh>(hidden, H, v);
            else row.issue(rhx, H);
            load_gain<NVH, 256>(pre_gain, H, gv);
            __builtin_amdgcn_sched_barrier(0);
            load_tile<QD>(down_w, g, H, F, wd[0]);
            __builtin_amdgcn_sched_barrier(0);
            if (l > 0 && !row.settle(rhx, H, (uint32_t)l, failed, v)) bad = 1;
            const float gx = quant_row_finish<kST, NVH, 256>(v, gv, H, pre != 0, pre_gain != nullptr, eps, lds,
                                                              dslot, fslot, fslot2, islot);
            __syncthreads();
            if (bad) return;
            int rs = 0;
#pragma unroll
            for (int q = 0; q < kSW; ++q) rs += islot[q];
            const float d = (gx * up_scale) / 127.0f;
            const int a = contract_tiles<QU, UT>(wu, lds, H, red);  // every thread takes part
            const int t = g + (int)(threadIdx.x / 16) * nwg;
            const int n = t * 16 + (int)(threadIdx.x % 16);
            if ((int)threadIdx.x < 16 * UT && n < F) {
                float y = (float)(a - rs) * d;
                y = y > 0.0f ? y : 0.0f;
                y = y * y;  // never negative: the sign bit is free for the flag
                store_coh4(__builtin_bit_cast(uint32_t, y) | ((uint32_t)(l & 1) << 31), ry, (uint32_t)n * 4u);
            }
        } else {
            load_tile<QD>(down_w, g, H, F, wd[0]);
        }

        // ---- down (the next layer's up weights go out right after the
        // row's first loads)
        if (has_dn) {
            float4 z[NVF], zg[NVF];
            Y1Row<NVF, VF> row;
            row.issue(ry, F);
            load_gain<NVF, VF>(sub_gain, F, zg);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < UT; ++j) load_tile<QU>(up_next, up_t0 + j * nwg, F, H, wu[j]);
            __builtin_amdgcn_sched_barrier(0);
            if (!row.settle(ry, F, (uint32_t)(l & 1) << 31, failed, z)) bad = 1;
            const float gx = quant_row_finish<kST, NVF, VF>(z, zg, F, true, sub_gain != nullptr, eps, lds, dslot,
                                                             fslot, fslot2, islot);
            __syncthreads();
            if (bad) return;
            int rs = 0;
#pragma unroll
            for (int q = 0; q < kSW; ++q) rs += islot[q];
            const float d = (gx * down_scale) / 127.0f;
            const int a = contract_tiles<QD, 1>(wd, lds, F, red);
            if (mine) {
                const float y = (float)(a - rs) * d;
                h_own = residual ? h_own + y : y;
                if (last)
                    store_coh4(__builtin_bit_cast(uint32_t, h_own), rh, (uint32_t)hn * 4u);
                else
                    store_coh8(uint2{__builtin_bit_cast(uint32_t, h_own), (uint32_t)(l + 1)}, rhx, (uint32_t)hn * 8u);
            }
        } else {
#pragma unroll
            for (int j = 0; j < UT; ++j) load_tile<QU>(up_next, up_t0 + j * nwg, F, H, wu[j]);
        }
    }
}

// Layer descriptors of one launch, passed by value (copied into the
// workspace by k_stack_prep, which also marks every published value stale
// and clears the failure record: no host copy and no memset, so the pair can
// be captured in a graph and replayed).
constexpr int kStackMaxLayers = 48;
constexpr int kStackMaxH = 4096;
struct StackLayers {
    bitnet_ffn_layer l[kStackMaxLayers];
};

__global__ void k_stack_prep(const StackLayers a, int n, bitnet_ffn_layer* dst, uint32_t* failed, uint2* hx, int H,
                             uint32_t* y1x, int F) {
    const int i = threadIdx.x;
    if (i < n) dst[i] = a.l[i];
    if (i == 0) *failed = 0u;
    for (int w = i; w < H; w += blockDim.x) hx[w] = uint2{0u, 0u};  // layer numbers start at 1
    for (int w = i; w < F; w += blockDim.x) y1x[w] = kSign;         // layer 0 publishes parity 0
}

}  // namespace

// Shapes of the persistent launch.  The row quantisers follow the
// standalone quantiser's workgroup sizes (256 threads up to 4096 wide, 512 up
// to 16384), so H <= 3072 (3 float4 per thread of 256) and F <= 8192 (4 of
// 256 or 512); quads per lane and up tiles per workgroup come from the shapes
// and the CU count.  The instantiated combinations are listed in kStackPlans.
struct StackPlan {
    int nvh, nvf, vf, qu, qd, ut;
};
constexpr StackPlan kStackPlans[] = {
    {3, 4, 512, 2, 4, 2},  // hidden 2560, intermediate 6912 on 216..431 CUs
    {3, 4, 512, 2, 4, 1},  // the same on 432 or more
    {1, 1, 256, 1, 1, 1},  // small shapes (tests): H <= 1024, F <= 1024
    {1, 2, 256, 1, 1, 1},  // H <= 1024, F <= 2048
};

static bool stack_plan(int64_t H, int64_t F, int64_t nwg, StackPlan& p) {
    if (H < 64 || F < 64 || H % 64 != 0 || F % 64 != 0 || (H + 15) / 16 > nwg || H > kStackMaxH || F > 16384)
        return false;
    p.nvh = (int)((H + 1023) / 1024);
    p.vf = F <= 4096 ? 256 : 512;
    p.nvf = (int)((F + 4 * p.vf - 1) / (4 * p.vf));
    p.qu = (int)(((H / 64 + 3) / 4 + kSW - 1) / kSW);
    p.qd = (int)(((F / 64 + 3) / 4 + kSW - 1) / kSW);
    p.ut = (int)(((F + 15) / 16 + nwg - 1) / nwg);
    for (const StackPlan& q : kStackPlans)
        if (q.nvh == p.nvh && q.nvf == p.nvf && q.vf == p.vf && q.qu == p.qu && q.qd == p.qd && q.ut == p.ut)
            return true;
    return false;
}

bool stack_supported(int64_t H, int64_t F) {
    StackPlan p;
    return stack_plan(H, F, cu_count(), p);
}

// [descriptors] [failure record: 256 bytes] [published hidden: kStackMaxH pairs]
size_t stack_ws_bytes() { return sizeof(bitnet_ffn_layer) * kStackMaxLayers + 256 + sizeof(uint2) * kStackMaxH; }

int stack_max_layers() { return kStackMaxLayers; }

hipError_t launch_stack(const bitnet_ffn_layer* layers, int n_layers, float* hidden, int64_t H, int64_t F,
                        bool pre, bool residual, float eps, float* y1, void* ws, hipStream_t s) {
    const int64_t nwg = cu_count();
    StackPlan p;
    if (n_layers < 1 || n_layers > kStackMaxLayers || !stack_plan(H, F, nwg, p)) return hipErrorInvalidValue;
    StackLayers a{};
    for (int i = 0; i < n_layers; ++i) a.l[i] = layers[i];
    char* w = static_cast<char*>(ws);
    bitnet_ffn_layer* layers_dev = reinterpret_cast<bitnet_ffn_layer*>(w);
    uint32_t* failed = reinterpret_cast<uint32_t*>(w + sizeof(bitnet_ffn_layer) * kStackMaxLayers);
    uint2* hx = reinterpret_cast<uint2*>(w + sizeof(bitnet_ffn_layer) * kStackMaxLayers + 256);
    uint32_t* y1x = reinterpret_cast<uint32_t*>(y1);
    hipLaunchKernelGGL(k_stack_prep, dim3(1), dim3(1024), 0, s, a, n_layers, layers_dev, failed, hx, (int)H, y1x,
                       (int)F);
    const size_t lds = (size_t)(H > F ? H : F) + (size_t)p.ut * kSW * 16 * sizeof(int);
#define BL_STK(NVH, NVF, VF, QU, QD, UT)                                                                       \
    if (p.nvh == NVH && p.nvf == NVF && p.vf == VF && p.qu == QU && p.qd == QD && p.ut == UT) {               \
        hipLaunchKernelGGL((k_stack<NVH, NVF, VF, QU, QD, UT>), dim3((unsigned)nwg), dim3(kST), lds, s,        \
                           layers_dev, n_layers, hidden, (int)H, (int)F, pre ? 1 : 0, residual ? 1 : 0, eps, y1x, \
                           hx, failed);                                                                          \
        return hipGetLastError();                                                                                \
    }
    BL_STK(3, 4, 512, 2, 4, 2)
    BL_STK(3, 4, 512, 2, 4, 1)
    BL_STK(1, 1, 256, 1, 1, 1)
    BL_STK(1, 2, 256, 1, 1, 1)
#undef BL_STK
    return hipErrorInvalidValue;
}

}  // namespace bl
