// Skinny contractions for decode and batched decode (M <= 64 tokens)
// (transformers "BitNet" page, "Model details" / Quantization: W1.58A8,
// int8 activations times ternary weights).  The work is a stream of packed
// weights against a few KB of activations, so it is laid out for memory
// parallelism and a short tail after the data lands:
//
//   - a workgroup owns 16 output rows (one MFMA column tile) or more; its
//     waves split K, and every lane issues its 16-byte weight loads before
//     anything that waits;
//   - the contraction runs on v_mfma_i32_16x16x64_i8 with the token rows as
//     the 16-row A operand: rows past M are don't-care (their outputs are
//     dropped), so one instruction serves 1..16 tokens; the MFMA does the
//     k-reduction, and expanding 16 weights costs one shift + mask per 4;
//   - lane (n, g) holds the whole 64-weight chunk 4s + g of row n (one 16-byte
//     load) and feeds its four 32-bit words to four MFMAs; the packed layout
//     puts chunk c of a 16-row tile's rows side by side (byte 16 (c R + n) of
//     the tile, R its row count), so the 16 adjacent lanes of a load read 256
//     contiguous bytes; the activation
//     operand of lane (m, g) is the matching 16 bytes of row m, so both
//     operands follow the same permutation of k and the sum is unchanged;
//   - per-wave partial tiles meet in LDS in a fixed wave order (exact integer
//     sums), then the epilogue subtracts the row sum of the code offset,
//     dequantises and applies ReLU^2 and the residual add or gating product.
//
// k_decode (M <= 4) takes fp32 rows that every workgroup quantises itself
// into LDS (the same quant_row_* as the standalone quantiser, so the same
// int8 values), which removes the quantiser launch from the decode chain.
// k_batch (M <= 64) takes the standalone quantiser's int8 rows.
#include <atomic>

#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// QMAX 16-byte weight chunks per lane; the fp32 activation row takes NV
// float4 per thread (quant_row_*: K <= 4 * NT * NV; NV is the quantiser's
// depth for K, at most QMAX by the plan below).  GATED: a second matrix Wg
// (the gate) of the same shape is streamed by the same lanes against the
// same quantised rows, and the output is ReLU^2(gate) * up (Wp is up).
template <int NWV, int QMAX, bool GATED, int NV>
__global__ __launch_bounds__(NWV* kWave) void k_decode(const float* __restrict__ X, int M, int K, int rmsnorm,
                                                        const float* __restrict__ gain, float eps,
                                                        const uint8_t* __restrict__ Wp,
                                                        const float* __restrict__ w_scale, int N,
                                                        uint32_t epi_flags, const float* aux, float* Y,
                                                        const uint8_t* __restrict__ Wg,
                                                        const float* __restrict__ g_scale) {
    constexpr int CT = 1;  // one 16-row output tile per workgroup
    static_assert(4 * 16 * CT <= NWV * kWave, "one epilogue thread per output");
    constexpr int NT = NWV * kWave;
    constexpr int COLS = 16 * CT;
    extern __shared__ __align__(16) int8_t lds[];  // [xq: M <= 4 rows of K] [partials]
    __shared__ double dslot[NWV];
    __shared__ float fslot[NWV], fslot2[NWV];
    __shared__ int islot[4][NWV];
    __shared__ float gx[4];

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int fr = lane & 15;      // column (output row) of the tile / activation row of the A operand
    const int fg = lane >> 4;      // k group
    const int n0 = blockIdx.x * COLS;
    const int C = K / 64;          // 64-weight chunks per row
    const int nq = (C + 3) / 4;    // chunk quads
    const float ws = *w_scale;
    const float gws = GATED ? *g_scale : 0.0f;

    // ---- every load up front, in the order they are needed: the first fp32
    // activation row (and the norm gain), the weights, then the epilogue's
    // operand for this thread's output.
    float4 v[NV], gv[NV];
    const bool has_gain = rmsnorm != 0 && gain != nullptr;
    quant_row_load<NT, NV>(X, has_gain ? gain : nullptr, K, v, gv);
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weights'
    uint4 w[CT][QMAX];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int r0 = n0 + 16 * ct;
        // readfirstlane: a clamp left in a VGPR would make the descriptor look
        // divergent (and every load a waterfall loop)
        const int rows = __builtin_amdgcn_readfirstlane(N - r0 < 0 ? 0 : (N - r0 < 16 ? N - r0 : 16));
        const Rsrc rw = make_rsrc(Wp + (int64_t)(rows > 0 ? r0 : 0) * (K / 4), (uint32_t)rows * (uint32_t)(K / 4));
#pragma unroll
        for (int i = 0; i < QMAX; ++i) {
            const int s = wave + i * NWV;
            const int c = 4 * s + fg;
            w[ct][i] = buf_load16(rw, (s < nq && c < C) ? (uint32_t)(c * rows + fr) * 16u : kOob);
        }
    }
    uint4 wg[GATED ? QMAX : 1];
    if constexpr (GATED) {
        const int rows = N - n0 < 16 ? N - n0 : 16;
        const Rsrc rg = make_rsrc(Wg + (int64_t)n0 * (K / 4), (uint32_t)rows * (uint32_t)(K / 4));
#pragma unroll
        for (int i = 0; i < QMAX; ++i) {
            const int s = wave + i * NWV;
            const int c = 4 * s + fg;
            wg[i] = buf_load16(rg, (s < nq && c < C) ? (uint32_t)(c * rows + fr) * 16u : kOob);
        }
    }
    const int e_m = threadIdx.x / COLS, e_n = n0 + (int)(threadIdx.x % COLS);
    const bool e_ok = (int)threadIdx.x < M * COLS && e_n < N;
    const float e_res = buf_load4f(make_rsrc(aux, (epi_flags & (kEpiResidual | kEpiMul)) ? 0x7FFFFFFFu : 0u),
                                   e_ok ? (uint32_t)((int64_t)e_m * N + e_n) * 4u : kOob);

    // ---- activation rows, quantised here.  Row 0 unconditionally (the host
    // launches with M >= 1): a guard would let the compiler sink its loads
    // behind the weights'.
    int8_t* xq = lds;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if (m == 0 || m < M) {
            if (m > 0) {
                __syncthreads();  // the reduction slots are reused
                quant_row_load_x<NT, NV>(X + (int64_t)m * K, K, v);
            }
            const float g = quant_row_finish<NT, NV>(v, gv, K, rmsnorm != 0, has_gain, eps, xq + m * K, dslot,
                                                       fslot, fslot2, islot[m]);
            if (threadIdx.x == 0) gx[m] = g;
        }
    }
    __syncthreads();
    const int8_t* arow = xq + (fr < M ? fr : M - 1) * K;

    // ---- contraction.  A chunk past the row end has zero weights (its load
    // was out of range), so its activation offset is clamped to 0 and it adds
    // nothing.
    v4i acc[CT], accg = v4i{0, 0, 0, 0};
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < QMAX; ++i) {
        const int s = wave + i * NWV;
        if (s < nq) {
            const int c = 4 * s + fg;
            const int koff = c < C ? 64 * c : 0;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const v4i a = *reinterpret_cast<const v4i*>(arow + koff + 16 * d);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const uint32_t wd = d == 0 ? w[ct][i].x : d == 1 ? w[ct][i].y : d == 2 ? w[ct][i].z : w[ct][i].w;
                    const v4i b = v4i{codes4(wd, 0), codes4(wd, 1), codes4(wd, 2), codes4(wd, 3)};
                    acc[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[ct], 0, 0, 0);
                }
                if constexpr (GATED) {
                    const uint32_t g4 = d == 0 ? wg[i].x : d == 1 ? wg[i].y : d == 2 ? wg[i].z : wg[i].w;
                    const v4i bg = v4i{codes4(g4, 0), codes4(g4, 1), codes4(g4, 2), codes4(g4, 3)};
                    accg = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bg, accg, 0, 0, 0);
                }
            }
        }
    }

    // ---- per-wave partial tiles -> LDS (a region of its own) -> epilogue,
    // summing the waves in index order
    int* red = reinterpret_cast<int*>(lds + 4 * K);  // [NWV][16 tokens][COLS], gate after it
    int* redg = red + NWV * 16 * 16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * fg + r;
        if (m < M) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) red[(wave * 16 + m) * COLS + 16 * ct + fr] = acc[ct][r];
            if constexpr (GATED) redg[(wave * 16 + m) * 16 + fr] = accg[r];
        }
    }
    __syncthreads();
    if (e_ok) {
        const int m = e_m, col = (int)threadIdx.x % COLS;
        int a = 0, ag = 0;
#pragma unroll
        for (int q = 0; q < NWV; ++q) a += red[(q * 16 + m) * COLS + col];
        if constexpr (GATED) {
#pragma unroll
            for (int q = 0; q < NWV; ++q) ag += redg[(q * 16 + m) * 16 + col];
        }
        int rs = 0;
#pragma unroll
        for (int q = 0; q < NWV; ++q) rs += islot[m][q];
        const float xs = gx[m];
        a -= rs;
        const float d = (xs * ws) / 127.0f;
        float y = (float)a * d;
        const int64_t o = (int64_t)m * N + e_n;
        if constexpr (GATED) {
            // ReLU^2(gate) * up, in that order
            ag -= rs;
            float t = (float)ag * ((xs * gws) / 127.0f);
            t = t > 0.0f ? t : 0.0f;
            y = (t * t) * y;
        } else {
            if (epi_flags & kEpiRelu2) {
                const float tt = y > 0.0f ? y : 0.0f;
                y = tt * tt;
            }
            if (epi_flags & kEpiMul) y = y * e_res;
            else if (epi_flags & kEpiResidual) y = y + e_res;
        }
        Y[o] = y;
    }
}

// Very tall matrices (thousands of 16-row tiles, e.g. an output layer over a
// large vocabulary), M <= 4, no gate: a persistent launch of about as many
// workgroups as fit on the device at once.  Each quantises the rows once
// (as k_decode does) and then walks the groups of CT tiles g = blockIdx.x,
// blockIdx.x + gridDim.x, ...; the weight loads (and epilogue operand) of
// the next group go out before the current group's MFMAs and epilogue, so
// every workgroup keeps one group in flight while it works and the launch
// streams the matrix with no second round of workgroups.
constexpr bool kStreamNT = true;  // non-temporal weight loads in the streaming launch

template <int NWV, int NV, int CT>
__global__ __launch_bounds__(NWV* kWave) void k_decode_stream(const float* __restrict__ X, int M, int K,
                                                               int rmsnorm, const float* __restrict__ gain,
                                                               float eps, const uint8_t* __restrict__ Wp,
                                                               const float* __restrict__ w_scale, int N,
                                                               uint32_t epi_flags, const float* aux, float* Y) {
    static_assert(4 * 16 * CT <= NWV * kWave, "one epilogue thread per output");
    constexpr int NT = NWV * kWave;
    constexpr int COLS = 16 * CT;
    // Chunk quads per wave: K <= 4 NT NV = 256 NWV NV, so NV covers them.
    constexpr int QMAX = NV;
    extern __shared__ __align__(16) int8_t lds[];  // [xq: M <= 4 rows of K] [partials]
    __shared__ double dslot[NWV];
    __shared__ float fslot[NWV], fslot2[NWV];
    __shared__ int islot[4][NWV];
    __shared__ float gx[4];

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int fr = lane & 15;
    const int fg = lane >> 4;
    const int C = K / 64;
    const int groups = (N + COLS - 1) / COLS;
    const float ws = *w_scale;
    const bool has_aux = (epi_flags & (kEpiResidual | kEpiMul)) != 0;
    const Rsrc raux = make_rsrc(aux, has_aux ? 0x7FFFFFFFu : 0u);
    const int e_m = threadIdx.x / COLS, e_col = (int)threadIdx.x % COLS;

    // This lane's chunk c of load i (quad wave + i NWV): byte offset 16 (c R
    // + fr) in a tile of R rows; past the row the top bit puts it past every
    // descriptor, so the load returns zeros (and adds nothing).
    uint32_t c16[QMAX], oob[QMAX];
#pragma unroll
    for (int i = 0; i < QMAX; ++i) {
        const int c = 4 * (wave + i * NWV) + fg;
        c16[i] = 16u * (uint32_t)c;
        oob[i] = c < C ? 0u : kOob;
    }
    // Weights of group g (a group past the matrix reads nothing: zero rows)
    // and this thread's epilogue operand for it.  Straight-line: no load
    // sits under a branch, so the loads of the next group can stay in
    // flight while the current one is contracted.
    auto load_group = [&](int g, uint4 (&w)[CT][QMAX], float& res) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int r0 = g * COLS + 16 * ct;
            const int rows = __builtin_amdgcn_readfirstlane(N - r0 < 0 ? 0 : (N - r0 < 16 ? N - r0 : 16));
            const Rsrc rw = make_rsrc(Wp + (int64_t)(rows > 0 ? r0 : 0) * (K / 4), (uint32_t)rows * (uint32_t)(K / 4));
#pragma unroll
            for (int i = 0; i < QMAX; ++i)
                w[ct][i] = kStreamNT ? buf_load16_nt(rw, (c16[i] * (uint32_t)rows + 16u * (uint32_t)fr) | oob[i])
                                     : buf_load16(rw, (c16[i] * (uint32_t)rows + 16u * (uint32_t)fr) | oob[i]);
        }
        const int e_n = g * COLS + e_col;
        const bool ok = (int)threadIdx.x < M * COLS && e_n < N;
        res = buf_load4f(raux, ok ? (uint32_t)((int64_t)e_m * N + e_n) * 4u : kOob);
    };

    float4 v[NV], gv[NV];
    const bool has_gain = rmsnorm != 0 && gain != nullptr;
    quant_row_load<NT, NV>(X, has_gain ? gain : nullptr, K, v, gv);
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weights'
    uint4 wa[CT][QMAX], wb[CT][QMAX];
    float ra, rb;
    int g = blockIdx.x;
    load_group(g, wa, ra);

    int8_t* xq = lds;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if (m == 0 || m < M) {
            if (m > 0) {
                __syncthreads();  // the reduction slots are reused
                quant_row_load_x<NT, NV>(X + (int64_t)m * K, K, v);
            }
            const float gq = quant_row_finish<NT, NV>(v, gv, K, rmsnorm != 0, has_gain, eps, xq + m * K, dslot,
                                                        fslot, fslot2, islot[m]);
            if (threadIdx.x == 0) gx[m] = gq;
        }
    }
    __syncthreads();
    const int8_t* arow = xq + (fr < M ? fr : M - 1) * K;
    int rs_m = 0;
    float d_m = 0.0f;
    if ((int)threadIdx.x < M * COLS) {
#pragma unroll
        for (int q = 0; q < NWV; ++q) rs_m += islot[e_m][q];
        d_m = (gx[e_m] * ws) / 127.0f;
    }
    int* red = reinterpret_cast<int*>(lds + 4 * K);  // [NWV][16 tokens][COLS]

    // One group: contraction, per-wave partial tiles summed in wave order,
    // epilogue.  Ends with a barrier, so the next group may reuse `red`.
    auto process = [&](int gg, const uint4 (&w)[CT][QMAX], float res) {
        v4i acc[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[ct] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < QMAX; ++i) {
            // every load is consumed (a wave short of quads multiplies zeros),
            // so no use of a load sits under a branch
            const int c = 4 * (wave + i * NWV) + fg;
            const int koff = c < C ? 64 * c : 0;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const v4i a = *reinterpret_cast<const v4i*>(arow + koff + 16 * d);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const uint32_t wd = d == 0 ? w[ct][i].x : d == 1 ? w[ct][i].y : d == 2 ? w[ct][i].z : w[ct][i].w;
                    const v4i b = v4i{codes4(wd, 0), codes4(wd, 1), codes4(wd, 2), codes4(wd, 3)};
                    acc[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[ct], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * fg + r;
            if (m < M) {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) red[(wave * 16 + m) * COLS + 16 * ct + fr] = acc[ct][r];
            }
        }
        __syncthreads();
        const int e_n = gg * COLS + e_col;
        if ((int)threadIdx.x < M * COLS && e_n < N) {
            int a = 0;
#pragma unroll
            for (int q = 0; q < NWV; ++q) a += red[(q * 16 + e_m) * COLS + e_col];
            a -= rs_m;
            float y = (float)a * d_m;
            if (epi_flags & kEpiRelu2) {
                const float tt = y > 0.0f ? y : 0.0f;
                y = tt * tt;
            }
            if (epi_flags & kEpiMul) y = y * res;
            else if (epi_flags & kEpiResidual) y = y + res;
            Y[(int64_t)e_m * N + e_n] = y;
        }
        __syncthreads();
    };

    // Two register sets alternate: while one group is contracted the next
    // group's loads are in flight.
    while (true) {
        load_group(g + (int)gridDim.x, wb, rb);
        process(g, wa, ra);
        g += gridDim.x;
        if (g >= groups) break;
        load_group(g + (int)gridDim.x, wa, ra);
        process(g, wb, rb);
        g += gridDim.x;
        if (g >= groups) break;
    }
}

// int8 rows from the standalone quantiser, M <= 64 tokens (batched decode).
// A workgroup owns 16 * CT output rows (CT column tiles) and all M tokens
// (MT token tiles of 16).  Its four waves split K in chunk quads (256 k),
// quad s going to wave s % 4, so a wave has Q or Q - 1 of them; every wave
// runs the same straight-line body of Q steps, and a missing last quad reads
// nothing (out-of-range offsets) and adds zeros.  Weights go to registers
// (every load issued first, as in k_decode).  Activations are the part that needs
// care: every workgroup reads all M x K of them from L2, and the MFMA
// operand layout (lane = token row) makes a direct load touch one cache line
// per lane, which the address unit serves at about a quarter of its rate.
// So they travel by direct buffer->LDS loads in whole-line order: one DMA
// instruction moves 8 rows x 128 bytes, adjacent lanes on adjacent 16-byte
// chunks, into a ring of NS stages private to the wave (no barrier in the
// loop); the operand reads then pick the MFMA layout out of LDS.  Inside a
// DMA block the chunk cc of row r lands at slot cc ^ (r / 2) (r = row of the
// 16-row tile, 3 bits), which keeps the 16 rows of an operand read on 16
// distinct bank groups.  Each operand fragment feeds all CT column tiles.
// A row past M or a chunk past the row end loads zeros or stale bytes: its
// outputs are dropped, or its weights are zero.
constexpr int kBatchWaves = 4;
constexpr int kTileBytes = 16 * 256;  // one token tile x one chunk quad
constexpr int kMaxGroups = 4;         // matrices per grouped launch

// s_waitcnt vmcnt(n) for a count that is a constant once the caller's loop
// is unrolled (the chain of ifs folds to one instruction); n <= 63.
template <int N = 63>
__device__ __forceinline__ void wait_vm_n(int n) {
    if constexpr (N > 0) {
        if (n >= N) {
            wait_vm<N>();
            return;
        }
        wait_vm_n<N - 1>(n);
    } else {
        wait_vm<0>();
    }
}

// Loads a wave issues after quad i's DMAs and before its wait for quad i,
// in the issue order of batch_body: (DMAs of quad j, weights of quad j) for
// j < NS - 1, then the remaining weights; iteration j of the loop then adds
// the DMAs of quad j + NS - 1.
constexpr int batch_loads_after(int i, int Q, int NS, int MT, int CT, bool H8) {
    const int dma = H8 ? 2 : 4 * MT;
    if (i <= NS - 2) {
        const int last_pro = NS - 2 < Q - 1 ? NS - 2 : Q - 1;
        const int rest = Q - (NS - 1) > 0 ? Q - (NS - 1) : 0;
        return CT + (last_pro - i) * (dma + CT) + CT * rest + (i < rest ? i : rest) * dma;
    }
    const int hi = Q - 1 < i + NS - 2 ? Q - 1 : i + NS - 2;
    return (hi - i) * dma;
}

// H8 (one token tile, M <= 8): only the tile's first 8 rows are moved; the
// other half of each stage is never written, and the operands read from it
// feed only outputs of rows past M, which are never stored.
template <int MT, int CT, int NS, int Q, bool H8>
__device__ __forceinline__ void batch_body(Rsrc ra, const uint32_t (&voff)[MT][2], const Rsrc (&rw)[CT],
                                           const int (&rows)[CT], int wave, int fr, int fg, int C, int nq,
                                           int8_t* ring, const uint32_t (&rd)[4], v4i (&acc)[CT][MT]) {
    constexpr int SB = MT * kTileBytes;  // bytes per stage
    uint4 w[CT][Q];
#define BL_WT(ii)                                                                                  \
    do {                                                                                           \
        const int c_ = 4 * (wave + (ii) * kBatchWaves) + fg;                                       \
        _Pragma("unroll") for (int ct = 0; ct < CT; ++ct)                                          \
            w[ct][ii] = buf_load16_nt(rw[ct], c_ < C ? (uint32_t)(c_ * rows[ct] + fr) * 16u : kOob); \
    } while (0)
    // quad i (the wave's i-th) -> stage i % NS: per token tile, 4 DMAs of 8 rows x 128 bytes
#define BL_DMA(ii)                                                                                        \
    do {                                                                                                  \
        const int s_ = wave + (ii) * kBatchWaves;                                                         \
        /* past every row for a missing quad (and no wrap when added to a kOob lane offset) */           \
        const uint32_t k0 = s_ < nq ? 256u * (uint32_t)s_ : 0x40000000u;                                  \
        int8_t* st_ = ring + ((ii) % NS) * SB;                                                            \
        _Pragma("unroll") for (int t = 0; t < MT; ++t)                                                    \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                     \
            if (!H8 || (j & 1) == 0)                                                                      \
                dma16(ra, (lds_ptr)(st_ + t * kTileBytes + j * 1024), voff[t][j & 1], k0 + 128u * (uint32_t)(j >> 1)); \
    } while (0)
    // issue order (pinned: the waits below count loads): each of the first
    // NS - 1 quads' DMAs then its weights, then the other weights.  Loads
    // complete in issue order, so the wait for quad i's activations leaves
    // its weights and every later load in flight (the MFMAs wait for the
    // weights they use).
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
        if (i < Q) {
            BL_DMA(i);
            __builtin_amdgcn_sched_barrier(0);
            BL_WT(i);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
    for (int i = NS - 1; i < Q; ++i) BL_WT(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < Q; ++i) {
        // quad i's activations have landed once only later loads are in flight
        wait_vm_n(batch_loads_after(i, Q, NS, MT, CT, H8));
        __builtin_amdgcn_sched_barrier(0);
        // all of quad i's operand fragments, then the DMA that refills the
        // stage read one step earlier (with every read in flight issued
        // before it, the compiler's own wait for LDS written by DMA is the
        // one above), then the MFMAs
        const int8_t* st = ring + (i % NS) * SB;
        v4i a[4][MT];
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int t = 0; t < MT; ++t) a[d][t] = *reinterpret_cast<const v4i*>(st + t * kTileBytes + rd[d]);
        __builtin_amdgcn_sched_barrier(0);
        if (i + NS - 1 < Q) BL_DMA(i + NS - 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const uint32_t wd = d == 0 ? w[ct][i].x : d == 1 ? w[ct][i].y : d == 2 ? w[ct][i].z : w[ct][i].w;
                const v4i b = v4i{codes4(wd, 0), codes4(wd, 1), codes4(wd, 2), codes4(wd, 3)};
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[ct][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[d][t], b, acc[ct][t], 0, 0, 0);
            }
        __builtin_amdgcn_sched_barrier(0);
    }
#undef BL_DMA
#undef BL_WT
}

// A launch may stream several weight matrices of the same K against the
// same int8 rows (a grouped launch: e.g. q, k and v, each with its own
// per-tensor scale): matrix i takes the workgroups from wg0 on, each with its
// own scale, output, epilogue and accumulator output.
struct BatchMat {
    const uint8_t* W;
    const float* w_scale;
    const float* aux;
    float* Y;
    int32_t* acc_out;
    int N;
    uint32_t epi_flags;
    int wg0;
};
struct BatchMats {
    BatchMat m[kMaxGroups];
    int count;
};

// GATED (CT = 2, one matrix): the two column tiles are the same 16 output
// rows of the up matrix (tile 0) and of the gate matrix Wg (tile 1), sharing
// every activation fragment, and the output is ReLU^2(gate) * up.
template <int MT, int CT, int NS, int QMAX, bool GATED = false, bool H8 = false>
__global__ __launch_bounds__(kBatchWaves* kWave) void k_batch(const int8_t* __restrict__ Xq,
                                                               const float* __restrict__ x_scale,
                                                               const int32_t* __restrict__ x_rowsum, int M, int K,
                                                               const BatchMats mats,
                                                               const uint8_t* __restrict__ Wg,
                                                               const float* __restrict__ g_scale) {
    static_assert(!GATED || CT == 2, "a gated tile pairs one up and one gate tile");
    static_assert(!H8 || MT == 1, "the half-tile copy is for one token tile");
    constexpr int NWV = kBatchWaves;
    constexpr int NT = NWV * kWave;
    constexpr int COLS = 16 * CT;                        // accumulated columns per workgroup
    constexpr int OCOLS = GATED ? 16 : COLS;             // output columns per workgroup
    constexpr int GROUPS = 16 * MT * OCOLS / 4;         // epilogue: 4 adjacent outputs of one row per group
    constexpr int EPG = (GROUPS + NT - 1) / NT;          // groups per thread
    constexpr int RING = NS * MT * kTileBytes;           // bytes per wave
    static_assert(NWV * 16 * MT * COLS * 4 <= NWV * RING, "partial tiles fit in the rings");
    __shared__ __align__(1024) int8_t lds[NWV * RING];   // activation rings, then partial tiles [NWV][M][COLS]
    __shared__ float sdq[16 * MT];  // per-row dequantisation factor (x_scale * w_scale) / 127
    __shared__ float sdqg[GATED ? 16 * MT : 1];  // the same with the gate's scale
    __shared__ int srs[16 * MT];

    // this workgroup's matrix: the last whose first workgroup is at or before
    // it (uniform: every field is picked by a scalar select, no indexing)
    int gi = 0;
#pragma unroll
    for (int i = 1; i < kMaxGroups; ++i)
        if (i < mats.count && (int)blockIdx.x >= mats.m[i].wg0) gi = i;
    const uint8_t* Wp = mats.m[0].W;
    const float* w_scale = mats.m[0].w_scale;
    const float* aux = mats.m[0].aux;
    float* Y = mats.m[0].Y;
    int32_t* acc_out = mats.m[0].acc_out;
    int N = mats.m[0].N;
    uint32_t epi_flags = mats.m[0].epi_flags;
    int wg0 = mats.m[0].wg0;
#pragma unroll
    for (int i = 1; i < kMaxGroups; ++i)
        if (gi == i) {
            Wp = mats.m[i].W;
            w_scale = mats.m[i].w_scale;
            aux = mats.m[i].aux;
            Y = mats.m[i].Y;
            acc_out = mats.m[i].acc_out;
            N = mats.m[i].N;
            epi_flags = mats.m[i].epi_flags;
            wg0 = mats.m[i].wg0;
        }

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int fr = lane & 15;  // activation row of the A operand / output column of the tile
    const int fg = lane >> 4;  // k group
    const int n0 = ((int)blockIdx.x - wg0) * OCOLS;
    const int C = K / 64;
    const int nq = (C + 3) / 4;
    const float ws = *w_scale;
    const float gws = GATED ? *g_scale : 0.0f;

    // ---- the epilogue's operands, loaded first: the rows' scales and sums
    // (thread t < M takes row t) and the residual or multiplier of every
    // output this thread finishes (group g = threadIdx.x + e * NT covers row
    // g / (COLS / 4), columns 4 (g % (COLS / 4)) .. + 3 of the tile).
    const float p_xs = buf_load4f(make_rsrc(x_scale, (uint32_t)M * 4u), (uint32_t)threadIdx.x * 4u);
    const int p_rs = buf_load4i(make_rsrc(x_rowsum, (uint32_t)M * 4u), (uint32_t)threadIdx.x * 4u);
    float e_aux[EPG][4];
    {
        const Rsrc rx = make_rsrc(aux, (!GATED && (epi_flags & (kEpiResidual | kEpiMul))) ? 0x7FFFFFFFu : 0u);
#pragma unroll
        for (int e = 0; e < EPG; ++e) {
            const int g = threadIdx.x + e * NT;
            const int m = g / (OCOLS / 4), n = n0 + 4 * (g % (OCOLS / 4));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                e_aux[e][j] = buf_load4f(rx, (m < M && n + j < N) ? (uint32_t)((int64_t)m * N + n + j) * 4u : kOob);
        }
    }

    Rsrc rw[CT];
    int rows[CT];  // rows of each column tile's 16-row weight tile (the last may have fewer)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int r0 = GATED ? n0 : n0 + 16 * ct;
        const uint8_t* W = GATED && ct == 1 ? Wg : Wp;
        // readfirstlane: a clamp the compiler leaves in a VGPR would make the
        // descriptor look divergent (and every load a waterfall loop)
        rows[ct] = __builtin_amdgcn_readfirstlane(N - r0 < 0 ? 0 : (N - r0 < 16 ? N - r0 : 16));
        rw[ct] = make_rsrc(W + (int64_t)(rows[ct] > 0 ? r0 : 0) * (K / 4), (uint32_t)rows[ct] * (uint32_t)(K / 4));
    }
    // DMA lane offsets: lane L moves row 8h + (L >> 3) of token tile t, 16-byte
    // chunk (L & 7) ^ (row / 2) of the 128-byte span (h = half of the tile)
    const Rsrc ra = make_rsrc(Xq, (uint32_t)M * (uint32_t)K);
    uint32_t voff[MT][2];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 8 * h + (lane >> 3);
            const int m = 16 * t + r;
            voff[t][h] = m < M ? (uint32_t)m * (uint32_t)K + 16u * (uint32_t)((lane & 7) ^ (r >> 1)) : kOob;
        }
    // operand reads: row fr, k bytes 64 fg + 16 d of the quad -> DMA block
    // 2 (fg / 2) + fr / 8, lane 8 (fr % 8) + ((4 (fg % 2) + d) ^ (fr / 2))
    uint32_t rd[4];
#pragma unroll
    for (int d = 0; d < 4; ++d)
        rd[d] = 1024u * (uint32_t)(2 * (fg >> 1) + (fr >> 3)) +
                16u * (uint32_t)(8 * (fr & 7) + ((4 * (fg & 1) + d) ^ (fr >> 1)));
    int8_t* ring = lds + wave * RING;

    v4i acc[CT][MT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[ct][t] = v4i{0, 0, 0, 0};
    batch_body<MT, CT, NS, QMAX, H8>(ra, voff, rw, rows, wave, fr, fg, C, nq, ring, rd, acc);

    // ---- per-wave partial tiles -> LDS (over the rings, once every wave is
    // done with its own) -> sum over the waves in index order
    if ((int)threadIdx.x < 16 * MT) {
        sdq[threadIdx.x] = (p_xs * ws) / 127.0f;
        if constexpr (GATED) sdqg[threadIdx.x] = (p_xs * gws) / 127.0f;
        srs[threadIdx.x] = p_rs;
    }
    __syncthreads();
    int* red = reinterpret_cast<int*>(lds);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * t + 4 * fg + r;
                if (m < M) red[(wave * M + m) * COLS + 16 * ct + fr] = acc[ct][t][r];
            }
    __syncthreads();
    // all partial-tile reads first (16 bytes: 4 adjacent columns), then the
    // arithmetic; a group past M reads row M - 1 and stores nothing
    int4 part[EPG][NWV], partg[GATED ? EPG : 1][NWV];
#pragma unroll
    for (int e = 0; e < EPG; ++e) {
        const int g = threadIdx.x + e * NT;
        const int m = g / (OCOLS / 4) < M ? g / (OCOLS / 4) : M - 1;
        const int c = 4 * (g % (OCOLS / 4));
#pragma unroll
        for (int q = 0; q < NWV; ++q) part[e][q] = *reinterpret_cast<const int4*>(red + (q * M + m) * COLS + c);
        if constexpr (GATED) {
#pragma unroll
            for (int q = 0; q < NWV; ++q)
                partg[e][q] = *reinterpret_cast<const int4*>(red + (q * M + m) * COLS + 16 + c);
        }
    }
    const bool vec = (N & 3) == 0;  // rows start 16-byte aligned
#pragma unroll
    for (int e = 0; e < EPG; ++e) {
        const int g = threadIdx.x + e * NT;
        const int m = g / (OCOLS / 4);
        const int n = n0 + 4 * (g % (OCOLS / 4));
        if (m < M && n < N) {
            int a[4] = {0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < NWV; ++q) {
                a[0] += part[e][q].x;
                a[1] += part[e][q].y;
                a[2] += part[e][q].z;
                a[3] += part[e][q].w;
            }
            const int rsum = srs[m];
            const float dq = sdq[m];
            float y[4];
            if constexpr (GATED) {
                int ag[4] = {0, 0, 0, 0};
#pragma unroll
                for (int q = 0; q < NWV; ++q) {
                    ag[0] += partg[e][q].x;
                    ag[1] += partg[e][q].y;
                    ag[2] += partg[e][q].z;
                    ag[3] += partg[e][q].w;
                }
                const float dqg = sdqg[m];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // ReLU^2(gate) * up, in that order
                    a[j] -= rsum;
                    const float u = (float)a[j] * dq;
                    float t = (float)(ag[j] - rsum) * dqg;
                    t = t > 0.0f ? t : 0.0f;
                    y[j] = (t * t) * u;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    a[j] -= rsum;
                    float v = (float)a[j] * dq;
                    if (epi_flags & kEpiRelu2) {
                        const float tt = v > 0.0f ? v : 0.0f;
                        v = tt * tt;
                    }
                    if (epi_flags & kEpiMul) v = v * e_aux[e][j];
                    else if (epi_flags & kEpiResidual) v = v + e_aux[e][j];
                    y[j] = v;
                }
            }
            const int64_t o = (int64_t)m * N + n;
            if (vec) {  // n + 3 < N as well
                if (Y != nullptr) *reinterpret_cast<float4*>(Y + o) = make_float4(y[0], y[1], y[2], y[3]);
                if (acc_out != nullptr) *reinterpret_cast<int4*>(acc_out + o) = make_int4(a[0], a[1], a[2], a[3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (n + j < N) {
                        if (Y != nullptr) Y[o + j] = y[j];
                        if (acc_out != nullptr) acc_out[o + j] = a[j];
                    }
            }
        }
    }
}

// Activation-stationary batched BitLinear (M <= 32 tokens, K <= 2560): every
// workgroup copies all M rows of int8 activations into LDS once (MT * 16 * K
// bytes, at most the whole 160 KB), then each wave contracts whole 16-row
// weight tiles over the full K by itself, one tile after another, with no
// cross-wave reduction and no barrier after the copy.  For launches of many
// tiles (a grouped launch of several matrices: q, k and v, or o, gate and
// up) this replaces the per-workgroup activation stream of k_batch, whose
// cost is M * K bytes through the CU for every 16 or 32 output rows, by one
// copy per CU.
//   LDS layout: row r of the activations at r * K, its 16-byte chunk j at
//   slot j ^ (r % 16) inside each whole group of 16 chunks (j ^ (r % 8) in a
//   last group of 8), so the 16 rows an operand read takes at one k fall on
//   distinct banks.  The copy is direct
//   buffer->LDS: instruction i fills LDS bytes [1024 i, 1024 i + 1024), each
//   lane fetching the global chunk that its slot holds.
//   A wave's tile: lane (fr, fg) loads chunk 4s + fg of weight row fr for
//   every quad s (all loads first); the A operand of MFMA (s, d) for token
//   tile t is row 16 t + fr, bytes 64 (4 s + fg) + 16 d.
constexpr int kStatLds = 160 * 1024;
constexpr int kStatWaves = 4;

// Byte offset of (row r, 16-byte chunk j) of the activation copy in LDS; nch
// chunks per row (K / 16), swizzled only inside whole groups of 16 (or of 8
// at the end of a row).  The map is its own inverse: a chunk and its image
// lie in the same group.
__device__ __forceinline__ uint32_t stat_slot(uint32_t r, uint32_t j, uint32_t K, uint32_t nch) {
    const uint32_t sj = ((j | 15u) < nch) ? (j ^ (r & 15u)) : ((j | 7u) < nch) ? (j ^ (r & 7u)) : j;
    return r * K + 16u * sj;
}

// One matrix of a grouped launch, as seen by the tile that works on it.
struct StatTile {
    const uint8_t* W;
    const float* w_scale;
    const float* aux;
    float* Y;
    int32_t* acc_out;
    int N;
    uint32_t epi_flags;
    int n0;    // first output row of the tile
    int rows;  // its rows (16, or fewer in a matrix's last tile)
};

// The matrix tile `tile` (counted over all matrices) belongs to: the last
// whose first tile (wg0) is at or before it; every field picked by a scalar
// select (the tile index is uniform), no indexing into the argument block.
__device__ __forceinline__ StatTile stat_tile(const BatchMats mats, int tile) {
    int gi = 0;
#pragma unroll
    for (int i = 1; i < kMaxGroups; ++i)
        if (i < mats.count && tile >= mats.m[i].wg0) gi = i;
    StatTile t{mats.m[0].W, mats.m[0].w_scale, mats.m[0].aux, mats.m[0].Y, mats.m[0].acc_out,
               mats.m[0].N, mats.m[0].epi_flags, mats.m[0].wg0, 0};
#pragma unroll
    for (int i = 1; i < kMaxGroups; ++i)
        if (gi == i)
            t = StatTile{mats.m[i].W, mats.m[i].w_scale, mats.m[i].aux, mats.m[i].Y, mats.m[i].acc_out,
                         mats.m[i].N, mats.m[i].epi_flags, mats.m[i].wg0, 0};
    t.n0 = (tile - t.n0) * 16;
    t.rows = __builtin_amdgcn_readfirstlane(t.N - t.n0 < 16 ? t.N - t.n0 : 16);
    return t;
}

template <int QMAX>
__device__ __forceinline__ void stat_load_weights(const uint8_t* W, int n0, int rows, int K, int C, int nq, int fr,
                                                  int fg, uint4 (&w)[QMAX]) {
    const Rsrc rw = make_rsrc(W + (int64_t)n0 * (K / 4), (uint32_t)rows * (uint32_t)(K / 4));
#pragma unroll
    for (int s = 0; s < QMAX; ++s) {
        const int c = 4 * s + fg;
        w[s] = buf_load16_nt(rw, (s < nq && c < C) ? (uint32_t)(c * rows + fr) * 16u : kOob);
    }
}

// The rows to quantise inside the launch (fp32, the quantiser's optional
// RMSNorm), or X == nullptr when the launch reads int8 rows.
struct StatQuant {
    const float* X;     // [M][K]
    const float* gain;  // [K] or nullptr
    float eps;
    int rms;
};

// One row as the 256-thread quantiser holds it, in one wave: lane l plays
// threads l + 64 u (u < 4), each with its float4 indices t + 256 i (i < NV).
template <int NV>
__device__ __forceinline__ void wrow_load(const float* X, int K, float4 (&v)[4][NV]) {
    const int lane = threadIdx.x % kWave;
    const Rsrc rx = make_rsrc(X, X != nullptr ? (uint32_t)K * 4u : 0u);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < NV; ++i) v[u][i] = buf_load16f(rx, (uint32_t)(lane + 64 * u + 256 * i) * 16u);
}

// quant_row_finish for NT = 256, run by one wave for row r of the copy: the
// same per-thread order, the same DPP tree per played wave and the four wave
// sums added in index order, so the same bits as the standalone quantiser.
// The int8 row goes into the copy's slots (float4 f = four bytes of chunk
// f / 4), gamma and the int8 row sum into s_xs[r], s_rs[r].
template <int NV>
__device__ __forceinline__ void wrow_quant(float4 (&v)[4][NV], const float4 (&gv)[4][NV], int K, bool rms,
                                           bool has_gain, float eps, int r, int8_t* act, uint32_t nch, float* s_xs,
                                           int* s_rs) {
    const int lane = threadIdx.x % kWave;
    const int n4 = K / 4;
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < NV; ++i)
            amax = fmaxf(fmaxf(amax, fmaxf(fabsf(v[u][i].x), fabsf(v[u][i].y))),
                         fmaxf(fabsf(v[u][i].z), fabsf(v[u][i].w)));
    float g;
    if (rms) {
        double t = 0.0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            double ss = 0.0;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                ss = __builtin_fma((double)v[u][i].x, (double)v[u][i].x, ss);
                ss = __builtin_fma((double)v[u][i].y, (double)v[u][i].y, ss);
                ss = __builtin_fma((double)v[u][i].z, (double)v[u][i].z, ss);
                ss = __builtin_fma((double)v[u][i].w, (double)v[u][i].w, ss);
            }
            t += wave_sum(ss);
        }
        const float rr = (float)(1.0 / sqrt(t / (double)K + (double)eps));
        float az = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                float4 z = v[u][i];
                z.x = z.x * rr;
                z.y = z.y * rr;
                z.z = z.z * rr;
                z.w = z.w * rr;
                if (has_gain) {
                    z.x = z.x * gv[u][i].x;
                    z.y = z.y * gv[u][i].y;
                    z.z = z.z * gv[u][i].z;
                    z.w = z.w * gv[u][i].w;
                    az = fmaxf(fmaxf(az, fmaxf(fabsf(z.x), fabsf(z.y))), fmaxf(fabsf(z.z), fabsf(z.w)));
                }
                v[u][i] = z;
            }
        g = has_gain ? wave_max(az) : wave_max(amax) * rr;
    } else {
        g = wave_max(amax);
    }
    if (!(g >= 1e-5f)) g = 1e-5f;
    const float sc = 127.0f / g;
    int sum = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int f = lane + 64 * u + 256 * i;
            const uint32_t packed = quant4(v[u][i], sc);
            sum = __builtin_amdgcn_sdot4((int)packed, 0x01010101, sum, false);  // slots past the row hold 0
            if (f < n4)
                *reinterpret_cast<uint32_t*>(act + stat_slot((uint32_t)r, (uint32_t)f / 4u, (uint32_t)K, nch) +
                                             4 * (f % 4)) = packed;
        }
    sum = wave_sum(sum);
    if (lane == 0) {
        s_xs[r] = g;
        s_rs[r] = sum;
    }
}

// NVQ > 0: the launch quantises the fp32 rows of sq itself (one token tile,
// M <= 8: wave w takes rows w and w + 4), NVQ float4 per played thread;
// Xq, x_scale and x_rowsum are then unused.
template <int MT, int QMAX, int NVQ>
__global__ __launch_bounds__(kStatWaves* kWave) void k_stat(const int8_t* __restrict__ Xq,
                                                             const float* __restrict__ x_scale,
                                                             const int32_t* __restrict__ x_rowsum, int M, int K,
                                                             const BatchMats mats, int tiles, uint32_t kdiv,
                                                             const StatQuant sq) {
    static_assert(NVQ == 0 || MT == 1, "in-launch quantisation covers one token tile");
    __shared__ __align__(1024) int8_t act[kStatLds];
    // quantised in the launch: gamma and row sums of the 16 rows in the last
    // 128 bytes (the rows themselves take at most 16 * 2560 bytes)
    float* s_xs = reinterpret_cast<float*>(act + kStatLds - 128);
    int* s_rs = reinterpret_cast<int*>(act + kStatLds - 64);
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int fr = lane & 15;
    const int fg = lane >> 4;
    const int C = K / 64;
    const int nq = (C + 3) / 4;
    const uint32_t nch = (uint32_t)K / 16u;
    const int stride = (int)gridDim.x * kStatWaves;
    int tile = (int)blockIdx.x * kStatWaves + wave;

    uint4 w[QMAX];
    StatTile T = stat_tile(mats, tile < tiles ? tile : 0);
    float xs[MT][4];
    int rsum[MT][4];
    if constexpr (NVQ > 0) {
        // ---- the rows' loads first (vector loads complete in issue order,
        // and the quantisation waits for them only), then the first tile's
        // weights, which land while the rows are quantised; rows past M are
        // left as they are (their outputs are never stored)
        const int r0 = wave, r1 = wave + kStatWaves;
        float4 v0[4][NVQ], v1[4][NVQ], gv[4][NVQ];
        wrow_load<NVQ>(r0 < M ? sq.X + (int64_t)r0 * K : nullptr, K, v0);
        wrow_load<NVQ>(r1 < M ? sq.X + (int64_t)r1 * K : nullptr, K, v1);
        const bool has_gain = sq.rms && sq.gain != nullptr;
        // without a gain its loads are skipped, not sent out of range: every
        // load instruction costs the CU's address unit the same time
        if (has_gain) {
            wrow_load<NVQ>(sq.gain, K, gv);
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < NVQ; ++i) gv[u][i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        __builtin_amdgcn_sched_barrier(0);
        stat_load_weights<QMAX>(T.W, T.n0, T.rows, K, C, nq, fr, fg, w);
        __builtin_amdgcn_sched_barrier(0);
        if (r0 < M) wrow_quant<NVQ>(v0, gv, K, sq.rms != 0, has_gain, sq.eps, r0, act, nch, s_xs, s_rs);
        if (r1 < M) wrow_quant<NVQ>(v1, gv, K, sq.rms != 0, has_gain, sq.eps, r1, act, nch, s_xs, s_rs);
    } else {
        // ---- the first tile's weights go out first, so their latency
        // overlaps the activation copy
        stat_load_weights<QMAX>(T.W, T.n0, T.rows, K, C, nq, fr, fg, w);

        // ---- the activation copy: MT * 16 rows (rows past M read zeros); one
        // token tile copies only the instructions that hold rows below M (the
        // rest of the tile is never stored from)
        const Rsrc rx = make_rsrc(Xq, (uint32_t)M * (uint32_t)K);
        const int ninst = MT == 1 ? (M * K + 1023) / 1024 : MT * 16 * K / 1024;
        // (rows of whole groups of 16 chunks, as at K = 2560, take the swizzle
        // without the per-lane test for a partial last group)
        const bool whole16 = (nch & 15u) == 0u;
#pragma unroll 4
        for (int i = wave; i < ninst; i += kStatWaves) {
            const uint32_t o = 1024u * (uint32_t)i + 16u * (uint32_t)lane;
            // r = o / K by a multiply-high with ceil(2^32 / K), then one correction
            uint32_t r = __umulhi(o, kdiv);
            if (r * (uint32_t)K > o) --r;
            if ((r + 1u) * (uint32_t)K <= o) ++r;
            const uint32_t j = (o - r * (uint32_t)K) / 16u;
            // the global chunk held by this LDS slot: the swizzle is its own inverse
            const uint32_t src = whole16 ? r * (uint32_t)K + 16u * (j ^ (r & 15u)) : stat_slot(r, j, (uint32_t)K, nch);
            dma16(rx, (lds_ptr)(act + 1024 * i), src, 0u);
        }

        // ---- the rows' scales and sums for this lane's outputs: acc[t][q] is
        // token 16 t + 4 fg + q, output column fr of the tile
        const Rsrc rs = make_rsrc(x_scale, (uint32_t)M * 4u);
        const Rsrc rr = make_rsrc(x_rowsum, (uint32_t)M * 4u);
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t m = (uint32_t)(16 * t + 4 * fg + q);
                xs[t][q] = buf_load4f(rs, m * 4u);
                rsum[t][q] = buf_load4i(rr, m * 4u);
            }
    }
    // operand addresses: row 16 t + fr, chunk 16 s + 4 fg + d of a whole group
    // of 16 sits at slot 16 s + ((4 fg + d) ^ fr), i.e. at ap[t][d] + 256 s
    const int8_t* ap[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int d = 0; d < 4; ++d) ap[t][d] = act + (16 * t + fr) * K + 16 * ((4 * fg + d) ^ fr);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copy (and first weights) have landed
    __syncthreads();                // and every other wave's copy
    if constexpr (NVQ > 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = 4 * fg + q;  // rows past M: never stored
            xs[0][q] = s_xs[m];
            rsum[0][q] = s_rs[m];
        }
    }

    for (bool first = true; tile < tiles; tile += stride, first = false) {
        if (!first) {
            T = stat_tile(mats, tile);
            stat_load_weights<QMAX>(T.W, T.n0, T.rows, K, C, nq, fr, fg, w);
        }
        const float ws = *T.w_scale;
        const int n = T.n0 + fr;
        const int N = T.N;
        float e_aux[MT][4];
        {
            const Rsrc ra =
                make_rsrc(T.aux, (T.epi_flags & (kEpiResidual | kEpiMul)) ? 0x7FFFFFFFu : 0u);
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int m = 16 * t + 4 * fg + q;
                    e_aux[t][q] = buf_load4f(ra, (m < M && n < N) ? (uint32_t)((int64_t)m * N + n) * 4u : kOob);
                }
        }

        v4i acc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = v4i{0, 0, 0, 0};
        // QMAX is the row's quad count (the launcher picks it so), and only the
        // last quad can be partial: earlier quads are whole groups of 16
        // chunks, read at the precomputed offsets plus 256 s; the last one
        // goes through the general map (a chunk past the row end has zero
        // weights, so its operand offset is clamped to chunk 0).  The operand
        // fragments of quad s + 1 are read from LDS while quad s's MFMAs run
        // (two register sets, pinned by scheduling barriers).
        auto read_quad = [&](int s, v4i (&a)[4][MT]) {
            const int c = 4 * s + fg;
            const uint32_t j0 = (uint32_t)(c < C ? 4 * c : 0);
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const int8_t* p = s + 1 < QMAX
                                          ? ap[t][d] + 256 * s
                                          : act + stat_slot((uint32_t)(16 * t + fr), j0 + d, (uint32_t)K, nch);
                    a[d][t] = *reinterpret_cast<const v4i*>(p);
                }
        };
        auto mma_quad = [&](int s, const v4i (&a)[4][MT]) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t wd = d == 0 ? w[s].x : d == 1 ? w[s].y : d == 2 ? w[s].z : w[s].w;
                const v4i b = v4i{codes4(wd, 0), codes4(wd, 1), codes4(wd, 2), codes4(wd, 3)};
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[d][t], b, acc[t], 0, 0, 0);
            }
        };
        v4i a0[4][MT], a1[4][MT];
        read_quad(0, a0);
#pragma unroll
        for (int s = 0; s < QMAX; ++s) {
            if (s + 1 < QMAX) {
                if (s % 2 == 0) read_quad(s + 1, a1);
                else read_quad(s + 1, a0);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (s % 2 == 0) mma_quad(s, a0);
            else mma_quad(s, a1);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- epilogue straight from the accumulators
        if (n < N) {
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int m = 16 * t + 4 * fg + q;
                    if (m < M) {
                        const int a = acc[t][q] - rsum[t][q];
                        float y = (float)a * ((xs[t][q] * ws) / 127.0f);
                        if (T.epi_flags & kEpiRelu2) {
                            const float tt = y > 0.0f ? y : 0.0f;
                            y = tt * tt;
                        }
                        if (T.epi_flags & kEpiMul) y = y * e_aux[t][q];
                        else if (T.epi_flags & kEpiResidual) y = y + e_aux[t][q];
                        const int64_t o = (int64_t)m * N + n;
                        if (T.Y != nullptr) T.Y[o] = y;
                        if (T.acc_out != nullptr) T.acc_out[o] = a;
                    }
                }
        }
    }
}

struct Plan {
    int nw, qmax;
};

// Waves per workgroup and weight loads per lane from the chunk-quad count:
// (4, 2) up to K = 2048, (4, 4) up to 4096, (8, 4) up to 8192, (8, 8) up to
// 16384.  In each case K <= 4 * 64 * nw * qmax, so an fp32 row fits in qmax
// float4 per thread.
bool plan(int64_t K, Plan& p) {
    const int64_t nq = (K / 64 + 3) / 4;
    p.nw = quant_threads(K) / kWave;  // 4 waves up to K = 4096, then 8 (same size as the quantiser)
    if (p.nw > 8) p.nw = 8;
    const int64_t per = (nq + p.nw - 1) / p.nw;
    if (per <= 2) p.qmax = 2;
    else if (per <= 4) p.qmax = 4;
    else if (per <= 8) p.qmax = 8;
    else return false;
    return true;
}

template <int NWV, int Q, bool G, int NV>
hipError_t go_decode(const float* X, int64_t M, int64_t K, bool rms, const float* gain, float eps,
                     const uint8_t* packed, const float* ws, int64_t N, uint32_t epi, const float* aux, float* Y,
                     const uint8_t* gate, const float* gate_scale, hipStream_t s) {
    const unsigned blocks = (unsigned)((N + 15) / 16);
    const size_t red = (size_t)NWV * 16 * 16 * sizeof(int) * (G ? 2 : 1);
    const size_t lds = 4 * (size_t)K + red;
    hipLaunchKernelGGL((k_decode<NWV, Q, G, NV>), dim3(blocks), dim3(NWV * kWave), lds, s, X, (int)M, (int)K,
                       rms ? 1 : 0, gain, eps, packed, ws, (int)N, epi, aux, Y, gate, gate_scale);
    return hipGetLastError();
}

// Very tall matrices (at least 2048 tiles of 16 rows, eight per CU): the
// persistent streaming launch, kStreamCT tiles per group.
constexpr int64_t kTallTiles = 2048;
constexpr int kStreamCT = 1;

template <int NWV, int NV, int CT>
hipError_t go_decode_stream(const float* X, int64_t M, int64_t K, bool rms, const float* gain, float eps,
                            const uint8_t* packed, const float* ws, int64_t N, uint32_t epi, const float* aux,
                            float* Y, hipStream_t s) {
    const size_t lds = 4 * (size_t)K + (size_t)NWV * 16 * 16 * CT * sizeof(int);
    // Resident workgroups per CU from the runtime's occupancy query, kept per
    // device for the last LDS size asked (one entry: lds << 16 | occupancy).
    static std::atomic<int64_t> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
    int occ = 0;
    const int64_t hit = dev >= 0 ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (hit != 0 && (size_t)(hit >> 16) == lds) {
        occ = (int)(hit & 0xFFFF);
    } else {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_decode_stream<NWV, NV, CT>, NWV * kWave, lds) !=
                hipSuccess ||
            occ < 1)
            occ = 1;
        if (occ > 0xFFFF) occ = 0xFFFF;
        if (dev >= 0) cache[dev].store(((int64_t)lds << 16) | occ, std::memory_order_relaxed);
    }
    const int64_t groups = (N + 16 * CT - 1) / (16 * CT);
    const int64_t resident = (int64_t)cu_count() * occ;
    const unsigned blocks = (unsigned)(groups < resident ? groups : resident);
    hipLaunchKernelGGL((k_decode_stream<NWV, NV, CT>), dim3(blocks), dim3(NWV * kWave), lds, s, X, (int)M,
                       (int)K, rms ? 1 : 0, gain, eps, packed, ws, (int)N, epi, aux, Y);
    return hipGetLastError();
}

// The quantiser's depth for K (which the plan bounds by qmax) picks NV.
template <bool G>
hipError_t go_decode_plan(const Plan& p, const float* X, int64_t M, int64_t K, bool rms, const float* gain,
                          float eps, const uint8_t* packed, const float* ws, int64_t N, uint32_t epi,
                          const float* aux, float* Y, hipStream_t s, const uint8_t* gate = nullptr,
                          const float* gate_scale = nullptr) {
    const int nv = quant_depth(K);
    const bool tall = !G && (N + 15) / 16 >= kTallTiles;
#define BL_DEC(NWV, Q, NV)                                                                                     \
    if (p.nw == NWV && p.qmax == Q && nv == NV)                                                                \
        return !tall ? go_decode<NWV, Q, G, NV>(X, M, K, rms, gain, eps, packed, ws, N, epi, aux, Y, gate, gate_scale, s) \
                     : go_decode_stream<NWV, NV, kStreamCT>(X, M, K, rms, gain, eps, packed, ws, N, epi, aux, Y, s);
    BL_DEC(4, 2, 1)
    BL_DEC(4, 2, 2)
    BL_DEC(4, 4, 3)
    BL_DEC(4, 4, 4)
    BL_DEC(8, 4, 3)
    BL_DEC(8, 4, 4)
    BL_DEC(8, 8, 5)
    BL_DEC(8, 8, 6)
    BL_DEC(8, 8, 7)
    BL_DEC(8, 8, 8)
#undef BL_DEC
    return hipErrorInvalidValue;
}

}  // namespace

// Batched kernel shape: four waves, up to 8 chunk quads each (K <= 8192;
// longer rows go to the GEMM); token tiles 1, 2 or 4 (M = 33..48 runs a
// zero tile) with 4, 3 or 2 ring stages (64, 96 or 128 KB of LDS); two
// column tiles per workgroup once several token tiles share each operand
// fragment, while that still leaves >= 128 workgroups, and four at four
// token tiles when that still gives every CU a workgroup (one workgroup per
// CU fits the LDS, so a launch of more takes a second round, whose weight
// stream starts only when the first round ends).
static bool batch_shape(int64_t M, int64_t K, int64_t N, int& q, int& mt, int& ct) {
    const int64_t nq = (K / 64 + 3) / 4;
    q = (int)((nq + kBatchWaves - 1) / kBatchWaves);
    mt = M <= 16 ? 1 : M <= 32 ? 2 : 4;
    ct = (mt == 4 && (N + 63) / 64 >= cu_count()) ? 4 : (mt >= 2 && (N + 31) / 32 >= 128) ? 2 : 1;
    return M >= 1 && M <= 64 && K >= 64 && K <= 8192 && q >= 1 && q <= 8;
}

// Output offsets are taken in 32-bit bytes by the buffer loads: M * N * 4 < 2^31.
bool gemv_supported(int64_t M, int64_t K, int64_t N) {
    int q, mt, ct;
    return M * N < (1LL << 29) && batch_shape(M, K, N, q, mt, ct);
}

// mats.m[i].wg0 is filled in here from each matrix's N and the launch's
// column tiles per workgroup.
template <int MT, int CT, int Q, bool G = false>
static hipError_t go_batch(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                           BatchMats mats, hipStream_t s, const uint8_t* gate = nullptr,
                           const float* gate_scale = nullptr) {
    constexpr int NS = MT == 1 ? 4 : MT == 2 ? 3 : 2;
    const int64_t cols = G ? 16 : 16 * CT;
    int64_t blocks = 0;
    for (int i = 0; i < mats.count; ++i) {
        mats.m[i].wg0 = (int)blocks;
        blocks += (mats.m[i].N + cols - 1) / cols;
    }
    if (MT == 1 && M <= 8)  // half the token tile: half the activation copy
        hipLaunchKernelGGL((k_batch<MT, CT, NS, Q, G, MT == 1>), dim3((unsigned)blocks), dim3(kBatchWaves * kWave), 0,
                           s, Xq, xs, rs, (int)M, (int)K, mats, gate, gate_scale);
    else
        hipLaunchKernelGGL((k_batch<MT, CT, NS, Q, G, false>), dim3((unsigned)blocks), dim3(kBatchWaves * kWave), 0,
                           s, Xq, xs, rs, (int)M, (int)K, mats, gate, gate_scale);
    return hipGetLastError();
}

template <int MT, int CT, bool G = false>
static hipError_t go_batch_q(int q, const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                             const BatchMats& mats, hipStream_t s, const uint8_t* gate = nullptr,
                             const float* gate_scale = nullptr) {
    switch (q) {
#define BL_BQ(Q) \
    case Q: return go_batch<MT, CT, Q, G>(Xq, xs, rs, M, K, mats, s, gate, gate_scale);
        BL_BQ(1) BL_BQ(2) BL_BQ(3) BL_BQ(4) BL_BQ(5) BL_BQ(6) BL_BQ(7) BL_BQ(8)
#undef BL_BQ
        default: return hipErrorInvalidValue;
    }
}

static BatchMat batch_mat(const uint8_t* packed, const float* ws, int64_t N, Epi epi, float* Y, int32_t* acc_out) {
    return BatchMat{packed, ws, epi.aux, Y, acc_out, (int)N, epi.flags, 0};
}

// The activation-stationary launch: up to 32 tokens, K <= 2560 (at most 10
// weight chunk quads per lane), and enough 16-row tiles for every CU (a
// launch of fewer tiles keeps k_batch, whose workgroups split K four ways).
// Measured on the grouped o + gate + up launch (1024 tiles, K = 2560): at
// 8 / 32 tokens 9.1 / 11.3 us against 10.3 / 12.6 us with k_batch, but at 64
// tokens 17.0 against 15.7 us (each wave then reads 160 KB of operands from
// LDS per tile, one wave per SIMD), so 33..64 tokens keep k_batch.
constexpr int64_t kStatMinTiles = 512;
constexpr int64_t kStatMaxM = 32;

static int stat_mt(int64_t M) { return M <= 16 ? 1 : 2; }

static bool stat_shape(int64_t M, int64_t K, int64_t tiles) {
    return M >= 1 && M <= kStatMaxM && K >= 64 && K <= 2560 && (int64_t)stat_mt(M) * 16 * K <= kStatLds &&
           tiles >= kStatMinTiles;
}

template <int MT, int Q, int NVQ = 0>
static hipError_t go_stat(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K, BatchMats mats,
                          hipStream_t s, const StatQuant sq = StatQuant{nullptr, nullptr, 0.0f, 0}) {
    int64_t tiles = 0;
    for (int i = 0; i < mats.count; ++i) {
        mats.m[i].wg0 = (int)tiles;
        tiles += (mats.m[i].N + 15) / 16;
    }
    const int64_t want = (tiles + kStatWaves - 1) / kStatWaves;
    const int64_t cus = cu_count();
    const unsigned blocks = (unsigned)(want < cus ? want : cus);
    const uint32_t kdiv = (uint32_t)((((uint64_t)1 << 32) + (uint64_t)K - 1) / (uint64_t)K);
    hipLaunchKernelGGL((k_stat<MT, Q, NVQ>), dim3(blocks), dim3(kStatWaves * kWave), 0, s, Xq, xs, rs, (int)M,
                       (int)K, mats, (int)tiles, kdiv, sq);
    return hipGetLastError();
}

static hipError_t go_stat_mt(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                             const BatchMats& mats, hipStream_t s) {
    const int q = (int)((K / 64 + 3) / 4);
#define BL_SQ(MT, Q) \
    if (stat_mt(M) == MT && q == Q) return go_stat<MT, Q>(Xq, xs, rs, M, K, mats, s);
#define BL_SQ_MT(MT) BL_SQ(MT, 1) BL_SQ(MT, 2) BL_SQ(MT, 3) BL_SQ(MT, 4) BL_SQ(MT, 5) \
    BL_SQ(MT, 6) BL_SQ(MT, 7) BL_SQ(MT, 8) BL_SQ(MT, 9) BL_SQ(MT, 10)
    BL_SQ_MT(1) BL_SQ_MT(2)
#undef BL_SQ_MT
#undef BL_SQ
    return hipErrorInvalidValue;
}

// The stationary launch that quantises its fp32 rows itself: at most 8
// tokens (each wave quantises two rows the way the 256-thread quantiser
// would, while the first tile's weights are in flight).
constexpr int64_t kStatQuantMaxM = 8;

static bool stat_quant_shape(int64_t M, int64_t K, int64_t tiles) {
    return M <= kStatQuantMaxM && quant_threads(K) == 256 && stat_shape(M, K, tiles);
}

static hipError_t go_stat_quant(const StatQuant& sq, int64_t M, int64_t K, const BatchMats& mats, hipStream_t s) {
    const int q = (int)((K / 64 + 3) / 4);  // NVQ: float4 per played thread of 256, (K / 4) / 256 rounded up
#define BL_SQQ(Q, NV) \
    if (q == Q) return go_stat<1, Q, NV>(nullptr, nullptr, nullptr, M, K, mats, s, sq);
    BL_SQQ(1, 1) BL_SQQ(2, 1) BL_SQQ(3, 1) BL_SQQ(4, 1) BL_SQQ(5, 2) BL_SQQ(6, 2) BL_SQQ(7, 2) BL_SQQ(8, 2)
    BL_SQQ(9, 3) BL_SQQ(10, 3)
#undef BL_SQQ
    return hipErrorInvalidValue;
}

// Column tiles per workgroup for a launch covering `rows` output rows in all.
static hipError_t go_batch_mats(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                                int64_t rows, const BatchMats& mats, hipStream_t s) {
    int64_t tiles = 0;
    for (int i = 0; i < mats.count; ++i) tiles += (mats.m[i].N + 15) / 16;
    if (stat_shape(M, K, tiles)) return go_stat_mt(Xq, xs, rs, M, K, mats, s);
    int q, mt, ct;
    if (!batch_shape(M, K, rows, q, mt, ct)) return hipErrorInvalidValue;
    switch (mt * 2 + ct - 1) {
        case 2: return go_batch_q<1, 1>(q, Xq, xs, rs, M, K, mats, s);
        case 4: return go_batch_q<2, 1>(q, Xq, xs, rs, M, K, mats, s);
        case 5: return go_batch_q<2, 2>(q, Xq, xs, rs, M, K, mats, s);
        case 8: return go_batch_q<4, 1>(q, Xq, xs, rs, M, K, mats, s);
        case 9: return go_batch_q<4, 2>(q, Xq, xs, rs, M, K, mats, s);
        case 11: return go_batch_q<4, 4>(q, Xq, xs, rs, M, K, mats, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                       const uint8_t* packed, const float* ws, int64_t N, Epi epi, float* Y, int32_t* acc_out,
                       hipStream_t s) {
    BatchMats mats{};
    mats.m[0] = batch_mat(packed, ws, N, epi, Y, acc_out);
    mats.count = 1;
    return go_batch_mats(Xq, xs, rs, M, K, N, mats, s);
}

int gemv_max_groups() { return kMaxGroups; }

hipError_t launch_gemv_grouped(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                               const GroupMat* g, int count, hipStream_t s) {
    if (count < 1 || count > kMaxGroups) return hipErrorInvalidValue;
    BatchMats mats{};
    int64_t rows = 0;
    for (int i = 0; i < count; ++i) {
        mats.m[i] = batch_mat(g[i].packed, g[i].w_scale, g[i].N, g[i].epi, g[i].Y, g[i].acc_out);
        rows += g[i].N;
    }
    mats.count = count;
    return go_batch_mats(Xq, xs, rs, M, K, rows, mats, s);
}

bool gemv_grouped_quant_supported(int64_t M, int64_t K, const GroupMat* g, int count) {
    if (count < 1 || count > kMaxGroups || M < 1) return false;
    int64_t tiles = 0;
    for (int i = 0; i < count; ++i) tiles += (g[i].N + 15) / 16;
    return stat_quant_shape(M, K, tiles);
}

hipError_t launch_gemv_grouped_quant(const float* X, int64_t M, int64_t K, bool rmsnorm, const float* gain, float eps,
                                     const GroupMat* g, int count, hipStream_t s) {
    if (!gemv_grouped_quant_supported(M, K, g, count)) return hipErrorInvalidValue;
    BatchMats mats{};
    for (int i = 0; i < count; ++i) mats.m[i] = batch_mat(g[i].packed, g[i].w_scale, g[i].N, g[i].epi, g[i].Y, g[i].acc_out);
    mats.count = count;
    return go_stat_quant(StatQuant{X, gain, eps, rmsnorm ? 1 : 0}, M, K, mats, s);
}

// The gated pair in one launch: one workgroup per 16 output rows, streaming
// those rows of up and of gate against one pass over the activations.
hipError_t launch_gemv_gated(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                             const uint8_t* up, const float* up_scale, const uint8_t* gate, const float* gate_scale,
                             int64_t N, float* Y, hipStream_t s) {
    int q, mt, ct;
    if (!batch_shape(M, K, N, q, mt, ct)) return hipErrorInvalidValue;
    BatchMats mats{};
    mats.m[0] = batch_mat(up, up_scale, N, Epi{0u, nullptr}, Y, nullptr);
    mats.count = 1;
    switch (mt) {
        case 1: return go_batch_q<1, 2, true>(q, Xq, xs, rs, M, K, mats, s, gate, gate_scale);
        case 2: return go_batch_q<2, 2, true>(q, Xq, xs, rs, M, K, mats, s, gate, gate_scale);
        case 4: return go_batch_q<4, 2, true>(q, Xq, xs, rs, M, K, mats, s, gate, gate_scale);
        default: return hipErrorInvalidValue;
    }
}

bool decode_supported(int64_t M, int64_t K, int64_t N) {
    Plan p;
    if (M < 1 || M > 4 || K < 64 || M * N >= (1LL << 29) || !plan(K, p) || quant_threads(K) != p.nw * kWave)
        return false;
    return quant_depth(K) <= p.qmax;  // the fp32 row fits the kernel's depth (it always does under plan())
}

hipError_t launch_decode_bitlinear(const float* X, int64_t M, int64_t K, bool rmsnorm, const float* gain, float eps,
                                   const uint8_t* packed, const float* w_scale, int64_t N, uint32_t epi,
                                   const float* aux, float* Y, hipStream_t s) {
    Plan p;
    if (!plan(K, p)) return hipErrorInvalidValue;
    return go_decode_plan<false>(p, X, M, K, rmsnorm, gain, eps, packed, w_scale, N, epi, aux, Y, s);
}

hipError_t launch_decode_gated(const float* X, int64_t M, int64_t K, bool rmsnorm, const float* gain, float eps,
                               const uint8_t* up, const float* up_scale, const uint8_t* gate,
                               const float* gate_scale, int64_t N, float* Y, hipStream_t s) {
    Plan p;
    if (!plan(K, p)) return hipErrorInvalidValue;
    return go_decode_plan<true>(p, X, M, K, rmsnorm, gain, eps, up, up_scale, N, 0u, nullptr, Y, s, gate,
                                gate_scale);
}

}  // namespace bl
