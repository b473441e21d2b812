// Prefill contraction: int8 MFMA GEMM over unpacked ternary weights
// (transformers "BitNet" page, "Model details" / Quantization: W1.58A8; with
// thousands of tokens the product is a dense contraction).
//
// Tiling.  A workgroup of WM x WN waves computes a BM x BN tile of acc; each
// wave owns a (BM/WM) x (BN/WN) block of 16x16 fragments and issues
// v_mfma_i32_16x16x64_i8, one per fragment pair and 64-k step.
// Weights stay packed (2 bits) all the way into LDS, 4x less traffic than
// int8; each wave expands its 32-bit words to int8 codes in registers: a
// shift and a mask per 4 weights give 16 consecutive k in order, which is one
// 16-byte MFMA operand, matching the 16 activation bytes of the same k.
// Tile order is XCD-aware: workgroups are dealt round-robin to the 8 XCDs,
// so consecutive tile indices are remapped to land on the same XCD and share
// its L2.
// The MFMA accumulates codes (q + 1); the epilogue subtracts the token's
// activation row sum, dequantises and applies the fused ReLU^2 and residual
// add or gating product, chosen at compile time (EP: kEpi* bits, MUL
// overriding RESIDUAL).
#include <atomic>

#include "bl_device.h"
#include "bl_internal.h"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;

// Pipeline: k advances 128 per stage and NBUF (4) stages ring through LDS,
// filled by direct buffer->LDS loads (buffer_load_dwordx4 ... lds) issued
// three stages ahead, so L2/HBM latency overlaps the MFMAs.
// A DMA instruction writes 64 lanes x 16 bytes contiguously; the global
// address each lane fetches is chosen so that:
//   - activations: one instruction covers 8 rows x 128 bytes (whole cache
//     lines); inside a row the 16-byte chunk c lands at slot c ^ (row % 8),
//     so the 16 rows of an MFMA fragment read at one k hit distinct banks;
//   - weights: one instruction covers 32 rows x both 16-byte chunks of the
//     stage, chunk-major, so a fragment read (word g of 16 rows) is one
//     contiguous 256-byte span; in the packed layout (16-row tiles, chunk c
//     of a tile's rows side by side) that is four 256-byte runs in memory.

constexpr int kBK = 128;             // k per stage

// Issue one stage of direct buffer->LDS loads for this wave.  A lane's byte
// offset is its part inside an 8-row (activations) or 32-row (weights)
// block: va fixed for the whole loop; for weights vb[i] + st * vs[i], since
// a stage's chunks advance by 32 bytes per row of the lane's weight tile
// (the last tile of a matrix may have fewer than 16 rows).  The block's row
// offset, the tile origin and (activations) the stage's k are wave-uniform
// and go in the scalar offset.
// Reads past the tensor return zero (the descriptor's size), so no row or
// k clamp is needed: rows past M or N are never stored, and when
// K % 128 == 64 the second half of the last stage is never read.
//   activations: A_BLKS instructions, block j = rows 8j..8j+7 of the tile;
//   weights: B_INS instructions, each 32 rows x both 64-k chunks.
template <int A_BLKS, int B_INS>
__device__ __forceinline__ void issue_stage(Rsrc ra, Rsrc rb, uint32_t va, const uint32_t (&vb)[B_INS],
                                            const uint32_t (&vs)[B_INS], int st, uint32_t a_s, uint32_t b_s,
                                            uint32_t a_blk, uint32_t b_blk, int8_t* base, int a_stage, int wave) {
#pragma unroll
    for (int i = 0; i < A_BLKS; ++i) {
        const int j = wave * A_BLKS + i;
        dma16(ra, (lds_ptr)(base + j * 1024), va, a_s + (uint32_t)j * a_blk);
    }
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
        const int j = wave * B_INS + i;
        dma16(rb, (lds_ptr)(base + a_stage + j * 1024), vb[i] + (uint32_t)st * vs[i], b_s + (uint32_t)j * b_blk);
    }
}

template <int BM, int BN, int WM, int WN, int NBUF, int OCC, uint32_t EP>
__global__ __launch_bounds__(WM* WN* kWave, OCC) void k_gemm_pipe(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ rowsum, int M, int K, const uint4* __restrict__ Wp,
    const float* __restrict__ w_scale, int N, Epi epi, float* Y,
    int32_t* __restrict__ acc_out) {
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
    constexpr int A_STAGE = BM * kBK;             // bytes
    constexpr int B_INS = (BN + 32 * NW - 1) / (32 * NW);  // weight DMAs per wave (32 rows each)
    constexpr int B_STAGE = B_INS * NW * 1024;    // bytes: 32 packed rows x 32 bytes per DMA
    constexpr int STAGE = A_STAGE + B_STAGE;
    constexpr int A_BLKS = (BM / 8) / NW;         // 1 KB activation blocks per wave
    constexpr int LOADS = A_BLKS + B_INS;         // DMA instructions per wave per stage
    static_assert((BM / 8) % NW == 0, "activation blocks must split evenly over waves");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "whole fragments");
    __shared__ __align__(1024) int8_t smem[NBUF * STAGE];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wave / WN;
    const int wn = wave % WN;

    const int tiles_n = (N + BN - 1) / BN;
    const int ntiles = gridDim.x;
    const int b = blockIdx.x;
    int t = b;
    if (ntiles % kXcds == 0) t = (b % kXcds) * (ntiles / kXcds) + b / kXcds;
    const int m0 = (t / tiles_n) * BM;
    const int n0 = (t % tiles_n) * BN;
    const int C = K / 64;
    const int nst = (K + kBK - 1) / kBK;

    const int fr = lane & 15;
    const int fg = lane >> 4;

    // DMA descriptors and this lane's fixed offsets (bytes).  Activations:
    // lane (r8 = lane/8, c = lane%8) of a block fetches row r8 of the block,
    // 16-byte chunk c ^ r8, stored at slot c of that row in LDS (so the 16
    // rows an MFMA fragment reads at one k sit in distinct banks).  Weights:
    // lane l of a block fetches row l%32, chunk l/32 of the stage
    // (chunk-major in LDS); in memory that row is row l%16 of weight tile
    // h = (l%32)/16 of the block, whose chunk c sits at 16 (c R + l%16).
    const Rsrc ra = make_rsrc(Xq, (uint32_t)M * (uint32_t)K);
    const Rsrc rb = make_rsrc(Wp, (uint32_t)N * (uint32_t)C * 16u);
    const uint32_t va = (uint32_t)(lane >> 3) * (uint32_t)K + (uint32_t)((lane & 7) ^ (lane >> 3)) * 16u;
    uint32_t vb[B_INS], vs[B_INS];
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
        const int h = (lane & 31) >> 4;
        const int r0 = n0 + 32 * (wave * B_INS + i) + 16 * h;  // first row of the lane's weight tile
        const int R = N - r0 < 16 ? N - r0 : 16;               // its rows (<= 0: past the matrix)
        vb[i] = R > 0 ? (uint32_t)h * 16u * (uint32_t)K / 4u + 16u * (uint32_t)((lane >> 5) * R + (lane & 15)) : kOob;
        vs[i] = R > 0 ? 32u * (uint32_t)R : 0u;
    }
    const uint32_t a_blk = 8u * (uint32_t)K, b_blk = 32u * (uint32_t)C * 16u;
    const uint32_t a_base = (uint32_t)m0 * (uint32_t)K, b_base = (uint32_t)n0 * (uint32_t)C * 16u;
    // A stage index past the last one gets a scalar offset past every
    // descriptor: its loads write zeros to LDS without touching memory, so
    // the issue is branch-free (those buffers are never read).
#define BL_ISSUE(st)                                                                                          \
    issue_stage<A_BLKS, B_INS>(ra, rb, va, vb, vs, (st), (st) < nst ? a_base + (uint32_t)(st) * kBK : kOob,    \
                               (st) < nst ? b_base : kOob, a_blk, b_blk, smem + ((st) % NBUF) * STAGE,       \
                               A_STAGE, wave)

    v4i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    static_assert(NBUF == 4, "two stages are read while two more are in flight");
#pragma unroll
    for (int p = 0; p < NBUF - 1; ++p) BL_ISSUE(p);

    // Fragments of one 64-k step: activation rows R (block R/8, slot
    // (4s + fg) ^ (R % 8)) and the packed weight word g of 16 rows.
    auto load_frags = [&](int st, int s, v4i (&a)[FM], uint32_t (&wq)[FN]) {
        const int8_t* sa = smem + (st % NBUF) * STAGE;
        const uint32_t* sb = reinterpret_cast<const uint32_t*>(sa + A_STAGE);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int R = wm * TM + fm * 16 + fr;
            const int slot = (4 * s + fg) ^ (R & 7);
            a[fm] = *reinterpret_cast<const v4i*>(sa + (R >> 3) * 1024 + (R & 7) * 128 + slot * 16);
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int col = wn * TN + fn * 16 + fr;
            wq[fn] = sb[(col >> 5) * 256 + s * 128 + (col & 31) * 4 + fg];
        }
    };
    auto mma = [&](const v4i (&a)[FM], const uint32_t (&wq)[FN]) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const v4i bv = v4i{codes4(wq[fn], 0), codes4(wq[fn], 1), codes4(wq[fn], 2), codes4(wq[fn], 3)};
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
                acc[fm][fn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bv, a[fm], acc[fm][fn], 0, 0, 0);
        }
    };
    auto mma_frag = [&](const v4i (&a)[FM], const uint32_t (&wq)[FN], int fn) {
        const v4i bv = v4i{codes4(wq[fn], 0), codes4(wq[fn], 1), codes4(wq[fn], 2), codes4(wq[fn], 3)};
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            acc[fm][fn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bv, a[fm], acc[fm][fn], 0, 0, 0);
    };
    // DMA instruction i (activation blocks first, then weight blocks) of a
    // stage, as in issue_stage.
    auto issue_one = [&](int st, int i) {
        const uint32_t as = st < nst ? a_base + (uint32_t)st * kBK : kOob;
        const uint32_t bs = st < nst ? b_base : kOob;
        int8_t* base = smem + (st % NBUF) * STAGE;
        if (i < A_BLKS) {
            const int j = wave * A_BLKS + i;
            dma16(ra, (lds_ptr)(base + j * 1024), va, as + (uint32_t)j * a_blk);
        } else {
            const int j = wave * B_INS + (i - A_BLKS);
            dma16(rb, (lds_ptr)(base + A_STAGE + j * 1024), vb[i - A_BLKS] + (uint32_t)st * vs[i - A_BLKS],
                  bs + (uint32_t)j * b_blk);
        }
    };
    auto interleave = [&](bool dma) {
        // per weight fragment: its unpack, then MFMAs with LDS reads between;
        // in the first step of a stage the DMA instructions of stage s+3 are
        // spread through the MFMA stream, one or two per fragment, instead
        // of leaving every wave to issue them in a burst after the barrier
#pragma unroll
        for (int g = 0; g < FN; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);   // VALU: unpack
            __builtin_amdgcn_sched_group_barrier(0x008, FM / 2, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, (FM + FN + FN - 1) / FN, 0);  // DS read
            if (dma) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM (DMA)
            if (dma && g == 0 && LOADS > FN)
                __builtin_amdgcn_sched_group_barrier(0x020, LOADS > FN ? LOADS - FN : 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, FM - FM / 2, 0);  // MFMA
        }
    };

    // Schedule.  Stages s and s+1 are readable while s+2 and s+3 are in
    // flight.  Within stage s the second 64-k step's fragments are read
    // during the first step's MFMAs, and the first fragments of stage s+1
    // during the second step's, so after a barrier the MFMAs resume at once.
    // The DMA of stage s+3 goes out during the first step, into the buffer
    // of stage s-1, which the barrier ending stage s-1 freed.  At the end of
    // stage s this wave waits for its own loads of stage s+2 (stage s+3 may
    // stay in flight) and the barrier makes stage s+2 visible from every
    // wave.
    wait_vm<LOADS>();
    __builtin_amdgcn_s_barrier();
    v4i a0[FM], a1[FM];
    uint32_t w0[FN], w1[FN];
    load_frags(0, 0, a0, w0);
    for (int st = 0; st + 1 < nst; ++st) {   // full 128-k stages
        load_frags(st, 1, a1, w1);
        if constexpr (FN >= LOADS) {
            // as many weight fragments as DMA instructions: one DMA after
            // each fragment's MFMAs, pinned there
#pragma unroll
            for (int g = 0; g < FN; ++g) {
                mma_frag(a0, w0, g);
                if (g < LOADS) issue_one(st + NBUF - 1, g);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            BL_ISSUE(st + NBUF - 1);
            mma(a0, w0);
            interleave(true);
        }
        __builtin_amdgcn_sched_barrier(0);
        load_frags(st + 1, 0, a0, w0);
        mma(a1, w1);
        interleave(false);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<LOADS>();
        __builtin_amdgcn_s_barrier();
    }
#undef BL_ISSUE
    // Last stage (one or two 64-k steps).  The token scales and row sums are
    // loaded between its two steps, into the registers the first step's
    // fragments free, so their latency hides under the second step's MFMAs.
    // In fragment fm this lane's outputs belong to token m0 + wm*TM + 16*fm
    // + fr (see the output layout below).  Buffer loads: rows past M read
    // zero (never stored), and the offsets stay 32-bit.
    int row_rs[FM];
    float row_d[FM];
    {
        const int st = nst - 1;
        const bool two = st * kBK + 64 < K;
        if (two) load_frags(st, 1, a1, w1);
        mma(a0, w0);
        __builtin_amdgcn_sched_barrier(0);
        const float wsc = *w_scale;
        // recomputed here rather than kept alive through the loop
        uint32_t mo = (uint32_t)(m0 + wm * TM + fr) * 4u;
        asm volatile("" : "+v"(mo));
        const Rsrc rxs = make_rsrc(x_scale, (uint32_t)M * 4u);
        const Rsrc rrs = make_rsrc(rowsum, (uint32_t)M * 4u);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            row_rs[fm] = buf_load4i(rrs, mo + fm * 64u);
            row_d[fm] = (buf_load4f(rxs, mo + fm * 64u) * wsc) / 127.0f;
        }
        __builtin_amdgcn_sched_barrier(0);
        if (two) mma(a1, w1);
        wait_vm<0>();   // no DMA may still write LDS when the workgroup ends
    }

    // Epilogue.  The weights are the MFMA's A operand and the tokens its B
    // operand, so a fragment is 16 outputs x 16 tokens and lane (fr, fg)
    // holds outputs 4fg..4fg+3 of token fr.  Stored from there, one 16-byte
    // store per lane would write 64-byte halves of 16 lines; a whole tile
    // (N % 4 == 0) instead goes through LDS, 16 tokens of a wave at a time
    // (the ring is free by then): each wave writes its fragments into a
    // private row-major block and reads it back by rows, so every store
    // instruction writes whole 128-byte lines (measured 30% less epilogue
    // time).  Partial tiles and the int32 accumulators take the element-wise
    // path.
    constexpr bool RELU2 = (EP & kEpiRelu2) != 0;
    constexpr bool MUL = (EP & kEpiMul) != 0;
    constexpr bool RES = !MUL && (EP & kEpiResidual) != 0;
    const bool whole = m0 + BM <= M && n0 + BN <= N && (N % 4) == 0;
    auto value = [&](int fm, int fn, int r) {
        float t = (float)(acc[fm][fn][r] - row_rs[fm]) * row_d[fm];
        if constexpr (RELU2) {
            t = t > 0.0f ? t : 0.0f;
            t = t * t;
        }
        return t;
    };
    if (whole && Y != nullptr && acc_out == nullptr) {
        __syncthreads();   // every wave is done with the ring
        constexpr int ROWB = TN * 4 + 16;     // staged row; +16 bytes puts the 16 rows on distinct banks
        constexpr int PER_ROW = TN / 4;       // float4 per row
        static_assert(NW * 16 * ROWB <= NBUF * STAGE, "staging fits in the ring");
        static_assert((16 * PER_ROW) % kWave == 0, "whole store instructions");
        int8_t* stg = smem + wave * (16 * ROWB);
        const int ncol = n0 + wn * TN;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                *reinterpret_cast<float4*>(stg + fr * ROWB + (fn * 16 + 4 * fg) * 4) =
                    make_float4(value(fm, fn, 0), value(fm, fn, 1), value(fm, fn, 2), value(fm, fn, 3));
            const int64_t mrow = m0 + wm * TM + fm * 16;
#pragma unroll
            for (int k = 0; k < 16 * PER_ROW / kWave; ++k) {
                const int i = k * kWave + lane;
                const int row = i / PER_ROW, c4 = i % PER_ROW;
                float4 y = *reinterpret_cast<const float4*>(stg + row * ROWB + c4 * 16);
                const int64_t o = (mrow + row) * N + ncol + 4 * c4;
                if constexpr (RES || MUL) {
                    const float4 x = *reinterpret_cast<const float4*>(epi.aux + o);
                    if constexpr (RES) {
                        y.x = y.x + x.x;
                        y.y = y.y + x.y;
                        y.z = y.z + x.z;
                        y.w = y.w + x.w;
                    } else {
                        y.x = y.x * x.x;
                        y.y = y.y * x.y;
                        y.z = y.z * x.z;
                        y.w = y.w * x.w;
                    }
                }
                *reinterpret_cast<float4*>(Y + o) = y;
            }
        }
    } else {
        // partial tiles, or the int32 accumulators requested: element-wise
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int m = m0 + wm * TM + fm * 16 + fr;
            if (m >= M) continue;
            const int64_t row = (int64_t)m * N;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int n = n0 + wn * TN + fn * 16 + 4 * fg;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (n + r < N) {
                        if (Y != nullptr) {
                            float t = value(fm, fn, r);
                            if constexpr (RES) t = t + epi.aux[row + n + r];
                            else if constexpr (MUL) t = t * epi.aux[row + n + r];
                            Y[row + n + r] = t;
                        }
                        if (acc_out != nullptr) acc_out[row + n + r] = acc[fm][fn][r] - row_rs[fm];
                    }
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, int NBUF, int OCC, uint32_t EP>
hipError_t launch_pipe_ep(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                          const uint8_t* packed, const float* ws, int64_t N, Epi epi, float* Y,
                          int32_t* acc_out, hipStream_t s) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL((k_gemm_pipe<BM, BN, WM, WN, NBUF, OCC, EP>), dim3((unsigned)tiles), dim3(WM * WN * kWave),
                       0, s, Xq, xs, rs, (int)M, (int)K, reinterpret_cast<const uint4*>(packed), ws,
                       (int)N, epi, Y, acc_out);
    return hipGetLastError();
}

// One kernel per epilogue: ReLU^2 on or off, then nothing, the residual add
// or the gating product (MUL overrides RESIDUAL).
template <int BM, int BN, int WM, int WN, int NBUF, int OCC>
hipError_t launch_pipe(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                       const uint8_t* packed, const float* ws, int64_t N, Epi epi, float* Y,
                       int32_t* acc_out, hipStream_t s) {
    uint32_t f = epi.flags & (kEpiRelu2 | kEpiResidual | kEpiMul);
    if (f & kEpiMul) f &= ~kEpiResidual;
#define BL_EP(e) launch_pipe_ep<BM, BN, WM, WN, NBUF, OCC, (e)>(Xq, xs, rs, M, K, packed, ws, N, epi, Y, acc_out, s)
    switch (f) {
        case kEpiRelu2: return BL_EP(kEpiRelu2);
        case kEpiResidual: return BL_EP(kEpiResidual);
        case kEpiRelu2 | kEpiResidual: return BL_EP(kEpiRelu2 | kEpiResidual);
        case kEpiMul: return BL_EP(kEpiMul);
        case kEpiRelu2 | kEpiMul: return BL_EP(kEpiRelu2 | kEpiMul);
        default: return BL_EP(0u);
    }
#undef BL_EP
}

}  // namespace

// Compute units of the current device, looked up once per device.
int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Tile choice.  One workgroup fits a CU (the LDS ring takes 160 KB), so the
// time goes as whole rounds of tiles over the CUs times the tile's work:
// 256x256 tiles (2x4 waves of 128x64: each unpacked weight fragment feeds 8
// MFMAs) unless 256x160 tiles (4x2 waves of 64x80, weighted 10% less
// efficient) need fewer rounds' worth of work -- e.g. N = 2560 at M = 4096
// is 160 tiles of 256 but 256 tiles of 160, one per CU.  128x128 tiles for
// M <= 128.
hipError_t launch_gemm(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                       const uint8_t* packed, const float* ws, int64_t N, Epi epi, float* Y,
                       int32_t* acc_out, hipStream_t s) {
    if (M > 128) {
        const int64_t cus = cu_count();
        const int64_t mt = (M + 255) / 256;
        const int64_t r256 = (mt * ((N + 255) / 256) + cus - 1) / cus;
        const int64_t r160 = (mt * ((N + 159) / 160) + cus - 1) / cus;
        if (r160 * 160 * 10 < r256 * 256 * 9)
            return launch_pipe<256, 160, 4, 2, 4, 1>(Xq, xs, rs, M, K, packed, ws, N, epi, Y, acc_out, s);
        return launch_pipe<256, 256, 2, 4, 4, 1>(Xq, xs, rs, M, K, packed, ws, N, epi, Y, acc_out, s);
    }
    return launch_pipe<128, 128, 2, 2, 4, 1>(Xq, xs, rs, M, K, packed, ws, N, epi, Y, acc_out, s);
}

hipError_t launch_contract(const int8_t* Xq, const float* x_scale, const int32_t* rowsum,
                           int64_t M, int64_t K, const uint8_t* packed, const float* w_scale,
                           int64_t N, Epi epi, float* Y, int32_t* acc_out, hipStream_t s) {
    if (gemv_supported(M, K, N))
        return launch_gemv(Xq, x_scale, rowsum, M, K, packed, w_scale, N, epi, Y, acc_out, s);
    return launch_gemm(Xq, x_scale, rowsum, M, K, packed, w_scale, N, epi, Y, acc_out, s);
}

}  // namespace bl
