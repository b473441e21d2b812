// Measurement support, not part of the BitLinear path: a plain streaming
// read of a device buffer, the read-bandwidth reference that decode
// throughput is set beside.  Each workgroup reads one contiguous share of the
// buffer, 8 sixteen-byte non-temporal loads per thread in flight, and folds
// the words with XOR so the loads cannot be dropped.  Raw buffer loads: an
// offset past the buffer reads zero, so the last share needs no bounds test.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr uint32_t kStep = kThreads * 16u * kUnroll;  // bytes per workgroup iteration

__global__ __launch_bounds__(kThreads) void k_stream_read(const uint8_t* buf, uint32_t bytes, uint32_t share,
                                                          uint32_t* sink) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf), (short)0,
                                                                       (int)bytes, 0x00020000);
    uint32_t acc = 0;
    const uint32_t b0 = blockIdx.x * share;
    for (uint32_t off = b0; off < b0 + share; off += kStep) {
        uint4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 r, off + (uint32_t)(u * kThreads + threadIdx.x) * 16u, 0, 2));
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x % 1024] = acc;  // practically never: keeps the reads live
}

}  // namespace

// Reads `bytes` (a multiple of 256 MiB, at most 2 GiB) of `buf` once on
// `stream` with 8192 workgroups, each byte by exactly one load.  sink: device buffer of 1024 uint32 (written
// only in the unlikely event that a share's XOR equals a fixed constant).
// Returns 0, -2 for a bad size, -5 for a launch error.
extern "C" int blbench_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t stream) {
    constexpr uint32_t kBlocks = 8192;
    if (bytes == 0 || bytes % (256ull << 20) != 0 || bytes > (2ull << 30)) return -2;
    const uint32_t share = (uint32_t)(bytes / kBlocks);  // a multiple of kStep: 32 KiB per 256 MiB
    hipLaunchKernelGGL(k_stream_read, dim3(kBlocks), dim3(kThreads), 0, stream,
                       static_cast<const uint8_t*>(buf), (uint32_t)bytes, share, sink);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
