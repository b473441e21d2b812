// C ABI of libbitlinear: argument validation, workspace carving and kernel
// dispatch.  Every check runs before the first launch, so a rejected call
// enqueues nothing.  See include/bitlinear.h for the contract of each call.
#include <stdarg.h>
#include <stdio.h>

#include "bitlinear.h"
#include "bl_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return BL_OK;
}

int hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return ok();
    return fail(BL_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int64_t kLimit = (int64_t)1 << 31;
constexpr size_t kWsAlign = 256;

size_t align_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Carves consecutive 256-byte aligned slices out of a workspace.
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <class T>
    T* take(size_t count) {
        T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
        off += align_up(count * sizeof(T));
        return p;
    }
};

int check_k(int64_t K, const char* name) {
    if (K < 64 || K % 64 != 0)
        return fail(BL_ERR_SHAPE, "%s = %lld must be a positive multiple of 64", name, (long long)K);
    return BL_OK;
}

int check_workspace(void* ws, size_t have, size_t need) {
    if (need == 0) return BL_OK;
    if (ws == nullptr) return fail(BL_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (!aligned(ws, kWsAlign)) return fail(BL_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (have < need) return fail(BL_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", have, need);
    return BL_OK;
}

size_t forward_ws(int64_t M, int64_t N, bool need_rowsum, bool need_y) {
    Carver c(nullptr);
    if (need_rowsum) c.take<int32_t>((size_t)M);
    if (need_y) c.take<float>((size_t)(M * N));
    return c.off;
}

size_t ffn_ws(int64_t M, int64_t H, int64_t F) {
    Carver c(nullptr);
    c.take<int8_t>((size_t)(M * H));
    c.take<float>((size_t)M);
    c.take<int32_t>((size_t)M);
    c.take<float>((size_t)(M * F));
    c.take<int8_t>((size_t)(M * F));
    c.take<float>((size_t)M);
    c.take<int32_t>((size_t)M);
    return c.off;
}

// The contraction kernels' epilogue from the public one: ReLU^2, then the
// residual add or the gating product (their common operand is aux).
bl::Epi kernel_epi(const bl_epilogue* epi) {
    if (!epi) return bl::Epi{0u, nullptr};
    uint32_t k = 0;
    const float* aux = nullptr;
    if (epi->flags & BL_EPI_RELU2) k |= bl::kEpiRelu2;
    if (epi->flags & BL_EPI_RESIDUAL) {
        k |= bl::kEpiResidual;
        aux = epi->residual;
    }
    if (epi->flags & BL_EPI_MUL) {
        k |= bl::kEpiMul;
        aux = epi->mul_by;
    }
    return bl::Epi{k, aux};
}

// Checks shared by forward and quant_forward for the residual / product operands.
int check_aux(const bl_epilogue* epi, uint32_t flags, const char* who) {
    if ((flags & BL_EPI_RESIDUAL) && (flags & BL_EPI_MUL))
        return fail(BL_ERR_UNSUPPORTED, "%s: BL_EPI_RESIDUAL and BL_EPI_MUL together", who);
    if ((flags & BL_EPI_RESIDUAL) && !epi->residual)
        return fail(BL_ERR_NULL, "%s: BL_EPI_RESIDUAL needs epi->residual", who);
    if ((flags & BL_EPI_MUL) && !epi->mul_by) return fail(BL_ERR_NULL, "%s: BL_EPI_MUL needs epi->mul_by", who);
    if (((flags & BL_EPI_RESIDUAL) && !aligned(epi->residual, 16)) ||
        ((flags & BL_EPI_MUL) && !aligned(epi->mul_by, 16)))
        return fail(BL_ERR_ALIGN, "%s: residual / mul_by need 16-byte alignment", who);
    return BL_OK;
}

}  // namespace

extern "C" {

const char* bitlinear_status_string(int status) {
    switch (status) {
        case BL_OK: return "ok";
        case BL_ERR_NULL: return "required pointer is NULL";
        case BL_ERR_SHAPE: return "invalid shape";
        case BL_ERR_ALIGN: return "misaligned pointer";
        case BL_ERR_WORKSPACE: return "workspace missing or too small";
        case BL_ERR_HIP: return "HIP runtime error";
        case BL_ERR_UNSUPPORTED: return "unsupported request";
        default: return "unknown status";
    }
}

const char* bitlinear_last_error(void) { return g_last_error; }

int bitlinear_abi_version(void) { return BITLINEAR_ABI_VERSION; }

// ---------------------------------------------------------------- packing

size_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K) {
    if (N < 1 || K < 1) return 0;
    return align_up(sizeof(double) * (size_t)bl::pack_partial_blocks(N * K));
}

int bitlinear_pack_weights(const float* W, int64_t N, int64_t K, uint8_t* packed, float* w_scale,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!W || !packed || !w_scale) return fail(BL_ERR_NULL, "pack: W, packed and w_scale are required");
    if (N < 1) return fail(BL_ERR_SHAPE, "pack: N = %lld must be >= 1", (long long)N);
    if (int r = check_k(K, "pack: K")) return r;
    if (N * K >= kLimit * 4) return fail(BL_ERR_SHAPE, "pack: N*K too large");
    if (!aligned(W, 16) || !aligned(packed, 16) || !aligned(w_scale, 4))
        return fail(BL_ERR_ALIGN, "pack: W and packed need 16-byte alignment, w_scale 4-byte");
    if (int r = check_workspace(ws, ws_bytes, bitlinear_pack_workspace_bytes(N, K))) return r;
    return hip_status(bl::launch_pack(W, false, N, K, packed, w_scale, static_cast<double*>(ws), stream),
                      "pack");
}

// ---------------------------------------------------------------- quantiser

int bitlinear_quant_act(const float* X, int64_t M, int64_t K, uint32_t flags, const float* norm_gain,
                        float norm_eps, int8_t* Xq, float* x_scale, int32_t* x_rowsum,
                        hipStream_t stream) {
    if (!X || !Xq || !x_scale) return fail(BL_ERR_NULL, "quant: X, Xq and x_scale are required");
    if (flags & ~BL_QUANT_RMSNORM) return fail(BL_ERR_UNSUPPORTED, "quant: unknown flags 0x%x", flags);
    if (M < 0) return fail(BL_ERR_SHAPE, "quant: M = %lld must be >= 0", (long long)M);
    if (int r = check_k(K, "quant: K")) return r;
    if (!bl::quant_supported(K)) return fail(BL_ERR_UNSUPPORTED, "quant: K = %lld above 32768", (long long)K);
    if (M * K >= kLimit) return fail(BL_ERR_SHAPE, "quant: M*K too large");
    if (!aligned(X, 16) || !aligned(Xq, 16) || !aligned(x_scale, 4) || !aligned(x_rowsum, 4) ||
        !aligned(norm_gain, 16))
        return fail(BL_ERR_ALIGN, "quant: X, Xq, norm_gain need 16-byte alignment, scales 4-byte");
    if (M == 0) return ok();
    const bool rms = (flags & BL_QUANT_RMSNORM) != 0;
    return hip_status(bl::launch_quant(X, M, K, rms, rms ? norm_gain : nullptr, norm_eps, Xq,
                                       x_scale, x_rowsum, stream),
                      "quant");
}

// ---------------------------------------------------------------- forward

size_t bitlinear_forward_workspace_bytes(int64_t M, int64_t K, int64_t N, uint32_t epi_flags) {
    (void)K;
    if (M < 1 || N < 1) return 0;
    // Conservative: room for the row sums and for the ReLU^2 output when the
    // caller gives no Y with BL_EPI_SUBLN_QUANT.
    return forward_ws(M, N, true, (epi_flags & BL_EPI_SUBLN_QUANT) != 0);
}

int bitlinear_forward(const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum, int64_t M,
                      int64_t K, const uint8_t* packed, const float* w_scale, int64_t N,
                      const bl_epilogue* epi, float* Y, int32_t* acc_out, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
    const uint32_t flags = epi ? epi->flags : 0u;
    const bool subln = (flags & BL_EPI_SUBLN_QUANT) != 0;
    if (!Xq || !x_scale || !packed || !w_scale)
        return fail(BL_ERR_NULL, "forward: Xq, x_scale, packed and w_scale are required");
    if (flags & ~(BL_EPI_RELU2 | BL_EPI_RESIDUAL | BL_EPI_SUBLN_QUANT | BL_EPI_MUL))
        return fail(BL_ERR_UNSUPPORTED, "forward: unknown epilogue flags 0x%x", flags);
    if (!Y && !subln) return fail(BL_ERR_NULL, "forward: Y is required without BL_EPI_SUBLN_QUANT");
    if (int r = epi ? check_aux(epi, flags, "forward") : BL_OK) return r;
    if (subln && (!epi->out_q || !epi->out_q_scale))
        return fail(BL_ERR_NULL, "forward: BL_EPI_SUBLN_QUANT needs out_q and out_q_scale");
    if (M < 0) return fail(BL_ERR_SHAPE, "forward: M = %lld must be >= 0", (long long)M);
    if (N < 1) return fail(BL_ERR_SHAPE, "forward: N = %lld must be >= 1", (long long)N);
    if (int r = check_k(K, "forward: K")) return r;
    if (subln) {
        if (int r = check_k(N, "forward: N (BL_EPI_SUBLN_QUANT)")) return r;
        if (!bl::quant_supported(N))
            return fail(BL_ERR_UNSUPPORTED, "forward: N = %lld above 32768 with subln", (long long)N);
    }
    if (M * K >= kLimit || M * N >= kLimit || N * K >= kLimit * 4)
        return fail(BL_ERR_SHAPE, "forward: sizes exceed 2^31 elements");
    if (!aligned(Xq, 16) || !aligned(packed, 16) || !aligned(Y, 16) || !aligned(acc_out, 16) ||
        !aligned(x_scale, 4) || !aligned(x_rowsum, 4) || !aligned(w_scale, 4))
        return fail(BL_ERR_ALIGN, "forward: Xq, packed, Y, acc_out need 16-byte alignment, scales 4-byte");
    if (subln && (!aligned(epi->out_q, 16) || !aligned(epi->out_q_scale, 4) ||
                  !aligned(epi->out_q_rowsum, 4) || !aligned(epi->norm_gain, 16)))
        return fail(BL_ERR_ALIGN, "forward: subln outputs/gain misaligned");
    const bool need_rowsum = (x_rowsum == nullptr);
    const bool need_y = subln && (Y == nullptr);
    if (int r = check_workspace(ws, ws_bytes, M == 0 ? 0 : forward_ws(M, N, need_rowsum, need_y)))
        return r;
    if (M == 0) return ok();

    Carver c(ws);
    int32_t* rs = need_rowsum ? c.take<int32_t>((size_t)M) : const_cast<int32_t*>(x_rowsum);
    float* y = need_y ? c.take<float>((size_t)(M * N)) : Y;
    hipError_t e = hipSuccess;
    if (need_rowsum) {
        e = bl::launch_rowsum(Xq, M, K, rs, stream);
        if (e != hipSuccess) return hip_status(e, "forward: rowsum");
    }
    e = bl::launch_contract(Xq, x_scale, rs, M, K, packed, w_scale, N, kernel_epi(epi), y, acc_out, stream);
    if (e != hipSuccess) return hip_status(e, "forward: contraction");
    if (subln) {
        e = bl::launch_quant(y, M, N, true, epi->norm_gain, epi->norm_eps, epi->out_q,
                             epi->out_q_scale, epi->out_q_rowsum, stream);
        if (e != hipSuccess) return hip_status(e, "forward: subln requant");
    }
    return ok();
}

// ---------------------------------------------------------------- fused quant + forward

size_t bitlinear_quant_forward_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    (void)N;
    if (M < 1 || K < 1) return 0;
    Carver c(nullptr);
    c.take<int8_t>((size_t)(M * K));
    c.take<float>((size_t)M);
    c.take<int32_t>((size_t)M);
    return c.off;
}

}  // extern "C"

namespace {
// Checks shared by bitlinear_quant_forward and bitlinear_latent_forward (the
// weight operand is checked by each caller).
int check_quant_forward(const char* who, const float* X, int64_t M, int64_t K, uint32_t quant_flags,
                        const float* norm_gain, int64_t N, const bl_epilogue* epi, float* Y) {
    const uint32_t flags = epi ? epi->flags : 0u;
    if (!X || !Y) return fail(BL_ERR_NULL, "%s: X and Y are required", who);
    if (quant_flags & ~BL_QUANT_RMSNORM) return fail(BL_ERR_UNSUPPORTED, "%s: unknown quant flags 0x%x", who, quant_flags);
    if (flags & ~(BL_EPI_RELU2 | BL_EPI_RESIDUAL | BL_EPI_MUL))
        return fail(BL_ERR_UNSUPPORTED, "%s: epilogue flags 0x%x not supported", who, flags);
    if (int r = epi ? check_aux(epi, flags, who) : BL_OK) return r;
    if (M < 0) return fail(BL_ERR_SHAPE, "%s: M = %lld must be >= 0", who, (long long)M);
    if (N < 1) return fail(BL_ERR_SHAPE, "%s: N = %lld must be >= 1", who, (long long)N);
    if (K < 64 || K % 64 != 0)
        return fail(BL_ERR_SHAPE, "%s: K = %lld must be a positive multiple of 64", who, (long long)K);
    if (!bl::quant_supported(K)) return fail(BL_ERR_UNSUPPORTED, "%s: K = %lld above 32768", who, (long long)K);
    if (M * K >= kLimit || M * N >= kLimit || N * K >= kLimit * 4)
        return fail(BL_ERR_SHAPE, "%s: sizes exceed 2^31 elements", who);
    if (!aligned(X, 16) || !aligned(Y, 16) || !aligned(norm_gain, 16))
        return fail(BL_ERR_ALIGN, "%s: X, Y, gain need 16-byte alignment", who);
    return BL_OK;
}

// Quantise X and run the BitLinear on packed weights: one fused launch for
// M <= 4 (no workspace), else the quantiser into `ws` then the contraction.
int run_quant_forward(const char* who, const float* X, int64_t M, int64_t K, uint32_t quant_flags,
                      const float* norm_gain, float norm_eps, const uint8_t* packed, const float* w_scale, int64_t N,
                      const bl_epilogue* epi, float* Y, void* ws, hipStream_t stream) {
    const bool rms = (quant_flags & BL_QUANT_RMSNORM) != 0;
    const bl::Epi ke = kernel_epi(epi);
    if (bl::decode_supported(M, K, N))
        return hip_status(bl::launch_decode_bitlinear(X, M, K, rms, rms ? norm_gain : nullptr, norm_eps, packed,
                                                      w_scale, N, ke.flags, ke.aux, Y, stream),
                          who);
    Carver c(ws);
    int8_t* xq = c.take<int8_t>((size_t)(M * K));
    float* xs = c.take<float>((size_t)M);
    int32_t* rs = c.take<int32_t>((size_t)M);
    hipError_t e = bl::launch_quant(X, M, K, rms, rms ? norm_gain : nullptr, norm_eps, xq, xs, rs, stream);
    if (e != hipSuccess) return hip_status(e, who);
    return hip_status(bl::launch_contract(xq, xs, rs, M, K, packed, w_scale, N, ke, Y, nullptr, stream), who);
}

size_t quant_forward_ws(int64_t M, int64_t K, int64_t N) {
    if (M < 1 || K < 1 || bl::decode_supported(M, K, N)) return 0;
    Carver c(nullptr);
    c.take<int8_t>((size_t)(M * K));
    c.take<float>((size_t)M);
    c.take<int32_t>((size_t)M);
    return c.off;
}
}  // namespace

extern "C" {

int bitlinear_quant_forward(const float* X, int64_t M, int64_t K, uint32_t quant_flags, const float* norm_gain,
                            float norm_eps, const uint8_t* packed, const float* w_scale, int64_t N,
                            const bl_epilogue* epi, float* Y, void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* who = "quant_forward";
    if (int r = check_quant_forward(who, X, M, K, quant_flags, norm_gain, N, epi, Y)) return r;
    if (!packed || !w_scale) return fail(BL_ERR_NULL, "quant_forward: packed and w_scale are required");
    if (!aligned(packed, 16) || !aligned(w_scale, 4))
        return fail(BL_ERR_ALIGN, "quant_forward: packed needs 16-byte alignment, w_scale 4-byte");
    if (int r = check_workspace(ws, ws_bytes, M == 0 ? 0 : quant_forward_ws(M, K, N))) return r;
    if (M == 0) return ok();
    return run_quant_forward(who, X, M, K, quant_flags, norm_gain, norm_eps, packed, w_scale, N, epi, Y, ws, stream);
}

// ---------------------------------------------------------------- forward from latent weights

size_t bitlinear_latent_forward_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M < 1 || K < 1 || N < 1) return 0;
    Carver c(nullptr);
    c.take<uint8_t>((size_t)(N * K / 4));
    c.take<float>(1);
    c.take<double>((size_t)bl::pack_partial_blocks(N * K));
    c.take<uint8_t>(quant_forward_ws(M, K, N));
    return c.off;
}

int bitlinear_latent_forward(const float* X, int64_t M, int64_t K, uint32_t quant_flags, const float* norm_gain,
                             float norm_eps, const void* W, uint32_t w_dtype, int64_t N, const bl_epilogue* epi,
                             float* Y, float* w_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* who = "latent_forward";
    if (int r = check_quant_forward(who, X, M, K, quant_flags, norm_gain, N, epi, Y)) return r;
    if (!W) return fail(BL_ERR_NULL, "latent_forward: W is required");
    if (w_dtype != BL_DTYPE_F32 && w_dtype != BL_DTYPE_BF16)
        return fail(BL_ERR_UNSUPPORTED, "latent_forward: w_dtype %u is neither BL_DTYPE_F32 nor BL_DTYPE_BF16", w_dtype);
    if (!aligned(W, 16) || !aligned(w_scale, 4))
        return fail(BL_ERR_ALIGN, "latent_forward: W needs 16-byte alignment, w_scale 4-byte");
    if (int r = check_workspace(ws, ws_bytes, M == 0 ? 0 : bitlinear_latent_forward_workspace_bytes(M, K, N)))
        return r;
    if (M == 0) return ok();
    Carver c(ws);
    uint8_t* packed = c.take<uint8_t>((size_t)(N * K / 4));
    float* gw = c.take<float>(1);
    double* partial = c.take<double>((size_t)bl::pack_partial_blocks(N * K));
    void* qws = c.take<uint8_t>(quant_forward_ws(M, K, N));
    if (w_scale) gw = w_scale;
    hipError_t e = bl::launch_pack(W, w_dtype == BL_DTYPE_BF16, N, K, packed, gw, partial, stream);
    if (e != hipSuccess) return hip_status(e, "latent_forward: pack");
    return run_quant_forward(who, X, M, K, quant_flags, norm_gain, norm_eps, packed, gw, N, epi, Y, qws, stream);
}

// ---------------------------------------------------------------- FFN stack

size_t bitnet_ffn_workspace_bytes(int64_t M, int64_t H, int64_t F) {
    if (M < 1 || H < 1 || F < 1) return 0;
    return ffn_ws(M, H, F);
}

int bitnet_ffn_forward(const bitnet_ffn_layer* layers, int32_t n_layers, float* hidden, int64_t M,
                       int64_t H, int64_t F, uint32_t flags, float norm_eps, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
    if (!hidden) return fail(BL_ERR_NULL, "ffn: hidden is required");
    if (n_layers < 0) return fail(BL_ERR_SHAPE, "ffn: n_layers = %d must be >= 0", n_layers);
    if (n_layers > 0 && !layers) return fail(BL_ERR_NULL, "ffn: layers is required");
    if (flags & ~(BL_FFN_PRE_NORM | BL_FFN_RESIDUAL))
        return fail(BL_ERR_UNSUPPORTED, "ffn: unknown flags 0x%x", flags);
    if (M < 0) return fail(BL_ERR_SHAPE, "ffn: M = %lld must be >= 0", (long long)M);
    if (int r = check_k(H, "ffn: H")) return r;
    if (int r = check_k(F, "ffn: F")) return r;
    if (!bl::quant_supported(H) || !bl::quant_supported(F))
        return fail(BL_ERR_UNSUPPORTED, "ffn: H and F must be <= 32768");
    if (M * H >= kLimit || M * F >= kLimit || H * F >= kLimit * 4)
        return fail(BL_ERR_SHAPE, "ffn: sizes exceed 2^31 elements");
    if (!aligned(hidden, 16)) return fail(BL_ERR_ALIGN, "ffn: hidden needs 16-byte alignment");
    for (int32_t l = 0; l < n_layers; ++l) {
        const bitnet_ffn_layer& L = layers[l];
        if (!L.up || !L.up_scale || !L.down || !L.down_scale)
            return fail(BL_ERR_NULL, "ffn: layer %d: up/down weights and scales are required", l);
        if ((L.gate != nullptr) != (L.gate_scale != nullptr))
            return fail(BL_ERR_NULL, "ffn: layer %d: gate and gate_scale go together", l);
        if (!aligned(L.up, 16) || !aligned(L.down, 16) || !aligned(L.up_scale, 4) ||
            !aligned(L.down_scale, 4) || !aligned(L.pre_norm_gain, 16) || !aligned(L.sub_norm_gain, 16) ||
            !aligned(L.gate, 16) || !aligned(L.gate_scale, 4))
            return fail(BL_ERR_ALIGN, "ffn: layer %d: misaligned pointer", l);
    }
    if (int r = check_workspace(ws, ws_bytes, M == 0 || n_layers == 0 ? 0 : ffn_ws(M, H, F))) return r;
    if (M == 0 || n_layers == 0) return ok();

    Carver c(ws);
    int8_t* xq1 = c.take<int8_t>((size_t)(M * H));
    float* s1 = c.take<float>((size_t)M);
    int32_t* rs1 = c.take<int32_t>((size_t)M);
    float* y1 = c.take<float>((size_t)(M * F));
    int8_t* xq2 = c.take<int8_t>((size_t)(M * F));
    float* s2 = c.take<float>((size_t)M);
    int32_t* rs2 = c.take<int32_t>((size_t)M);
    const bool pre = (flags & BL_FFN_PRE_NORM) != 0;
    const bool res = (flags & BL_FFN_RESIDUAL) != 0;

    // Few tokens: two launches per layer, each quantising its own input rows
    // (a gated layer streams gate and up in the first one).
    if (bl::decode_supported(M, H, F) && bl::decode_supported(M, F, H)) {
        for (int32_t l = 0; l < n_layers; ++l) {
            const bitnet_ffn_layer& L = layers[l];
            hipError_t e = L.gate ? bl::launch_decode_gated(hidden, M, H, pre, L.pre_norm_gain, norm_eps, L.up,
                                                            L.up_scale, L.gate, L.gate_scale, F, y1, stream)
                                  : bl::launch_decode_bitlinear(hidden, M, H, pre, L.pre_norm_gain, norm_eps, L.up,
                                                                L.up_scale, F, bl::kEpiRelu2, nullptr, y1, stream);
            if (e != hipSuccess) return hip_status(e, "ffn: decode up/gate");
            e = bl::launch_decode_bitlinear(y1, M, F, true, L.sub_norm_gain, norm_eps, L.down, L.down_scale, H,
                                            res ? bl::kEpiResidual : 0u, res ? hidden : nullptr, hidden, stream);
            if (e != hipSuccess) return hip_status(e, "ffn: decode down");
        }
        return ok();
    }

    for (int32_t l = 0; l < n_layers; ++l) {
        const bitnet_ffn_layer& L = layers[l];
        hipError_t e = bl::launch_quant(hidden, M, H, pre, pre ? L.pre_norm_gain : nullptr, norm_eps,
                                        xq1, s1, rs1, stream);
        if (e != hipSuccess) return hip_status(e, "ffn: input quant");
        const bool gated = L.gate != nullptr;
        if (gated && bl::gemv_supported(M, H, F)) {
            // few tokens: gate and up streamed by one launch
            e = bl::launch_gemv_gated(xq1, s1, rs1, M, H, L.up, L.up_scale, L.gate, L.gate_scale, F, y1, stream);
            if (e != hipSuccess) return hip_status(e, "ffn: gate and up");
        } else {
            e = bl::launch_contract(xq1, s1, rs1, M, H, L.up, L.up_scale, F,
                                    bl::Epi{gated ? 0u : bl::kEpiRelu2, nullptr}, y1, nullptr, stream);
            if (e != hipSuccess) return hip_status(e, "ffn: up");
        }
        if (gated && !bl::gemv_supported(M, H, F)) {
            e = bl::launch_contract(xq1, s1, rs1, M, H, L.gate, L.gate_scale, F,
                                    bl::Epi{bl::kEpiRelu2 | bl::kEpiMul, y1}, y1, nullptr, stream);
            if (e != hipSuccess) return hip_status(e, "ffn: gate");
        }
        e = bl::launch_quant(y1, M, F, true, L.sub_norm_gain, norm_eps, xq2, s2, rs2, stream);
        if (e != hipSuccess) return hip_status(e, "ffn: subln requant");
        e = bl::launch_contract(xq2, s2, rs2, M, F, L.down, L.down_scale, H,
                                bl::Epi{res ? bl::kEpiResidual : 0u, res ? hidden : nullptr}, hidden,
                                nullptr, stream);
        if (e != hipSuccess) return hip_status(e, "ffn: down");
    }
    return ok();
}

}  // extern "C"
