// C ABI of libbitlinear: argument validation, workspace carving and kernel
// dispatch.  Every check runs before the first launch, so a rejected call
// enqueues nothing.  See include/bitlinear.h for the contract of each call.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

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

// Whether the byte ranges [a, a + na) and [b, b + nb) share a byte (NULL or
// empty ranges share none).
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

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
    c.take<uint8_t>(bl::stack_ws_bytes());  // the persistent launch's layer descriptors and counter
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

// ---------------------------------------------------------------- packed-layout conversion

}  // extern "C"

namespace {
int check_layout(const char* who, const void* in, size_t in_align, const void* out, size_t out_align,
                 size_t out_elem, int64_t N, int64_t K) {
    if (!in || !out) return fail(BL_ERR_NULL, "%s: input and output are required", who);
    if (N < 1) return fail(BL_ERR_SHAPE, "%s: N = %lld must be >= 1", who, (long long)N);
    if (K < 64 || K % 64 != 0)
        return fail(BL_ERR_SHAPE, "%s: K = %lld must be a positive multiple of 64", who, (long long)K);
    if (N * K >= kLimit * 4) return fail(BL_ERR_SHAPE, "%s: N*K too large", who);
    if (!aligned(in, in_align) || !aligned(out, out_align))
        return fail(BL_ERR_ALIGN, "%s: input needs %zu-byte, output %zu-byte alignment", who, in_align, out_align);
    if (overlap(in, (size_t)(N * K / 4), out, (size_t)(N * K) * out_elem / 4))
        return fail(BL_ERR_UNSUPPORTED, "%s: input and output overlap", who);
    return BL_OK;
}
}  // namespace

extern "C" {

int bitlinear_import_canonical(const uint8_t* canonical, int64_t N, int64_t K, uint8_t* packed,
                               hipStream_t stream) {
    if (int r = check_layout("import_canonical", canonical, 4, packed, 16, 1, N, K)) return r;
    return hip_status(bl::launch_relayout(canonical, N, K, true, packed, stream), "import_canonical");
}

int bitlinear_export_canonical(const uint8_t* packed, int64_t N, int64_t K, uint8_t* canonical,
                               hipStream_t stream) {
    if (int r = check_layout("export_canonical", packed, 16, canonical, 4, 1, N, K)) return r;
    return hip_status(bl::launch_relayout(packed, N, K, false, canonical, stream), "export_canonical");
}

int bitlinear_unpack_weights(const uint8_t* packed, int64_t N, int64_t K, int8_t* q, hipStream_t stream) {
    if (int r = check_layout("unpack_weights", packed, 16, q, 16, 4, N, K)) return r;
    return hip_status(bl::launch_unpack(packed, N, K, q, stream), "unpack_weights");
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
    {
        const void* outs[3] = {Xq, x_scale, x_rowsum};
        const size_t ob[3] = {(size_t)(M * K), (size_t)M * 4, (size_t)M * 4};
        for (int o = 0; o < 3; ++o) {
            if (overlap(outs[o], ob[o], X, (size_t)(M * K) * 4) ||
                overlap(outs[o], ob[o], (flags & BL_QUANT_RMSNORM) ? norm_gain : nullptr, (size_t)K * 4))
                return fail(BL_ERR_UNSUPPORTED, "quant: an output overlaps X or the norm gain");
            for (int o2 = o + 1; o2 < 3; ++o2)
                if (overlap(outs[o], ob[o], outs[o2], ob[o2]))
                    return fail(BL_ERR_UNSUPPORTED, "quant: two outputs overlap");
        }
    }
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

}  // extern "C"

namespace {
// Every check of bitlinear_forward but the workspace: null pointers, flags,
// shapes, alignment, and no output overlapping an input or another output
// (Y may equal residual / mul_by).
int check_forward(const char* who, const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum, int64_t M,
                  int64_t K, const uint8_t* packed, const float* w_scale, int64_t N, const bl_epilogue* epi,
                  float* Y, int32_t* acc_out) {
    const uint32_t flags = epi ? epi->flags : 0u;
    const bool subln = (flags & BL_EPI_SUBLN_QUANT) != 0;
    if (!Xq || !x_scale || !packed || !w_scale)
        return fail(BL_ERR_NULL, "%s: Xq, x_scale, packed and w_scale are required", who);
    if (flags & ~(BL_EPI_RELU2 | BL_EPI_RESIDUAL | BL_EPI_SUBLN_QUANT | BL_EPI_MUL))
        return fail(BL_ERR_UNSUPPORTED, "%s: unknown epilogue flags 0x%x", who, flags);
    if (!Y && !subln) return fail(BL_ERR_NULL, "%s: Y is required without BL_EPI_SUBLN_QUANT", who);
    if (int r = epi ? check_aux(epi, flags, who) : BL_OK) return r;
    if (subln && (!epi->out_q || !epi->out_q_scale))
        return fail(BL_ERR_NULL, "%s: BL_EPI_SUBLN_QUANT needs out_q and out_q_scale", who);
    if (M < 0) return fail(BL_ERR_SHAPE, "%s: M = %lld must be >= 0", who, (long long)M);
    if (N < 1) return fail(BL_ERR_SHAPE, "%s: N = %lld must be >= 1", who, (long long)N);
    if (K < 64 || K % 64 != 0)
        return fail(BL_ERR_SHAPE, "%s: K = %lld must be a positive multiple of 64", who, (long long)K);
    if (subln) {
        if (N < 64 || N % 64 != 0)
            return fail(BL_ERR_SHAPE, "%s: N = %lld must be a positive multiple of 64 with subln", who,
                        (long long)N);
        if (!bl::quant_supported(N))
            return fail(BL_ERR_UNSUPPORTED, "%s: N = %lld above 32768 with subln", who, (long long)N);
    }
    if (M * K >= kLimit || M * N >= kLimit || N * K >= kLimit * 4)
        return fail(BL_ERR_SHAPE, "%s: sizes exceed 2^31 elements", who);
    if (!aligned(Xq, 16) || !aligned(packed, 16) || !aligned(Y, 16) || !aligned(acc_out, 16) ||
        !aligned(x_scale, 4) || !aligned(x_rowsum, 4) || !aligned(w_scale, 4))
        return fail(BL_ERR_ALIGN, "%s: Xq, packed, Y, acc_out need 16-byte alignment, scales 4-byte", who);
    if (subln && (!aligned(epi->out_q, 16) || !aligned(epi->out_q_scale, 4) ||
                  !aligned(epi->out_q_rowsum, 4) || !aligned(epi->norm_gain, 16)))
        return fail(BL_ERR_ALIGN, "%s: subln outputs/gain misaligned", who);
    {
        const size_t xb = (size_t)(M * K), yb = (size_t)(M * N) * 4, wb = (size_t)(N * K / 4);
        const void* outs[5] = {Y, acc_out, subln ? epi->out_q : nullptr, subln ? epi->out_q_scale : nullptr,
                               subln ? epi->out_q_rowsum : nullptr};
        const size_t ob[5] = {yb, yb, (size_t)(M * N), (size_t)M * 4, (size_t)M * 4};
        const void* ins[5] = {Xq, x_scale, x_rowsum, packed, w_scale};
        const size_t ib[5] = {xb, (size_t)M * 4, (size_t)M * 4, wb, 4};
        const float* aux = (flags & BL_EPI_RESIDUAL) ? epi->residual : (flags & BL_EPI_MUL) ? epi->mul_by : nullptr;
        for (int o = 0; o < 5; ++o) {
            for (int i = 0; i < 5; ++i)
                if (overlap(outs[o], ob[o], ins[i], ib[i]))
                    return fail(BL_ERR_UNSUPPORTED, "%s: an output overlaps an input", who);
            for (int o2 = o + 1; o2 < 5; ++o2)
                if (overlap(outs[o], ob[o], outs[o2], ob[o2]))
                    return fail(BL_ERR_UNSUPPORTED, "%s: two outputs overlap", who);
            if (aux && !(o == 0 && outs[o] == aux) && overlap(outs[o], ob[o], aux, yb))
                return fail(BL_ERR_UNSUPPORTED, "%s: an output overlaps residual / mul_by (only Y == it is allowed)",
                            who);
        }
    }
    return BL_OK;
}
}  // namespace

extern "C" {

int bitlinear_forward(const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum, int64_t M,
                      int64_t K, const uint8_t* packed, const float* w_scale, int64_t N,
                      const bl_epilogue* epi, float* Y, int32_t* acc_out, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
    if (int r = check_forward("forward", Xq, x_scale, x_rowsum, M, K, packed, w_scale, N, epi, Y, acc_out))
        return r;
    const uint32_t flags = epi ? epi->flags : 0u;
    const bool subln = (flags & BL_EPI_SUBLN_QUANT) != 0;
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

// ---------------------------------------------------------------- grouped forward

}  // extern "C"

namespace {
// Every check of bitlinear_forward_grouped: each matrix as bitlinear_forward
// would check it, and no output of one matrix overlapping another's data.
int check_grouped(const char* who, const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum, int64_t M,
                  int64_t K, const bl_group* groups, int32_t n_groups) {
    if (n_groups < 1 || n_groups > BL_MAX_GROUPS)
        return fail(BL_ERR_UNSUPPORTED, "%s: n_groups = %d outside 1..%d", who, n_groups, BL_MAX_GROUPS);
    if (!groups) return fail(BL_ERR_NULL, "%s: groups is required", who);
    if (!x_rowsum) return fail(BL_ERR_NULL, "%s: x_rowsum is required", who);
    char what[64];
    for (int32_t g = 0; g < n_groups; ++g) {
        const bl_group& G = groups[g];
        snprintf(what, sizeof(what), "%s: matrix %d", who, g);
        if (!G.Y) return fail(BL_ERR_NULL, "%s: Y is required", what);
        if (int r = check_forward(what, Xq, x_scale, x_rowsum, M, K, G.packed, G.w_scale, G.N, &G.epi, G.Y,
                                  G.acc_out))
            return r;
    }
    // across matrices: no output of one may overlap another's inputs or outputs
    for (int32_t a = 0; a < n_groups; ++a)
        for (int32_t b = 0; b < n_groups; ++b) {
            if (a == b) continue;
            const bl_group& A = groups[a];
            const bl_group& B = groups[b];
            const bool sa = (A.epi.flags & BL_EPI_SUBLN_QUANT) != 0;
            const size_t ya = (size_t)(M * A.N) * 4, yb = (size_t)(M * B.N) * 4;
            const void* outs[5] = {A.Y, A.acc_out, sa ? A.epi.out_q : nullptr, sa ? A.epi.out_q_scale : nullptr,
                                   sa ? A.epi.out_q_rowsum : nullptr};
            const size_t ob[5] = {ya, ya, (size_t)(M * A.N), (size_t)M * 4, (size_t)M * 4};
            const bool sb = (B.epi.flags & BL_EPI_SUBLN_QUANT) != 0;
            const float* bx = (B.epi.flags & BL_EPI_RESIDUAL) ? B.epi.residual
                              : (B.epi.flags & BL_EPI_MUL) ? B.epi.mul_by : nullptr;
            const void* other[8] = {B.packed, B.w_scale, bx, B.Y, B.acc_out, sb ? B.epi.out_q : nullptr,
                                    sb ? B.epi.out_q_scale : nullptr, sb ? B.epi.out_q_rowsum : nullptr};
            const size_t otb[8] = {(size_t)(B.N * K / 4), 4, yb, yb, yb, (size_t)(M * B.N), (size_t)M * 4,
                                   (size_t)M * 4};
            for (int o = 0; o < 5; ++o)
                for (int i = 0; i < 8; ++i)
                    if (overlap(outs[o], ob[o], other[i], otb[i]))
                        return fail(BL_ERR_UNSUPPORTED, "%s: an output of matrix %d overlaps matrix %d's data", who,
                                    a, b);
        }
    return BL_OK;
}

void group_mats(const bl_group* groups, int32_t n_groups, bl::GroupMat (&mats)[BL_MAX_GROUPS]) {
    for (int32_t g = 0; g < n_groups; ++g) {
        const bl_group& G = groups[g];
        mats[g] = bl::GroupMat{G.packed, G.w_scale, G.N, kernel_epi(&G.epi), G.Y, G.acc_out};
    }
}

// The subln requant of every matrix that asks for it, after its contraction.
int grouped_requant(const char* who, int64_t M, const bl_group* groups, int32_t n_groups, hipStream_t stream) {
    for (int32_t g = 0; g < n_groups; ++g) {
        const bl_group& G = groups[g];
        if (!(G.epi.flags & BL_EPI_SUBLN_QUANT)) continue;
        hipError_t e = bl::launch_quant(G.Y, M, G.N, true, G.epi.norm_gain, G.epi.norm_eps, G.epi.out_q,
                                        G.epi.out_q_scale, G.epi.out_q_rowsum, stream);
        if (e != hipSuccess) return hip_status(e, who);
    }
    return ok();
}

// The contraction launches of a checked grouped forward from int8 rows: one
// launch when every matrix fits the skinny kernels, else one per matrix;
// then the subln requants.
int run_grouped(const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum, int64_t M, int64_t K,
                const bl_group* groups, int32_t n_groups, hipStream_t stream) {
    bl::GroupMat mats[BL_MAX_GROUPS];
    group_mats(groups, n_groups, mats);
    bool one_launch = n_groups <= bl::gemv_max_groups();
    for (int32_t g = 0; g < n_groups; ++g) one_launch = one_launch && bl::gemv_supported(M, K, mats[g].N);
    hipError_t e = hipSuccess;
    if (one_launch) {
        e = bl::launch_gemv_grouped(Xq, x_scale, x_rowsum, M, K, mats, n_groups, stream);
        if (e != hipSuccess) return hip_status(e, "forward_grouped: contraction");
    } else {
        for (int32_t g = 0; g < n_groups; ++g) {
            e = bl::launch_contract(Xq, x_scale, x_rowsum, M, K, mats[g].packed, mats[g].w_scale, mats[g].N,
                                    mats[g].epi, mats[g].Y, mats[g].acc_out, stream);
            if (e != hipSuccess) return hip_status(e, "forward_grouped: contraction");
        }
    }
    return grouped_requant("forward_grouped: subln requant", M, groups, n_groups, stream);
}

// A stand-in address for the workspace rows of a call with no rows.
alignas(256) char g_no_rows[16];

size_t quant_grouped_ws(int64_t M, int64_t K) {
    Carver c(nullptr);
    c.take<int8_t>((size_t)(M * K));
    c.take<float>((size_t)M);
    c.take<int32_t>((size_t)M);
    return c.off;
}
}  // namespace

extern "C" {

int bitlinear_forward_grouped(const int8_t* Xq, const float* x_scale, const int32_t* x_rowsum, int64_t M,
                              int64_t K, const bl_group* groups, int32_t n_groups, hipStream_t stream) {
    if (int r = check_grouped("forward_grouped", Xq, x_scale, x_rowsum, M, K, groups, n_groups)) return r;
    if (M == 0) return ok();
    return run_grouped(Xq, x_scale, x_rowsum, M, K, groups, n_groups, stream);
}

size_t bitlinear_quant_forward_grouped_workspace_bytes(int64_t M, int64_t K) {
    if (M < 1 || K < 1) return 0;
    return quant_grouped_ws(M, K);
}

int bitlinear_quant_forward_grouped(const float* X, int64_t M, int64_t K, uint32_t quant_flags,
                                    const float* norm_gain, float norm_eps, const bl_group* groups,
                                    int32_t n_groups, void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* who = "quant_forward_grouped";
    if (!X) return fail(BL_ERR_NULL, "%s: X is required", who);
    if (quant_flags & ~BL_QUANT_RMSNORM) return fail(BL_ERR_UNSUPPORTED, "%s: unknown quant flags 0x%x", who, quant_flags);
    if (M < 0) return fail(BL_ERR_SHAPE, "%s: M = %lld must be >= 0", who, (long long)M);
    if (K < 64 || K % 64 != 0)
        return fail(BL_ERR_SHAPE, "%s: K = %lld must be a positive multiple of 64", who, (long long)K);
    if (!bl::quant_supported(K)) return fail(BL_ERR_UNSUPPORTED, "%s: K = %lld above 32768", who, (long long)K);
    if (M * K >= kLimit) return fail(BL_ERR_SHAPE, "%s: sizes exceed 2^31 elements", who);
    if (!aligned(X, 16) || !aligned(norm_gain, 16)) return fail(BL_ERR_ALIGN, "%s: X and gain need 16-byte alignment", who);
    if (int r = check_workspace(ws, ws_bytes, M == 0 ? 0 : quant_grouped_ws(M, K))) return r;
    Carver c(ws);
    int8_t* xq = c.take<int8_t>((size_t)(M * K));
    float* xs = c.take<float>((size_t)M);
    int32_t* rs = c.take<int32_t>((size_t)M);
    if (M == 0) {  // no rows: nothing is read or written, only the checks run
        xq = reinterpret_cast<int8_t*>(g_no_rows);
        xs = reinterpret_cast<float*>(g_no_rows);
        rs = reinterpret_cast<int32_t*>(g_no_rows);
    }
    // the matrices against the quantised rows in the workspace, and X (and
    // the gain) against every output, which other workgroups write while
    // every workgroup still reads X
    if (int r = check_grouped(who, xq, xs, rs, M, K, groups, n_groups)) return r;
    const size_t xb = (size_t)(M * K) * 4;
    if (overlap(X, xb, ws, quant_grouped_ws(M, K)) || (norm_gain && overlap(norm_gain, (size_t)K * 4, ws, quant_grouped_ws(M, K))))
        return fail(BL_ERR_UNSUPPORTED, "%s: X or the gain overlaps the workspace", who);
    for (int32_t g = 0; g < n_groups; ++g) {
        const bl_group& G = groups[g];
        const bool sg = (G.epi.flags & BL_EPI_SUBLN_QUANT) != 0;
        const size_t yb = (size_t)(M * G.N) * 4;
        const void* outs[5] = {G.Y, G.acc_out, sg ? G.epi.out_q : nullptr, sg ? G.epi.out_q_scale : nullptr,
                               sg ? G.epi.out_q_rowsum : nullptr};
        const size_t ob[5] = {yb, yb, (size_t)(M * G.N), (size_t)M * 4, (size_t)M * 4};
        for (int o = 0; o < 5; ++o)
            if (overlap(outs[o], ob[o], X, xb) || (norm_gain && overlap(outs[o], ob[o], norm_gain, (size_t)K * 4)))
                return fail(BL_ERR_UNSUPPORTED, "%s: an output of matrix %d overlaps X or the gain", who, g);
    }
    if (M == 0) return ok();
    const bool rms = (quant_flags & BL_QUANT_RMSNORM) != 0;
    bl::GroupMat mats[BL_MAX_GROUPS];
    group_mats(groups, n_groups, mats);
    // the one launch also needs every matrix within the skinny kernels' 32-bit
    // output offsets (M * N < 2^29), as run_grouped's single launch does
    bool fused = bl::gemv_grouped_quant_supported(M, K, mats, n_groups);
    for (int32_t g = 0; g < n_groups; ++g) fused = fused && bl::gemv_supported(M, K, mats[g].N);
    if (fused) {
        hipError_t e = bl::launch_gemv_grouped_quant(X, M, K, rms, rms ? norm_gain : nullptr, norm_eps, mats,
                                                     n_groups, stream);
        if (e != hipSuccess) return hip_status(e, "quant_forward_grouped: contraction");
        return grouped_requant("quant_forward_grouped: subln requant", M, groups, n_groups, stream);
    }
    hipError_t e = bl::launch_quant(X, M, K, rms, rms ? norm_gain : nullptr, norm_eps, xq, xs, rs, stream);
    if (e != hipSuccess) return hip_status(e, "quant_forward_grouped: quantise");
    return run_grouped(xq, xs, rs, M, K, groups, n_groups, stream);
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
    // Every workgroup of the few-token launch reads all of X while others
    // write Y, so Y may not overlap X (or the gain); it may equal residual or
    // mul_by, and overlap them in no other way.
    const size_t yb = (size_t)(M * N) * 4;
    if (overlap(X, (size_t)(M * K) * 4, Y, yb) || overlap(norm_gain, (size_t)K * 4, Y, yb))
        return fail(BL_ERR_UNSUPPORTED, "%s: Y overlaps X or the norm gain", who);
    const float* aux = (flags & BL_EPI_RESIDUAL) ? epi->residual : (flags & BL_EPI_MUL) ? epi->mul_by : nullptr;
    if (aux && aux != Y && overlap(aux, yb, Y, yb))
        return fail(BL_ERR_UNSUPPORTED, "%s: Y overlaps residual / mul_by (only Y == it is allowed)", who);
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

}  // extern "C"

namespace {
// Everything bitnet_ffn_forward checks before its workspace.
int ffn_check(const bitnet_ffn_layer* layers, int32_t n_layers, float* hidden, int64_t M, int64_t H, int64_t F,
              uint32_t flags) {
    if (!hidden) return fail(BL_ERR_NULL, "ffn: hidden is required");
    if (n_layers < 0) return fail(BL_ERR_SHAPE, "ffn: n_layers = %d must be >= 0", n_layers);
    if (n_layers > 0 && !layers) return fail(BL_ERR_NULL, "ffn: layers is required");
    if (flags & ~(BL_FFN_PRE_NORM | BL_FFN_RESIDUAL | BL_FFN_PERSISTENT))
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
        if ((flags & BL_FFN_PERSISTENT) && L.gate)
            return fail(BL_ERR_UNSUPPORTED, "ffn: BL_FFN_PERSISTENT: layer %d is gated", l);
    }
    if (flags & BL_FFN_PERSISTENT) {
        if (M > 1) return fail(BL_ERR_UNSUPPORTED, "ffn: BL_FFN_PERSISTENT runs one token, M = %lld", (long long)M);
        if (!bl::stack_supported(H, F))
            return fail(BL_ERR_UNSUPPORTED, "ffn: BL_FFN_PERSISTENT: no persistent launch for H = %lld, F = %lld",
                        (long long)H, (long long)F);
    }
    return BL_OK;
}

// The layer launches, with scratch `ws` of ffn_ws(M, H, F) bytes (M >= 1).
int ffn_launch(const bitnet_ffn_layer* layers, int32_t n_layers, float* hidden, int64_t M, int64_t H, int64_t F,
               uint32_t flags, float norm_eps, void* ws, hipStream_t stream) {
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
    void* stack_ws = c.take<uint8_t>(bl::stack_ws_bytes());

    // One token, persistent: every layer in one launch (chunks of
    // stack_max_layers() layers).
    if (flags & BL_FFN_PERSISTENT) {
        for (int32_t l0 = 0; l0 < n_layers; l0 += bl::stack_max_layers()) {
            const int32_t n = n_layers - l0 < bl::stack_max_layers() ? n_layers - l0 : bl::stack_max_layers();
            hipError_t e = bl::launch_stack(layers + l0, n, hidden, H, F, pre, res, norm_eps, y1, stack_ws, stream);
            if (e != hipSuccess) return hip_status(e, "ffn: persistent stack");
        }
        return ok();
    }

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

}  // namespace

extern "C" {

int bitnet_ffn_forward(const bitnet_ffn_layer* layers, int32_t n_layers, float* hidden, int64_t M,
                       int64_t H, int64_t F, uint32_t flags, float norm_eps, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
    if (int r = ffn_check(layers, n_layers, hidden, M, H, F, flags)) return r;
    if (int r = check_workspace(ws, ws_bytes, M == 0 || n_layers == 0 ? 0 : ffn_ws(M, H, F))) return r;
    if (M == 0 || n_layers == 0) return ok();
    if (overlap(hidden, (size_t)(M * H) * 4, ws, ffn_ws(M, H, F)))
        return fail(BL_ERR_UNSUPPORTED, "ffn: hidden overlaps the workspace");
    return ffn_launch(layers, n_layers, hidden, M, H, F, flags, norm_eps, ws, stream);
}

// ---------------------------------------------------------------- FFN stack without allocation

}  // extern "C"

namespace {
// Scratch of bitnet_ffn_forward_noalloc: a fixed array in device memory, one
// copy per GPU the library runs on, held until the process ends.  In host
// code `scratch` names a host-side stand-in, not the device array: its device
// address comes from hipGetSymbolAddress, once per device (with that device
// current), and only that address is handed to kernels.
constexpr size_t kScratchBytes = BITNET_FFN_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "ffn_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(BL_ERR_UNSUPPORTED, "ffn_noalloc: device %d beyond the %d devices the library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "ffn_noalloc: hipGetSymbolAddress");
        if (p == nullptr) return fail(BL_ERR_HIP, "ffn_noalloc: hipGetSymbolAddress returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return BL_OK;
}
}  // namespace

extern "C" {

int bitnet_ffn_forward_noalloc(const bitnet_ffn_layer* layers, int32_t n_layers, float* hidden, int64_t M,
                               int64_t H, int64_t F, uint32_t flags, float norm_eps, hipStream_t stream) {
    if (int r = ffn_check(layers, n_layers, hidden, M, H, F, flags)) return r;
    if (M == 0 || n_layers == 0) return ok();
    const size_t need = ffn_ws(M, H, F);
    if (need > kScratchBytes)
        return fail(BL_ERR_WORKSPACE,
                    "ffn_noalloc: M = %lld, H = %lld, F = %lld need %zu bytes of scratch, above the library's "
                    "fixed %zu (use bitnet_ffn_forward with a workspace)",
                    (long long)M, (long long)H, (long long)F, need, kScratchBytes);
    void* ws = nullptr;
    if (int r = scratch_address(&ws)) return r;
    return ffn_launch(layers, n_layers, hidden, M, H, F, flags, norm_eps, ws, stream);
}

}  // extern "C"
