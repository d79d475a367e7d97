// fuse_api.cpp -- the C ABI declared in include/fuse.h: argument checks, then
// the kernel launch(es) on the caller's stream.
//
// Checks mirror the shape verifier that the "LLMBoost" fused op runs before
// execution (section 1): every argument is validated on the host, with no
// HIP call, so a rejected call leaves the device untouched and can be tested
// without a GPU.
#include "../../include/fuse.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "launch.h"

namespace {

static_assert(lf::kScratchBytes == FUSE_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");

// Per tensor: byte offsets of 16-bit elements, plus a K step and the
// out-of-range bit, must stay below 2^32 (buffer offsets are 32-bit).
constexpr int64_t kMaxElems = int64_t(1) << 29;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};
Span span(const void* p, int64_t elems, int elem_bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + static_cast<uintptr_t>(elems) * static_cast<uintptr_t>(elem_bytes)};
}
bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

int check_dtype(int dtype, bool* bf16, bool* out_f32) {
    if ((dtype & ~(FUSE_OUT_F32 | 0xff)) != 0) return FUSE_E_ENUM;
    const int base = dtype & 0xff;
    if (base != FUSE_F16 && base != FUSE_BF16) return FUSE_E_ENUM;
    *bf16 = base == FUSE_BF16;
    *out_f32 = (dtype & FUSE_OUT_F32) != 0;
    return FUSE_OK;
}

int check_dims(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 8 || K < 8 || (N % 8) != 0 || (K % 8) != 0) return FUSE_E_SHAPE;
    if (M > kMaxElems || N > kMaxElems || K > kMaxElems) return FUSE_E_SHAPE;
    if (M * K >= kMaxElems || K * N >= kMaxElems || M * N >= kMaxElems) return FUSE_E_SHAPE;
    return FUSE_OK;
}

int check_eps(float eps) {
    if (!std::isfinite(eps) || eps < 0.0f) return FUSE_E_EPS;
    return FUSE_OK;
}

thread_local int t_last_hip = 0;

int run(const lf::Problem& p, void* stream, bool noalloc = false) {
    if (p.M == 0) return FUSE_OK;
    const hipError_t e = lf::launch(p, static_cast<hipStream_t>(stream), noalloc);
    if (e != hipSuccess) {
        t_last_hip = static_cast<int>(e);
        return FUSE_E_HIP;
    }
    return FUSE_OK;
}

// fuse_rmsnorm_gemm and its allocation-free variant: checks, then launch.
int rmsnorm_gemm(const void* X, const void* gamma, float eps, const void* W, const void* bias, void* Y,
                 int64_t M, int64_t N, int64_t K, int act, int dtype, void* stream, bool noalloc) {
    if (!gamma || !W || (M > 0 && (!X || !Y))) return FUSE_E_NULL;
    bool bf16 = false, out_f32 = false;
    if (int rc = check_dtype(dtype, &bf16, &out_f32)) return rc;
    if (act < FUSE_ACT_NONE || act > FUSE_ACT_SILU) return FUSE_E_ENUM;
    if (int rc = check_dims(M, N, K)) return rc;
    if (int rc = check_eps(eps)) return rc;
    if (!aligned16(X) || !aligned16(gamma) || !aligned16(W) || !aligned16(Y) ||
        (bias && !aligned16(bias)))
        return FUSE_E_ALIGN;
    const Span y = span(Y, M * N, out_f32 ? 4 : 2);
    if (M > 0 && (overlaps(y, span(X, M * K, 2)) || overlaps(y, span(gamma, K, 2)) ||
                  overlaps(y, span(W, K * N, 2)) || (bias && overlaps(y, span(bias, N, 2)))))
        return FUSE_E_ALIAS;
    lf::Problem p{};
    p.op = lf::Op::RmsGemm;
    p.A = X;
    p.W = W;
    p.bias = bias;
    p.gamma = gamma;
    p.Y = Y;
    p.M = M;
    p.N = N;
    p.K = K;
    p.eps = eps;
    p.act = act;
    p.bf16 = bf16;
    p.out_f32 = out_f32;
    if (noalloc && lf::workspace_bytes(p) > lf::kScratchBytes) return FUSE_E_WORKSPACE;
    return run(p, stream, noalloc);
}

}  // namespace

extern "C" {

int fuse_gemm_epilogue(const void* A, const void* W, const void* bias, const void* residual,
                       void* Y, int64_t M, int64_t N, int64_t K, int act, int dtype,
                       void* stream) {
    // Operands with M rows may be NULL when M == 0 (an empty tensor).
    if (!W || (M > 0 && (!A || !Y))) return FUSE_E_NULL;
    bool bf16 = false, out_f32 = false;
    if (int rc = check_dtype(dtype, &bf16, &out_f32)) return rc;
    if (act < FUSE_ACT_NONE || act > FUSE_ACT_SILU) return FUSE_E_ENUM;
    if (int rc = check_dims(M, N, K)) return rc;
    if (!aligned16(A) || !aligned16(W) || !aligned16(Y) || (bias && !aligned16(bias)) ||
        (residual && !aligned16(residual)))
        return FUSE_E_ALIGN;
    const Span y = span(Y, M * N, out_f32 ? 4 : 2);
    if (M > 0) {
        if (overlaps(y, span(A, M * K, 2)) || overlaps(y, span(W, K * N, 2)) ||
            (bias && overlaps(y, span(bias, N, 2))))
            return FUSE_E_ALIAS;
        if (residual && overlaps(y, span(residual, M * N, 2)) && !(residual == Y && !out_f32))
            return FUSE_E_ALIAS;
    }
    lf::Problem p{};
    p.op = lf::Op::GemmEpilogue;
    p.A = A;
    p.W = W;
    p.bias = bias;
    p.resid = residual;
    p.Y = Y;
    p.M = M;
    p.N = N;
    p.K = K;
    p.act = act;
    p.bf16 = bf16;
    p.out_f32 = out_f32;
    return run(p, stream);
}

int fuse_rmsnorm_gemm(const void* X, const void* gamma, float eps, const void* W,
                      const void* bias, void* Y, int64_t M, int64_t N, int64_t K, int act,
                      int dtype, void* stream) {
    return rmsnorm_gemm(X, gamma, eps, W, bias, Y, M, N, K, act, dtype, stream, false);
}

int fuse_rmsnorm_gemm_noalloc(const void* X, const void* gamma, float eps, const void* W,
                              const void* bias, void* Y, int64_t M, int64_t N, int64_t K, int act,
                              int dtype, void* stream) {
    return rmsnorm_gemm(X, gamma, eps, W, bias, Y, M, N, K, act, dtype, stream, true);
}

int fuse_rmsnorm_gemm_swiglu(const void* X, const void* gamma, float eps, const void* Wg,
                             const void* Wu, void* H, int64_t M, int64_t F, int64_t K, int dtype,
                             void* stream) {
    if (!gamma || !Wg || !Wu || (M > 0 && (!X || !H))) return FUSE_E_NULL;
    bool bf16 = false, out_f32 = false;
    if (int rc = check_dtype(dtype, &bf16, &out_f32)) return rc;
    if (int rc = check_dims(M, F, K)) return rc;
    if (int rc = check_eps(eps)) return rc;
    if (!aligned16(X) || !aligned16(gamma) || !aligned16(Wg) || !aligned16(Wu) || !aligned16(H))
        return FUSE_E_ALIGN;
    const Span h = span(H, M * F, out_f32 ? 4 : 2);
    if (M > 0 && (overlaps(h, span(X, M * K, 2)) || overlaps(h, span(gamma, K, 2)) ||
                  overlaps(h, span(Wg, K * F, 2)) || overlaps(h, span(Wu, K * F, 2))))
        return FUSE_E_ALIAS;
    lf::Problem p{};
    p.op = lf::Op::RmsSwiglu;
    p.A = X;
    p.W = Wg;
    p.W2 = Wu;
    p.gamma = gamma;
    p.Y = H;
    p.M = M;
    p.N = F;
    p.K = K;
    p.eps = eps;
    p.act = FUSE_ACT_SILU;
    p.bf16 = bf16;
    p.out_f32 = out_f32;
    return run(p, stream);
}

int fuse_layernorm_gemm(const void* X, const void* gamma, const void* beta, float eps, const void* W,
                        const void* bias, void* Y, int64_t M, int64_t N, int64_t K, int act, int dtype,
                        void* stream) {
    if (!gamma || !W || (M > 0 && (!X || !Y))) return FUSE_E_NULL;
    bool bf16 = false, out_f32 = false;
    if (int rc = check_dtype(dtype, &bf16, &out_f32)) return rc;
    if (act < FUSE_ACT_NONE || act > FUSE_ACT_SILU) return FUSE_E_ENUM;
    if (int rc = check_dims(M, N, K)) return rc;
    if (int rc = check_eps(eps)) return rc;
    if (!aligned16(X) || !aligned16(gamma) || (beta && !aligned16(beta)) || !aligned16(W) || !aligned16(Y) ||
        (bias && !aligned16(bias)))
        return FUSE_E_ALIGN;
    const Span y = span(Y, M * N, out_f32 ? 4 : 2);
    if (M > 0 && (overlaps(y, span(X, M * K, 2)) || overlaps(y, span(gamma, K, 2)) ||
                  (beta && overlaps(y, span(beta, K, 2))) || overlaps(y, span(W, K * N, 2)) ||
                  (bias && overlaps(y, span(bias, N, 2)))))
        return FUSE_E_ALIAS;
    lf::Problem p{};
    p.op = lf::Op::LnGemm;
    p.A = X;
    p.W = W;
    p.bias = bias;
    p.gamma = gamma;
    p.beta = beta;
    p.Y = Y;
    p.M = M;
    p.N = N;
    p.K = K;
    p.eps = eps;
    p.act = act;
    p.bf16 = bf16;
    p.out_f32 = out_f32;
    return run(p, stream);
}

int fuse_gemm_prologue_bias(const void* A, const void* abias, const void* W, const void* bias,
                            const void* residual, void* Y, int64_t M, int64_t N, int64_t K, int act, int dtype,
                            void* stream) {
    if (!abias || !W || (M > 0 && (!A || !Y))) return FUSE_E_NULL;
    bool bf16 = false, out_f32 = false;
    if (int rc = check_dtype(dtype, &bf16, &out_f32)) return rc;
    if (act < FUSE_ACT_NONE || act > FUSE_ACT_SILU) return FUSE_E_ENUM;
    if (int rc = check_dims(M, N, K)) return rc;
    if (!aligned16(A) || !aligned16(abias) || !aligned16(W) || !aligned16(Y) || (bias && !aligned16(bias)) ||
        (residual && !aligned16(residual)))
        return FUSE_E_ALIGN;
    const Span y = span(Y, M * N, out_f32 ? 4 : 2);
    if (M > 0) {
        if (overlaps(y, span(A, M * K, 2)) || overlaps(y, span(abias, K, 2)) || overlaps(y, span(W, K * N, 2)) ||
            (bias && overlaps(y, span(bias, N, 2))))
            return FUSE_E_ALIAS;
        if (residual && overlaps(y, span(residual, M * N, 2)) && !(residual == Y && !out_f32))
            return FUSE_E_ALIAS;
    }
    lf::Problem p{};
    p.op = lf::Op::BiasGemm;
    p.A = A;
    p.gamma = abias;
    p.W = W;
    p.bias = bias;
    p.resid = residual;
    p.Y = Y;
    p.M = M;
    p.N = N;
    p.K = K;
    p.act = act;
    p.bf16 = bf16;
    p.out_f32 = out_f32;
    return run(p, stream);
}

const char* fuse_plan_name(int op, int64_t M, int64_t N, int64_t K, int dtype) {
    if (op < 0 || op > 4) return "invalid";
    lf::Problem p{};
    p.op = static_cast<lf::Op>(op);
    p.M = M;
    p.N = N;
    p.K = K;
    p.bf16 = (dtype & 0xff) == FUSE_BF16;
    p.out_f32 = (dtype & FUSE_OUT_F32) != 0;
    return lf::plan_name(p);
}

int64_t fuse_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int dtype) {
    if (op < 0 || op > 4) return -1;
    bool bf16 = false, out_f32 = false;
    if (check_dtype(dtype, &bf16, &out_f32) != FUSE_OK || check_dims(M, N, K) != FUSE_OK) return -1;
    lf::Problem p{};
    p.op = static_cast<lf::Op>(op);
    p.M = M;
    p.N = N;
    p.K = K;
    p.bf16 = bf16;
    p.out_f32 = out_f32;
    return static_cast<int64_t>(lf::workspace_bytes(p));
}

int fuse_set_plan(const char* name) { return lf::set_plan(name) ? FUSE_OK : FUSE_E_ENUM; }

namespace {
int shape_problem(int op, int64_t M, int64_t N, int64_t K, int dtype, lf::Problem* p) {
    if (op < 0 || op > 4) return FUSE_E_ENUM;
    bool bf16 = false, out_f32 = false;
    if (int rc = check_dtype(dtype, &bf16, &out_f32)) return rc;
    if (int rc = check_dims(M, N, K)) return rc;
    *p = lf::Problem{};
    p->op = static_cast<lf::Op>(op);
    p->M = M;
    p->N = N;
    p->K = K;
    p->bf16 = bf16;
    p->out_f32 = out_f32;
    return FUSE_OK;
}
}  // namespace

int fuse_tune_set(int op, int64_t M, int64_t N, int64_t K, int dtype, const char* plan) {
    lf::Problem p;
    if (int rc = shape_problem(op, M, N, K, dtype, &p)) return rc;
    return lf::tune_set(p, plan) == 0 ? FUSE_OK : FUSE_E_ENUM;
}

int fuse_tune_clear(void) {
    lf::tune_clear();
    return FUSE_OK;
}

int fuse_plan_count(void) { return lf::plan_count(); }

const char* fuse_plan_info(int i, int32_t* fields) { return fields ? lf::plan_info(i, fields) : nullptr; }

int fuse_plan_applies(int op, int64_t M, int64_t N, int64_t K, int dtype, const char* plan) {
    lf::Problem p;
    if (!plan || shape_problem(op, M, N, K, dtype, &p) != FUSE_OK) return 0;
    return lf::plan_applies(p, plan) ? 1 : 0;
}

int fuse_kernel_resources(int op, int64_t M, int64_t N, int64_t K, int dtype, int32_t* out) {
    if (!out) return FUSE_E_NULL;
    lf::Problem p;
    if (int rc = shape_problem(op, M, N, K, dtype, &p)) return rc;
    if (M == 0) return FUSE_E_SHAPE;
    const hipError_t e = lf::kernel_resources(p, out);
    if (e != hipSuccess) {
        t_last_hip = static_cast<int>(e);
        return FUSE_E_HIP;
    }
    return FUSE_OK;
}

const char* fuse_strerror(int status) {
    switch (status) {
    case FUSE_OK: return "success";
    case FUSE_E_NULL: return "a required pointer is NULL";
    case FUSE_E_SHAPE: return "invalid shape (M < 0, N or K < 8 or not a multiple of 8, or tensor too large)";
    case FUSE_E_ALIGN: return "a pointer is not 16-byte aligned";
    case FUSE_E_ENUM: return "unknown activation, dtype or flag";
    case FUSE_E_EPS: return "eps is negative or not finite";
    case FUSE_E_ALIAS: return "output overlaps an input";
    case FUSE_E_HIP: return "HIP runtime error at launch";
    case FUSE_E_WORKSPACE: return "the call needs more split-K scratch than the fixed buffer holds";
    default: return "unknown status";
    }
}

int fuse_version(void) { return FUSE_ABI_VERSION; }

int fuse_last_hip_error(void) { return t_last_hip; }

}  // extern "C"
