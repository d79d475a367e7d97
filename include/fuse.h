/*
 * fuse.h -- C ABI of libfuse: fused GEMM + epilogue and RMSNorm -> Linear
 * operators for AMD Instinct MI355X (gfx950).
 *
 * Operations (page title, section that defines them):
 *
 *  fuse_gemm_epilogue
 *      Y = act(A . W + bias) + residual.
 *      "llm-fusion-compiler" (JohnScheuer): pattern table (gemm_bias_gelu,
 *      gemm_bias_silu, gemm_bias_relu, gemm_bias, gemm_bias_residual,
 *      gemm_gelu, gemm_silu) and the usage example, which builds
 *      gemm -> bias -> activation on x (M,K), w (K,N), bias (N,).
 *
 *  fuse_rmsnorm_gemm
 *      Y = act(RMSNorm_{gamma,eps}(X) . W + bias), the normalised activation
 *      never written to memory.
 *      "LLMBoost" (saitejasrivilli): problem statement (the RMSNorm output is
 *      written out and read straight back by the next Linear; fusion keeps it
 *      on chip), section 1 (fused op taking x, the norm weight, the
 *      projection weight and an epsilon attribute; shapes verified before
 *      execution), section 3 (per-row rsqrt(sum_sq / d_in + eps)); deplodock
 *      post, RMSNorm loop nest (mean square, plus eps, rsqrt, times x, times
 *      weight).
 *
 *  fuse_layernorm_gemm
 *      Y = act(LayerNorm_{gamma,beta,eps}(X) . W + bias).
 *      "llm-fusion-compiler": pattern table (layernorm_gemm, LayerNorm + GEMM).
 *      LayerNorm(X)[m,k] = (X[m,k] - mu[m]) / sqrt(var[m] + eps) * gamma[k]
 *      + beta[k], mu and var the mean and the biased (centred) variance of
 *      row m.  Two kernels: the row statistics (written to the library
 *      workspace, 24 bytes per row), then the GEMM, whose prologue
 *      normalises each X element on its way to the matrix cores; the
 *      normalised activation is never written to memory.
 *
 *  fuse_gemm_prologue_bias
 *      Y = act((A + abias) . W + bias) + residual, abias [K] added to every row
 *      of A inside the reduction.  deplodock post ("A hackable compiler to
 *      generate efficient fused GPU kernels"), Loop IR worked example
 *      relu((x + bias) @ w): the add is the prologue inside the reduce, the
 *      activation the epilogue after it.
 *
 *  fuse_rmsnorm_gemm_swiglu
 *      H = SiLU(Xhat . Wg) * (Xhat . Wu), Xhat = RMSNorm_{gamma,eps}(X): the
 *      gate and up projections of a SwiGLU FFN sharing one normalised input
 *      tile, with the gating product in the epilogue.
 *      "llm-fusion-compiler": FFN block (SwiGLU style), fused into a
 *      gemm + SiLU kernel and a gemm + bias + residual kernel; the second
 *      kernel is fuse_gemm_epilogue(H, Wd, bias, X, FUSE_ACT_NONE).
 *
 * Conventions shared by every entry point:
 *
 *  Layout      Dense, row-major, contiguous, no strides.  A/X is [M,K], W/Wg/Wu
 *              is [K,N] (N contiguous), bias is [N], residual and Y are [M,N],
 *              gamma is [K].
 *  dtype       FUSE_F16 or FUSE_BF16 gives the type of every input (A/X, W,
 *              bias, residual, gamma) and, by default, of the output.  OR-ing
 *              FUSE_OUT_F32 makes the output float32 instead.  Products are
 *              accumulated in float32; bias, activation, residual and the
 *              normalisation's per-row factor are applied in float32; the
 *              output is rounded once, to nearest even.  With a prologue the
 *              matrix-core operand is rounded once to the input dtype:
 *              RMSNorm round(x * gamma), its row factor 1/sqrt(ms + eps)
 *              applied to the float32 accumulator; LayerNorm round((x - mu) *
 *              gamma + beta * s) with s = sqrt(var + eps) and 1/s applied to
 *              the accumulator (the register-staged tiles round the
 *              normalised value itself); input bias round(x + b).  A tile
 *              whose rows fall outside the range where these operands keep
 *              their precision (RMSNorm: mean square + eps below 2^-30 for
 *              fp16 or 2^-120 for bf16, or mean square above 2^100;
 *              LayerNorm: var + eps below 2^-24 or s at the fp16 maximum for
 *              fp16, outside [2^-120, 2^100] for bf16), or whose accumulators came out
 *              non-finite, is recomputed exactly: float64 row factors,
 *              float32 operands and float32 accumulation.
 *  Shapes      M >= 0 (M == 0 is a no-op returning FUSE_OK), N >= 8, K >= 8,
 *              N % 8 == 0, K % 8 == 0; every tensor below 2^29 elements.
 *  Alignment   Every pointer 16-byte aligned.
 *  Ownership   All pointers are device memory owned by the caller.  The library
 *              keeps no pointer after the call returns.
 *  Workspace   Plans that split K across workgroups exchange float32 partial
 *              sums through a library-owned device buffer, one per (device,
 *              stream), allocated (hipMalloc) by the first call on that stream
 *              that needs it: at least 64 MiB, including 1 MiB of arrival
 *              counters, which a small kernel zeroes on the caller's stream.
 *              fuse_workspace_bytes reports what a call needs; the automatic
 *              plans stay within the 64 MiB minimum.  A call needing more than
 *              the stream's buffer holds allocates a new one of at least twice
 *              the size; the old buffer is kept (never freed before the process
 *              ends), since a HIP graph captured earlier may still use it.
 *              Calls on one stream use the buffer in stream order; calls on
 *              different streams never share it.  A graph replay uses the
 *              buffer of the stream it was captured on, so it must not run
 *              concurrently with other split-K work from that stream.  A call
 *              captured into a HIP graph must come after an eager call on the
 *              capturing stream that needed at least as much workspace: an
 *              allocation during capture fails with FUSE_E_HIP
 *              (hipErrorStreamCaptureUnsupported).  This buffer, the plan
 *              override of fuse_set_plan and the tuned-plan table of
 *              fuse_tune_set are the library's only state.
 *  Stream      `stream` is a hipStream_t (NULL: the default stream).  Calls are
 *              asynchronous: they return once the kernel is enqueued.
 *  Aliasing    Y must not overlap any input, except Y == residual exactly
 *              (in-place residual update, allowed only when the output dtype
 *              equals the input dtype).
 *  Errors      Returned as a status code; nothing is printed and no exception
 *              crosses the ABI.  All argument checks finish before any HIP
 *              call, so a rejected call has no effect on the device.  Faults
 *              inside a kernel surface at the caller's next synchronisation.
 *  Threads     Entry points may be called from several host threads.
 */
#ifndef LIBFUSE_FUSE_H
#define LIBFUSE_FUSE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FUSE_ABI_VERSION 1

/* Epilogue activation applied to (accumulator + bias). */
enum fuse_act {
    FUSE_ACT_NONE = 0,      /* identity                                        */
    FUSE_ACT_RELU = 1,      /* max(0, z)                                       */
    FUSE_ACT_GELU_TANH = 2, /* 0.5 z (1 + tanh(sqrt(2/pi)(z + 0.044715 z^3)))  */
    FUSE_ACT_SILU = 3       /* z * sigmoid(z)                                  */
};

/* Element types; FUSE_OUT_F32 is a flag OR-ed onto the input type. */
enum fuse_dtype {
    FUSE_F16 = 0,
    FUSE_BF16 = 1,
    FUSE_OUT_F32 = 0x100
};

/* Status codes. */
enum fuse_status {
    FUSE_OK = 0,
    FUSE_E_NULL = 1,  /* a required pointer is NULL                         */
    FUSE_E_SHAPE = 2, /* M < 0, N or K < 8 or not a multiple of 8, too big   */
    FUSE_E_ALIGN = 3, /* a pointer is not 16-byte aligned                    */
    FUSE_E_ENUM = 4,  /* unknown act, dtype or flag                          */
    FUSE_E_EPS = 5,   /* eps < 0 or not finite                               */
    FUSE_E_ALIAS = 6, /* output overlaps an input (other than Y == residual) */
    FUSE_E_HIP = 7,   /* the HIP runtime reported an error at launch         */
    FUSE_E_WORKSPACE = 8 /* fuse_rmsnorm_gemm_noalloc: the call needs more
                            split-K scratch than FUSE_NOALLOC_SCRATCH_BYTES    */
};

/*
 * Y[M,N] = act(A[M,K] . W[K,N] + bias[N]) + residual[M,N]
 *
 * A, W, Y required (A, Y and residual may be NULL when M == 0); bias and
 * residual may be NULL (read as zero).  The
 * residual is added after the activation.  `act` is an enum fuse_act, `dtype`
 * an enum fuse_dtype value (optionally | FUSE_OUT_F32).
 */
int fuse_gemm_epilogue(const void* A, const void* W, const void* bias,
                       const void* residual, void* Y, int64_t M, int64_t N,
                       int64_t K, int act, int dtype, void* stream);

/*
 * Y[M,N] = act(RMSNorm(X)[M,K] . W[K,N] + bias[N])
 * RMSNorm(X)[m,k] = X[m,k] * gamma[k] / sqrt(mean_k(X[m,k]^2) + eps)
 *
 * X, gamma, W, Y required (X and Y may be NULL when M == 0); bias may be NULL.  eps is a float32 >= 0.  The
 * normalisation runs over K, the GEMM's reduction axis.
 */
int fuse_rmsnorm_gemm(const void* X, const void* gamma, float eps,
                      const void* W, const void* bias, void* Y, int64_t M,
                      int64_t N, int64_t K, int act, int dtype, void* stream);

/*
 * Y[M,N] = act(LayerNorm_{gamma,beta,eps}(X)[M,K] . W[K,N] + bias[N])
 *
 * X, gamma, W, Y required (X and Y may be NULL when M == 0); beta and bias may
 * be NULL (zero).  The row statistics come from a first kernel (float64
 * accumulation; the mean from float32 sums of 8 values) and go to the
 * stream's workspace (M * 24 bytes, after any split-K partials);
 * the operand is formed as described under dtype above.
 */
int fuse_layernorm_gemm(const void* X, const void* gamma, const void* beta,
                        float eps, const void* W, const void* bias, void* Y,
                        int64_t M, int64_t N, int64_t K, int act, int dtype,
                        void* stream);

/*
 * Y[M,N] = act((A[M,K] + abias[K]) . W[K,N] + bias[N]) + residual[M,N]
 *
 * A, abias, W, Y required (A, Y and residual may be NULL when M == 0); bias
 * and residual may be NULL.  A + abias is rounded once to the input dtype as
 * the matrix-core operand (fp16: one packed fp16 add; bf16: the sum in
 * float32, then rounded).  Aliasing as for fuse_gemm_epilogue.
 */
int fuse_gemm_prologue_bias(const void* A, const void* abias, const void* W,
                            const void* bias, const void* residual, void* Y,
                            int64_t M, int64_t N, int64_t K, int act,
                            int dtype, void* stream);

/*
 * fuse_rmsnorm_gemm for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks and results (bit for bit) as
 * fuse_rmsnorm_gemm; it calls no hipMalloc, hipFree or allocating routine.
 * A plan that splits K exchanges its partials through a fixed buffer of
 * FUSE_NOALLOC_SCRATCH_BYTES that every device holds from its first such call
 * until the process ends; a call whose plan needs more (fuse_workspace_bytes
 * with op 1 tells beforehand; every automatic plan fits) returns
 * FUSE_E_WORKSPACE before any HIP call.  Calls on one GPU share that buffer
 * and its arrival counters whatever their stream, so calls that overlap in
 * time on one GPU race and must be ordered by the caller (one stream, or
 * events).  The first call on a device zeroes the counters on its stream and,
 * outside capture, waits for that; a call captured before any eager call on
 * its device captures the zeroing too.
 */
#define FUSE_NOALLOC_SCRATCH_BYTES (48u << 20)
int fuse_rmsnorm_gemm_noalloc(const void* X, const void* gamma, float eps,
                              const void* W, const void* bias, void* Y,
                              int64_t M, int64_t N, int64_t K, int act,
                              int dtype, void* stream);

/*
 * H[M,F] = SiLU(Xhat . Wg) * (Xhat . Wu),  Xhat = RMSNorm_{gamma,eps}(X)
 *
 * X [M,K], gamma [K], Wg and Wu [K,F], H [M,F]; all required (X and H may be
 * NULL when M == 0).  F follows the
 * same rules as N above.
 */
int fuse_rmsnorm_gemm_swiglu(const void* X, const void* gamma, float eps,
                             const void* Wg, const void* Wu, void* H,
                             int64_t M, int64_t F, int64_t K, int dtype,
                             void* stream);

/*
 * Tile plans.  Each entry point picks a kernel configuration ("plan") from the
 * problem shape.  fuse_plan_name reports the plan a call with these arguments
 * would use (op: 0 = fuse_gemm_epilogue, 1 = fuse_rmsnorm_gemm,
 * 2 = fuse_rmsnorm_gemm_swiglu, 3 = fuse_layernorm_gemm,
 * 4 = fuse_gemm_prologue_bias); it returns "invalid" for an unknown op.
 * fuse_set_plan forces one plan by name, "<plan>" or "<plan>:k<S>" for S-way
 * split K, for every later call of this process that the plan fits (a
 * gate/up dual plan only fuse_rmsnorm_gemm_swiglu, the others the two
 * single-GEMM entry points; a call it does not fit keeps the automatic
 * choice).  It is for tuning and testing only; NULL or "" restores the
 * automatic choice, and an unknown name returns FUSE_E_ENUM.  The override is
 * process-wide; calls racing with it see either the old or the new plan.
 */
const char* fuse_plan_name(int op, int64_t M, int64_t N, int64_t K, int dtype);
int fuse_set_plan(const char* name);

/*
 * Bytes of workspace (float32 split-K partials or LayerNorm row statistics,
 * plus arrival counters) a call of entry point `op` (numbered as for
 * fuse_plan_name) with these arguments uses under the current plan choice; 0
 * when it needs none, -1 for an unknown op, dtype or invalid shape.  No HIP
 * call.
 */
int64_t fuse_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int dtype);

/*
 * Tuned plans ("llm-fusion-compiler", Auto-Tuner: a search over tile
 * configurations under the hardware's limits, timed on the device, with a
 * persistent cache per pattern, shape and architecture).  The search and the
 * cache live in the Python tuner (gemm_epilogue_fuse_amd.tuner); the library
 * holds its results in a process-wide table of exact (op, M, N, K, dtype)
 * keys, consulted after a plan forced by fuse_set_plan and before the static
 * shape rules.
 *
 * fuse_tune_set     registers `plan` ("<plan>" or "<plan>:k<S>") for calls of
 *                   entry point `op` (numbered as for fuse_plan_name) with
 *                   exactly these M, N, K and input dtype; NULL or "" removes
 *                   the entry.  FUSE_E_ENUM for an unknown plan or one that
 *                   cannot serve such calls, FUSE_E_SHAPE for a bad shape.
 * fuse_tune_clear   empties the table.
 * fuse_plan_count / fuse_plan_info
 *                   enumerate the compiled plans: the name, and in fields[8]
 *                   {BM, BN, BK, LDS stages, threads, can split K, dual GEMM,
 *                   kernel family}; NULL past the end.
 * fuse_plan_applies 1 if `plan` can serve such calls, else 0.  No HIP call.
 * fuse_kernel_resources
 *                   the kernel a call with these arguments would run, as the
 *                   HIP runtime reports it: out[5] = {LDS bytes, launch
 *                   threads, max threads per block, registers, scratch bytes
 *                   per lane}; FUSE_E_HIP where no device is present.
 * Calls racing with fuse_tune_set see either the old or the new entry.
 */
int fuse_tune_set(int op, int64_t M, int64_t N, int64_t K, int dtype, const char* plan);
int fuse_tune_clear(void);
int fuse_plan_count(void);
const char* fuse_plan_info(int i, int32_t* fields);
int fuse_plan_applies(int op, int64_t M, int64_t N, int64_t K, int dtype, const char* plan);
int fuse_kernel_resources(int op, int64_t M, int64_t N, int64_t K, int dtype, int32_t* out);

/* Static, human-readable text for a status code (never NULL). */
const char* fuse_strerror(int status);

/* FUSE_ABI_VERSION of the loaded library. */
int fuse_version(void);

/* The hipError_t behind the most recent FUSE_E_HIP returned on the calling
 * thread (0 if none). */
int fuse_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBFUSE_FUSE_H */
