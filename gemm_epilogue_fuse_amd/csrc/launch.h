// launch.h -- internal interface between the host entry points (fuse_api.cpp)
// and the gfx950 kernels (gemm_fused.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lf {

enum class Op : int { GemmEpilogue = 0, RmsGemm = 1, RmsSwiglu = 2, LnGemm = 3, BiasGemm = 4 };

// One fused call, already validated.  Pointers are device pointers.
struct Problem {
    Op op;
    const void* A;      // A or X, [M,K]
    const void* W;      // W or Wg, [K,N]
    const void* W2;     // Wu for RmsSwiglu, else nullptr
    const void* bias;   // [N] or nullptr
    const void* resid;  // [M,N] or nullptr
    const void* gamma;  // [K]: gamma of the RMS and LayerNorm ops, the input bias of BiasGemm
    const void* beta;   // [K] LayerNorm beta or nullptr
    void* Y;            // [M,N]
    int64_t M, N, K;
    float eps;
    int act;        // enum fuse_act
    bool bf16;      // input dtype is bf16 (else fp16)
    bool out_f32;   // output is float32
};

// Bytes of the fixed split-K scratch each device holds for calls that must
// not allocate (1 MiB of arrival counters, then fp32 partials).
constexpr size_t kScratchBytes = size_t(48) << 20;  // FUSE_NOALLOC_SCRATCH_BYTES

// Enqueue the kernel(s) for `p` on `stream`.  Returns hipSuccess or the
// launch error.  With `noalloc`, a split-K plan exchanges its partials through
// the fixed scratch instead of a per-stream workspace (no allocation; the
// caller has checked that workspace_bytes(p) <= kScratchBytes).
hipError_t launch(const Problem& p, hipStream_t stream, bool noalloc = false);

// Bytes of split-K workspace (partials and arrival counters) `launch` uses
// for `p`; 0 when its plan does not split K.  No HIP call.
size_t workspace_bytes(const Problem& p);

// Name of the tile configuration `launch` would use for `p` (static string).
const char* plan_name(const Problem& p);

// Force a single-GEMM plan by name (nullptr or "" = automatic).  Returns
// false for an unknown name.
bool set_plan(const char* name);

// Tuned plan for calls with exactly p's (op, M, N, K, dtype): "<plan>" or
// "<plan>:k<S>"; nullptr or "" removes the entry.  0 on success, -1 for an
// unknown name, -2 for a plan that does not fit such calls.
int tune_set(const Problem& p, const char* name);
void tune_clear();

// The compiled plans: name and {bm, bn, bk, stages, threads, can split K,
// dual GEMM, kernel family} (nullptr past the end).
int plan_count();
const char* plan_info(int i, int32_t* fields);

// Whether plan `name` ("<plan>" or "<plan>:k<S>") can serve calls like p.
bool plan_applies(const Problem& p, const char* name);

// Resources of the kernel `launch` would use for p, from the HIP runtime:
// {LDS bytes, launch threads, max threads per block, registers, scratch bytes}.
hipError_t kernel_resources(const Problem& p, int32_t* out);

}  // namespace lf
