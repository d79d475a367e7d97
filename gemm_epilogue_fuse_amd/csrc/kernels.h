// kernels.h -- internal table between the tile plans (gemm_fused.hip) and
// the translation units that instantiate the gfx950 kernels (k_*.hip).  Each
// unit compiles one family, so the library builds in parallel.  Not part of
// the public ABI.
#pragma once

namespace lf {

// Plan indices; the table itself (names, tile sizes) is in gemm_fused.hip.
enum PlanIndex : int {
    kDma256 = 0,
    kDma128 = 1,
    kReg256 = 2,
    kReg128 = 3,
    kDual = 4,
    kRegDual = 5,
    kDma256W8 = 6,
    kDma128G2 = 7,
    kDma128S8G2 = 8,
    kDec = 9,
    kStrip16 = 10,
    kStrip32 = 11,
    kDma256x128W8 = 12,
    kDma256x128x64W8 = 13,
    kWStrip16 = 14,
    kWStrip32 = 15,
    kDma64x128G2 = 16,
    kDma256x128S3 = 17,
    kNumPlanIndices = 18
};

// Which instantiation of a plan's kernel a call needs.
struct KernelSel {
    int plan;    // PlanIndex
    bool bf16;   // bf16 inputs (else fp16)
    bool rms;    // RMSNorm prologue (RmsGemm, RmsSwiglu)
    int pro;     // A prologue: 0 none, 1 RMSNorm, 2 input bias, 3 LayerNorm (dev::Prologue)
    bool split;  // split-K partial exchange compiled in
    int K;       // reduction length (the register-staged kernel has a K-tail variant)
};

// Host-side kernel handles for hipLaunchKernel, or nullptr when the unit
// holds no kernel for `s`.
const void* kernels_dma_square(const KernelSel& s);  // k_dma_square.hip: 128x128 and 256x256 tiles
const void* kernels_dma_wide(const KernelSel& s);    // k_dma_wide.hip: 256x128 and 64x128 tiles, dual gate/up
const void* kernels_reg(const KernelSel& s);         // k_reg.hip: register-staged tiles, every prologue
const void* kernels_small(const KernelSel& s);       // k_small.hip: small-M and strip kernels
const void* kernels_dma_pro(const KernelSel& s);     // k_dma_pro.hip: 4 x 1 wave tiles, input-bias and LayerNorm

}  // namespace lf
