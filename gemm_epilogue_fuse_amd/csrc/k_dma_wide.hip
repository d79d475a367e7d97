// k_dma_wide.hip -- instantiations of the LDS-DMA kernel for non-square tiles:
// the single GEMM with 8 waves as 4 x 2, 64x64 per wave (a 32-wide K step in
// 6 stages with whole-step fragment read-ahead, or a 64-wide step in 3 stages
// with sub-step read-ahead, which keeps a 64x64 wave within its registers),
// with and without the split-K exchange; the 64x128 tile with 4 waves in two K
// groups of 1 x 2 (64x64 per wave); and the SwiGLU gate/up dual GEMM: 4 waves
// as 4 x 1, each holding 64 rows x 128 columns of both operands, so every A
// row is scaled by gamma in one wave only (a 2 x 2 grid scales each row in
// two waves and measured 3-10% slower despite its fewer transposing reads).
#include "kernels.h"
#include "kernel_dma.h"

namespace lf {

namespace {
template <bool BF, bool RMS>
const void* wide(const KernelSel& s) {
    using namespace dev;
    constexpr int PRO = RMS ? kProRms : kProNone;
    switch (s.plan) {
    case kDma256x128W8:
        return s.split ? reinterpret_cast<const void*>(&gemm_dma_kernel<256, 128, 32, 6, 4, 2, 1, true, BF, PRO, 1, true>)
                       : reinterpret_cast<const void*>(&gemm_dma_kernel<256, 128, 32, 6, 4, 2, 1, true, BF, PRO, 1, false>);
    case kDma256x128x64W8:
        return s.split ? reinterpret_cast<const void*>(&gemm_dma_kernel<256, 128, 64, 3, 4, 2, 1, false, BF, PRO, 1, true>)
                       : reinterpret_cast<const void*>(&gemm_dma_kernel<256, 128, 64, 3, 4, 2, 1, false, BF, PRO, 1, false>);
    case kDma64x128G2:
        return s.split ? reinterpret_cast<const void*>(&gemm_dma_kernel<64, 128, 64, 4, 1, 2, 2, true, BF, PRO, 1, true>)
                       : reinterpret_cast<const void*>(&gemm_dma_kernel<64, 128, 64, 4, 1, 2, 2, true, BF, PRO, 1, false>);
    case kDual:
        if constexpr (RMS)
            return reinterpret_cast<const void*>(&gemm_dma_kernel<256, 128, 32, 4, 4, 1, 1, false, BF, kProRms, 2, false>);
        return nullptr;
    default:
        return nullptr;
    }
}
}  // namespace

const void* kernels_dma_wide(const KernelSel& s) {
    if (s.bf16) return s.rms ? wide<true, true>(s) : wide<true, false>(s);
    return s.rms ? wide<false, true>(s) : wide<false, false>(s);
}

}  // namespace lf
