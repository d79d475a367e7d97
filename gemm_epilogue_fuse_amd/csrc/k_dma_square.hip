// k_dma_square.hip -- instantiations of the LDS-DMA kernel for the square
// tiles: 256x256 (4 or 8 waves) and 128x128 (4 waves, or 8 waves in two K
// groups with a 64- or 32-wide K step), with and without the split-K
// exchange.
#include "kernels.h"
#include "kernel_dma.h"

namespace lf {

namespace {
template <bool BF, bool RMS>
const void* square(const KernelSel& s) {
    using namespace dev;
    constexpr int PRO = RMS ? kProRms : kProNone;
    switch (s.plan) {
    case kDma256:
        // RMS: 4 x 1 waves, so every A row is scaled by gamma in one wave only
        if constexpr (RMS)
            return reinterpret_cast<const void*>(&gemm_dma_kernel<256, 256, 32, 4, 4, 1, 1, false, BF, kProRms, 1, false>);
        return reinterpret_cast<const void*>(&gemm_dma_kernel<256, 256, 32, 4, 2, 2, 1, false, BF, PRO, 1, false>);
    case kDma256W8:
        return reinterpret_cast<const void*>(&gemm_dma_kernel<256, 256, 32, 4, 2, 4, 1, false, BF, PRO, 1, false>);
    case kDma128:
        return s.split ? reinterpret_cast<const void*>(&gemm_dma_kernel<128, 128, 64, 4, 2, 2, 1, false, BF, PRO, 1, true>)
                       : reinterpret_cast<const void*>(&gemm_dma_kernel<128, 128, 64, 4, 2, 2, 1, false, BF, PRO, 1, false>);
    case kDma128G2:
        return s.split ? reinterpret_cast<const void*>(&gemm_dma_kernel<128, 128, 64, 4, 2, 2, 2, true, BF, PRO, 1, true>)
                       : reinterpret_cast<const void*>(&gemm_dma_kernel<128, 128, 64, 4, 2, 2, 2, true, BF, PRO, 1, false>);
    case kDma128S8G2:
        return s.split ? reinterpret_cast<const void*>(&gemm_dma_kernel<128, 128, 32, 8, 2, 2, 2, true, BF, PRO, 1, true>)
                       : reinterpret_cast<const void*>(&gemm_dma_kernel<128, 128, 32, 8, 2, 2, 2, true, BF, PRO, 1, false>);
    default:
        return nullptr;
    }
}
}  // namespace

const void* kernels_dma_square(const KernelSel& s) {
    if (s.bf16) return s.rms ? square<true, true>(s) : square<true, false>(s);
    return s.rms ? square<false, true>(s) : square<false, false>(s);
}

}  // namespace lf
