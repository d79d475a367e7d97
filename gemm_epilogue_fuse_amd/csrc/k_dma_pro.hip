// k_dma_pro.hip -- instantiations of the LDS-DMA kernel with 4 x 1 waves:
// every wave holds whole rows of the tile, so each A element passes through
// the prologue (input bias, LayerNorm) in exactly one wave.  256x256 (64 x 256
// per wave), 128x128 with a 64-wide K step (32 x 128 per wave, with or
// without the split-K exchange) for the bias and LayerNorm GEMMs, and
// 256x128 with a 64-wide K step in 3 stages (64 x 128 per wave) for every
// prologue.  Also the input bias in the plain GEMM's 8-wave tiles (256x256
// as 2 x 4 waves, 256x128 as 4 x 2), where its one add per value costs
// little even though two or four waves repeat it for each row.
#include "kernels.h"
#include "kernel_dma.h"

namespace lf {

namespace {
template <bool BF, int PRO>
const void* pro(const KernelSel& s) {
    using namespace dev;
    constexpr bool LB = PRO == kProBias || PRO == kProLn;
    switch (s.plan) {
    case kDma256:
        if constexpr (LB)
            return reinterpret_cast<const void*>(&gemm_dma_kernel<256, 256, 32, 4, 4, 1, 1, false, BF, PRO, 1, false>);
        return nullptr;
    case kDma128:
        if constexpr (LB)
            return s.split
                       ? reinterpret_cast<const void*>(&gemm_dma_kernel<128, 128, 64, 4, 4, 1, 1, false, BF, PRO, 1, true>)
                       : reinterpret_cast<const void*>(&gemm_dma_kernel<128, 128, 64, 4, 4, 1, 1, false, BF, PRO, 1, false>);
        return nullptr;
    case kDma256x128S3:
        return s.split ? reinterpret_cast<const void*>(&gemm_dma_kernel<256, 128, 64, 3, 4, 1, 1, false, BF, PRO, 1, true>)
                       : reinterpret_cast<const void*>(&gemm_dma_kernel<256, 128, 64, 3, 4, 1, 1, false, BF, PRO, 1, false>);
    case kDma256W8:
        if constexpr (PRO == kProBias)
            return reinterpret_cast<const void*>(&gemm_dma_kernel<256, 256, 32, 4, 2, 4, 1, false, BF, PRO, 1, false>);
        return nullptr;
    case kDma256x128x64W8:
        if constexpr (PRO == kProBias)
            return s.split
                       ? reinterpret_cast<const void*>(&gemm_dma_kernel<256, 128, 64, 3, 4, 2, 1, false, BF, PRO, 1, true>)
                       : reinterpret_cast<const void*>(&gemm_dma_kernel<256, 128, 64, 3, 4, 2, 1, false, BF, PRO, 1, false>);
        return nullptr;
    default:
        return nullptr;
    }
}

template <bool BF>
const void* by_prologue(const KernelSel& s) {
    switch (s.pro) {
    case dev::kProNone: return pro<BF, dev::kProNone>(s);
    case dev::kProRms: return pro<BF, dev::kProRms>(s);
    case dev::kProBias: return pro<BF, dev::kProBias>(s);
    case dev::kProLn: return pro<BF, dev::kProLn>(s);
    default: return nullptr;
    }
}
}  // namespace

const void* kernels_dma_pro(const KernelSel& s) { return s.bf16 ? by_prologue<true>(s) : by_prologue<false>(s); }

}  // namespace lf
