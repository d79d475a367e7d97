// k_reg.hip -- instantiations of the register-staged kernel (any K that is
// a multiple of 8): 256x256 and 128x128 single GEMMs with every A prologue
// (none, RMSNorm, input bias, LayerNorm) and the 256x128 SwiGLU gate/up dual
// GEMM, each with a K-tail variant.
#include "kernels.h"
#include "kernel_reg.h"

namespace lf {

namespace {
template <int BM, int BN, int WM, int WN, bool BF, int PRO, int NB, int NREG>
const void* reg_fn(int K) {
    return (K % dev::kBK == 0)
               ? reinterpret_cast<const void*>(&dev::gemm_fused_kernel<BM, BN, WM, WN, BF, PRO, NB, NREG, false>)
               : reinterpret_cast<const void*>(&dev::gemm_fused_kernel<BM, BN, WM, WN, BF, PRO, NB, NREG, true>);
}

template <bool BF, int PRO>
const void* reg(const KernelSel& s) {
    switch (s.plan) {
    case kReg256:
        return reg_fn<256, 256, 2, 2, BF, PRO, 1, 1>(s.K);
    case kReg128:
        return reg_fn<128, 128, 2, 2, BF, PRO, 1, 2>(s.K);
    case kRegDual:
        if constexpr (PRO == dev::kProRms) return reg_fn<256, 128, 2, 2, BF, PRO, 2, 1>(s.K);
        return nullptr;
    default:
        return nullptr;
    }
}

template <bool BF>
const void* reg_pro(const KernelSel& s) {
    switch (s.pro) {
    case dev::kProRms: return reg<BF, dev::kProRms>(s);
    case dev::kProBias: return reg<BF, dev::kProBias>(s);
    case dev::kProLn: return reg<BF, dev::kProLn>(s);
    default: return reg<BF, dev::kProNone>(s);
    }
}
}  // namespace

const void* kernels_reg(const KernelSel& s) { return s.bf16 ? reg_pro<true>(s) : reg_pro<false>(s); }

}  // namespace lf
