// k_reg.hip -- instantiations of the register-staged kernel (any K that is
// a multiple of 8): 256x256 and 128x128 single GEMMs and the 256x128 SwiGLU
// gate/up dual GEMM, each with a K-tail variant.
#include "kernels.h"
#include "kernel_reg.h"

namespace lf {

namespace {
template <int BM, int BN, int WM, int WN, bool BF, bool RMS, int NB, int NREG>
const void* reg_fn(int K) {
    return (K % dev::kBK == 0)
               ? reinterpret_cast<const void*>(&dev::gemm_fused_kernel<BM, BN, WM, WN, BF, RMS, NB, NREG, false>)
               : reinterpret_cast<const void*>(&dev::gemm_fused_kernel<BM, BN, WM, WN, BF, RMS, NB, NREG, true>);
}

template <bool BF, bool RMS>
const void* reg(const KernelSel& s) {
    switch (s.plan) {
    case kReg256:
        return reg_fn<256, 256, 2, 2, BF, RMS, 1, 1>(s.K);
    case kReg128:
        return reg_fn<128, 128, 2, 2, BF, RMS, 1, 2>(s.K);
    case kRegDual:
        if constexpr (RMS) return reg_fn<256, 128, 2, 2, BF, true, 2, 1>(s.K);
        return nullptr;
    default:
        return nullptr;
    }
}
}  // namespace

const void* kernels_reg(const KernelSel& s) {
    if (s.bf16) return s.rms ? reg<true, true>(s) : reg<true, false>(s);
    return s.rms ? reg<false, true>(s) : reg<false, false>(s);
}

}  // namespace lf
