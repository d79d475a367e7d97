// k_small.hip -- instantiations of the few-row kernels: the small-M kernel
// (32x64 tiles, split K) and the strip kernels (16 or 32 rows, 16-column
// strips over all of K).
#include "kernels.h"
#include "kernel_decode.h"
#include "kernel_strip.h"

namespace lf {

namespace {
template <bool BF, bool RMS>
const void* small(const KernelSel& s) {
    using namespace dev;
    switch (s.plan) {
    case kDec:
        return reinterpret_cast<const void*>(&gemm_decode_kernel<64, BF, RMS>);
    case kStrip16:
        return reinterpret_cast<const void*>(&gemm_strip_kernel<1, 16, BF, RMS>);
    case kStrip32:
        return reinterpret_cast<const void*>(&gemm_strip_kernel<2, 11, BF, RMS>);
    default:
        return nullptr;
    }
}
}  // namespace

const void* kernels_small(const KernelSel& s) {
    if (s.bf16) return s.rms ? small<true, true>(s) : small<true, false>(s);
    return s.rms ? small<false, true>(s) : small<false, false>(s);
}

}  // namespace lf
