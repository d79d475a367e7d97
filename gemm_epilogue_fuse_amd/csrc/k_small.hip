// k_small.hip -- instantiations of the few-row kernels: the small-M kernel
// (32x64 tiles, split K), the strip kernels (16 or 32 rows, 16-column strips
// over all of K through a workgroup-wide LDS ring) and the whole-strip
// kernels (16 or 32 rows, each wave streaming its K share of the strip).
#include "kernels.h"
#include "kernel_decode.h"
#include "kernel_strip.h"
#include "kernel_wstrip.h"

namespace lf {

namespace {
// The whole-strip kernel walks 4, 8 or 16 blocks of 32 k per wave: the
// fewest that cover K / 256.
template <int RB, bool BF, bool RMS>
const void* wstrip(int K) {
    using namespace dev;
    const int nb = K / (kWStripWaves * 32);
    if (nb <= 4) return reinterpret_cast<const void*>(&gemm_wstrip_kernel<RB, 4, BF, RMS>);
    if (nb <= 8) return reinterpret_cast<const void*>(&gemm_wstrip_kernel<RB, 8, BF, RMS>);
    return reinterpret_cast<const void*>(&gemm_wstrip_kernel<RB, 16, BF, RMS>);
}

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
    case kWStrip16:
        return wstrip<1, BF, RMS>(s.K);
    case kWStrip32:
        return wstrip<2, BF, RMS>(s.K);
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
