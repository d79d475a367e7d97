// gemm_fused.hip -- tile plans and kernel dispatch for the fused GEMM +
// epilogue, the RMSNorm -> Linear operator and the SwiGLU gate/up dual GEMM
// on gfx950 (MI355X).
//
// What every kernel computes ("llm-fusion-compiler" pattern table and usage
// example; "LLMBoost" problem statement and section 3; deplodock post,
// RMSNorm loop nest):
//     C[m,n]  = sum_k Aop[m,k] * W[k,n]                   (fp32 accumulate)
//     Aop     = A                                          (plain GEMM)
//             = round_T(X[m,k] * gamma[k])                 (RMS ops)
//     z       = r[m] * C[m,n] + bias[n]                    (r = 1 for plain GEMM)
//     Y[m,n]  = act(z) + R[m,n],  rounded once to the output type
//     r[m]    = 1 / sqrt( sum_k X[m,k]^2 / K + eps )
// For the SwiGLU dual GEMM: H = SiLU(r*Cg) * (r*Cu).
//
// RMSNorm fusion.  x_hat[m,k] = X[m,k] * r[m] * gamma[k]; r[m] is one scalar
// per row, so it factors out of the k-sum: x_hat . W = r[m] * ((X*gamma) . W).
// The kernels scale the A operand by gamma on its way to the matrix cores,
// accumulate sum_k X^2 from the same data, and apply r[m] to the fp32
// accumulator in the epilogue.  X is read once, the normalised activation is
// never written anywhere, and no separate pass over X is needed.
#include "launch.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <shared_mutex>
#include <tuple>
#include <utility>
#include <vector>
#include <algorithm>

#include "common.h"
#include "kernel_strip.h"
#include "kernel_wstrip.h"
#include "kernels.h"

namespace lf {
namespace {

using dev::KArgs;

enum class Kind { Reg, Dma, Dec, Strip, WStrip };

// A tile plan: kernel family, tile sizes, K step, LDS stages, wave grid
// (wm x wn waves, kg K groups; the register-staged kernel always uses 2x2x1),
// and whether it can split K across workgroups.
struct Plan {
    const char* name;
    Kind kind;
    int bm, bn, bk, ns;
    int wm, wn, kg;
    bool dual;
    bool split;
    int threads() const { return wm * wn * kg * 64; }
};

constexpr Plan kPlans[] = {
    {"dma_256x256x32_s4", Kind::Dma, 256, 256, 32, 4, 2, 2, 1, false, false},  // every prologue: 4 x 1 waves
    {"dma_128x128x64_s4", Kind::Dma, 128, 128, 64, 4, 2, 2, 1, false, true},  // bias, LayerNorm: 4 x 1
    {"reg_256x256x64", Kind::Reg, 256, 256, 64, 2, 2, 2, 1, false, false},
    {"reg_128x128x64", Kind::Reg, 128, 128, 64, 2, 2, 2, 1, false, false},
    {"dma_dual_256x128x32_s4", Kind::Dma, 256, 128, 32, 4, 4, 1, 1, true, false},
    {"reg_dual_256x128x64", Kind::Reg, 256, 128, 64, 2, 2, 2, 1, true, false},
    {"dma_256x256x32_s4_w8", Kind::Dma, 256, 256, 32, 4, 2, 4, 1, false, false},
    {"dma_128x128x64_s4_g2", Kind::Dma, 128, 128, 64, 4, 2, 2, 2, false, true},
    {"dma_128x128x32_s8_g2", Kind::Dma, 128, 128, 32, 8, 2, 2, 2, false, true},
    {"dec_32x64", Kind::Dec, 32, 64, 64, 8, 1, 1, 4, false, true},
    {"strip_16x16", Kind::Strip, 16, 16, 128, 16, 1, 1, 4, false, false},
    {"strip_32x16", Kind::Strip, 32, 16, 128, 11, 1, 1, 4, false, false},
    {"dma_256x128x32_s6_w8", Kind::Dma, 256, 128, 32, 6, 4, 2, 1, false, true},
    {"dma_256x128x64_s3_w8", Kind::Dma, 256, 128, 64, 3, 4, 2, 1, false, true},
    {"wstrip_16x16", Kind::WStrip, 16, 16, 256, 0, 1, 1, 8, false, false},
    {"wstrip_32x16", Kind::WStrip, 32, 16, 256, 0, 1, 1, 8, false, false},
    {"dma_64x128x64_s4_g2", Kind::Dma, 64, 128, 64, 4, 1, 2, 2, false, true},
    {"dma_256x128x64_s3", Kind::Dma, 256, 128, 64, 3, 4, 1, 1, false, true},
};
constexpr int kNumPlans = sizeof(kPlans) / sizeof(kPlans[0]);
static_assert(kNumPlans == kNumPlanIndices, "plan table and PlanIndex (kernels.h) agree");

std::atomic<int> g_override{-1};        // forced plan index, -1 = automatic
std::atomic<int> g_override_splits{0};  // forced split count with a forced plan, 0 = one split


// The LayerNorm and input-bias prologues run in the register-staged kernel
// and in the LDS-DMA tiles with 4 x 1 waves (each A row transformed by one
// wave): 256x256, 256x128 and 128x128.  The input bias also runs in the
// 8-wave 256x256 and 256x128 tiles (forced or tuned plans).
bool ln_or_bias(const Problem& p) { return p.op == Op::LnGemm || p.op == Op::BiasGemm; }

bool pro_plan(int idx, const Problem& p) {
    if (idx == kDma256 || idx == kDma128 || idx == kDma256x128S3) return true;
    return p.op == Op::BiasGemm && (idx == kDma256W8 || idx == kDma256x128x64W8);
}

bool plan_fits(const Plan& pl, const Problem& p) {
    if (pl.dual != (p.op == Op::RmsSwiglu)) return false;
    if (ln_or_bias(p) && pl.kind != Kind::Reg && !pro_plan((int)(&pl - kPlans), p)) return false;
    if (pl.kind != Kind::Reg && (p.K % pl.bk) != 0) return false;
    if (pl.kind == Kind::Strip && p.op != Op::GemmEpilogue && p.K > dev::kStripMaxK) return false;
    if (pl.kind == Kind::WStrip && p.K > dev::kWStripMaxK) return false;
    return true;
}

// Rows up to which a call counts as decode-shaped: streaming W once at HBM
// rate bounds it, and the small-M kernel serves it.
constexpr int64_t kDecodeMaxM = 128;
// K steps of 64 a small-M workgroup holds at most (its whole W chunk is in
// flight at once).
constexpr int kDecodeMaxSteps = 8;
// The small-M kernel reads W once per 32-row tile.  Past this much W traffic
// the 128-row split tile, which reads W once per 128 rows, is faster (the
// crossover lies between 33 rows at 4096x4096 and 128 rows at 2048x2048).
constexpr int64_t kDecodeMaxWBytes = int64_t(32) << 20;

// Workgroups a plan keeps busy at once: the chip has 256 CUs and every
// tile plan here holds one workgroup per CU.
constexpr int kCUs = 256;

struct Choice {
    const Plan* plan;
    int splits;
};

// Split K when the output has too few tiles to occupy the CUs: the splits
// of a tile run on different CUs and are reduced in a fixed order.  Each
// split keeps at least 8 K steps so the pipeline has room to fill.  The
// small-M kernel takes the largest K chunk (at most 8 steps) that still
// gives two workgroups per CU.
int auto_splits(const Plan& pl, const Problem& p) {
    if (!pl.split) return 1;
    if (pl.kind == Kind::Dec) {
        // Longest chunks the kernel holds: measured on 1..128 rows and
        // K = 1024..4096, every further split (more workgroups, shorter
        // chunks) costs more in partial-sum traffic than it gains.
        return (int)((p.K / pl.bk + kDecodeMaxSteps - 1) / kDecodeMaxSteps);
    }
    const int64_t tiles = ((p.M + pl.bm - 1) / pl.bm) * ((p.N + pl.bn - 1) / pl.bn);
    const int64_t nk = p.K / pl.bk;
    int s = 1;
    while (tiles * s * 2 <= kCUs && nk / (s * 2) >= 8) s *= 2;
    return s;
}

// Plan `idx` with `s` requested K splits (0 or 1: none), as it runs for `p`
// (a plan that fits it): the split count is clamped to the K steps, and the
// small-M kernel takes at least enough splits for chunks of 8 steps.
Choice pinned(int idx, int s, const Problem& p) {
    const int64_t nk = p.K / kPlans[idx].bk;
    if (kPlans[idx].kind == Kind::Dec) {
        const int64_t lo = (nk + kDecodeMaxSteps - 1) / kDecodeMaxSteps;
        return {&kPlans[idx], (int)std::min<int64_t>(std::max<int64_t>(s, lo), nk)};
    }
    return {&kPlans[idx], (kPlans[idx].split && s > 1) ? (int)std::min<int64_t>(s, nk) : 1};
}

// Tuned plans: exact (op, M, N, K, dtype) keys filled by fuse_tune_set (the
// tuner measures every fitting plan and split count and loads its winners
// from a persistent cache).  Consulted after a forced plan, before the
// static rules.
struct TuneKey {
    int op;
    int64_t M, N, K;
    int bf16;
    bool operator<(const TuneKey& o) const {
        return std::tie(op, M, N, K, bf16) < std::tie(o.op, o.M, o.N, o.K, o.bf16);
    }
};
std::shared_mutex g_tune_mu;
std::map<TuneKey, std::pair<int, int>> g_tune;  // key -> (plan index, splits)
std::atomic<int> g_tune_n{0};

TuneKey tune_key(const Problem& p) { return {(int)p.op, p.M, p.N, p.K, p.bf16 ? 1 : 0}; }

Choice choose(const Problem& p) {
    const int ov = g_override.load(std::memory_order_relaxed);
    if (ov >= 0 && plan_fits(kPlans[ov], p)) return pinned(ov, g_override_splits.load(std::memory_order_relaxed), p);
    if (g_tune_n.load(std::memory_order_acquire) > 0) {
        std::shared_lock<std::shared_mutex> lk(g_tune_mu);
        const auto it = g_tune.find(tune_key(p));
        if (it != g_tune.end() && plan_fits(kPlans[it->second.first], p))
            return pinned(it->second.first, it->second.second, p);
    }
    const Plan* pl;
    if (ln_or_bias(p)) {
        // the 4 x 1 LDS-DMA tiles, largest first while the output still
        // fills the chip, then 128x128 with split K; K not a multiple of the
        // K step: the register-staged kernel
        const int64_t t256 = ((p.M + 255) / 256) * ((p.N + 255) / 256);
        const int64_t t256x128 = ((p.M + 255) / 256) * ((p.N + 127) / 128);
        if (p.K % 64 != 0) return {(t256 >= 224) ? &kPlans[kReg256] : &kPlans[kReg128], 1};
        // (cold 4096^3 input-bias GEMM: 126.6 us on 4 x 1 waves against 130.6 us
        // on the 8-wave tile in fp16, 136.3 against 177.1 us in bf16)
        pl = (t256 >= 224) ? &kPlans[kDma256] : (t256x128 >= 224) ? &kPlans[kDma256x128S3] : &kPlans[kDma128];
        return {pl, auto_splits(*pl, p)};
    }
    if (p.op != Op::RmsSwiglu && p.M <= 128 && p.K <= 1024 && plan_fits(kPlans[kWStrip16], p)) {
        // a few rows and a short K: one workgroup per 16-column strip over
        // all of K (no partial sums cross the device), the whole strip in
        // flight at once (1024x1024: 4.8 us against 6.0 us for the LDS-ring
        // strip).  At longer K the 16-column strips read a quarter of each
        // 128-byte line per workgroup and lose to 64-column tiles with split K.
        // Past 64 rows the 32-row strip, which reads each W strip half as
        // often (cold, 128x1024x1024: 6.5 us against 8.3 us for the small-M
        // kernel; 64x256x256 GEMM: 3.8 against 4.1 us with 16-row strips).
        pl = &kPlans[p.M <= 64 ? kWStrip16 : kWStrip32];
    } else if (p.op != Op::RmsSwiglu && p.M <= 32 && p.K <= 1024 && plan_fits(kPlans[kStrip16], p)) {
        pl = &kPlans[kStrip16];
    } else if (p.op != Op::RmsSwiglu && p.M <= kDecodeMaxM && p.K % 64 == 0 &&
               ((p.M + 31) / 32) * p.K * p.N * 2 <= kDecodeMaxWBytes) {
        pl = &kPlans[kDec];
    } else if (p.op == Op::RmsSwiglu) {
        pl = (p.K % 32 == 0) ? &kPlans[kDual] : &kPlans[kRegDual];
    } else {
        const int64_t t256 = ((p.M + 255) / 256) * ((p.N + 255) / 256);
        const int64_t t256x128 = ((p.M + 255) / 256) * ((p.N + 127) / 128);
        if (t256 >= 224) {
            // the plain GEMM on 8 waves of 128x64 (cold 4096^3: 116-122 us
            // against 124-135 us with 4 waves); with RMSNorm 4 x 1 waves, so
            // each row is scaled once
            const PlanIndex big = (p.op == Op::GemmEpilogue) ? kDma256W8 : kDma256;
            pl = (p.K % 32 == 0) ? &kPlans[big] : &kPlans[kReg256];
        } else if (t256x128 >= 224 && p.K % 64 == 0) {
            // Enough 256x128 tiles to fill the chip without splitting K: 8
            // waves of 64x64 keep LDS reads in flight, and the taller tile
            // halves the W traffic per row of the 128x128 tile.  Measured
            // 18-20% faster than the 128x128 K-group tile at 2048x4096x4096
            // and 2048x4096x11008.  With RMSNorm the 4 x 1 wave tile, which
            // scales each A row in one wave (cold 2048x4096x4096: 84.0 us
            // against 88.8 us).
            pl = &kPlans[p.op == Op::RmsGemm ? kDma256x128S3 : kDma256x128x64W8];
        } else if (p.op == Op::RmsGemm && p.bf16 && t256x128 >= 112 && p.K % 64 == 0) {
            // bf16 RMSNorm, whose gamma scaling costs the most VALU: the 4 x 1
            // wave 256x128 tile with K split in two (cold 1024x4096x4096:
            // 55.7 us against 61.4 us for the 8-wave 128x128 tile; in fp16
            // the 128x128 tile stays ahead, 51.4 against 53.1 us)
            pl = &kPlans[kDma256x128S3];
        } else if (p.K % 64 == 0) {
            // The 8-wave tile: its second K group keeps twice the LDS reads
            // in flight and halves each wave's share of the RMS scaling.
            // Measured equal or faster than the 4-wave 128x128 tile from
            // 512 to 2048 rows with and without RMSNorm.  Outputs too small
            // to fill the chip also split K.
            pl = &kPlans[kDma128G2];
            // Exchanging 128x128 fp32 partials pays off only when each split
            // keeps at least 32 K steps; with shorter splits the 64x128 tile
            // (twice the tiles, half the partial per tile, fewer splits) is
            // faster: 128x4096x4096 22.8 -> 18.2 us, 512x2048x2048 18.1 ->
            // 15.3 us, 512x1024x1024 12.3 -> 9.8 us.
            const int s128 = auto_splits(*pl, p);
            if (s128 > 1 && p.K / 64 / s128 < 32) pl = &kPlans[kDma64x128G2];
        } else {
            pl = &kPlans[kReg128];
        }
    }
    return {pl, auto_splits(*pl, p)};
}

// Split-K workspace, one per (device, stream) so calls on different
// streams never share partials or counters.  It grows geometrically on
// demand; a buffer it outgrows is retired, never freed, because a HIP graph
// captured earlier may still hold its address.  The arrival counters of a new
// buffer are zeroed by a fill kernel on the caller's stream (stream-ordered
// before the call that needs them); every reducing workgroup puts its counter
// back to zero.  The lock is held from the lookup through the launch, so a
// second host thread on the same stream cannot retire the buffer in between.
struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
std::vector<void*> g_ws_retired;
constexpr size_t kCounterBytes = 1 << 20;  // 256K tiles
constexpr size_t kMinWorkspace = size_t(64) << 20;
static_assert(kScratchBytes >= kCounterBytes, "scratch holds the arrival counters");

__global__ void __launch_bounds__(256) zero_words_kernel(unsigned* p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

hipError_t zero_words(unsigned* p, size_t bytes, hipStream_t stream) {
    const int n = (int)(bytes / sizeof(unsigned));
    void* args[] = {&p, const_cast<int*>(&n)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&zero_words_kernel), dim3((n + 255) / 256), dim3(256),
                           args, 0, stream);
}

// LayerNorm row statistics ("llm-fusion-compiler" pattern table:
// layernorm_gemm, the statistics pass of a two-kernel LayerNorm + GEMM): one
// wave per row, mean and centred variance over two passes of the row: the mean
// from float32 sums of 8 values accumulated in float64, the variance from
// float64 squares of the float32 differences.
// Two forms per row:
//   rec[m]  16 bytes for the LDS-DMA kernel, which forms
//           (x - mean) * gamma + beta * s in the input type (s = sqrt(var +
//           eps)) and scales its accumulator by 1/s: fp16 words 0-2 are the
//           half pairs (mu_hi, mu_hi), (mu_lo, mu_lo), (s, s) with mean =
//           mu_hi + mu_lo to about 22 bits; bf16 words 0 and 2 are mean and s
//           as floats; word 3 is 1/s as a float, negated when var + eps lies
//           outside the window where those operands keep their precision
//           (fp16: [2^-24, s below the fp16 maximum]; bf16: [2^-120, 2^100]),
//           which sends the row's tiles to the exact path;
//   ab[m]   the fp32 pair (a, b) = (1/s, -mean * a) for the register-staged
//           kernel, which forms (a*x + b) * gamma + beta in fp32.
// Rows are 16-byte aligned (K % 8 == 0), so each lane reads 8 values at a time.
template <bool BF>
__global__ void __launch_bounds__(256) ln_stats_kernel(const uint16_t* X, int M, int K, float eps, dev::u32x4* rec,
                                                       float2* out) {
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    const uint16_t* x = X + (size_t)m * K;
    // A lane holds R 16-byte chunks at once, all loads in flight together:
    // rows of up to 512 R values are read from memory once for both passes.
    constexpr int R = 8;
    dev::u32x4 v[R];
    auto load = [&](int base) {
#pragma unroll
        for (int c = 0; c < R; ++c) {
            const int k = base + 8 * (lane + 64 * c);
            v[c] = k < K ? *reinterpret_cast<const dev::u32x4*>(x + k) : dev::u32x4{0u, 0u, 0u, 0u};
        }
    };
    const bool held = K <= 512 * R;
    // Sums of 8 values in float32, pairwise, then float64 across chunks and
    // lanes: a chunk sum is off by at most 3 roundings of 2^-24 of its
    // magnitude, far below what the fp16/bf16 operand keeps.
    auto chunk_sum = [&](const dev::u32x4& w) {
        float e[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            e[2 * q] = dev::lo_f32<BF>(w[q]);
            e[2 * q + 1] = dev::hi_f32<BF>(w[q]);
        }
        return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    };
    double s = 0.0;
    for (int base = 0; base < K; base += 512 * R) {
        load(base);
#pragma unroll
        for (int c = 0; c < R; ++c) s += (double)chunk_sum(v[c]);
    }
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    const double mu = s / (double)K;
    // Squares about the float32 mean, squared and summed in float64 (a float32
    // square of a bf16 difference can leave the float32 range or fall into its
    // subnormals): sum (x - mu_f)^2 = sum (x - mu)^2 + K (mu - mu_f)^2, and
    // (mu - mu_f)^2 is at most 2^-48 mu^2.
    const float muf = (float)mu;
    double v2 = 0.0;
    for (int base = 0; base < K; base += 512 * R) {
        if (!held) load(base);
#pragma unroll
        for (int c = 0; c < R; ++c) {
            if (base + 8 * (lane + 64 * c) >= K) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const double d0 = (double)(dev::lo_f32<BF>(v[c][q]) - muf);
                const double d1 = (double)(dev::hi_f32<BF>(v[c][q]) - muf);
                v2 = fma(d0, d0, fma(d1, d1, v2));
            }
        }
    }
    for (int o = 32; o > 0; o >>= 1) v2 += __shfl_xor(v2, o);
    if (lane == 0) {
        const double ve = v2 / (double)K + (double)eps;
        const double sd = sqrt(ve);
        const double a = 1.0 / sd;
        out[m] = make_float2((float)a, (float)(-mu * a));
        dev::u32x4 r;
        bool inside;
        if constexpr (BF) {
            r[0] = __float_as_uint((float)mu);
            r[1] = 0u;
            r[2] = __float_as_uint((float)sd);
            inside = ve >= 0x1p-120 && ve <= 0x1p100;
        } else {
            const _Float16 mh = (_Float16)mu;
            const _Float16 ml = (_Float16)(mu - (double)mh);
            const _Float16 sh = (_Float16)sd;
            const uint32_t bh = __builtin_bit_cast(uint16_t, mh), bl = __builtin_bit_cast(uint16_t, ml);
            const uint32_t bs = __builtin_bit_cast(uint16_t, sh);
            r[0] = bh | (bh << 16);
            r[1] = bl | (bl << 16);
            r[2] = bs | (bs << 16);
            inside = ve >= 0x1p-24 && sd < 65504.0;
        }
        r[3] = __float_as_uint(inside ? (float)a : -(float)a);
        rec[m] = r;
    }
}

// Caller holds g_ws_mu.
hipError_t get_workspace(hipStream_t stream, size_t part_bytes, float** ws, unsigned** cnt) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    Workspace& w = g_ws[{dev, stream}];
    const size_t need = kCounterBytes + part_bytes;
    if (w.bytes < need) {
        // allocating inside a stream capture is not allowed: capture after
        // an eager call on this stream that needed at least as much
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess) return e;
        if (cs != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
        const size_t bytes = std::max({need, kMinWorkspace, 2 * w.bytes});
        void* ptr = nullptr;
        e = hipMalloc(&ptr, bytes);
        if (e != hipSuccess) return e;
        e = zero_words(static_cast<unsigned*>(ptr), kCounterBytes, stream);
        if (e != hipSuccess) {
            (void)hipFree(ptr);
            return e;
        }
        if (w.ptr) g_ws_retired.push_back(w.ptr);
        w.ptr = ptr;
        w.bytes = bytes;
    }
    *cnt = static_cast<unsigned*>(w.ptr);
    *ws = reinterpret_cast<float*>(static_cast<char*>(w.ptr) + kCounterBytes);
    return hipSuccess;
}

hipError_t launch_fn(const void* fn, const KArgs& a, int nwg, int threads, hipStream_t s) {
    // hipLaunchKernel reports the status of this launch itself, so an error
    // left behind by an unrelated earlier call is not picked up.
    void* args[] = {const_cast<KArgs*>(&a)};
    return hipLaunchKernel(fn, dim3(nwg), dim3(threads), args, 0, s);
}

// The kernel of plan `pi` for this call, from the unit that instantiates it.
int prologue_of(const Problem& p) {
    switch (p.op) {
    case Op::RmsGemm:
    case Op::RmsSwiglu: return dev::kProRms;
    case Op::BiasGemm: return dev::kProBias;
    case Op::LnGemm: return dev::kProLn;
    default: return dev::kProNone;
    }
}

const void* kernel_for(int pi, const Problem& p, bool split) {
    const int pro = prologue_of(p);
    const KernelSel s{pi, p.bf16, pro == dev::kProRms, pro, split, (int)p.K};
    switch (kPlans[pi].kind) {
    case Kind::Reg: return kernels_reg(s);
    case Kind::Dec:
    case Kind::Strip:
    case Kind::WStrip: return kernels_small(s);
    case Kind::Dma:
        if (pro == dev::kProBias || pro == dev::kProLn || pi == kDma256x128S3) return kernels_dma_pro(s);
        return (kPlans[pi].bm == kPlans[pi].bn) ? kernels_dma_square(s) : kernels_dma_wide(s);
    }
    return nullptr;
}

}  // namespace

const char* plan_name(const Problem& p) {
    // "<plan>" or "<plan>:k<S>" for S-way split K (static strings)
    static thread_local char buf[64];
    const Choice c = choose(p);
    if (c.splits == 1) return c.plan->name;
    snprintf(buf, sizeof(buf), "%s:k%d", c.plan->name, c.splits);
    return buf;
}

namespace {

// "<plan>" or "<plan>:k<S>" (S in 1..64, only for plans that split K).
bool parse_plan(const char* name, int* idx, int* splits) {
    const char* colon = std::strchr(name, ':');
    const size_t len = colon ? (size_t)(colon - name) : std::strlen(name);
    *splits = 0;
    if (colon) {
        if (colon[1] != 'k') return false;
        char* end = nullptr;
        const long v = std::strtol(colon + 2, &end, 10);
        if (end == colon + 2 || *end != 0 || v < 1 || v > 64) return false;
        *splits = (int)v;
    }
    for (int i = 0; i < kNumPlans; ++i) {
        if (std::strlen(kPlans[i].name) == len && std::strncmp(name, kPlans[i].name, len) == 0) {
            if (*splits > 1 && !kPlans[i].split) return false;
            *idx = i;
            return true;
        }
    }
    return false;
}

}  // namespace

bool set_plan(const char* name) {
    if (name == nullptr || name[0] == 0) {
        g_override.store(-1);
        g_override_splits.store(0);
        return true;
    }
    int idx = 0, splits = 0;
    if (!parse_plan(name, &idx, &splits)) return false;
    g_override_splits.store(splits);
    g_override.store(idx);
    return true;
}

int tune_set(const Problem& p, const char* name) {
    std::unique_lock<std::shared_mutex> lk(g_tune_mu);
    if (name == nullptr || name[0] == 0) {
        g_tune.erase(tune_key(p));
    } else {
        int idx = 0, splits = 0;
        if (!parse_plan(name, &idx, &splits)) return -1;
        if (!plan_fits(kPlans[idx], p)) return -2;
        g_tune[tune_key(p)] = {idx, splits};
    }
    g_tune_n.store((int)g_tune.size(), std::memory_order_release);
    return 0;
}

void tune_clear() {
    std::unique_lock<std::shared_mutex> lk(g_tune_mu);
    g_tune.clear();
    g_tune_n.store(0, std::memory_order_release);
}

int plan_count() { return kNumPlans; }

const char* plan_info(int i, int32_t* f) {
    if (i < 0 || i >= kNumPlans) return nullptr;
    const Plan& pl = kPlans[i];
    f[0] = pl.bm;
    f[1] = pl.bn;
    f[2] = pl.bk;
    f[3] = pl.ns;
    f[4] = pl.threads();
    f[5] = pl.split ? 1 : 0;
    f[6] = pl.dual ? 1 : 0;
    f[7] = (int)pl.kind;
    return pl.name;
}

bool plan_applies(const Problem& p, const char* name) {
    int idx = 0, splits = 0;
    return parse_plan(name, &idx, &splits) && plan_fits(kPlans[idx], p);
}

namespace {

// Kernel arguments of a call (without the workspace pointers) and its plan.
Choice setup(const Problem& p, KArgs& a) {
    const Choice c = choose(p);
    const Plan& pl = *c.plan;
    a.A = static_cast<const uint16_t*>(p.A);
    a.W = static_cast<const uint16_t*>(p.W);
    a.W2 = static_cast<const uint16_t*>(p.W2);
    a.bias = static_cast<const uint16_t*>(p.bias);
    a.resid = static_cast<const uint16_t*>(p.resid);
    a.gamma = static_cast<const uint16_t*>(p.gamma);
    a.beta = static_cast<const uint16_t*>(p.beta);
    a.stats = nullptr;
    a.lnstats = nullptr;
    a.Y = p.Y;
    a.M = (int)p.M;
    a.N = (int)p.N;
    a.K = (int)p.K;
    a.tiles_m = (int)((p.M + pl.bm - 1) / pl.bm);
    a.tiles_n = (int)((p.N + pl.bn - 1) / pl.bn);
    // small M: the row tiles of a W column tile share an XCD
    a.group_m = (pl.kind == Kind::Dec || pl.kind == Kind::Strip || pl.kind == Kind::WStrip) ? a.tiles_m : 4;
    a.act = p.act;
    a.out_f32 = p.out_f32 ? 1 : 0;
    a.eps = p.eps;
    a.splits = 1;
    a.kchunk = a.K;
    a.ws = nullptr;
    a.cnt = nullptr;
    if (c.splits > 1) {
        // K steps per split, rounded up; the last split may get fewer
        const int nk = a.K / pl.bk;
        const int per = (nk + c.splits - 1) / c.splits;
        a.splits = (nk + per - 1) / per;
        a.kchunk = per * pl.bk;
    }
    return c;
}

// Bytes of fp32 partials a split call exchanges: per tile and split, the
// accumulators of every operand and the RMS partial sums of squares (the
// small-M kernel: 8 floats plus one sum per thread).
size_t split_bytes(const Plan& pl, const Problem& p, const KArgs& a) {
    const size_t tiles = (size_t)a.tiles_m * a.tiles_n;
    const size_t nb = (p.op == Op::RmsSwiglu) ? 2 : 1;
    const size_t acc_floats = nb * pl.bm * pl.bn;
    // 4 x 1 waves: 256x256 with any prologue, 128x128 with the bias and LayerNorm prologues
    const int idx = (int)(&pl - kPlans);
    const int wm = ((idx == kDma256 && p.op != Op::GemmEpilogue) || (idx == kDma128 && ln_or_bias(p))) ? 4 : pl.wm;
    const size_t ss_floats = (size_t)pl.threads() * (pl.bm / wm / 32 / pl.kg);
    const size_t per_split = (pl.kind == Kind::Dec) ? 256 * 36 : (acc_floats + ss_floats) * sizeof(float);
    return tiles * a.splits * per_split;
}

// Fixed split-K scratch for callers that cannot allocate: counters first,
// partials after.  Each device holds its own copy until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host it names
// a stand-in, not device memory): its device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_zeroed[kMaxDevices] = {};

// Device address of this device's scratch, its arrival counters zeroed on
// `stream`.  The first call on a device looks the address up; until a zeroing
// has run eagerly (and been waited for) on some stream of the device, every
// call zeroes the counters on its own stream first, so a call captured into a
// graph carries its own zeroing.
hipError_t get_scratch(hipStream_t stream, float** ws, unsigned** cnt) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = ptr;
    }
    unsigned char* base = static_cast<unsigned char*>(g_scratch_ptr[dev]);
    if (!g_scratch_zeroed[dev]) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess) return e;
        e = zero_words(reinterpret_cast<unsigned*>(base), kCounterBytes, stream);
        if (e != hipSuccess) return e;
        if (cs == hipStreamCaptureStatusNone) {
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return e;
            g_scratch_zeroed[dev] = true;
        }
    }
    *cnt = reinterpret_cast<unsigned*>(base);
    *ws = reinterpret_cast<float*>(base + kCounterBytes);
    return hipSuccess;
}

}  // namespace

// Bytes of LayerNorm row statistics a call keeps in the workspace: the
// 16-byte record and the (a, b) pair per row.
size_t stats_bytes(const Problem& p) { return p.op == Op::LnGemm ? (size_t)p.M * 24 : 0; }

// Split partials rounded up to 256 bytes, so the statistics after them stay aligned.
size_t split_area(const Plan& pl, const Problem& p, const KArgs& a) {
    return a.splits > 1 ? (split_bytes(pl, p, a) + 255) / 256 * 256 : 0;
}

size_t workspace_bytes(const Problem& p) {
    if (p.M == 0) return 0;
    KArgs a;
    const Choice c = setup(p, a);
    if (a.splits == 1 && stats_bytes(p) == 0) return 0;
    return kCounterBytes + split_area(*c.plan, p, a) + stats_bytes(p);
}

hipError_t launch(const Problem& p, hipStream_t stream, bool noalloc) {
    if (p.M == 0) return hipSuccess;
    KArgs a;
    const Choice c = setup(p, a);
    const Plan& pl = *c.plan;
    if (a.splits > 1 && (size_t)a.tiles_m * a.tiles_n >= kCounterBytes / sizeof(unsigned))
        return hipErrorInvalidValue;
    const int nwg = a.tiles_m * a.tiles_n * a.splits;
    const void* fn = kernel_for((int)(c.plan - kPlans), p, a.splits > 1);
    if (fn == nullptr) return hipErrorInvalidDeviceFunction;
    if (noalloc && p.op == Op::LnGemm) return hipErrorInvalidValue;  // its statistics live in the workspace
    if (a.splits > 1 && noalloc) {
        if (kCounterBytes + split_bytes(pl, p, a) > kScratchBytes) return hipErrorInvalidValue;
        const hipError_t e = get_scratch(stream, &a.ws, &a.cnt);
        if (e != hipSuccess) return e;
        return launch_fn(fn, a, nwg, pl.threads(), stream);
    }
    if (p.op == Op::LnGemm) {
        // two kernels: the row statistics into the workspace, then the GEMM
        // whose prologue normalises each A element on its way to LDS
        // (workspace: counters, split partials, then the statistics)
        std::lock_guard<std::mutex> lk(g_ws_mu);
        const size_t part = split_area(pl, p, a);
        hipError_t e = get_workspace(stream, part + stats_bytes(p), &a.ws, &a.cnt);
        if (e != hipSuccess) return e;
        char* st = reinterpret_cast<char*>(a.ws) + part;
        dev::u32x4* rec = reinterpret_cast<dev::u32x4*>(st);
        float2* out = reinterpret_cast<float2*>(st + (size_t)a.M * 16);
        a.lnstats = reinterpret_cast<const uint32_t*>(rec);
        a.stats = out;
        const uint16_t* X = a.A;
        int M = a.M, K = a.K;
        float eps = a.eps;
        void* sargs[] = {&X, &M, &K, &eps, &rec, &out};
        const void* sfn = p.bf16 ? reinterpret_cast<const void*>(&ln_stats_kernel<true>)
                                 : reinterpret_cast<const void*>(&ln_stats_kernel<false>);
        e = hipLaunchKernel(sfn, dim3((M + 3) / 4), dim3(256), sargs, 0, stream);
        if (e != hipSuccess) return e;
        return launch_fn(fn, a, nwg, pl.threads(), stream);
    }
    if (a.splits > 1) {
        std::lock_guard<std::mutex> lk(g_ws_mu);
        const hipError_t e = get_workspace(stream, split_bytes(pl, p, a), &a.ws, &a.cnt);
        if (e != hipSuccess) return e;
        return launch_fn(fn, a, nwg, pl.threads(), stream);
    }
    return launch_fn(fn, a, nwg, pl.threads(), stream);
}

hipError_t kernel_resources(const Problem& p, int32_t* out) {
    KArgs a;
    const Choice c = setup(p, a);
    const void* fn = kernel_for((int)(c.plan - kPlans), p, a.splits > 1);
    if (fn == nullptr) return hipErrorInvalidDeviceFunction;
    hipFuncAttributes attr{};
    const hipError_t e = hipFuncGetAttributes(&attr, fn);
    if (e != hipSuccess) return e;
    out[0] = (int32_t)attr.sharedSizeBytes;
    out[1] = c.plan->threads();
    out[2] = (int32_t)attr.maxThreadsPerBlock;
    out[3] = (int32_t)attr.numRegs;
    out[4] = (int32_t)attr.localSizeBytes;
    return hipSuccess;
}

}  // namespace lf
