// kernel_wstrip.h -- few-row fused GEMM on gfx950 with the whole W strip in
// flight at once.
//
// At a handful of rows (decode: M = B <= 32) the call streams W [K, N] once
// and does almost no arithmetic, so its time is one HBM stream plus fixed
// latency.  Here a workgroup owns a 16-column output strip over all of K
// (no partial sums cross the device), and its 8 waves each own K/8 of the
// strip.  Each wave
//   * loads its X fragments and gamma straight into registers (X is tiny and
//     shared by every workgroup, so it comes from L2),
//   * then requests its entire share of the W strip global -> LDS with
//     buffer_load_dwordx4 ... lds, one 1 KiB DMA row (32 k-rows x 16
//     columns) per 32-k block, all issued before the first is used,
//   * and consumes the blocks in arrival order with no workgroup barrier:
//     wait for block j (vmcnt), two transposing LDS reads for the B operand,
//     one v_mfma_f32_16x16x32 per 16-row block.
// Every vector-memory instruction a wave issues comes before its first wait
// and completes in issue order, so waiting until at most NBT-1-j remain
// outstanding means block j has landed.
// With K <= 4096 a CU holds its whole strip (<= 128 KiB) in flight.  The
// waves' sums are added through LDS in wave order at the end, so results do
// not depend on timing.
//
// Matrix-core layouts (v_mfma_f32_16x16x32): A lane l holds row l%16, k
// 8(l/16)..+7; B lane l holds column l%16, same k; C register r of lane l is
// row 4(l/16)+r, column l%16.
//
// Requires K % 256 == 0 and K <= 4096.
#pragma once

#include "common.h"
#include "kernel_dma.h"

namespace lf {
namespace dev {

constexpr int kWStripWaves = 8;
constexpr int kWStripMaxBlocks = 16;  // 32-k blocks per wave
constexpr int kWStripMaxK = kWStripWaves * kWStripMaxBlocks * 32;

// f(ic<J>{}) for J = J0 .. N-1, in order.
template <int J, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (J < N) {
        f(ic<J>{});
        static_for<J + 1, N>(f);
    }
}

template <bool BF>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
}

// NBT: 32-k blocks each wave walks (4, 8 or 16).  A wave's real share is
// nb = K / 256 <= NBT blocks; the blocks past it are padding whose DMA rows
// and X fragments are out of range (zeros), so every count and wait in the
// loop is a compile-time constant.
template <int RB, int NBT, bool BF, bool RMS>
__global__ void __launch_bounds__(kWStripWaves * 64, 1)
gemm_wstrip_kernel(const KArgs p) {
    constexpr int NW = kWStripWaves, MAXB = NBT;
    static_assert(NBT <= kWStripMaxBlocks, "at most 16 blocks per wave");
    constexpr int BM = 16 * RB, BN = 16;
    constexpr int RED_FLOATS = NW * RB * 256;  // per-wave 16x16 sums per row block
    constexpr int W_BYTES = NW * MAXB * 1024;
    constexpr int RED_BYTES = (RED_FLOATS + NW * RB * 64) * 4;
    __shared__ __attribute__((aligned(1024))) char smem[W_BYTES > RED_BYTES ? W_BYTES : RED_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int tm, tn, kz;
    map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, 1, tm, tn, kz);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K;
    const int nb = K / (NW * 32);  // real 32-k blocks per wave, 1..MAXB
    const int kw = wave * nb * 32;  // first k of this wave's share

    // X and gamma fragments first (their loads complete before any W block,
    // so waiting for W block j also covers them).  Rows past M read as zero.
    const __amdgpu_buffer_rsrc_t rsX = make_rsrc(p.A + (size_t)m0 * K, (uint32_t)((size_t)(M - m0) * K * 2));
    const __amdgpu_buffer_rsrc_t rsG = make_rsrc(RMS ? p.gamma : p.A, RMS ? (uint32_t)K * 2u : 0u);
    const int kl = 8 * (lane >> 4);
    u32x4 xa[MAXB][RB];
    u32x4 gv[MAXB];
#pragma unroll
    for (int j = 0; j < MAXB; ++j) {
        const bool real = j < nb;
        const int k = kw + 32 * (real ? j : 0) + kl;
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int row = 16 * i + (lane & 15);
            xa[j][i] = bload16(rsX, oob_or((uint32_t)(row * K + k) * 2u, real && m0 + row < M), 0);
        }
        if constexpr (RMS) gv[j] = bload16(rsG, oob_or((uint32_t)k * 2u, real), 0);
    }

    // The wave's W share: block j (k-rows kw+32j..+31, 16 columns) into its
    // own 1 KiB slot; lane l moves the 16-byte half l%2 of k-row l/2.
    const i32x4 rsW = rsrc128(p.W, (uint32_t)((size_t)K * N * 2));
    const uint32_t voffW = oob_or((uint32_t)((lane >> 1) * N + n0 + 8 * (lane & 1)) * 2u, n0 + 8 * (lane & 1) < N);
    const uint32_t lds_w = lds_u32(smem) + (uint32_t)(wave * MAXB * 1024);
#pragma unroll
    for (int j = 0; j < MAXB; ++j) {
        const bool real = j < nb;  // padding rows read as zero
        dma16(rsW, lds_w + (uint32_t)(j * 1024), real ? voffW : kOOB,
              real ? (uint32_t)(kw + 32 * j) * (uint32_t)N * 2u : 0u);
    }

    // Transposing reads of a block: 16-lane group g covers k-rows 8g+4h..+3
    // (h = 0, 1); lane j of the group points at k-row j/4, columns 4(j%4)..+3.
    const int boff = wave * MAXB * 1024 + (8 * ((lane >> 4) & 3) + ((lane >> 2) & 3)) * (BN * 2) + 8 * (lane & 3);
    f32x4 acc[RB];
    float ss[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        ss[i] = 0.0f;
    }
    auto block = [&](auto J) {
        constexpr int j = decltype(J)::value;
        wait_vmcnt<MAXB - 1 - j>();  // block j of this wave landed (and every X / gamma load)
        u32x4 b;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x2 v = ds_tr16(smem + boff + j * 1024 + 4 * h * (BN * 2));
            b[2 * h] = v[0];
            b[2 * h + 1] = v[1];
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            u32x4 a = xa[j][i];
            if constexpr (RMS) a = rms_scale<BF>(a, gv[j], ss[i]);
            acc[i] = mfma16x16x32<BF>(a, b, acc[i]);
        }
        __builtin_amdgcn_sched_barrier(0);  // block j's work stays ahead of block j+1's wait
    };
    static_for<0, MAXB>(block);
    __syncthreads();  // every wave is done with its W slots

    // add the waves' sums in wave order: red[w][i][row][col], sred[w][i][lane]
    float* red = reinterpret_cast<float*>(smem);
    float* sred = red + RED_FLOATS;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            red[((wave * RB + i) * 16 + 4 * (lane >> 4) + r) * 16 + (lane & 15)] = acc[i][r];
        if constexpr (RMS) sred[(wave * RB + i) * 64 + lane] = ss[i];
    }
    __syncthreads();
    // thread t < 2 BM finishes row t/2, columns 8(t%2)..+7
    const int row = tid >> 1, c0 = 8 * (tid & 1);
    const int grow = m0 + row, gcol = n0 + c0;
    const bool active = tid < 2 * BM && grow < M && gcol < N;  // N % 8 == 0: 8 columns all in or all out
    const int blk = row >> 4, rr = row & 15;
    float v[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    float s = 0.0f;  // the row's sum of squares
    if (tid < 2 * BM) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = red[(blk * 16 + rr) * 16 + c0 + e];
#pragma unroll
        for (int w = 1; w < NW; ++w)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += red[((w * RB + blk) * 16 + rr) * 16 + c0 + e];
        if constexpr (RMS) {
            // lanes rr, rr+16, rr+32, rr+48 of each wave hold the row's four k-groups
#pragma unroll
            for (int w = 0; w < NW; ++w)
#pragma unroll
                for (int q = 0; q < 4; ++q) s += sred[(w * RB + blk) * 64 + 16 * q + rr];
        }
    }
    if constexpr (RMS) {
        // rows outside the fast path's range: recompute the tile exactly (an
        // overflowed operand leaves non-finite sums)
        bool bad = false;
        if (active) {
            float t = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) t += v[e];
            bad = rms_outside<BF>(s, K, p.eps) || !__builtin_isfinite(t);
        }
        if (__syncthreads_or(bad)) {
            prologue_exact_tile<BF, 1, NW * 64, BN>(p, smem, m0, BM, n0);
            return;
        }
    }
    if (!active) return;
    finish_store8<BF>(p, v, RMS ? 1.0f / sqrtf(s / (float)K + p.eps) : 1.0f, grow, gcol);
}

}  // namespace dev
}  // namespace lf
