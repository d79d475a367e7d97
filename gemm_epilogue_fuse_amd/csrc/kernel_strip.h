// kernel_strip.h -- the few-row fused GEMM on gfx950: one workgroup per
// 16-column strip of the output, all of K, no cross-workgroup reduction.
//
// At a handful of rows (decode: M = B <= 32) the call streams W [K, N] once
// and does almost no arithmetic, so its time is the HBM stream plus any fixed
// latency.  Splitting K across workgroups would need partial sums to cross the
// device (a write-through store, an arrival atomic and the reducer's loads:
// three device-scope round trips, each about a microsecond).  Instead each
// workgroup owns a 16-column strip over the whole of K, and the chip is filled
// by strips (N / 16 workgroups: 256 at N = 4096):
//
//   * W, X and gamma travel global -> LDS with buffer_load_dwordx4 ... lds
//     through an NS-deep ring of 128-wide K steps, so NS-2 steps of W are in
//     flight per CU;
//   * the matrix-core instruction is v_mfma_f32_16x16x32 (A lane l: row
//     l%16, k 8(l/16)..+7; B lane l: column l%16, same k; C register r of
//     lane l: row 4(l/16)+r, column l%16), RB blocks of 16 rows;
//   * each of the four waves takes 32 k of every step and the waves' sums
//     are added through LDS in wave order at the end, so results do not
//     depend on timing.
//
// LDS stage (one 128-wide K step):
//   W [128 k-rows][16 columns]   32 bytes per k-row as in memory; B fragments
//                                 come from ds_read_b64_tr_b16 (16-lane group
//                                 g reads k-rows 8g+4h..+3 for h = 0, 1).
//   A [16 RB rows][128 k]         row-major, 16-byte chunk c of row r stored at
//                                 c ^ (r % 16), conflict-free for the fragment
//                                 reads (16 rows at one chunk).
// gamma [K] sits in its own LDS region, loaded once.
//
// Requires K % 128 == 0 and K <= 8192.
#pragma once

#include "common.h"
#include "kernel_dma.h"

namespace lf {
namespace dev {

typedef float f32x4v __attribute__((ext_vector_type(4)));

template <bool BF>
__device__ __forceinline__ f32x4v mfma16(u32x4 a, u32x4 b, f32x4v c) {
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
}

constexpr int kStripMaxK = 8192;

template <int RB, int NS, bool BF, bool RMS>
__global__ void __launch_bounds__(256, 1)
gemm_strip_kernel(const KArgs p) {
    constexpr int BM = 16 * RB, BN = 16, BK = 128, NT = 256;
    constexpr int W_BYTES = BK * BN * 2;   // 4 KiB: one DMA row per wave
    constexpr int A_BYTES = BM * BK * 2;   // RB * 4 KiB: RB DMA rows per wave
    constexpr int STAGE = W_BYTES + A_BYTES;
    constexpr int G_BYTES = RMS ? kStripMaxK * 2 : 0;
    constexpr int LPT = 1 + RB;            // DMA loads per thread and step
    static_assert((NS - 2) * LPT <= 63, "vmcnt range");
    static_assert(4 * RB * 256 * 4 + 4 * RB * 64 * 4 <= NS * STAGE, "wave reduction fits in the stages");

    __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE + G_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int tm, tn, kz;
    map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, 1, tm, tn, kz);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K;
    const int nk = K / BK;
    const uint32_t lds0 = lds_u32(smem);

    // Per-lane DMA offsets.  W: wave w moves k-rows 32w..32w+31 of a step,
    // lane l the 16-byte half l%2 of k-row 32w + l/2.  A: DMA row d = 4i + w
    // (i < RB) moves rows 4d..4d+3, lane l row 4d + l/16, global chunk
    // (l%16) ^ (row%16) so that LDS chunk l%16 holds it swizzled.
    const i32x4 rsW = rsrc128(p.W, (uint32_t)((size_t)K * N * 2));
    const uint32_t voffW =
        oob_or((uint32_t)((32 * wave + (lane >> 1)) * N + n0 + 8 * (lane & 1)) * 2u, n0 + 8 * (lane & 1) < N);
    const i32x4 rsA = rsrc128(p.A + (size_t)m0 * K, (uint32_t)((size_t)(M - m0) * K * 2));
    uint32_t voffA[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        const int row = 4 * (4 * i + wave) + (lane >> 4);
        voffA[i] = oob_or((uint32_t)(row * K + 8 * ((lane & 15) ^ (row & 15))) * 2u, m0 + row < M);
    }
    auto issue = [&](int stage, int t) {
        const uint32_t base = lds0 + (uint32_t)(stage * STAGE);
        const uint32_t k0 = (uint32_t)(min(t, nk - 1) * BK);  // steps past the end re-read the last one
        dma16(rsW, base + (uint32_t)(wave * 1024), voffW, k0 * (uint32_t)N * 2u);
#pragma unroll
        for (int i = 0; i < RB; ++i)
            dma16(rsA, base + (uint32_t)(W_BYTES + (4 * i + wave) * 1024), voffA[i], k0 * 2u);
    };

    // gamma once, whole K (issued before the ring, so the first step's wait covers it)
    if constexpr (RMS) {
        const i32x4 rsG = rsrc128(p.gamma, (uint32_t)K * 2u);
        const uint32_t gbase = lds0 + (uint32_t)(NS * STAGE);
        for (int c = wave; c * 512 < K; c += 4)
            dma16(rsG, gbase + (uint32_t)(c * 1024), oob_or((uint32_t)(c * 1024 + 16 * lane), c * 512 + 8 * lane < K), 0u);
    }
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(s, s);

    f32x4v acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[i] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    float ss[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) ss[i] = 0.0f;

    // fragment addresses within a stage (this wave's 32 k of the step)
    const int kq = 32 * wave + 8 * (lane >> 4);  // first k of the lane's 8
    int aoff[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        const int row = 16 * i + (lane & 15);
        aoff[i] = W_BYTES + row * (BK * 2) + (((kq >> 3) ^ (row & 15)) << 4);
    }
    // transposing reads: 16-lane group g covers k-rows 8g+4h..+3 of the wave's slice;
    // lane j of the group points at k-row j/4, columns 4(j%4)..+3
    const int g16 = (lane >> 4) & 3;
    const int boff = (32 * wave + 8 * g16 + ((lane >> 2) & 3)) * (BN * 2) + 8 * (lane & 3);

    for (int t = 0; t < nk; ++t) {
        wait_vmcnt<(NS - 2) * LPT>();
        __syncthreads();  // step t landed for every wave; every wave is done with step t-1
        issue((t + NS - 1) % NS, t + NS - 1);
        const int sb = (t % NS) * STAGE;
        u32x4 b;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x2 v = ds_tr16(smem + sb + boff + 4 * h * (BN * 2));
            b[2 * h] = v[0];
            b[2 * h + 1] = v[1];
        }
        u32x4 gv = {0u, 0u, 0u, 0u};
        if constexpr (RMS) gv = *reinterpret_cast<const u32x4*>(smem + NS * STAGE + (t * BK + kq) * 2);
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            u32x4 a = *reinterpret_cast<const u32x4*>(smem + sb + aoff[i]);
            if constexpr (RMS) a = rms_scale<BF>(a, gv, ss[i]);
            acc[i] = mfma16<BF>(a, b, acc[i]);
        }
    }
    wait_vmcnt<0>();
    __syncthreads();  // the trailing loads landed; every wave is done with the stages

    // add the four waves' sums in wave order: red[w][i][row][col], sred[w][i][lane]
    float* red = reinterpret_cast<float*>(smem);
    float* sred = red + 4 * RB * 256;
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
        for (int w = 1; w < 4; ++w)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += red[((w * RB + blk) * 16 + rr) * 16 + c0 + e];
        if constexpr (RMS) {
            // lanes rr, rr+16, rr+32, rr+48 of each wave hold the row's four k-groups
#pragma unroll
            for (int w = 0; w < 4; ++w)
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
            prologue_exact_tile<BF, 1, NT, BN>(p, smem, m0, BM, n0);
            return;
        }
    }
    if (!active) return;
    finish_store8<BF>(p, v, RMS ? 1.0f / sqrtf(s / (float)K + p.eps) : 1.0f, grow, gcol);
}

}  // namespace dev
}  // namespace lf
