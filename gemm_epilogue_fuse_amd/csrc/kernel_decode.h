// kernel_decode.h -- the small-M (decode-shaped) fused GEMM on gfx950.
//
// With M = B a handful of rows, Y = act(r * (X*gamma) W + bias) + R is bound
// by streaming W [K, N] from HBM once ("LLMBoost", decode-shape sweep: the
// speedup is highest at small batch).  What matters is that every CU keeps a
// large share of W in flight, so:
//
//   * a workgroup owns a 32-row x BN-column output tile and a K chunk of at
//     most 8 steps of 64; all of its W chunk (<= 64 KiB) is requested from
//     HBM at once, global -> LDS with buffer_load_dwordx4 ... lds, and two
//     workgroups share a CU;
//   * X and gamma never touch LDS: the A operand of the 32x32x16 matrix-core
//     instruction is K-contiguous (lane l: row l%32, 8 consecutive k), which
//     is how X is stored, so each lane loads its fragment straight into
//     registers, all of them up front;
//   * the four waves split every 64-wide K step (wave w takes k 16w..16w+15),
//     so each W element is read from LDS exactly once, and their partial sums
//     are added through LDS in wave order;
//   * K chunks are split across workgroups and reduced in chunk order by the
//     last workgroup of a tile to finish (deterministic), as in the tiled
//     kernel.
//
// W in LDS: stage t holds k-rows 64t..64t+63 of the chunk, row kr of BN
// halves with 16-byte chunk c stored at c ^ swz(kr); B fragments come from
// ds_read_b64_tr_b16 exactly as in the tiled kernel.
//
// Requires K % 64 == 0 and a K chunk of at most 8 * 64.
#pragma once

#include "common.h"
#include "kernel_dma.h"

namespace lf {
namespace dev {

// W row swizzle for a tile of BN halves per k-row, conflict-free for the
// transposing reads (4 k-rows at the same columns per 16-lane group).
template <int BN>
__device__ __forceinline__ int swz_w(int kr) {
    if constexpr (BN >= 128) return (kr & 3) << 2;  // rows fill 256-byte bank lines
    else return ((kr >> 1) & 1) << 2;                // two 128-byte rows per bank line
}

template <int BN, bool BF, bool RMS>
__global__ void __launch_bounds__(256, 2)
gemm_decode_kernel(const KArgs p) {
    constexpr int BM = 32, BK = 64, NT = 256, NS = 8;
    constexpr int FN = BN / 32;
    constexpr int BCH = BN / 8;                  // 16-byte chunks per W k-row
    constexpr int STAGE = BK * BN * 2;           // bytes of W per 64-wide K step
    constexpr int W_LD = STAGE / (NT * 16);      // DMA rows per thread and step
    constexpr int CPR = BN / 8;                  // 8-column chunks per output row
    static_assert(BN == 64 || BN == 128, "BN must be 64 or 128");
    static_assert(STAGE % (NT * 16) == 0, "W stage splits into 1 KiB DMA rows");
    static_assert(BM * CPR == NT, "one 8-column output chunk per thread");
    static_assert(4 * BM * BN * 4 <= NS * STAGE, "wave reduction fits in the W stages");

    __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE + 4 * 64 * 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int tm, tn, kz;
    map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, p.splits, tm, tn, kz);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K;
    const int kbeg = kz * p.kchunk;
    const int nk = min(p.kchunk, K - kbeg) / BK;  // 1..NS steps

    // ---- requests: every W row of the chunk, then every A and gamma fragment
    const i32x4 rsW = rsrc128(p.W + n0, (uint32_t)(((size_t)K * N - n0) * 2));
    const uint32_t lds0 = lds_u32(smem);
#pragma unroll
    for (int t = 0; t < NS; ++t) {
        if (t < nk) {
#pragma unroll
            for (int i = 0; i < W_LD; ++i) {
                const int q = (i * 4 + wave) * 64 + lane;
                const int kr = q / BCH, lc = (q % BCH) ^ swz_w<BN>(q / BCH);
                const uint32_t voff = oob_or((uint32_t)(kr * N + lc * 8) * 2u, n0 + lc * 8 < N);
                dma16(rsW, lds0 + (uint32_t)(t * STAGE + (i * 4 + wave) * 1024), voff,
                      (uint32_t)(kbeg + t * BK) * (uint32_t)N * 2u);
            }
        }
    }
    // A fragment of sub-step (t, wave): row m0 + lane%32, k = kbeg + 64t + 16*wave + 8*(lane/32).
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A + (size_t)m0 * K, (uint32_t)((size_t)(M - m0) * K * 2));
    const int arow = lane & 31;
    const uint32_t avoff = oob_or((uint32_t)(arow * K + kbeg + 16 * wave + 8 * (lane >> 5)) * 2u, m0 + arow < M);
    u32x4 af[NS], gf[NS];
#pragma unroll
    for (int t = 0; t < NS; ++t) {
        if (t < nk) af[t] = bload16(rA, avoff, (uint32_t)(t * BK * 2));
    }
    if constexpr (RMS) {
        const __amdgpu_buffer_rsrc_t rG = make_rsrc(p.gamma, (uint32_t)K * 2u);
        const uint32_t gvoff = (uint32_t)(kbeg + 16 * wave + 8 * (lane >> 5)) * 2u;
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            if (t < nk) gf[t] = bload16(rG, gvoff, (uint32_t)(t * BK * 2));
        }
    }
    wait_vmcnt<0>();
    __syncthreads();

    // ---- this wave's sub-steps
    f32x16 acc[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    float ss = 0.0f;
    const int bkr = 8 * (lane >> 5) + ((lane >> 2) & 3);
    const int bcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    // all B fragments of the chunk first, so the LDS reads overlap
    u32x4 bf[NS][FN];
#pragma unroll
    for (int t = 0; t < NS; ++t) {
        if (t < nk) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int kr = 16 * wave + bkr + 4 * h;
                    const int n = bcol + 32 * j;
                    const int off = t * STAGE + kr * (BN * 2) + (((n >> 3) ^ swz_w<BN>(kr)) << 4) +
                                    (((n >> 2) & 1) << 3);
                    const u32x2 v = ds_tr16(smem + off);
                    bf[t][j][2 * h] = v[0];
                    bf[t][j][2 * h + 1] = v[1];
                }
        }
    }
#pragma unroll
    for (int t = 0; t < NS; ++t) {
        if (t < nk) {
            u32x4 a = af[t];
            if constexpr (RMS) a = rms_scale<BF>(a, gf[t], ss);
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[j] = mfma32<BF>(a, bf[t][j], acc[j]);
        }
    }
    __syncthreads();  // every wave is done with the W stages

    // ---- add the four waves' sums, in wave order, through LDS
    float* red = reinterpret_cast<float*>(smem);         // [4][BM][BN]
    float* sred = reinterpret_cast<float*>(smem + NS * STAGE);  // [4][64]
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            red[(wave * BM + row) * BN + 32 * j + (lane & 31)] = acc[j][r];
        }
    if constexpr (RMS) sred[wave * 64 + lane] = ss;
    __syncthreads();
    // thread t finishes row t / CPR, columns 8 * (t % CPR) .. +7
    const int row = tid / CPR, c0 = 8 * (tid % CPR);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = red[row * BN + c0 + e];
#pragma unroll
    for (int w = 1; w < 4; ++w)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += red[(w * BM + row) * BN + c0 + e];
    float srow = 0.0f;  // sum of squares of this row over the chunk (lanes row and row+32 of each wave)
    if constexpr (RMS) {
#pragma unroll
        for (int w = 0; w < 4; ++w) srow += sred[w * 64 + row] + sred[w * 64 + 32 + row];
    }
    const bool row_ok = m0 + row < M;

    if (p.splits > 1) {
        // Split-K, as in the tiled kernel: device-coherent partials, the last
        // workgroup of the tile adds chunks 0..S-1 in that order.
        constexpr int SPLIT_BYTES = NT * 36;  // 8 floats + the row's sum of squares per thread
        const int tile = tm * p.tiles_n + tn;
        float* part = p.ws + (size_t)tile * p.splits * (SPLIT_BYTES / 4);
        const __amdgpu_buffer_rsrc_t rsP = make_rsrc(part, (uint32_t)(p.splits * SPLIT_BYTES));
        const uint32_t own_off = (uint32_t)(kz * SPLIT_BYTES);
        if (row_ok) {
            const u32x4 v0 = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
            const u32x4 v1 = {__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])};
            __builtin_amdgcn_raw_buffer_store_b128(v0, rsP, (uint32_t)(tid * 32), own_off, 16);
            __builtin_amdgcn_raw_buffer_store_b128(v1, rsP, (uint32_t)(tid * 32 + 16), own_off, 16);
            if constexpr (RMS)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(srow), rsP, (uint32_t)(NT * 32 + tid * 4),
                                                      own_off, 16);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        __shared__ unsigned arrived;
        if (tid == 0) arrived = __hip_atomic_fetch_add(p.cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (arrived != (unsigned)(p.splits - 1)) return;
        if (row_ok) {
            // chunks z = 0..S-1 in order, eight in flight at a time
            constexpr int BATCH = 8;
            float s[8], sq = 0.0f;
            for (int z0 = 0; z0 < p.splits; z0 += BATCH) {
                f32x4 a0[BATCH], a1[BATCH];
                float aq[BATCH];
#pragma unroll
                for (int i = 0; i < BATCH; ++i) {
                    const int z = z0 + i;
                    if (z < p.splits && z != kz) {
                        const uint32_t zo = (uint32_t)(z * SPLIT_BYTES);
                        a0[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsP, (uint32_t)(tid * 32), zo, 16));
                        a1[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsP, (uint32_t)(tid * 32 + 16), zo, 16));
                        aq[i] = RMS ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsP, (uint32_t)(NT * 32 + tid * 4), zo, 16))
                                    : 0.0f;
                    }
                }
#pragma unroll
                for (int i = 0; i < BATCH; ++i) {
                    const int z = z0 + i;
                    if (z >= p.splits) break;
                    float w8[8], wsq;
                    if (z == kz) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) w8[e] = v[e];
                        wsq = srow;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            w8[e] = a0[i][e];
                            w8[4 + e] = a1[i][e];
                        }
                        wsq = aq[i];
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) s[e] = (z == 0) ? w8[e] : s[e] + w8[e];
                    sq = (z == 0) ? wsq : sq + wsq;
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = s[e];
            srow = sq;
        }
        // ready for the next call on this workspace (stream order separates calls)
        if (tid == 0) __hip_atomic_store(p.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- epilogue: r[m], bias, activation, residual, one rounding, 16-byte store
    const int gcol = n0 + c0;
    const bool active = row_ok && gcol < N;  // N % 8 == 0: a thread's 8 columns are all in or all out
    if constexpr (RMS) {
        // rows outside the fast path's range: recompute the tile exactly (an
        // overflowed operand leaves non-finite sums)
        bool bad = false;
        if (active) {
            float t = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) t += v[e];
            bad = rms_outside<BF>(srow, K, p.eps) || !__builtin_isfinite(t);
        }
        if (__syncthreads_or(bad)) {
            prologue_exact_tile<BF, 1, NT, BN>(p, smem, m0, BM, n0);
            return;
        }
    }
    if (!active) return;
    finish_store8<BF>(p, v, RMS ? 1.0f / sqrtf(srow / (float)K + p.eps) : 1.0f, m0 + row, gcol);
}

}  // namespace dev
}  // namespace lf
