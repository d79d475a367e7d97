// kernel_dma.h -- LDS-DMA pipeline for the fused GEMM kernels on gfx950.
//
// Both operands travel global -> LDS with buffer_load_dwordx4 ... lds: no
// staging registers, so NS LDS stages (NS-1 K steps of loads in flight) cost
// only LDS.  A wave's DMA instruction fills 1 KiB of LDS (lane l writes bytes
// [16 l, 16 l + 16) of it); which global 16-byte chunk each lane fetches is
// free, so the XOR swizzles below are applied on the global side.
//
//   A tile  [BM rows][BK k]   K-contiguous, 16-byte chunk c of row r stored
//                             at chunk c ^ swz_a(r); fragments for the matrix
//                             cores are plain ds_read_b128.
//   W tile  [BK rows][BN n]   N-contiguous as in memory, chunk c of k-row kr
//                             stored at c ^ 4 (kr % 4); B fragments come from
//                             ds_read_b64_tr_b16, the gfx950 transposing LDS
//                             read: within each 16-lane group, lane i gets
//                             element i%4 of the 8 bytes addressed by lane
//                             4e + i/4, for e = 0..3.  With lane j of the group
//                             pointing at k-row (j/4), columns 4(j%4)..+3, lane
//                             i receives column i at four consecutive k, i.e.
//                             the K-contiguous operand the matrix core needs.
//   gamma   [BK]             (RMS only) one 1 KiB slot per stage.
//
// Synchronisation per K step: wait until this wave's loads for the step have
// landed (vmcnt), barrier (every wave's loads landed, every wave done with
// the stage about to be refilled), issue the loads NS-1 steps ahead, compute.
// The DMA and transposing reads are issued from inline assembly, so the
// compiler neither waits for them (it does not know they are in flight) nor
// reorders memory operations across them; the waits are explicit here.
//
// Requires K % BK == 0 (the register-staged kernel covers other K).
#pragma once

#include "common.h"

namespace lf {
namespace dev {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (gfx9 layout): base, stride 0, num_records bytes.
__device__ __forceinline__ i32x4 rsrc128(const void* p, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(p);
    i32x4 r;
    r[0] = (int)(uint32_t)b;
    r[1] = (int)((uint32_t)(b >> 32) & 0xffffu);
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    return r;
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane, global -> LDS at m0 + 16*lane.  m0 is written here and
// nowhere else in these kernels (the compiler does not use it on gfx950), so
// clobbering it cannot disturb compiler-generated code.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

__device__ __forceinline__ u32x2 ds_tr16(uint32_t addr) {
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr) : "memory");
    return r;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

template <int ACH>
__device__ __forceinline__ int swz_a(int r) {
    if constexpr (ACH == 8) return (r ^ (r >> 3)) & 7;
    else return (r >> 2) & 3;
}
__device__ __forceinline__ int swz_b(int kr) { return (kr & 3) << 2; }

// x * gamma, rounded to the 16-bit type (nearest even), and sum x^2 in fp32.
// (Vector elements are copied to scalars before __builtin_bit_cast: applied
// to an element subscript directly, clang takes element 0 every time.)
template <bool BF>
__device__ __forceinline__ u32x4 rms_scale(u32x4 x, u32x4 g, float& ss) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t xq = x[q];
        const uint32_t gq = g[q];
        if constexpr (BF) {
            const bf16x2 xv = __builtin_bit_cast(bf16x2, xq);
            ss = __builtin_amdgcn_fdot2_f32_bf16(xv, xv, ss, false);
            o[q] = pack2<true>(lo_f32<true>(xq) * lo_f32<true>(gq), hi_f32<true>(xq) * hi_f32<true>(gq));
        } else {
            const f16x2 xv = __builtin_bit_cast(f16x2, xq);
            ss = __builtin_amdgcn_fdot2(xv, xv, ss, false);
            const f16x2 prod = xv * __builtin_bit_cast(f16x2, gq);
            o[q] = __builtin_bit_cast(uint32_t, prod);
        }
    }
    return o;
}

template <int BM, int BN, int BK, int NS, int WM, int WN, bool BF, bool RMS, int NB, bool SPLIT>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_dma_kernel(const KArgs p) {
    constexpr int NT = WM * WN * 64;
    constexpr int NW = NT / 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int ACH = BK / 8;
    constexpr int BCH = BN / 8;
    constexpr int A_BYTES = BM * BK * 2;
    constexpr int B_BYTES = BK * BN * 2;
    constexpr int G_OFF = A_BYTES + NB * B_BYTES;
    constexpr int STAGE = G_OFF + (RMS ? 1024 : 0);
    constexpr int A_LD = A_BYTES / (NT * 16);
    constexpr int B_LD = B_BYTES / (NT * 16);
    constexpr int LPT = A_LD + NB * B_LD + (RMS ? 1 : 0);
    static_assert(ACH == 4 || ACH == 8, "BK must be 32 or 64");
    static_assert(BCH >= 16, "BN must be at least 128 for the W swizzle");
    static_assert(A_BYTES % (NT * 16) == 0 && B_BYTES % (NT * 16) == 0, "tiles must split into 1 KiB DMA rows");
    static_assert(BK * 2 <= 1024, "gamma slot");
    static_assert((NS - 2) * LPT <= 63, "vmcnt range");
    using Store = TileStore<BM, BN, WM, WN, BF, RMS, NB>;
    static_assert(Store::kBytes <= NS * STAGE, "epilogue staging must fit in the LDS stages");

    __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE + BM * 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;

    int tm, tn, kz;
    map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, SPLIT ? p.splits : 1, tm, tn, kz);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = SPLIT ? kz * p.kchunk : 0;
    const int M = p.M, N = p.N, K = p.K;

    const i32x4 rsA = rsrc128(p.A + (size_t)m0 * K, (uint32_t)((size_t)(M - m0) * K * 2));
    const uint32_t w_bytes = (uint32_t)(((size_t)K * N - n0) * 2);
    const i32x4 rsW = rsrc128(p.W + n0, w_bytes);
    const i32x4 rsW2 = rsrc128((NB == 2 ? p.W2 : p.W) + n0, w_bytes);
    const i32x4 rsG = rsrc128(RMS ? p.gamma : p.W, RMS ? (uint32_t)K * 2u : 0u);

    // Loop-invariant per-lane global offsets of the DMA rows (bytes).  Rows
    // past M and columns past N carry the out-of-range bit.
    uint32_t voffA[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int q = (i * NW + wave) * 64 + lane;
        const int r = q / ACH, lc = (q % ACH) ^ swz_a<ACH>(q / ACH);
        voffA[i] = oob_or((uint32_t)(r * K + lc * 8) * 2u, m0 + r < M);
    }
    uint32_t voffB[B_LD];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int q = (i * NW + wave) * 64 + lane;
        const int kr = q / BCH, lc = (q % BCH) ^ swz_b(q / BCH);
        voffB[i] = oob_or((uint32_t)(kr * N + lc * 8) * 2u, n0 + lc * 8 < N);
    }
    const uint32_t voffG = oob_or((uint32_t)lane * 16u, lane < ACH);
    const uint32_t lds0 = lds_u32(smem);

    auto issue = [&](int s, int k0) {
        const uint32_t base = lds0 + (uint32_t)(s * STAGE);
        const uint32_t sa = (uint32_t)k0 * 2u;
        const uint32_t sw = (uint32_t)k0 * (uint32_t)N * 2u;
#pragma unroll
        for (int i = 0; i < A_LD; ++i) dma16(rsA, base + (uint32_t)((i * NW + wave) * 1024), voffA[i], sa);
#pragma unroll
        for (int o = 0; o < NB; ++o)
#pragma unroll
            for (int i = 0; i < B_LD; ++i)
                dma16(o ? rsW2 : rsW, base + (uint32_t)(A_BYTES + o * B_BYTES + (i * NW + wave) * 1024), voffB[i],
                      sw);
        if constexpr (RMS) dma16(rsG, base + (uint32_t)G_OFF, voffG, sa);
    };

    f32x16 acc[NB][FM][FN];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[b][i][j][r] = 0.0f;
    float ss[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) ss[i] = 0.0f;

    // Per-lane parts of the fragment addresses that do not depend on the step.
    int arow[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) arow[i] = wm * TM + i * 32 + (lane & 31);
    const int bkr = 8 * (lane >> 5) + ((lane >> 2) & 3);           // k-row within a 16-k step
    const int bcol = wn * TN + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // Fragments of one 16-wide K sub-step, read from LDS by assembly so the
    // waits below are the only ones: two sets alternate, the reads for
    // sub-step t+1 (possibly in the next stage) are in flight while the
    // matrix cores work on sub-step t.
    struct Frags {
        u32x4 a[FM];
        u32x2 b0[NB][FN], b1[NB][FN];
        u32x4 g;
    };
    // One LDS read of the fragments of sub-step ks of stage s: pieces
    // 0..FM-1 are the A rows, then two transposing reads per (operand,
    // column block), then gamma.
    constexpr int NREAD = FM + 2 * NB * FN + (RMS ? 1 : 0);
    auto read_piece = [&](Frags& f, int s, int ks, int r) {
        const uint32_t sbase = lds0 + (uint32_t)(s * STAGE);
        const int lc = 2 * ks + (lane >> 5);
        if (r < FM) {
            const int i = r;
            const uint32_t addr = sbase + (uint32_t)(arow[i] * (BK * 2) + ((lc ^ swz_a<ACH>(arow[i])) << 4));
            asm volatile("ds_read_b128 %0, %1" : "=v"(f.a[i]) : "v"(addr) : "memory");
        } else if (r < FM + 2 * NB * FN) {
            const int t = r - FM;
            const int o = t / (2 * FN), j = (t / 2) % FN, h = t & 1;
            const int kr = 16 * ks + bkr + 4 * h;
            const int n = bcol + 32 * j;
            const uint32_t addr = sbase + (uint32_t)(A_BYTES + o * B_BYTES + kr * (BN * 2) +
                                                     (((n >> 3) ^ swz_b(kr)) << 4) + (((n >> 2) & 1) << 3));
            if (h == 0) f.b0[o][j] = ds_tr16(addr);
            else f.b1[o][j] = ds_tr16(addr);
        } else {
            const uint32_t addr = sbase + (uint32_t)(G_OFF + (lc << 4));
            asm volatile("ds_read_b128 %0, %1" : "=v"(f.g) : "v"(addr) : "memory");
        }
    };
    // One DMA row of stage s (k offset k0): A rows, then W rows per operand,
    // then gamma.
    auto dma_piece = [&](int s, int k0, int d) {
        const uint32_t base = lds0 + (uint32_t)(s * STAGE);
        if (d < A_LD) {
            dma16(rsA, base + (uint32_t)((d * NW + wave) * 1024), voffA[d], (uint32_t)k0 * 2u);
        } else if (d < A_LD + NB * B_LD) {
            const int o = (d - A_LD) / B_LD, i = (d - A_LD) % B_LD;
            dma16(o ? rsW2 : rsW, base + (uint32_t)(A_BYTES + o * B_BYTES + (i * NW + wave) * 1024), voffB[i],
                  (uint32_t)k0 * (uint32_t)N * 2u);
        } else {
            dma16(rsG, base + (uint32_t)G_OFF, voffG, (uint32_t)k0 * 2u);
        }
    };
    // Wait for every outstanding LDS read and tie the fragment registers to
    // the wait, so nothing consumes them before it.
    auto wait_frags = [&](Frags& f) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(f.a[i]));
#pragma unroll
        for (int o = 0; o < NB; ++o)
#pragma unroll
            for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(f.b0[o][j]), "+v"(f.b1[o][j]));
        if constexpr (RMS) asm volatile("" : "+v"(f.g));
    };

    constexpr int KS = BK / 16;
    constexpr int NMMA = NB * FM * FN;
    const int nk = (SPLIT ? min(p.kchunk, K - kbeg) : K) / BK;
    // Prologue: NS-1 stages in flight, wait for the first, queue the next.
    // Steps past the end of K are never computed; they re-read the last
    // tile so every address stays inside the tensors.
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(s, kbeg + min(s, nk - 1) * BK);
    wait_vmcnt<(NS - 2) * LPT>();
    __syncthreads();
    issue(NS - 1, kbeg + min(NS - 1, nk - 1) * BK);
    Frags F0, F1;
#pragma unroll
    for (int r = 0; r < NREAD; ++r) read_piece(F0, 0, 0, r);
    // Sub-step t = kt*KS + ks computes from fragment set t%2.  Its
    // matrix-core instructions are interleaved one by one with the LDS reads
    // of sub-step t+1 and, on the first sub-step of a stage, with the DMA of
    // the stage NS-1 ahead, so neither the LDS queue nor the texture address
    // FIFOs hold the matrix cores up.  When t+1 opens a new stage this wave
    // first waits for its own loads of that stage, then a barrier makes every
    // wave's loads visible and guarantees that no wave still reads the stage
    // that the DMA is about to refill.
    auto substep = [&](Frags& cur, Frags& nxt, int kt, int ks) {
        wait_frags(cur);
        if constexpr (RMS) {
#pragma unroll
            for (int i = 0; i < FM; ++i) cur.a[i] = rms_scale<BF>(cur.a[i], cur.g, ss[i]);
        }
        const bool more_in_stage = ks + 1 < KS;
        const bool next_stage = !more_in_stage && kt + 1 < nk;
        if (next_stage) {
            wait_vmcnt<(NS - 2) * LPT>();
            __syncthreads();
        }
        const int rs_stage = more_in_stage ? kt % NS : (kt + 1) % NS;
        const int rs_ks = more_in_stage ? ks + 1 : 0;
        const int k_dma = kbeg + min(kt + NS, nk - 1) * BK;
#pragma unroll
        for (int m = 0; m < NMMA; ++m) {
            const int o = m / (FM * FN), i = (m / FN) % FM, j = m % FN;
            const u32x4 bfrag = {cur.b0[o][j][0], cur.b0[o][j][1], cur.b1[o][j][0], cur.b1[o][j][1]};
            acc[o][i][j] = mfma32<BF>(cur.a[i], bfrag, acc[o][i][j]);
            __builtin_amdgcn_sched_barrier(0);
            if (m < NREAD && (more_in_stage || next_stage)) read_piece(nxt, rs_stage, rs_ks, m);
            if (m < LPT && next_stage) dma_piece(kt % NS, k_dma, m);
            __builtin_amdgcn_sched_barrier(0);
        }
        // reads that did not fit between the matrix-core instructions
#pragma unroll
        for (int m = NMMA; m < NREAD; ++m)
            if (more_in_stage || next_stage) read_piece(nxt, rs_stage, rs_ks, m);
#pragma unroll
        for (int m = NMMA; m < LPT; ++m)
            if (next_stage) dma_piece(kt % NS, k_dma, m);
    };
    static_assert(KS % 2 == 0, "sub-steps per stage must be even so the fragment sets line up");
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
        for (int ks = 0; ks < KS; ks += 2) {
            substep(F0, F1, kt, ks);
            substep(F1, F0, kt, ks + 1);
        }
    }
    wait_vmcnt<0>();
    __syncthreads();

    if (SPLIT && p.splits > 1) {
        // Split-K.  Every split stores its fp32 partial accumulators (and
        // partial sums of squares) with device-coherent stores, waits for
        // them to complete, then counts in on the tile's counter.  The last
        // split to arrive adds the partials of splits 0..S-1 in that order --
        // its own from registers at its place in the sequence -- so the sum
        // does not depend on arrival order, and finishes the tile.  Device-
        // scope relaxed atomics reach the coherence point directly, so no
        // cache-wide write-back or invalidate is needed.
        constexpr int NACC = NB * FM * FN * 16;  // floats per thread
        const size_t split_floats = (size_t)NT * (NACC + FM);
        const int tile = tm * p.tiles_n + tn;
        float* part = p.ws + (size_t)tile * p.splits * split_floats;
        float* mine = part + (size_t)kz * split_floats;
        // Only outputs inside the [M, N] range travel (decode shapes fill a
        // tile with a handful of rows).  Accumulator register r of a 32x32
        // block holds row 8*(r/4) + 4*(lane/32) + r%4, column lane%32.
        auto in_range = [&](int i, int j, int r) {
            const int row = m0 + wm * TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int col = n0 + wn * TN + j * 32 + (lane & 31);
            return row < M && col < N;
        };
#pragma unroll
        for (int o = 0; o < NB; ++o)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int e = ((o * FM + i) * FN + j) * 16 + r;
                        if (in_range(i, j, r))
                            __hip_atomic_store(mine + (size_t)e * NT + tid, acc[o][i][j][r], __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                    }
        if constexpr (RMS) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                __hip_atomic_store(mine + (size_t)(NACC + i) * NT + tid, ss[i], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        __shared__ unsigned arrived;
        if (tid == 0) arrived = __hip_atomic_fetch_add(p.cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (arrived != (unsigned)(p.splits - 1)) return;
        auto gather = [&](int e, float own) {
            const float* src = part + (size_t)e * NT + tid;
            float v = (kz == 0) ? own : __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int z = 1; z < p.splits; ++z)
                v += (z == kz) ? own
                               : __hip_atomic_load(src + (size_t)z * split_floats, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            return v;
        };
#pragma unroll
        for (int o = 0; o < NB; ++o)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (in_range(i, j, r))
                            acc[o][i][j][r] = gather(((o * FM + i) * FN + j) * 16 + r, acc[o][i][j][r]);
        if constexpr (RMS) {
#pragma unroll
            for (int i = 0; i < FM; ++i) ss[i] = gather(NACC + i, ss[i]);
        }
        // ready for the next call on this workspace (stream order separates calls)
        if (tid == 0) __hip_atomic_store(p.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    float* rs = reinterpret_cast<float*>(smem + NS * STAGE);
    if constexpr (RMS) {
        // lanes l and l+32 hold the two k-halves of row l%32 of each fragment
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const float s = ss[i] + __shfl_xor(ss[i], 32);
            if (wn == 0 && lane < 32) rs[arow[i]] = 1.0f / sqrtf(s / (float)K + p.eps);
        }
        __syncthreads();
    }
    Store::run(p, acc, reinterpret_cast<float*>(smem), rs, m0, n0);
}

}  // namespace dev
}  // namespace lf
