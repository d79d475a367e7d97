// kernel_reg.h -- register-staged pipeline for the fused GEMM kernels.
//
// Structure of one workgroup (256 threads = 4 wave64s in a 2x2 grid):
//   * tile BM x BN of the output, K walked in steps of 64;
//   * A and W tiles fetched with 128-bit buffer loads into registers
//     (out-of-range lanes read zero, which handles the M, N and K tails);
//   * W arrives N-contiguous; each thread transposes a KB(k) x 8(n) block in
//     registers so LDS holds both operands K-contiguous;
//   * LDS rows of 64 halves (8 chunks of 16 B) with the chunk index
//     XOR-swizzled by the row, so fragment reads and tile writes avoid bank
//     conflicts;
//   * two LDS stages and one or two register sets of lookahead;
//   * v_mfma_f32_32x32x16_{f16,bf16}; the A prologue folded into the staging,
//     once per element and workgroup: RMSNorm (X scaled by gamma, sum of
//     squares from the same registers), an input bias (x + b), or LayerNorm
//     (a*x + b from the row statistics, then * gamma + beta), each computed
//     in fp32 and rounded once to the input type.
// Handles any K that is a multiple of 8 (the KT variant masks the K tail).
#pragma once

#include "common.h"

namespace lf {
namespace dev {

constexpr int kBK = 64;          // K step per LDS stage
constexpr int kKCH = kBK / 8;    // 16-byte chunks per LDS row

// ---------------------------------------------------------------- kernel

template <int BM, int BN, int WM, int WN, bool BF, int PRO, int NB, int NREG, bool KT>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_fused_kernel(const KArgs p) {
    constexpr bool RMS = PRO == kProRms;
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int A_CH = BM * kKCH;             // 16 B chunks in an A tile
    static_assert(A_CH % NT == 0, "A tile must split evenly over threads");
    constexpr int A_PER = A_CH / NT;
    constexpr int A_ROW_STEP = NT / kKCH;
    // W tiles move as KB(k) x 8(n) blocks, one per thread per pass; KB = 4
    // when 8x8 blocks would leave threads idle.
    constexpr int KB = (NB * (kBK / 8) * (BN / 8) >= NT) ? 8 : 4;
    constexpr int B_BLK = (kBK / KB) * (BN / 8);   // blocks in one W tile
    constexpr int B_ALL = NB * B_BLK;               // blocks over all W operands
    static_assert(B_ALL % NT == 0, "W tile blocks must split evenly over threads");
    constexpr int B_PER = B_ALL / NT;
    constexpr int A_STAGE = BM * kKCH;          // chunks
    constexpr int B_STAGE = BN * kKCH;
    constexpr int STAGE = A_STAGE + NB * B_STAGE;

    // 2 stages + the per-row RMS factors; static, so the size is part of the
    // kernel descriptor (gfx950 has 160 KiB of LDS per CU).
    __shared__ u32x4 lds[2 * STAGE + (BM * 4 + 15) / 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    int tm, tn, kz_unused;
    map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, 1, tm, tn, kz_unused);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K;

    const auto rsA = make_rsrc(p.A + (size_t)m0 * K, (uint32_t)((size_t)(M - m0) * K * 2));
    const uint32_t w_bytes = (uint32_t)(((size_t)K * N - n0) * 2);
    const auto rsW = make_rsrc(p.W + n0, w_bytes);
    const auto rsW2 = make_rsrc(NB == 2 ? p.W2 + n0 : p.W + n0, w_bytes);
    const auto rsG = make_rsrc(p.gamma, PRO != kProNone ? (uint32_t)K * 2 : 0u);
    // LayerNorm beta; absent, its loads read zeros
    const auto rsBe = make_rsrc(p.beta ? p.beta : p.A, (PRO == kProLn && p.beta) ? (uint32_t)K * 2 : 0u);

    // Thread -> A chunk mapping: row a_row0 + i*A_ROW_STEP, chunk a_kc.
    const int a_kc = tid % kKCH;
    const int a_row0 = tid / kKCH;

    // One register set holds a whole A/W (and gamma) tile on its way from
    // global memory to LDS.  Two sets give the loads two K steps of lead time.
    struct Regs {
        u32x4 a[A_PER];
        u32x4 b[B_PER][KB];
        u32x4 g;   // gamma, or the input bias
        u32x4 be;  // LayerNorm beta
    };
    Regs R0;
    Regs R1;  // unused when NREG == 1
    float ss[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) ss[i] = 0.0f;
    // LayerNorm: the operand of row m is (a[m] x + b[m]) * gamma + beta
    float2 lnab[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        const int row = m0 + a_row0 + i * A_ROW_STEP;
        lnab[i] = make_float2(0.0f, 0.0f);
        if (PRO == kProLn && row < M) lnab[i] = p.stats[row];
    }

    f32x16 acc[NB][FM][FN];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[b][i][j][r] = 0.0f;

    // Per-lane byte offsets, fixed for the whole K loop; rows past M and
    // columns past N carry the out-of-range bit, so they read zeros.  The
    // K step enters through the scalar offset.
    uint32_t offA[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        const int row = a_row0 + i * A_ROW_STEP;
        offA[i] = oob_or((uint32_t)(row * K + a_kc * 8) * 2u, m0 + row < M);
    }
    uint32_t offB[B_PER][KB];
    int opnd_of[B_PER];
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
        const int ball = tid + i * NT;
        // B_BLK is a multiple of 64, so the operand index is the same across a wave
        opnd_of[i] = __builtin_amdgcn_readfirstlane(ball / B_BLK);
        const int b = ball % B_BLK;
        const int nb = b % (BN / 8), kb = b / (BN / 8);
        const bool nok = (n0 + nb * 8) < N;
#pragma unroll
        for (int j = 0; j < KB; ++j) offB[i][j] = oob_or((uint32_t)((kb * KB + j) * N + nb * 8) * 2u, nok);
    }

    auto gload = [&](Regs& R, int k0) {
        const uint32_t sA = (uint32_t)k0 * 2u;
        const uint32_t sW = (uint32_t)k0 * (uint32_t)N * 2u;
        // K tail (KT only): chunks at or past K read zeros
        const bool kaok = !KT || (k0 + a_kc * 8 < K);
#pragma unroll
        for (int i = 0; i < A_PER; ++i) R.a[i] = bload16(rsA, KT ? oob_or(offA[i], kaok) : offA[i], sA);
        if constexpr (PRO != kProNone) R.g = bload16(rsG, oob_or((uint32_t)a_kc * 16u, k0 + a_kc * 8 < K), sA);
        if constexpr (PRO == kProLn) R.be = bload16(rsBe, oob_or((uint32_t)a_kc * 16u, k0 + a_kc * 8 < K), sA);
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const auto rs = (NB == 2 && opnd_of[i] == 1) ? rsW2 : rsW;
            const int kb = ((tid + i * NT) % B_BLK) / (BN / 8);
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                const bool kok = !KT || (k0 + kb * KB + j < K);
                R.b[i][j] = bload16(rs, KT ? oob_or(offB[i][j], kok) : offB[i][j], sW);
            }
        }
    };

    auto lstore = [&](const Regs& R, int stage) {
        u32x4* sA = lds + stage * STAGE;
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            const int row = a_row0 + i * A_ROW_STEP;
            u32x4 v = R.a[i];
            if constexpr (RMS) {
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float x0 = lo_f32<BF>(v[q]), x1 = hi_f32<BF>(v[q]);
                    ss[i] = fmaf(x0, x0, ss[i]);
                    ss[i] = fmaf(x1, x1, ss[i]);
                    o[q] = pack2<BF>(x0 * lo_f32<BF>(R.g[q]), x1 * hi_f32<BF>(R.g[q]));
                }
                v = o;
            } else if constexpr (PRO == kProBias) {
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    o[q] = pack2<BF>(lo_f32<BF>(v[q]) + lo_f32<BF>(R.g[q]), hi_f32<BF>(v[q]) + hi_f32<BF>(R.g[q]));
                v = o;
            } else if constexpr (PRO == kProLn) {
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float t0 = fmaf(lo_f32<BF>(v[q]), lnab[i].x, lnab[i].y);
                    const float t1 = fmaf(hi_f32<BF>(v[q]), lnab[i].x, lnab[i].y);
                    o[q] = pack2<BF>(fmaf(t0, lo_f32<BF>(R.g[q]), lo_f32<BF>(R.be[q])),
                                     fmaf(t1, hi_f32<BF>(R.g[q]), hi_f32<BF>(R.be[q])));
                }
                v = o;
            }
            sA[row * kKCH + (a_kc ^ swz(row))] = v;
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            const int b = (tid + i * NT) % B_BLK;
            const int nb = b % (BN / 8), kb = b / (BN / 8);
            u32x4* sB = sA + A_STAGE + opnd_of[i] * B_STAGE;
            u32x4 cols[8];
            transpose_k8<KB>(R.b[i], cols);
            const int kc = (kb * KB) >> 3;
#pragma unroll
            for (int jn = 0; jn < 8; ++jn) {
                const int n = nb * 8 + jn;
                u32x4* dst = sB + n * kKCH + (kc ^ swz(n));
                if constexpr (KB == 8) {
                    *dst = cols[jn];
                } else {
                    // half of a 16-byte chunk: k in [kb*4, kb*4+4)
                    uint2* d2 = reinterpret_cast<uint2*>(dst) + (kb & 1);
                    *d2 = make_uint2(cols[jn][0], cols[jn][1]);
                }
            }
        }
    };

    auto compute = [&](int stage) {
        const u32x4* sA = lds + stage * STAGE;
        const u32x4* sB = sA + A_STAGE;
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int kc = 2 * ks + (lane >> 5);
            u32x4 af[FM];
            u32x4 bfr[NB][FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * TM + i * 32 + (lane & 31);
                af[i] = sA[row * kKCH + (kc ^ swz(row))];
            }
#pragma unroll
            for (int nbi = 0; nbi < NB; ++nbi)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int n = wn * TN + j * 32 + (lane & 31);
                    bfr[nbi][j] = sB[nbi * B_STAGE + n * kKCH + (kc ^ swz(n))];
                }
#pragma unroll
            for (int nbi = 0; nbi < NB; ++nbi)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[nbi][i][j] = mfma32<BF>(af[i], bfr[nbi][j], acc[nbi][i][j]);
        }
    };

    const int nk = (K + kBK - 1) / kBK;
    if constexpr (NREG == 2) {
        // Step kt computes on LDS stage kt%2.  At its start it writes tile
        // kt+1 (held in register set (kt+1)%2 since step kt-2) into the other
        // stage, which every wave finished reading before the previous
        // barrier, and refills that register set with tile kt+3: loads get two
        // steps of lead time.  Loads past the end of K read zeros and are
        // never stored.
        // Steps past the end of K re-read the last tile (never stored), so
        // every address stays inside the tensors.
        const int klast = (nk - 1) * kBK;
        gload(R0, 0);
        gload(R1, min(kBK, klast));
        lstore(R0, 0);
        gload(R0, min(2 * kBK, klast));
        __syncthreads();
        auto step = [&](Regs& Rw, int kt) {
            if (kt + 1 < nk) {
                lstore(Rw, (kt + 1) & 1);
                gload(Rw, min((kt + 3) * kBK, klast));
            }
            compute(kt & 1);
            __syncthreads();
        };
        for (int kt = 0; kt < nk; kt += 2) {
            step(R1, kt);
            if (kt + 1 < nk) step(R0, kt + 1);
        }
    } else {
        // One register set: tile kt+1 is fetched while step kt computes and is
        // written to the other stage after the matrix-core work is issued.
        gload(R0, 0);
        lstore(R0, 0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const bool more = kt + 1 < nk;
            if (more) gload(R0, (kt + 1) * kBK);
            compute(kt & 1);
            if (more) lstore(R0, (kt + 1) & 1);
            __syncthreads();
        }
    }

    // Per-row RMS factor: reduce the sum of squares over the kKCH lanes that
    // loaded the same row, then r = 1/sqrt(ss/K + eps) into LDS.
    float* rs = reinterpret_cast<float*>(lds + 2 * STAGE);
    if constexpr (RMS) {
        bool bad = false;
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            float s = ss[i];
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            s += __shfl_xor(s, 4);
            const int row = a_row0 + i * A_ROW_STEP;
            if (a_kc == 0) rs[row] = 1.0f / sqrtf(s / (float)K + p.eps);
            bad |= m0 + row < M && rms_outside<BF>(s, K, p.eps);
        }
        // rows outside the fast path's range: recompute the tile exactly
        // (an overflowed operand leaves a non-finite accumulator)
        float t = 0.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) t += acc[b][i][j][r];
        bad |= !__builtin_isfinite(t);
        __syncthreads();
        if (__syncthreads_or(bad)) {
            prologue_exact_tile<BF, NB, NT, BN>(p, reinterpret_cast<char*>(lds), m0, BM, n0);
            return;
        }
    } else if constexpr (PRO == kProBias || PRO == kProLn) {
        // an operand that left the input type's range (x + b, or a normalised
        // value past the fp16 maximum) leaves a non-finite accumulator:
        // recompute the tile with fp32 operands
        float t = 0.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) t += acc[b][i][j][r];
        if (__syncthreads_or(!__builtin_isfinite(t))) {
            prologue_exact_tile<BF, NB, NT, BN, PRO>(p, reinterpret_cast<char*>(lds), m0, BM, n0);
            return;
        }
    }

    using Store = TileStore<BM, BN, WM, WN, BF, RMS, NB>;
    static_assert(Store::kBytes <= 2 * STAGE * 16, "staging must fit in the LDS stages");
    Store::run(p, acc, reinterpret_cast<float*>(lds), rs, m0, n0, wm, wn);
}

}  // namespace dev
}  // namespace lf
