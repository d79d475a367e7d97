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
//   gamma   [BK]             (with a prologue) one 1 KiB slot per stage for
//                             gamma (RMSNorm, LayerNorm) or the input bias,
//                             and a second one for LayerNorm's beta; with 8
//                             waves loaded by wave 0 alone (the other waves
//                             issue fewer DMA rows per step and wait on counts
//                             that much lower), with 4 waves by every wave.
//
// Synchronisation per K step: wait until this wave's loads for the step have
// landed (vmcnt), barrier (every wave's loads landed, every wave done with
// the stage about to be refilled), issue the loads NS-1 steps ahead, compute.
// The DMA is issued from inline assembly (it has no register result), so the
// compiler neither waits for it nor reorders memory operations across it;
// its waits are explicit here.  Fragment reads are ordinary LDS loads the
// compiler tracks: an asm load would let the compiler copy its destination
// register before the data has landed.
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

template <int N>
using ic = std::integral_constant<int, N>;

typedef short i16x4 __attribute__((ext_vector_type(4)));
// ds_read_b64_tr_b16 through the compiler builtin, so the compiler knows the
// load is in flight and waits for it before the result is used.
__device__ __forceinline__ u32x2 ds_tr16(const char* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p)));
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
// bf16 has no packed multiply, so each product comes from a two-term dot
// product against gamma with the other half zeroed: a bf16 x bf16 product is
// exact in fp32, so this equals the fp32 multiply, and the one rounding is the
// conversion back to bf16.  (Vector elements are copied to scalars before
// __builtin_bit_cast: applied to an element subscript directly, clang takes
// element 0 every time.)
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
            // (compiler builtins, not inline assembly: x comes from an LDS
            // read the compiler must see consumed to place its wait)
            const float plo = __builtin_amdgcn_fdot2_f32_bf16(xv, __builtin_bit_cast(bf16x2, gq & 0xffffu), 0.0f, false);
            const float phi =
                __builtin_amdgcn_fdot2_f32_bf16(xv, __builtin_bit_cast(bf16x2, gq & 0xffff0000u), 0.0f, false);
            o[q] = pack2<true>(plo, phi);
        } else {
            const f16x2 xv = __builtin_bit_cast(f16x2, xq);
            ss = __builtin_amdgcn_fdot2(xv, xv, ss, false);
            const f16x2 prod = xv * __builtin_bit_cast(f16x2, gq);
            o[q] = __builtin_bit_cast(uint32_t, prod);
        }
    }
    return o;
}

// bf16 scaling of one 8-value A fragment, o = round_bf16(x * gamma) pairwise,
// and ss += x.x, for the one-slot-ahead path.  Each product is one
// three-operand dot2 against gamma with the other half masked to zero (exact:
// the product of two bf16 values fits fp32), which saves the zeroing move the
// compiler pairs with its two-operand form.  gl/gh hold gamma masked to its
// low / high halves.  t is scratch that stays live across the whole K loop,
// so its registers are never operands of matrix-core instructions still in
// flight; every dot2 result is read at least three instructions after it is
// written, and so is the running ss.
__device__ __forceinline__ void rms_scale_bf16_ahead(u32x4& x, const uint32_t (&gl)[4], const uint32_t (&gh)[4],
                                                     float& ss, float (&t)[8]) {
    asm volatile(
        "v_dot2c_f32_bf16 %[ss], %[x0], %[x0]\n\t"
        "v_dot2_f32_bf16 %[t0], %[x0], %[l0], 0\n\t"
        "v_dot2_f32_bf16 %[t1], %[x0], %[h0], 0\n\t"
        "v_dot2_f32_bf16 %[t2], %[x1], %[l1], 0\n\t"
        "v_dot2c_f32_bf16 %[ss], %[x1], %[x1]\n\t"
        "v_dot2_f32_bf16 %[t3], %[x1], %[h1], 0\n\t"
        "v_dot2_f32_bf16 %[t4], %[x2], %[l2], 0\n\t"
        "v_dot2_f32_bf16 %[t5], %[x2], %[h2], 0\n\t"
        "v_dot2c_f32_bf16 %[ss], %[x2], %[x2]\n\t"
        "v_dot2_f32_bf16 %[t6], %[x3], %[l3], 0\n\t"
        "v_dot2_f32_bf16 %[t7], %[x3], %[h3], 0\n\t"
        "v_cvt_pk_bf16_f32 %[x0], %[t0], %[t1]\n\t"
        "v_dot2c_f32_bf16 %[ss], %[x3], %[x3]\n\t"
        "v_cvt_pk_bf16_f32 %[x1], %[t2], %[t3]\n\t"
        "v_cvt_pk_bf16_f32 %[x2], %[t4], %[t5]\n\t"
        "v_cvt_pk_bf16_f32 %[x3], %[t6], %[t7]"
        : [x0] "+v"(x[0]), [x1] "+v"(x[1]), [x2] "+v"(x[2]), [x3] "+v"(x[3]), [ss] "+v"(ss), [t0] "+v"(t[0]),
          [t1] "+v"(t[1]), [t2] "+v"(t[2]), [t3] "+v"(t[3]), [t4] "+v"(t[4]), [t5] "+v"(t[5]), [t6] "+v"(t[6]),
          [t7] "+v"(t[7])
        : [l0] "v"(gl[0]), [l1] "v"(gl[1]), [l2] "v"(gl[2]), [l3] "v"(gl[3]), [h0] "v"(gh[0]), [h1] "v"(gh[1]),
          [h2] "v"(gh[2]), [h3] "v"(gh[3]));
}

// bf16 pairs {1, 0} and {0, 1}: a two-term dot product against them with an
// fp32 addend picks one half of x and adds to it in fp32.  The pair is moved
// into a scalar register by hand: left as a constant, the compiler encodes
// {1, 0} as the inline constant 1.0, which the bf16 dot instruction does not
// read as that pair (the results came out wrong).
constexpr uint32_t kBf16OneLo = 0x00003f80u, kBf16OneHi = 0x3f800000u;
template <uint32_t V>
__device__ __forceinline__ bf16x2 bf16_pair() {
    uint32_t r;
    asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(V));
    return __builtin_bit_cast(bf16x2, r);
}

// Input-bias prologue: x + b for dwords q0..q0+nq-1 of one 8-value A
// fragment, in place, rounded once to the 16-bit type (fp16: one packed add;
// bf16: the sum in fp32, then rounded).
template <bool BF>
__device__ __forceinline__ void bias_add(u32x4& x, const u32x4& b, int q0 = 0, int nq = 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (q < q0 || q >= q0 + nq) continue;
        const uint32_t xq = x[q];
        const uint32_t bq = b[q];
        if constexpr (BF) {
            const bf16x2 xv = __builtin_bit_cast(bf16x2, xq);
            const float lo = __builtin_amdgcn_fdot2_f32_bf16(xv, bf16_pair<kBf16OneLo>(),
                                                             __uint_as_float(bq << 16), false);
            const float hi = __builtin_amdgcn_fdot2_f32_bf16(xv, bf16_pair<kBf16OneHi>(),
                                                             __uint_as_float(bq & 0xffff0000u), false);
            x[q] = pack2<true>(lo, hi);
        } else {
            x[q] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, xq) + __builtin_bit_cast(f16x2, bq));
        }
    }
}

// LayerNorm prologue.  The statistics pass stores per row a 16-byte record:
// for fp16 inputs the mean as a two-term fp16 sum mu_hi + mu_lo and
// s = sqrt(var + eps), each as a half pair; for bf16 inputs mu and s as
// floats (words 0 and 2); in both the float rstd = 1/s in word 3, negative
// for a row outside the fast path's window.  The operand of x is
//     round((x - mu) * gamma + beta * s),
// and rstd multiplies the fp32 accumulator, so that rstd * sum_k op_k W[k,n]
// is the GEMM of the normalised activation (x - mu) * rstd * gamma + beta.
// Subtracting the mean before any rounding keeps rows whose mean is large
// against their spread exact; fp16 does it in packed fp16 (mu_hi, then mu_lo,
// then one fused multiply-add), bf16 in fp32.  Dwords q0..q0+nq-1, in place.
template <bool BF>
__device__ __forceinline__ void ln_apply(u32x4& x, const u32x4& g, const u32x4& be, const u32x4& st, int q0 = 0,
                                         int nq = 4) {
    if constexpr (BF) {
        const float mu = __uint_as_float(st[0]), sd = __uint_as_float(st[2]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q < q0 || q >= q0 + nq) continue;
            const uint32_t xq = x[q], gq = g[q], bq = be[q];
            const bf16x2 xv = __builtin_bit_cast(bf16x2, xq);
            const float dlo = __builtin_amdgcn_fdot2_f32_bf16(xv, bf16_pair<kBf16OneLo>(), -mu, false);
            const float dhi = __builtin_amdgcn_fdot2_f32_bf16(xv, bf16_pair<kBf16OneHi>(), -mu, false);
            const float lo = __builtin_fmaf(dlo, __uint_as_float(gq << 16), __uint_as_float(bq << 16) * sd);
            const float hi = __builtin_fmaf(dhi, __uint_as_float(gq & 0xffff0000u), __uint_as_float(bq & 0xffff0000u) * sd);
            x[q] = pack2<true>(lo, hi);
        }
    } else {
        const uint32_t w0 = st[0], w1 = st[1], w2 = st[2];
        const f16x2 mh = __builtin_bit_cast(f16x2, w0), ml = __builtin_bit_cast(f16x2, w1);
        const f16x2 sd = __builtin_bit_cast(f16x2, w2);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q < q0 || q >= q0 + nq) continue;
            const uint32_t xq = x[q], gq = g[q], bq = be[q];
            const f16x2 d = (__builtin_bit_cast(f16x2, xq) - mh) - ml;
            const f16x2 bs = __builtin_bit_cast(f16x2, bq) * sd;
            x[q] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(d, __builtin_bit_cast(f16x2, gq), bs));
        }
    }
}

// The workgroup is KG groups of WM x WN waves.  Group g computes the whole
// BM x BN tile over its own share of every K step (16-wide sub-steps
// g*KSG .. g*KSG+KSG-1 of each stage), so KG = 2 doubles the waves that keep
// LDS reads in flight without shrinking the per-wave tile; the groups' sums
// are added through LDS at the end, after which each wave owns FM/KG of its
// row blocks.
template <int BM, int BN, int BK, int NS, int WM, int WN, int KG, bool SRA, bool BF, int PRO, int NB, bool SPLIT>
__global__ void __launch_bounds__(WM * WN * KG * 64)
gemm_dma_kernel(const KArgs p) {
    constexpr bool RMS = PRO == kProRms;
    constexpr bool LN = PRO == kProLn;
    constexpr bool PV = PRO != kProNone;      // a per-k prologue vector (gamma, the input bias) travels with A
    constexpr int NPV = LN ? 2 : (PV ? 1 : 0);  // 1 KiB slots per stage: gamma or the input bias, then beta
    constexpr bool ROWSCALE = RMS || LN;      // a per-row factor multiplies the accumulator
    static_assert(!SRA || PRO == kProNone || RMS, "step read-ahead carries the RMS prologue only");
    static_assert(PRO <= kProRms || KG == 1, "the bias and LayerNorm prologues use one K group");
    constexpr int NWT = WM * WN;  // waves per K group
    constexpr int NT = NWT * KG * 64;
    constexpr int NW = NT / 64;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int FMO = FM / KG;  // row blocks a wave owns after the group reduction
    constexpr int KS = BK / 16, KSG = KS / KG;
    constexpr int ACH = BK / 8;
    constexpr int BCH = BN / 8;
    constexpr int A_BYTES = BM * BK * 2;
    constexpr int B_BYTES = BK * BN * 2;
    constexpr int G_OFF = A_BYTES + NB * B_BYTES;
    constexpr int STAGE = G_OFF + NPV * 1024;
    constexpr int A_LD = A_BYTES / (NT * 16);
    constexpr int B_LD = B_BYTES / (NT * 16);
    constexpr int LPT = A_LD + NB * B_LD + NPV;  // DMA loads per thread and step (wave 0)
    constexpr bool G1 = PV && NW >= 8;           // the prologue vectors loaded by wave 0 alone
    constexpr int NMMA = NB * FM * FN;
    constexpr int NREAD = FM + 2 * NB * FN + NPV;
    constexpr int WIN = KSG * NMMA;  // matrix-core slots that carry one step's DMA
    static_assert(ACH == 4 || ACH == 8, "BK must be 32 or 64");
    static_assert(BCH >= 16, "BN must be at least 128 for the W swizzle");
    static_assert(A_BYTES % (NT * 16) == 0 && B_BYTES % (NT * 16) == 0, "tiles must split into 1 KiB DMA rows");
    static_assert(BK * 2 <= 1024, "gamma slot");
    static_assert((NS - 2) * LPT <= 63, "vmcnt range");
    static_assert(KG == 1 || KG == 2, "one or two K groups");
    static_assert(FM % KG == 0 && KS % KG == 0, "groups split row blocks and sub-steps evenly");
    static_assert(NS >= 3, "two stages ahead of the one being read");
    static_assert(SRA || KSG % 2 == 0, "sub-step read-ahead alternates fragment sets within a step");
    static_assert(WIN >= LPT, "one DMA row per matrix-core slot at most");
    using Store = TileStore<BM, BN, WM * KG, WN, BF, ROWSCALE, NB>;
    // The epilogue staging reuses the stages' LDS, extended where it needs more.
    constexpr int SMEM_MAIN = (Store::kBytes > NS * STAGE) ? Store::kBytes : NS * STAGE;
    static_assert(SMEM_MAIN + BM * 4 <= 160 * 1024, "LDS per workgroup");
    static_assert(KG == 1 || KG * NWT * FMO * (NB * FN * 16 + 1) * 64 * 4 <= NS * STAGE,
                  "group reduction must fit in the LDS stages");

    __shared__ __attribute__((aligned(1024))) char smem[SMEM_MAIN + BM * 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = KG == 1 ? 0 : wave / NWT, wl = KG == 1 ? wave : wave % NWT;
    const int wm = wl / WN, wn = wl % WN;

    int tm, tn, kz;
    map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, SPLIT ? p.splits : 1, tm, tn, kz);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = SPLIT ? kz * p.kchunk : 0;
    const int M = p.M, N = p.N, K = p.K;

    const i32x4 rsA = rsrc128(p.A + (size_t)m0 * K, (uint32_t)((size_t)(M - m0) * K * 2));
    const uint32_t w_bytes = (uint32_t)(((size_t)K * N - n0) * 2);
    const i32x4 rsW = rsrc128(p.W + n0, w_bytes);
    const i32x4 rsW2 = rsrc128((NB == 2 ? p.W2 : p.W) + n0, w_bytes);
    const i32x4 rsG = rsrc128(PV ? p.gamma : p.W, PV ? (uint32_t)K * 2u : 0u);
    // LayerNorm beta; absent, its loads read zeros
    const i32x4 rsBe = rsrc128((LN && p.beta) ? p.beta : p.W, (LN && p.beta) ? (uint32_t)K * 2u : 0u);

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
        } else if (!G1 || wave == 0) {
            // with 8 waves one wave loads the step's gamma for the workgroup
            // (the barrier that follows its wait makes it visible to every
            // wave): measured 1-3.5% faster there, 3% slower with 4 waves
            const int v = d - A_LD - NB * B_LD;  // 0: gamma or the input bias, 1: beta
            dma16(v ? rsBe : rsG, base + (uint32_t)(G_OFF + v * 1024), voffG, (uint32_t)k0 * 2u);
        }
    };
    // Wait until at most `steps` whole steps of this wave's DMA rows are in
    // flight: LPT rows per step, one fewer on the waves that skip gamma.
    auto wait_steps = [&](auto STEPS) {
        constexpr int n = decltype(STEPS)::value;
        if (!G1 || wave == 0) wait_vmcnt<n * LPT>();
        else wait_vmcnt<n * (G1 ? LPT - NPV : LPT)>();
    };
    auto issue = [&](int s, int k0) {
#pragma unroll
        for (int d = 0; d < LPT; ++d) dma_piece(s, k0, d);
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
    // LayerNorm: this lane's row record of each row block (rows past M: zeros)
    u32x4 lnst[LN ? FM : 1];
#pragma unroll
    for (int i = 0; i < (LN ? FM : 1); ++i) {
        lnst[i] = u32x4{0u, 0u, 0u, 0u};
        if (LN && m0 + arow[i] < M) lnst[i] = *reinterpret_cast<const u32x4*>(p.lnstats + 4 * (size_t)(m0 + arow[i]));
    }
    const int bkr = 8 * (lane >> 5) + ((lane >> 2) & 3);  // k-row within a 16-k step
    const int bcol = wn * TN + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // Fragment read-ahead.  SRA: two sets of a whole K step (the group's KSG
    // sub-steps of 16) alternate, every read of step kt+1 in flight while the
    // matrix cores work on step kt -- for few matrix-core instructions per
    // sub-step.  Otherwise two sets of one sub-step alternate, the reads of
    // sub-step t+1 in flight during sub-step t, which keeps the deepest DMA
    // lookahead.  The reads are ordinary LDS loads, so the compiler tracks
    // them and waits for each fragment right before its first use.
    constexpr int KH = SRA ? KSG : 1;  // sub-steps one set holds
    struct Frags {
        u32x4 a[KH][FM];
        u32x4 b[KH][NB][FN];  // k 0..3 of the lane's group from the first transposing read, 4..7 from the second
        u32x4 g[KH];          // gamma or the input bias
        u32x4 be[KH];         // LayerNorm beta
    };
    // One LDS read of local sub-step ls of stage s into slot h of a set.
    // With sub-step read-ahead pieces come in the order the matrix cores
    // consume them: A block 0 (and gamma), the transposing reads of every
    // (operand, column block), then A blocks 1..FM-1.  With step read-ahead
    // A blocks and gamma come first, so they can be scaled early.
    constexpr int NRB = 2 * NB * FN;  // transposing reads per sub-step
    constexpr int G0 = NPV;
    // With sub-step read-ahead and enough matrix-core slots per sub-step,
    // the next sub-step's A blocks and gamma are read first and scaled a
    // few slots later, while this sub-step's matrix-core work runs, so no
    // matrix-core instruction waits on the scaling.  RMS scales them all in
    // slot AHEAD_SLOT; the bias and LayerNorm prologues spread them (below),
    // which needs a slot after every A and vector read is issued.
    constexpr int AHEAD_SLOT = RMS ? FM + G0 + 2 : FM + G0;
    constexpr bool AHEAD = PV && !SRA && AHEAD_SLOT < NMMA;
    // Bias and LayerNorm spread their transform (below).  RMS scales all
    // blocks in one slot: spread like the others it measured 2-7% slower.
    constexpr bool SPREAD = AHEAD && !RMS;
    // The prologue of dwords q0..q0+nq-1 of A block i of slot h of a
    // fragment set (bias, LayerNorm; RMS scales whole blocks in its own forms).
    auto pro_apply = [&](Frags& f, int h, int i, int q0 = 0, int nq = 4) {
        if constexpr (PRO == kProBias) bias_add<BF>(f.a[h][i], f.g[h], q0, nq);
        else if constexpr (LN) ln_apply<BF>(f.a[h][i], f.g[h], f.be[h], lnst[i], q0, nq);
        else f.a[h][i] = rms_scale<BF>(f.a[h][i], f.g[h], ss[i]);
    };
    // Bias and LayerNorm with sub-step read-ahead: the next sub-step's A
    // blocks are transformed in half blocks (two dwords) spread over the slots
    // from AHEAD_SLOT to the end of the sub-step, so no burst of VALU work
    // holds up the next matrix-core instruction (the wave issues in order).
    constexpr int PSLOT0 = AHEAD_SLOT, PSPAN = NMMA - PSLOT0;
    auto read_piece = [&](Frags& f, int s, int ls, int h, int r) {
        const int ks = g * KSG + ls;
        const int sbase = s * STAGE;
        const int lc = 2 * ks + (lane >> 5);
        if (SRA || AHEAD) {
            // order: A0, gamma, A1..A(FM-1), B pieces -> map to the other order's numbering
            if (r >= 1 + G0 && r < G0 + FM) r = r - G0 - 1 + 1 + G0 + NRB;          // A1..
            else if (r >= G0 + FM) r = r - (G0 + FM) + 1 + G0;                      // B pieces
        }
        if (r == 0 || r >= 1 + G0 + NRB) {
            const int i = (r == 0) ? 0 : r - G0 - NRB;
            const int off = sbase + arow[i] * (BK * 2) + ((lc ^ swz_a<ACH>(arow[i])) << 4);
            f.a[h][i] = *reinterpret_cast<const u32x4*>(smem + off);
        } else if (PV && r >= 1 && r <= G0) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(smem + sbase + G_OFF + (r - 1) * 1024 + (lc << 4));
            if (r == 1) f.g[h] = v;
            else f.be[h] = v;
        } else {
            const int t = r - 1 - G0;
            const int o = t / (2 * FN), j = (t / 2) % FN, q = t & 1;
            const int kr = 16 * ks + bkr + 4 * q;
            const int n = bcol + 32 * j;
            const int off = sbase + A_BYTES + o * B_BYTES + kr * (BN * 2) + (((n >> 3) ^ swz_b(kr)) << 4) +
                            (((n >> 2) & 1) << 3);
            const u32x2 v = ds_tr16(smem + off);
            f.b[h][o][j][2 * q] = v[0];
            f.b[h][o][j][2 * q + 1] = v[1];
        }
    };
    // The matrix-core instruction of slot m of a sub-step on slot h of a
    // set.  With sub-step read-ahead A block i is scaled by gamma just before
    // its first use; with step read-ahead the scaling runs a sub-step ahead
    // (see below).
    auto mma = [&](Frags& cur, int h, int m) {
        const int o = m / (FM * FN), i = (m / FN) % FM, j = m % FN;
        if constexpr (PV && !SRA && !AHEAD)
            if (o == 0 && j == 0) pro_apply(cur, h, i);
        acc[o][i][j] = mfma32<BF>(cur.a[h][i], cur.b[h][o][j], acc[o][i][j]);
    };

    const int nk = (SPLIT ? min(p.kchunk, K - kbeg) : K) / BK;
    auto kstep = [&](int t) { return kbeg + min(t, nk - 1) * BK; };
    // Steps past the end of K are never computed; their loads re-read the
    // last tile so every address stays inside the tensors.
    Frags F0, F1;
    if constexpr (SRA) {
        // Prologue: steps 0..NS-2 in flight, wait for the first, read it.
#pragma unroll
        for (int s = 0; s < NS - 1; ++s) issue(s, kstep(s));
        wait_steps(ic<NS - 2>{});
        __syncthreads();
#pragma unroll
        for (int ls = 0; ls < KSG; ++ls)
#pragma unroll
            for (int r = 0; r < NREAD; ++r) read_piece(F0, 0, ls, ls, r);
        if constexpr (RMS) {
#pragma unroll
            for (int i = 0; i < FM; ++i) F0.a[0][i] = rms_scale<BF>(F0.a[0][i], F0.g[0], ss[i]);
        }
        // Step kt.  Unless it is the last: wait for this wave's loads of
        // step kt+1, then a barrier makes every wave's loads visible and
        // guarantees that no wave still reads stage kt-1 (its fragments were
        // consumed in step kt-1).  The matrix-core instructions of step kt
        // are interleaved one by one with the LDS reads of step kt+1 and with
        // the DMA of step kt+NS-1 into the freed stage, each spread evenly
        // over the WIN slots.  RMS: the A blocks of the following sub-step
        // (the next step's first, on the last sub-step) are scaled by gamma
        // in the slots of the current one, off the matrix cores' dependency
        // path.  FINAL marks the last step, so the steady-state steps carry
        // no conditions at all.
        constexpr int RT = KSG * NREAD;  // fragment reads per step
        // scratch of the bf16 scaling, live across the loop
        float sct[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) sct[q] = 0.0f;
        auto step = [&](Frags& cur, Frags& nxt, int kt, auto FINAL) {
            constexpr bool fin = decltype(FINAL)::value;
            if constexpr (!fin) {
                wait_steps(ic<NS - 3>{});
                __syncthreads();
            }
            const int rs_stage = (kt + 1) % NS;
            const int dstage = (kt + NS - 1) % NS;
            const int k_dma = kstep(kt + NS - 1);
#pragma unroll
            for (int ls = 0; ls < KSG; ++ls) {
                uint32_t gl[4], gh[4];  // gamma of the following sub-step, masked to each half
#pragma unroll
                for (int m = 0; m < NMMA; ++m) {
                    mma(cur, ls, m);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (!fin) {
                        const int slot = ls * NMMA + m;
#pragma unroll
                        for (int q = 0; q < RT; ++q)
                            if ((q * WIN) / RT == slot) read_piece(nxt, rs_stage, q / NREAD, q / NREAD, q % NREAD);
#pragma unroll
                        for (int d = 0; d < LPT; ++d)
                            if ((d * WIN) / LPT == slot) dma_piece(dstage, k_dma, d);
                    }
                    if constexpr (RMS) {
                        // block i of the following sub-step at slot NMMA-FM+i
                        const int i = m - (NMMA - FM);
                        if (i >= 0 && (ls + 1 < KSG || !fin)) {
                            Frags& f = (ls + 1 < KSG) ? cur : nxt;
                            const int h = (ls + 1 < KSG) ? ls + 1 : 0;
                            if constexpr (BF) {
                                if (i == 0) {
#pragma unroll
                                    for (int q = 0; q < 4; ++q) {
                                        gl[q] = f.g[h][q] & 0xffffu;
                                        gh[q] = f.g[h][q] & 0xffff0000u;
                                    }
                                }
                                rms_scale_bf16_ahead(f.a[h][i], gl, gh, ss[i], sct);
                            } else {
                                f.a[h][i] = rms_scale<BF>(f.a[h][i], f.g[h], ss[i]);
                            }
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        int kt = 0;
        for (; kt + 2 < nk; kt += 2) {
            step(F0, F1, kt, std::false_type{});
            step(F1, F0, kt + 1, std::false_type{});
        }
        if (nk - kt == 2) {
            step(F0, F1, kt, std::false_type{});
            step(F1, F0, kt + 1, std::true_type{});
        } else {
            step(F0, F1, kt, std::true_type{});
        }
    } else {
        // Prologue: NS-1 stages in flight, wait for the first, queue the
        // next, read the first sub-step.
#pragma unroll
        for (int s = 0; s < NS - 1; ++s) issue(s, kstep(s));
        wait_steps(ic<NS - 2>{});
        __syncthreads();
        issue(NS - 1, kstep(NS - 1));
#pragma unroll
        for (int r = 0; r < NREAD; ++r) read_piece(F0, 0, 0, 0, r);
        if constexpr (AHEAD) {
#pragma unroll
            for (int i = 0; i < FM; ++i) pro_apply(F0, 0, i);
        }
        // scratch of the bf16 one-slot-ahead scaling, live across the loop
        float sct[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) sct[q] = 0.0f;
        // Local sub-step s of step kt computes from set s%2.  Its
        // matrix-core instructions are interleaved one by one with the LDS
        // reads of the next local sub-step and with DMA rows.  On the last
        // local sub-step of a step the wave first waits for its own loads of
        // the next stage, then a barrier makes every wave's loads visible and
        // guarantees that no wave still reads the current stage; the loads of
        // step kt+NS into that stage are then spread over the WIN
        // matrix-core slots from there to the end of step kt+1's
        // second-to-last local sub-step (before the barrier that waits for
        // them).  FIRST / FINAL mark the first and last step, so the
        // steady-state steps carry no conditions at all.
        auto substep = [&](Frags& cur, Frags& nxt, int kt, auto S, auto FIRST, auto FINAL) {
            constexpr int s = decltype(S)::value;
            constexpr bool first = decltype(FIRST)::value, fin = decltype(FINAL)::value;
            constexpr bool last = s == KSG - 1;
            constexpr bool next_stage = last && !fin;
            constexpr bool do_read = !last || next_stage;
            constexpr bool do_dma = last ? !fin : !first;
            constexpr int widx = last ? 0 : s + 1;
            if constexpr (next_stage) {
                wait_steps(ic<NS - 2>{});
                __syncthreads();
            }
            const int rs_stage = last ? (kt + 1) % NS : kt % NS;
            constexpr int rs_ls = last ? 0 : s + 1;
            const int dstep = last ? kt : kt - 1;
            const int k_dma = kstep(dstep + NS);
#pragma unroll
            for (int m = 0; m < NMMA; ++m) {
                mma(cur, 0, m);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (do_read)
                    if (m < NREAD) read_piece(nxt, rs_stage, rs_ls, 0, m);
                if constexpr (SPREAD && do_read) {
#pragma unroll
                    for (int pp = 0; pp < 2 * FM; ++pp)
                        if (m == PSLOT0 + (pp * PSPAN) / (2 * FM)) pro_apply(nxt, 0, pp >> 1, 2 * (pp & 1), 2);
                }
                if constexpr (AHEAD && !SPREAD && do_read)
                    if (m == AHEAD_SLOT) {
                        // all blocks in one slot: independent chains the
                        // scheduler can interleave
                        if constexpr (BF && RMS) {
                            uint32_t gl[4], gh[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                gl[q] = nxt.g[0][q] & 0xffffu;
                                gh[q] = nxt.g[0][q] & 0xffff0000u;
                            }
#pragma unroll
                            for (int i = 0; i < FM; ++i) rms_scale_bf16_ahead(nxt.a[0][i], gl, gh, ss[i], sct);
                        } else {
#pragma unroll
                            for (int i = 0; i < FM; ++i) pro_apply(nxt, 0, i);
                        }
                    }
                if constexpr (do_dma) {
#pragma unroll
                    for (int d = 0; d < LPT; ++d)
                        if (widx * NMMA + m == (d * WIN) / LPT) dma_piece(dstep % NS, k_dma, d);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // reads that did not fit between the matrix-core instructions
            if constexpr (do_read) {
#pragma unroll
                for (int m = NMMA; m < NREAD; ++m) read_piece(nxt, rs_stage, rs_ls, 0, m);
            }
        };
        auto step = [&](int kt, auto FIRST, auto FINAL) {
            substep(F0, F1, kt, ic<0>{}, FIRST, FINAL);
            substep(F1, F0, kt, ic<1>{}, FIRST, FINAL);
            if constexpr (KSG == 4) {
                substep(F0, F1, kt, ic<2>{}, FIRST, FINAL);
                substep(F1, F0, kt, ic<3>{}, FIRST, FINAL);
            }
        };
        if (nk == 1) {
            step(0, std::true_type{}, std::true_type{});
        } else {
            step(0, std::true_type{}, std::false_type{});
            for (int kt = 1; kt < nk - 1; ++kt) step(kt, std::false_type{}, std::false_type{});
            step(nk - 1, std::false_type{}, std::true_type{});
        }
    }
    wait_vmcnt<0>();
    __syncthreads();

    // Add the K groups.  Wave (g, wm, wn) keeps row blocks g*FMO..g*FMO+FMO-1
    // of its wave tile and hands the others to the wave of the other group
    // through LDS (one region per writing group); the sum of a block is
    // group 0's plus group 1's either way (fp32 addition commutes), so
    // results do not depend on which wave adds.
    f32x16 acco[NB][FMO][FN];
    float sso[FMO];
    if constexpr (KG == 1) {
#pragma unroll
        for (int o = 0; o < NB; ++o)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acco[o][i][j] = acc[o][i][j];
#pragma unroll
        for (int i = 0; i < FM; ++i) sso[i] = ss[i];
    } else {
        constexpr int RED = NWT * FMO * NB * FN * 16 * 64;  // floats per group
        float* red = reinterpret_cast<float*>(smem);
        float* sred = red + KG * RED;
        float* red_mine = red + g * RED;
        const float* red_other = red + (1 - g) * RED;
        float* sred_mine = sred + g * NWT * FMO * 64;
        const float* sred_other = sred + (1 - g) * NWT * FMO * 64;
#pragma unroll
        for (int i = 0; i < FMO; ++i) {
#pragma unroll
            for (int o = 0; o < NB; ++o)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        red_mine[((((wl * FMO + i) * NB + o) * FN + j) * 16 + r) * 64 + lane] =
                            g ? acc[o][i][j][r] : acc[o][FMO + i][j][r];
            if constexpr (RMS) sred_mine[(wl * FMO + i) * 64 + lane] = g ? ss[i] : ss[FMO + i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < FMO; ++i) {
#pragma unroll
            for (int o = 0; o < NB; ++o)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acco[o][i][j][r] = (g ? acc[o][FMO + i][j][r] : acc[o][i][j][r]) +
                                           red_other[((((wl * FMO + i) * NB + o) * FN + j) * 16 + r) * 64 + lane];
            if constexpr (RMS) sso[i] = (g ? ss[FMO + i] : ss[i]) + sred_other[(wl * FMO + i) * 64 + lane];
        }
        __syncthreads();
    }
    // From here the wave holds the (wme, wn) tile of a (WM*KG) x WN grid.
    constexpr int TME = TM / KG;
    const int wme = wm * KG + g;

    if (SPLIT && p.splits > 1) {
        // Split-K.  Every split stores its fp32 partial accumulators (and
        // partial sums of squares) with device-coherent stores, waits for
        // them to complete, then counts in on the tile's counter.  The last
        // split to arrive adds the partials of splits 0..S-1 in that order --
        // its own from registers at its place in the sequence -- so the sum
        // does not depend on arrival order, and finishes the tile.  Device-
        // scope (sc1) accesses reach the coherence point directly, so no
        // cache-wide write-back or invalidate is needed.
        constexpr int NQ = NB * FMO * FN * 4;  // 16-byte groups per thread
        constexpr int SPLIT_BYTES = NT * (NQ * 16 + FMO * 4);
        const int tile = tm * p.tiles_n + tn;
        float* part = p.ws + (size_t)tile * p.splits * (SPLIT_BYTES / 4);
        const __amdgpu_buffer_rsrc_t rsP = make_rsrc(part, (uint32_t)(p.splits * SPLIT_BYTES));
        // Only groups of four rows that start inside [M, N] travel (decode
        // shapes fill a tile with a handful of rows).  Accumulator register
        // r of a 32x32 block holds row 8*(r/4) + 4*(lane/32) + r%4, column
        // lane%32; registers 4q..4q+3 are one group.
        auto in_range = [&](int i, int j, int q) {
            const int row = m0 + wme * TME + i * 32 + 8 * q + 4 * (lane >> 5);
            const int col = n0 + wn * TN + j * 32 + (lane & 31);
            return row < M && col < N;
        };
        const uint32_t own_off = (uint32_t)(kz * SPLIT_BYTES);
#pragma unroll
        for (int o = 0; o < NB; ++o)
#pragma unroll
            for (int i = 0; i < FMO; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int e = ((o * FMO + i) * FN + j) * 4 + q;
                        if (in_range(i, j, q)) {
                            const u32x4 v = {__float_as_uint(acco[o][i][j][4 * q]),
                                             __float_as_uint(acco[o][i][j][4 * q + 1]),
                                             __float_as_uint(acco[o][i][j][4 * q + 2]),
                                             __float_as_uint(acco[o][i][j][4 * q + 3])};
                            __builtin_amdgcn_raw_buffer_store_b128(v, rsP, (uint32_t)((e * NT + tid) * 16), own_off,
                                                                   16);
                        }
                    }
        if constexpr (RMS) {
#pragma unroll
            for (int i = 0; i < FMO; ++i)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sso[i]), rsP,
                                                      (uint32_t)(NQ * NT * 16 + (i * NT + tid) * 4), own_off, 16);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        __shared__ unsigned arrived;
        if (tid == 0) arrived = __hip_atomic_fetch_add(p.cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (arrived != (unsigned)(p.splits - 1)) return;
        // Sum the partials in split order 0..S-1.  Each pass issues all of one
        // split's loads before using any, so a split costs one round trip to
        // the coherence point rather than one per 16-byte group.
        f32x16 sum[NB][FMO][FN];
        float ssum[FMO];
        for (int z = 0; z < p.splits; ++z) {
            const uint32_t zoff = (uint32_t)(z * SPLIT_BYTES);
            f32x16 v[NB][FMO][FN];
            float vs[FMO];
            if (z == kz) {
#pragma unroll
                for (int o = 0; o < NB; ++o)
#pragma unroll
                    for (int i = 0; i < FMO; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j) v[o][i][j] = acco[o][i][j];
#pragma unroll
                for (int i = 0; i < FMO; ++i) vs[i] = sso[i];
            } else {
#pragma unroll
                for (int o = 0; o < NB; ++o)
#pragma unroll
                    for (int i = 0; i < FMO; ++i)
#pragma unroll
                        for (int j = 0; j < FN; ++j)
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
                                if (in_range(i, j, q)) {
                                    const int e = ((o * FMO + i) * FN + j) * 4 + q;
                                    t = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                      rsP, (uint32_t)((e * NT + tid) * 16), zoff, 16));
                                }
#pragma unroll
                                for (int t4 = 0; t4 < 4; ++t4) v[o][i][j][4 * q + t4] = t[t4];
                            }
#pragma unroll
                for (int i = 0; i < FMO; ++i)
                    vs[i] = RMS ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                      rsP, (uint32_t)(NQ * NT * 16 + (i * NT + tid) * 4), zoff, 16))
                                : 0.0f;
            }
#pragma unroll
            for (int o = 0; o < NB; ++o)
#pragma unroll
                for (int i = 0; i < FMO; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) sum[o][i][j] = (z == 0) ? v[o][i][j] : sum[o][i][j] + v[o][i][j];
#pragma unroll
            for (int i = 0; i < FMO; ++i) ssum[i] = (z == 0) ? vs[i] : ssum[i] + vs[i];
        }
#pragma unroll
        for (int o = 0; o < NB; ++o)
#pragma unroll
            for (int i = 0; i < FMO; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acco[o][i][j] = sum[o][i][j];
        if constexpr (RMS) {
#pragma unroll
            for (int i = 0; i < FMO; ++i) sso[i] = ssum[i];
        }
        // ready for the next call on this workspace (stream order separates calls)
        if (tid == 0) __hip_atomic_store(p.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    float* rs = reinterpret_cast<float*>(smem + SMEM_MAIN);
    if constexpr (PV) {
        // lanes l and l+32 hold the two k-halves of row l%32 of each block
        bool bad = false;
#pragma unroll
        for (int i = 0; i < FMO; ++i) {
            const int rl = wme * TME + i * 32 + (lane & 31);
            if constexpr (RMS) {
                const float s = sso[i] + __shfl_xor(sso[i], 32);
                if (wn == 0 && lane < 32) rs[rl] = 1.0f / sqrtf(s / (float)K + p.eps);
                bad |= m0 + rl < M && rms_outside<BF>(s, K, p.eps);
            } else if constexpr (LN) {
                const float rstd = __uint_as_float(lnst[i][3]);
                if (wn == 0 && lane < 32) rs[rl] = fabsf(rstd);
                bad |= m0 + rl < M && !(rstd > 0.0f);
            }
        }
        // an operand that overflowed leaves a non-finite accumulator (and
        // the sum of non-finite and finite values is never finite)
        float t = 0.0f;
#pragma unroll
        for (int o = 0; o < NB; ++o)
#pragma unroll
            for (int i = 0; i < FMO; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) t += acco[o][i][j][r];
        bad |= !__builtin_isfinite(t);
        __syncthreads();
        if (__syncthreads_or(bad)) {
            prologue_exact_tile<BF, NB, NT, BN, PRO>(p, smem, m0, BM, n0);
            return;
        }
    }
    Store::run(p, acco, reinterpret_cast<float*>(smem), rs, m0, n0, wme, wn);
}

}  // namespace dev
}  // namespace lf
