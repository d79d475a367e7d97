// gemm_fused.hip -- gfx950 (MI355X) kernels for the fused GEMM + epilogue,
// the RMSNorm -> Linear operator and the SwiGLU gate/up dual GEMM.
//
// What is computed ("llm-fusion-compiler" pattern table and usage example;
// "LLMBoost" problem statement and section 3; deplodock post, RMSNorm loop
// nest):
//     C[m,n]  = sum_k Aop[m,k] * W[k,n]                   (fp32 accumulate)
//     Aop     = A                                          (plain GEMM)
//             = round_T(X[m,k] * gamma[k])                 (RMS ops; see below)
//     z       = r[m] * C[m,n] + bias[n]                    (r = 1 for plain GEMM)
//     Y[m,n]  = act(z) + R[m,n],  rounded once to the output type
//     r[m]    = 1 / sqrt( sum_k X[m,k]^2 / K + eps )
// For the SwiGLU dual GEMM: H = SiLU(r*Cg) * (r*Cu).
//
// RMSNorm fusion.  x_hat[m,k] = X[m,k] * r[m] * gamma[k]; r[m] is one scalar
// per row, so it factors out of the k-sum: x_hat . W = r[m] * ((X*gamma) . W).
// The kernel therefore scales each A tile by gamma as it is staged into LDS,
// accumulates sum_k X^2 from the same registers, and applies r[m] to the fp32
// accumulator in the epilogue.  X is read once, the normalised activation is
// never written anywhere, and no separate pass over X is needed.
//
// Structure of one workgroup (256 threads = 4 wave64s in a 2x2 grid):
//   * tile BM x BN of the output, K walked in steps of BK = 64;
//   * A and W tiles fetched with 128-bit buffer loads (out-of-range lanes
//     return zero, which handles the M, N and K tails);
//   * W arrives N-contiguous; each thread transposes an 8(k) x 8(n) block in
//     registers so LDS holds both operands K-contiguous, as the matrix cores
//     want them;
//   * LDS rows of 64 halves (8 chunks of 16 B) with chunk index XOR-swizzled
//     by the row, so fragment reads and tile writes avoid bank conflicts;
//   * two LDS stages: the global loads for step k+1 are in flight while the
//     matrix cores work on step k;
//   * v_mfma_f32_32x32x16_{f16,bf16}: each wave owns (BM/2) x (BN/2) of the
//     tile as 32x32 fp32 accumulator blocks;
//   * epilogue in fp32: accumulators staged through LDS so that every lane
//     finishes 8 consecutive columns of a row and writes them with one
//     16-byte store.
#include "launch.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstring>
#include <type_traits>

namespace lf {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;          // K step per LDS stage
constexpr int kKCH = kBK / 8;    // 16-byte chunks per LDS row
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset that reads as zero

struct KArgs {
    const uint16_t* A;
    const uint16_t* W;
    const uint16_t* W2;
    const uint16_t* bias;
    const uint16_t* resid;
    const uint16_t* gamma;
    void* Y;
    int M, N, K;
    int tiles_m, tiles_n, group_m;
    int act;
    int out_f32;
    float eps;
};

// ---------------------------------------------------------------- elements

template <bool BF>
__device__ __forceinline__ float lo_f32(uint32_t w) {
    if constexpr (BF) return __uint_as_float(w << 16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <bool BF>
__device__ __forceinline__ float hi_f32(uint32_t w) {
    if constexpr (BF) return __uint_as_float(w & 0xffff0000u);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
template <bool BF>
__device__ __forceinline__ float h_f32(uint16_t h) {
    if constexpr (BF) return __uint_as_float((uint32_t)h << 16);
    else return (float)__builtin_bit_cast(_Float16, h);
}
// Round to the 16-bit type, nearest-even.
template <bool BF>
__device__ __forceinline__ uint16_t f32_h(float x) {
    if constexpr (BF) return __builtin_bit_cast(uint16_t, (__bf16)x);
    else return __builtin_bit_cast(uint16_t, (_Float16)x);
}
template <bool BF>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return (uint32_t)f32_h<BF>(a) | ((uint32_t)f32_h<BF>(b) << 16);
}

template <bool BF>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- memory

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Byte offset for a buffer load, or one past the 2 GiB window when the lane
// is out of range (the buffer bounds check then returns zero).  Built with
// integer arithmetic so the compiler keeps the loads branch-free.
__device__ __forceinline__ uint32_t oob_or(uint32_t off, bool valid) {
    return off | ((uint32_t)(!valid) << 31);
}

// Chunk swizzle of an LDS row: conflict-free for 8 or 16 consecutive rows
// read at the same logical chunk, and for 8 rows 8 apart written at the same
// logical chunk.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// KB x 8 transpose of 16-bit elements (KB = 4 or 8): in[j] holds row j
// (8 halves), out[i] holds column i (KB halves in its first KB/2 words).
template <int KB>
__device__ __forceinline__ void transpose_k8(const u32x4 (&in)[KB], u32x4 (&out)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int d = 0; d < KB / 2; ++d) {
            const uint32_t a = in[2 * d][i >> 1];
            const uint32_t b = in[2 * d + 1][i >> 1];
            out[i][d] = (i & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
    }
}

// ---------------------------------------------------------------- epilogue math

// exp(x) as 2^(x log2 e) on the hardware exp2 unit.
__device__ __forceinline__ float exp_fast(float x) {
    return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}
// GeLU, tanh form; tanh(u) = 1 - 2 / (exp(2u) + 1) saturates cleanly at +-1.
__device__ __forceinline__ float gelu_tanh(float z) {
    const float u = 0.79788456080286536f * (z + 0.044715f * z * z * z);
    const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(exp_fast(2.0f * u) + 1.0f);
    return 0.5f * z * (1.0f + t);
}
__device__ __forceinline__ float silu(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + exp_fast(-z));
}
template <int ACT>
__device__ __forceinline__ float apply_act(float z) {
    if constexpr (ACT == 1) return fmaxf(z, 0.0f);
    else if constexpr (ACT == 2) return gelu_tanh(z);
    else if constexpr (ACT == 3) return silu(z);
    else return z;
}

// ---------------------------------------------------------------- schedule

// Workgroups are handed to the 8 XCDs round-robin by id.  Give every XCD a
// contiguous range of logical tiles, and walk logical tiles in groups of
// `group_m` tile-rows (column-major inside a group), so the workgroups that
// share an XCD's L2 also share A rows and W columns.
__device__ __forceinline__ void map_tile(int bid, int nwg, int tiles_m, int tiles_n, int group_m,
                                         int& tm, int& tn) {
    const int xcd = bid & 7, idx = bid >> 3;
    const int q = nwg >> 3, r = nwg & 7;
    const int l = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
    const int per_group = group_m * tiles_n;
    const int g = l / per_group;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int li = l - g * per_group;
    tm = first_m + li % gm;
    tn = li / gm;
}

// ---------------------------------------------------------------- kernel

template <int BM, int BN, int WM, int WN, bool BF, bool RMS, int NB, int NREG, bool KT>
__global__ void __launch_bounds__(WM * WN * 64)
gemm_fused_kernel(const KArgs p) {
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

    int tm, tn;
    map_tile(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.M, N = p.N, K = p.K;

    const auto rsA = make_rsrc(p.A + (size_t)m0 * K, (uint32_t)((size_t)(M - m0) * K * 2));
    const uint32_t w_bytes = (uint32_t)(((size_t)K * N - n0) * 2);
    const auto rsW = make_rsrc(p.W + n0, w_bytes);
    const auto rsW2 = make_rsrc(NB == 2 ? p.W2 + n0 : p.W + n0, w_bytes);
    const auto rsG = make_rsrc(p.gamma, RMS ? (uint32_t)K * 2 : 0u);

    // Thread -> A chunk mapping: row a_row0 + i*A_ROW_STEP, chunk a_kc.
    const int a_kc = tid % kKCH;
    const int a_row0 = tid / kKCH;

    // One register set holds a whole A/W (and gamma) tile on its way from
    // global memory to LDS.  Two sets give the loads two K steps of lead time.
    struct Regs {
        u32x4 a[A_PER];
        u32x4 b[B_PER][KB];
        u32x4 g;
    };
    Regs R0;
    Regs R1;  // unused when NREG == 1
    float ss[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) ss[i] = 0.0f;

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
        if constexpr (RMS) R.g = bload16(rsG, oob_or((uint32_t)a_kc * 16u, k0 + a_kc * 8 < K), sA);
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
        gload(R0, 0);
        gload(R1, kBK);
        lstore(R0, 0);
        gload(R0, 2 * kBK);
        __syncthreads();
        auto step = [&](Regs& Rw, int kt) {
            if (kt + 1 < nk) {
                lstore(Rw, (kt + 1) & 1);
                gload(Rw, (kt + 3) * kBK);
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
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            float s = ss[i];
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            s += __shfl_xor(s, 4);
            if (a_kc == 0) rs[a_row0 + i * A_ROW_STEP] = 1.0f / sqrtf(s / (float)K + p.eps);
        }
        __syncthreads();
    }

    // Epilogue.  The accumulators go through LDS one 32-row slab of the wave
    // tile at a time (register r of a 32x32 block holds row
    // 8*(r/4) + 4*(lane/32) + r%4, column lane%32), are read back with each
    // lane owning 8 consecutive columns of one row, finished in fp32 (RMS
    // factor, bias, activation, residual), rounded once and written with
    // 16-byte stores.  Each wave uses its own LDS region.
    constexpr int SROW = TN + 8;            // staged row stride (floats)
    constexpr int LPR = TN / 8;             // lanes per staged row
    constexpr int RPI = 64 / LPR;           // rows per read-back step
    static_assert(4 * NB * 32 * SROW * 4 <= 2 * STAGE * 16, "staging must fit in the LDS stages");
    float* stg = reinterpret_cast<float*>(lds) + wave * (NB * 32 * SROW);
    const int ec = (lane % LPR) * 8;
    const int er = lane / LPR;
    const int gcol = n0 + wn * TN + ec;
    const bool colok = gcol < N;  // N % 8 == 0: a lane's 8 columns are all in or all out
    const bool has_res = p.resid != nullptr;
    float bias8[8];
    {
        u32x4 bw = {0u, 0u, 0u, 0u};
        if (p.bias != nullptr && colok) bw = *reinterpret_cast<const u32x4*>(p.bias + gcol);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bias8[2 * q] = lo_f32<BF>(bw[q]);
            bias8[2 * q + 1] = hi_f32<BF>(bw[q]);
        }
    }

    auto epilogue = [&](auto act_tag) {
        constexpr int ACT = decltype(act_tag)::value;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int nbi = 0; nbi < NB; ++nbi)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        stg[nbi * 32 * SROW + (8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * SROW + j * 32 +
                            (lane & 31)] = acc[nbi][i][j][r];
            __syncthreads();
            for (int it = 0; it < 32 / RPI; ++it) {
                const int rr = it * RPI + er;
                const int rl = wm * TM + i * 32 + rr;
                const int grow = m0 + rl;
                const float4* src = reinterpret_cast<const float4*>(stg + rr * SROW + ec);
                const float4 v0 = src[0], v1 = src[1];
                float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                const float rsc = RMS ? rs[rl] : 1.0f;
                if constexpr (NB == 2) {
                    const float4* srcu = reinterpret_cast<const float4*>(stg + 32 * SROW + rr * SROW + ec);
                    const float4 u0 = srcu[0], u1 = srcu[1];
                    const float u[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = silu(v[e] * rsc) * (u[e] * rsc);
                } else {
                    u32x4 rw = {0u, 0u, 0u, 0u};
                    if (has_res && grow < M && colok)
                        rw = *reinterpret_cast<const u32x4*>(p.resid + (size_t)grow * N + gcol);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float z = (RMS ? v[e] * rsc : v[e]) + bias8[e];
                        z = apply_act<ACT>(z);
                        if (has_res) z += (e & 1) ? hi_f32<BF>(rw[e >> 1]) : lo_f32<BF>(rw[e >> 1]);
                        v[e] = z;
                    }
                }
                if (grow < M && colok) {
                    const size_t o = (size_t)grow * N + gcol;
                    if (p.out_f32) {
                        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.Y) + o);
                        dst[0] = make_float4(v[0], v[1], v[2], v[3]);
                        dst[1] = make_float4(v[4], v[5], v[6], v[7]);
                    } else {
                        u32x4 ow;
#pragma unroll
                        for (int q = 0; q < 4; ++q) ow[q] = pack2<BF>(v[2 * q], v[2 * q + 1]);
                        *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.Y) + o) = ow;
                    }
                }
            }
            __syncthreads();
        }
    };
    if constexpr (NB == 2) {
        epilogue(std::integral_constant<int, 0>{});
    } else {
        switch (p.act) {
        case 1: epilogue(std::integral_constant<int, 1>{}); break;
        case 2: epilogue(std::integral_constant<int, 2>{}); break;
        case 3: epilogue(std::integral_constant<int, 3>{}); break;
        default: epilogue(std::integral_constant<int, 0>{}); break;
        }
    }
}

// ---------------------------------------------------------------- host side

template <int BM, int BN, int WM, int WN, bool BF, bool RMS, int NB, int NREG>
struct Cfg {
    static hipError_t run(const KArgs& a, int nwg, hipStream_t s) {
        // hipLaunchKernel reports the status of this launch itself, so an
        // error left behind by an unrelated earlier call is not picked up.
        void* args[] = {const_cast<KArgs*>(&a)};
        const void* fn = (a.K % kBK == 0)
                             ? reinterpret_cast<const void*>(&gemm_fused_kernel<BM, BN, WM, WN, BF, RMS, NB, NREG, false>)
                             : reinterpret_cast<const void*>(&gemm_fused_kernel<BM, BN, WM, WN, BF, RMS, NB, NREG, true>);
        return hipLaunchKernel(fn, dim3(nwg), dim3(WM * WN * 64), args, 0, s);
    }
};

struct Tile {
    int bm, bn;
    const char* name;
};

constexpr Tile kSingleTiles[] = {
    {256, 256, "256x256x64_w2x2"},
    {128, 128, "128x128x64_w2x2"},
};
constexpr Tile kDualTile = {256, 128, "dual_256x128x64_w2x2"};

std::atomic<int> g_override{-1};

Tile choose_tile(const Problem& p) {
    if (p.op == Op::RmsSwiglu) return kDualTile;
    const int ov = g_override.load(std::memory_order_relaxed);
    if (ov >= 0) return kSingleTiles[ov];
    const int64_t t256 = ((p.M + 255) / 256) * ((p.N + 255) / 256);
    if (t256 >= 224) return kSingleTiles[0];
    return kSingleTiles[1];
}

template <bool BF, bool RMS>
hipError_t dispatch_single(const Problem& p, const KArgs& a, const Tile& t, int nwg, hipStream_t s) {
    if (t.bm == 256) return Cfg<256, 256, 2, 2, BF, RMS, 1, 1>::run(a, nwg, s);
    return Cfg<128, 128, 2, 2, BF, RMS, 1, 2>::run(a, nwg, s);
}

}  // namespace

const char* plan_name(const Problem& p) { return choose_tile(p).name; }

bool set_plan(const char* name) {
    if (name == nullptr || name[0] == 0) {
        g_override.store(-1);
        return true;
    }
    for (int i = 0; i < (int)(sizeof(kSingleTiles) / sizeof(kSingleTiles[0])); ++i) {
        if (std::strcmp(name, kSingleTiles[i].name) == 0) {
            g_override.store(i);
            return true;
        }
    }
    return false;
}

hipError_t launch(const Problem& p, hipStream_t stream) {
    if (p.M == 0) return hipSuccess;
    const Tile t = choose_tile(p);
    KArgs a;
    a.A = static_cast<const uint16_t*>(p.A);
    a.W = static_cast<const uint16_t*>(p.W);
    a.W2 = static_cast<const uint16_t*>(p.W2);
    a.bias = static_cast<const uint16_t*>(p.bias);
    a.resid = static_cast<const uint16_t*>(p.resid);
    a.gamma = static_cast<const uint16_t*>(p.gamma);
    a.Y = p.Y;
    a.M = (int)p.M;
    a.N = (int)p.N;
    a.K = (int)p.K;
    a.tiles_m = (int)((p.M + t.bm - 1) / t.bm);
    a.tiles_n = (int)((p.N + t.bn - 1) / t.bn);
    a.group_m = 4;
    a.act = p.act;
    a.out_f32 = p.out_f32 ? 1 : 0;
    a.eps = p.eps;
    const int nwg = a.tiles_m * a.tiles_n;
    const bool rms = p.op != Op::GemmEpilogue;
    if (p.op == Op::RmsSwiglu) {
        if (p.bf16) return Cfg<256, 128, 2, 2, true, true, 2, 1>::run(a, nwg, stream);
        return Cfg<256, 128, 2, 2, false, true, 2, 1>::run(a, nwg, stream);
    }
    if (p.bf16) {
        return rms ? dispatch_single<true, true>(p, a, t, nwg, stream)
                   : dispatch_single<true, false>(p, a, t, nwg, stream);
    }
    return rms ? dispatch_single<false, true>(p, a, t, nwg, stream)
               : dispatch_single<false, false>(p, a, t, nwg, stream);
}

}  // namespace lf
