// common.h -- device-side building blocks shared by the gfx950 kernels:
// element conversions, matrix-core wrappers, buffer loads, LDS swizzles, the
// epilogue activations, the XCD-aware tile order and the LDS-staged epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lf {
namespace dev {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kOOB = 0x80000000u;  // buffer offset that reads as zero

struct KArgs {
    const uint16_t* A;
    const uint16_t* W;
    const uint16_t* W2;
    const uint16_t* bias;
    const uint16_t* resid;
    const uint16_t* gamma;  // [K]: RMSNorm/LayerNorm gamma, or the input bias of the prologue-bias GEMM
    const uint16_t* beta;   // [K] LayerNorm beta (nullptr: zero)
    const float2* stats;    // [M] LayerNorm row statistics (a, b): the operand is a*x + b before gamma, beta
    const uint32_t* lnstats;  // [M][4] LayerNorm row record of the LDS-DMA kernel (mean, spread, 1/spread)
    void* Y;
    int M, N, K;
    int tiles_m, tiles_n, group_m;
    int act;
    int out_f32;
    float eps;
    // split-K (DMA kernel only): `splits` workgroups share each output tile,
    // split z covering K range [z*kchunk, min(K, (z+1)*kchunk)); fp32
    // partials and per-tile arrival counters live in a library workspace.
    int splits, kchunk;
    float* ws;
    unsigned* cnt;
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
// Two values rounded to the 16-bit type (nearest even) and packed, low half
// first: one v_cvt_pk_{f16,bf16}_f32.
template <bool BF>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2 v = {a, b};
    if constexpr (BF) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
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
// GeLU, tanh form.  0.5 z (1 + tanh u) = z * sigmoid(2u) = z / (1 + e^(-2u)) with
// u = sqrt(2/pi) (z + 0.044715 z^3); -2u log2(e) = z (c0 + c1 z^2) feeds the exp2 unit
// directly.  Saturates cleanly: e^(-2u) -> inf gives -0, -> 0 gives z.
__device__ __forceinline__ float gelu_tanh(float z) {
    constexpr float c0 = -2.302208198144325f;   // -2 sqrt(2/pi) log2(e)
    constexpr float c1 = -0.1029432395800235f;  // c0 * 0.044715
    const float e = __builtin_amdgcn_exp2f(z * __builtin_fmaf(c1, z * z, c0));
    return z * __builtin_amdgcn_rcpf(1.0f + e);
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

// ---------------------------------------------------------------- RMS range check and exact path
//
// The fast RMS path multiplies each X element by gamma on its way to the matrix
// cores, rounds that product to the input type, and applies the row factor
// r = 1/sqrt(mean(x^2) + eps) to the fp32 accumulator; the sum of squares is
// accumulated in fp32.  x * r * gamma = r * (x * gamma) exactly, but the two
// roundings differ in range: round(x * gamma) overflows the fp16 maximum when
// |x * gamma| >= 65520 even though x * r * gamma is small; for a row whose mean
// square plus eps is tiny, r multiplies the absolute rounding error of subnormal
// products; and in bf16 the fp32 sum of squares can overflow.  A workgroup
// therefore checks its rows after the reduction -- mean square plus eps inside
// [lo, hi] and every accumulator finite (an operand that overflowed leaves an
// inf or NaN in every column of its row) -- and if any row fails, recomputes
// its whole tile with prologue_exact_tile: r in fp64, the normalised activation
// x * r * gamma (deplodock post, RMSNorm loop nest; "LLMBoost", section 3) as
// an fp32 operand, products accumulated in fp32.  Inside the window the fast
// path's operand error stays at or below the rounding of the normalised value
// itself: an fp16 subnormal product is off by at most 2^-25, times r <= 2^15.

constexpr float kRmsLoF16 = 0x1p-30f;    // mean square + eps below this: fp16 subnormal rounding matters
constexpr float kRmsLoBF16 = 0x1p-120f;  // bf16 (and fp32) subnormal range
constexpr float kRmsHi = 0x1p100f;       // mean square above this: the fp32 sum of squares nears overflow

template <bool BF>
__device__ __forceinline__ bool rms_outside(float ss, int K, float eps) {
    const float ms = ss / (float)K;
    return !(ms + eps >= (BF ? kRmsLoBF16 : kRmsLoF16)) || !(ms <= kRmsHi);
}

// Prologue of the A operand, applied elementwise on the way to the matrix
// cores: none, RMSNorm (x * gamma, row factor applied after the reduction),
// input bias (x + b), LayerNorm (per-row a*x + b from precomputed statistics,
// then * gamma + beta).
enum Prologue : int { kProNone = 0, kProRms = 1, kProBias = 2, kProLn = 3 };

// Recompute output rows [m0, m0 + BM) x columns [n0, n0 + BN) with plain
// arithmetic from global memory: the exact path of the prologue PRO (RMS
// calls: also NB = 2, the SwiGLU gate/up pair, H = SiLU(g) * u).  The
// operand is the method's value in fp32, never rounded to the input type:
//   RMS   x * r * gamma,            r = 1 / sqrt(mean(x^2) + eps) in fp64
//   bias  x + b
//   LN    (x - mu) * rstd * gamma + beta, mu and rstd = 1/sqrt(var + eps) in fp64
// and products are accumulated in fp32; bias, activation and residual follow.
// Every thread of the NT-thread workgroup calls it; `lds` needs
// 16 * 16 + 16 * 64 * 4 bytes.  Slow (no matrix cores, no staging of W), and
// only reached by tiles whose fast path left its range.
template <bool BF, int NB, int NT, int BN, int PRO = kProRms>
__device__ __forceinline__ void prologue_exact_tile(const KArgs& p, char* lds, int m0, int BM, int n0) {
    constexpr int RC = 16, KC = 64, NW = NT / 64;
    static_assert(NT % BN == 0, "whole threads per output column");
    constexpr int TPC = NT / BN;               // threads per output column
    static_assert(TPC >= RC || RC % TPC == 0, "rows of a chunk split evenly");
    constexpr int RPT = (RC + TPC - 1) / TPC;  // rows of a chunk per thread
    double* rr = reinterpret_cast<double*>(lds);       // RMS r, LN rstd
    double* mu = rr + RC;                              // LN mean
    float* op = reinterpret_cast<float*>(lds + 2 * RC * sizeof(double));
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int N = p.N, K = p.K;
    const int rows = min(BM, p.M - m0);
    const int c = tid % BN, rsub = tid / BN;
    const bool mine = n0 + c < N && rsub < RC;
    __syncthreads();  // the caller's LDS use is over
    for (int r0 = 0; r0 < rows; r0 += RC) {
        const int rc = min(RC, rows - r0);
        // per-row factors in fp64, one wave per row
        if constexpr (PRO == kProRms || PRO == kProLn) {
            for (int i = wave; i < rc; i += NW) {
                const uint16_t* x = p.A + (size_t)(m0 + r0 + i) * K;
                double m = 0.0;
                if constexpr (PRO == kProLn) {
                    for (int k = lane; k < K; k += 64) m += (double)h_f32<BF>(x[k]);
                    for (int o = 32; o > 0; o >>= 1) m += __shfl_xor(m, o);
                    m /= (double)K;
                }
                double s = 0.0;
                for (int k = lane; k < K; k += 64) {
                    const double v = (double)h_f32<BF>(x[k]) - m;
                    s = fma(v, v, s);
                }
                for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
                if (lane == 0) {
                    rr[i] = 1.0 / sqrt(s / (double)K + (double)p.eps);
                    mu[i] = m;
                }
            }
        }
        float acc[NB][RPT];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int j = 0; j < RPT; ++j) acc[b][j] = 0.0f;
        for (int k0 = 0; k0 < K; k0 += KC) {
            __syncthreads();  // the row factors are written; the previous chunk is consumed
            for (int e = tid; e < RC * KC; e += NT) {
                const int i = e / KC, k = k0 + e % KC;
                float v = 0.0f;
                if (i < rc && k < K) {
                    const double x = (double)h_f32<BF>(p.A[(size_t)(m0 + r0 + i) * K + k]);
                    const double g = (double)h_f32<BF>(p.gamma[k]);
                    if constexpr (PRO == kProRms) v = (float)(x * rr[i] * g);
                    else if constexpr (PRO == kProBias) v = (float)(x + g);
                    else if constexpr (PRO == kProLn)
                        v = (float)((x - mu[i]) * rr[i] * g + (p.beta ? (double)h_f32<BF>(p.beta[k]) : 0.0));
                    else v = (float)x;
                }
                op[e] = v;
            }
            __syncthreads();
            if (mine) {
                const int kn = min(KC, K - k0);
                for (int kk = 0; kk < kn; ++kk) {
                    const size_t wo = (size_t)(k0 + kk) * N + n0 + c;
                    const float w0 = h_f32<BF>(p.W[wo]);
                    const float w1 = (NB == 2) ? h_f32<BF>(p.W2[wo]) : 0.0f;
#pragma unroll
                    for (int j = 0; j < RPT; ++j) {
                        const float a = op[(rsub + j * TPC) * KC + kk];  // rows past rc hold zeros
                        acc[0][j] = fmaf(a, w0, acc[0][j]);
                        if constexpr (NB == 2) acc[NB - 1][j] = fmaf(a, w1, acc[NB - 1][j]);
                    }
                }
            }
        }
        if (mine) {
            const float bias = (NB == 1 && p.bias != nullptr) ? h_f32<BF>(p.bias[n0 + c]) : 0.0f;
#pragma unroll
            for (int j = 0; j < RPT; ++j) {
                const int i = rsub + j * TPC;
                if (i >= rc) continue;
                const size_t o = (size_t)(m0 + r0 + i) * N + n0 + c;
                float z;
                if constexpr (NB == 2) {
                    z = silu(acc[0][j]) * acc[NB - 1][j];
                } else {
                    z = acc[0][j] + bias;
                    switch (p.act) {
                    case 1: z = apply_act<1>(z); break;
                    case 2: z = apply_act<2>(z); break;
                    case 3: z = apply_act<3>(z); break;
                    default: break;
                    }
                    if (p.resid != nullptr) z += h_f32<BF>(p.resid[o]);
                }
                if (p.out_f32) static_cast<float*>(p.Y)[o] = z;
                else static_cast<uint16_t*>(p.Y)[o] = f32_h<BF>(z);
            }
        }
        __syncthreads();  // before the next chunk's row factors overwrite rr
    }
}

// Finish and store 8 consecutive output columns [gcol, gcol + 8) of row grow:
// r[m] (rsc), bias, activation, residual, one rounding, 16-byte stores.  Used by
// the few-row kernels, where one thread owns such a piece.
template <bool BF>
__device__ __forceinline__ void finish_store8(const KArgs& p, float (&v)[8], float rsc, int grow, int gcol) {
    const int N = p.N;
    float bias8[8];
    {
        u32x4 bw = {0u, 0u, 0u, 0u};
        if (p.bias != nullptr) bw = *reinterpret_cast<const u32x4*>(p.bias + gcol);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bias8[2 * q] = lo_f32<BF>(bw[q]);
            bias8[2 * q + 1] = hi_f32<BF>(bw[q]);
        }
    }
    u32x4 rw = {0u, 0u, 0u, 0u};
    const bool has_res = p.resid != nullptr;
    if (has_res) rw = *reinterpret_cast<const u32x4*>(p.resid + (size_t)grow * N + gcol);
    auto finish = [&](auto ACT) {
        constexpr int A = decltype(ACT)::value;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float z = v[e] * rsc + bias8[e];
            z = apply_act<A>(z);
            if (has_res) z += (e & 1) ? hi_f32<BF>(rw[e >> 1]) : lo_f32<BF>(rw[e >> 1]);
            v[e] = z;
        }
    };
    switch (p.act) {
    case 1: finish(std::integral_constant<int, 1>{}); break;
    case 2: finish(std::integral_constant<int, 2>{}); break;
    case 3: finish(std::integral_constant<int, 3>{}); break;
    default: finish(std::integral_constant<int, 0>{}); break;
    }
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

// ---------------------------------------------------------------- schedule

// Workgroups are handed to the 8 XCDs round-robin by id.  Give every XCD a
// contiguous range of logical tiles, and walk logical tiles in groups of
// `group_m` tile-rows (column-major inside a group), so the workgroups that
// share an XCD's L2 also share A rows and W columns.
__device__ __forceinline__ void map_tile(int bid, int nwg, int tiles_m, int tiles_n, int group_m, int splits,
                                         int& tm, int& tn, int& kz) {
    const int xcd = bid & 7, idx = bid >> 3;
    const int q = nwg >> 3, r = nwg & 7;
    int l = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
    // the splits of one tile are consecutive, hence on the same XCD
    kz = l % splits;
    l /= splits;
    const int per_group = group_m * tiles_n;
    const int g = l / per_group;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int li = l - g * per_group;
    tm = first_m + li % gm;
    tn = li / gm;
}

// ---------------------------------------------------------------- epilogue

// Finish and store one BM x BN output tile.  The accumulators go through LDS
// one 32-row slab of the wave tile at a time (register r of a 32x32 block
// holds row 8*(r/4) + 4*(lane/32) + r%4, column lane%32), are read back with
// each lane owning 8 consecutive columns of one row, finished in fp32 (RMS
// factor, bias, activation, residual; SiLU(gate)*up for the dual GEMM),
// rounded once and written with 16-byte stores.  The calling wave holds the
// (wm, wn) wave tile of a WM x WN grid; each wave uses its own LDS region of
// kStageFloats floats at `stage`; every thread of the workgroup must call
// this.
template <int BM, int BN, int WM, int WN, bool BF, bool RMS, int NB>
struct TileStore {
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int SROW = TN + 8;   // staged row stride (floats)
    static constexpr int LPR = TN / 8;    // lanes per staged row
    static constexpr int RPI = 64 / LPR;  // rows per read-back step
    static constexpr int kStageFloats = NB * 32 * SROW;
    static constexpr int kBytes = WM * WN * kStageFloats * 4;

    // Orders this wave's LDS accesses in program order for the compiler; the
    // LDS executes one wave's instructions in issue order, and each wave
    // stages through its own region, so no workgroup barrier is needed.
    static __device__ __forceinline__ void wave_lds_order() {
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    }

    template <int ACT, bool RES>
    static __device__ __forceinline__ void run_act(const KArgs& p, f32x16 (&acc)[NB][FM][FN], float* stage,
                                                   const float* rs, int m0, int n0, int wm, int wn) {
        constexpr int NIT = 32 / RPI;  // read-back steps per 32-row slab
        const int lane = threadIdx.x & 63;
        const int wave = threadIdx.x >> 6;
        const int M = p.M, N = p.N;
        float* stg = stage + wave * kStageFloats;
        const int ec = (lane % LPR) * 8;
        const int er = lane / LPR;
        const int gcol = n0 + wn * TN + ec;
        const bool colok = gcol < N;  // N % 8 == 0: a lane's 8 columns are all in or all out
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
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            // The slab's residual rows are requested before the staging so
            // their latency hides behind it.  Each lane reads exactly the
            // elements it later writes, so Y may be the residual buffer.
            u32x4 rw[RES ? NIT : 1];
            if constexpr (RES) {
#pragma unroll
                for (int it = 0; it < NIT; ++it) {
                    const int grow = m0 + wm * TM + i * 32 + it * RPI + er;
                    rw[it] = u32x4{0u, 0u, 0u, 0u};
                    if (grow < M && colok)
                        rw[it] = *reinterpret_cast<const u32x4*>(p.resid + (size_t)grow * N + gcol);
                }
            }
#pragma unroll
            for (int nbi = 0; nbi < NB; ++nbi)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        stg[nbi * 32 * SROW + (8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * SROW + j * 32 +
                            (lane & 31)] = acc[nbi][i][j][r];
            wave_lds_order();
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
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
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float z = (RMS ? v[e] * rsc : v[e]) + bias8[e];
                        z = apply_act<ACT>(z);
                        if constexpr (RES) z += (e & 1) ? hi_f32<BF>(rw[it][e >> 1]) : lo_f32<BF>(rw[it][e >> 1]);
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
            wave_lds_order();
        }
    }

    template <bool RES>
    static __device__ __forceinline__ void run_res(const KArgs& p, f32x16 (&acc)[NB][FM][FN], float* stage,
                                                   const float* rs, int m0, int n0, int wm, int wn) {
        switch (p.act) {
        case 1: run_act<1, RES>(p, acc, stage, rs, m0, n0, wm, wn); break;
        case 2: run_act<2, RES>(p, acc, stage, rs, m0, n0, wm, wn); break;
        case 3: run_act<3, RES>(p, acc, stage, rs, m0, n0, wm, wn); break;
        default: run_act<0, RES>(p, acc, stage, rs, m0, n0, wm, wn); break;
        }
    }

    static __device__ __forceinline__ void run(const KArgs& p, f32x16 (&acc)[NB][FM][FN], float* stage,
                                               const float* rs, int m0, int n0, int wm, int wn) {
        if constexpr (NB == 2) {
            run_act<0, false>(p, acc, stage, rs, m0, n0, wm, wn);
        } else {
            if (p.resid != nullptr)
                run_res<true>(p, acc, stage, rs, m0, n0, wm, wn);
            else
                run_res<false>(p, acc, stage, rs, m0, n0, wm, wn);
        }
    }
};

}  // namespace dev
}  // namespace lf
