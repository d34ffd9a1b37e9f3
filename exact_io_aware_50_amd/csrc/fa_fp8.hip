// FP8 (OCP E4M3) forward pass and the per-tensor quantiser that feeds it.
//
// The FlashAttention legal glossary (FlashAttention-3 paragraph) and "flash
// attention io aware" (section "Flash Attention 2 and 3") name FP8 attention
// on low-precision matrix units without a recipe.  Here: one descale per
// tensor (real value = code * s_X), both products on the fp8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales) with float32
// accumulation, the softmax in float32, and P multiplied by 256 before its
// E4M3 rounding so that small probabilities stay out of the E4M3 subnormal
// range (the factor is a power of two and is divided out exactly with l).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------ quantiser
__global__ void q8_clear_kernel(float* descale) {
    if (threadIdx.x == 0) descale[0] = 0.f;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__global__ __launch_bounds__(256) void q8_absmax_kernel(const uint16_t* __restrict__ x, size_t n,
                                                       float* __restrict__ descale) {
    float m = 0.f;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        m = fmaxf(m, fabsf(bf16_to_f32(x[i])));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __shared__ float wmax[4];
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        // non-negative floats order like their bit patterns
        atomicMax(reinterpret_cast<unsigned int*>(descale), __float_as_uint(m));
    }
}

__device__ __forceinline__ float q8_scale(float absmax) {
    return fmaxf(absmax, 0x1p-120f) / 448.0f;   // IEEE division, as the format recipe states
}

// float32 -> E4M3 code, round to nearest even, saturating at +-448.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    uint32_t code;
    if (a >= 0x43e00000u) {                    // |f| >= 448
        code = 0x7e;
    } else if (a < 0x3c800000u) {              // |f| < 2^-6: multiples of 2^-9
        code = (uint32_t)rintf(__uint_as_float(a) * 512.0f);
    } else {
        uint32_t base = a >> 20;               // biased exponent and top 3 mantissa bits
        const uint32_t rem = a & 0xfffffu, half = 0x80000u;
        base += (rem > half || (rem == half && (base & 1u))) ? 1u : 0u;
        code = base - (120u << 3);             // rebias 127 -> 7
        if (code > 0x7e) code = 0x7e;
    }
    return sign | code;
}

__global__ __launch_bounds__(256) void q8_cast_kernel(const uint16_t* __restrict__ x, size_t n,
                                                     uint8_t* __restrict__ out,
                                                     const float* __restrict__ descale) {
    const float s = q8_scale(descale[0]);
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        out[i] = (uint8_t)e4m3_rne_sat(bf16_to_f32(x[i]) / s);
}

__global__ void q8_finalize_kernel(float* descale) {
    if (threadIdx.x == 0) descale[0] = q8_scale(descale[0]);
}

hipError_t launch_quantize_fp8(const void* x, size_t n, void* out, float* descale, hipStream_t st) {
    hipLaunchKernelGGL(q8_clear_kernel, dim3(1), dim3(64), 0, st, descale);
    if (n > 0) {
        size_t blocks = (n + 1023) / 1024;
        if (blocks > 2048) blocks = 2048;
        hipLaunchKernelGGL(q8_absmax_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint16_t*)x, n,
                           descale);
        hipLaunchKernelGGL(q8_cast_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint16_t*)x, n,
                           (uint8_t*)out, (const float*)descale);
    }
    hipLaunchKernelGGL(q8_finalize_kernel, dim3(1), dim3(64), 0, st, descale);
    return hipGetLastError();
}

// ------------------------------------------------------------ fp8 forward
//
// Operands are 32 bytes per lane: lane l supplies row (A) or column (B) l % 32
// and 32 contraction slots.  S^T = K Q^T uses d-slots 64*s + 32*hh + e.  For
// O^T += V^T P^T the B operand is this lane's P: byte e is accumulator
// register e % 16 of key block e / 16, i.e. key 32*(e/16) + row(e%16, hh).  The
// transposed V tile stores key kappa at the position this lane reads it from:
//   pos(kappa) = 32*hh + 16*kb + 4*a + b  for kappa = 32*kb + 8*a + 4*hh + b.
__device__ __forceinline__ int fp8_vpos(int key) {
    return 32 * ((key >> 2) & 1) + 16 * ((key >> 5) & 1) + 4 * ((key >> 3) & 3) + (key & 3);
}

__device__ __forceinline__ f32x16 mma_fp8(const u32x8& a, const u32x8& b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a),
                                                           __builtin_bit_cast(i32x8, b), c,
                                                           0, 0,        // A and B are E4M3
                                                           0, 127,      // A block scale 2^0
                                                           0, 127);     // B block scale 2^0
}

template <int D>
struct Fp8Cfg {
    static constexpr int kThreads = 256;
    static constexpr int BM = 128;
    static constexpr int BN = 64;
    static constexpr int KS = D + 16;                      // bytes per K row in LDS
    static constexpr int VS = BN + 16;                     // bytes per V^T row in LDS
    static constexpr int kKBytes = BN * KS;
    static constexpr int kVBytes = D * VS;
    static constexpr int kStage = kKBytes + kVBytes;
    static constexpr int kKChunks = BN * D / 16;           // 16-byte chunks of a K tile
    static constexpr int kKPer = kKChunks / kThreads;
    static constexpr int kVTasks = (BN / 4) * (D / 16);    // 4 keys x 16 columns per task
    static_assert(kKChunks % kThreads == 0, "K tile chunks cover the threads evenly");
    static_assert(kVTasks <= kThreads, "one V task per thread at most");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_fp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
                                                      const uint8_t* __restrict__ V, uint16_t* __restrict__ O,
                                                      float* __restrict__ LSE, const float* __restrict__ descale,
                                                      int Hq, int Hkv, int N, float scale) {
    using Cfg = Fp8Cfg<D>;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, KS = Cfg::KS, VS = Cfg::VS;
    __shared__ __attribute__((aligned(64))) uint8_t smem[2 * Cfg::kStage];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;

    const int nmb = (N + BM - 1) / BM;
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    const int mbi = lin % nmb, bh = lin / nmb;
    const int h = bh % Hq, b = bh / Hq;
    const int mb = CAUSAL ? nmb - 1 - mbi : mbi;
    const int g = h / (Hq / Hkv);
    const uint8_t* Qh = Q + ((int64_t)b * Hq + h) * N * D;
    const uint8_t* Kh = K + ((int64_t)b * Hkv + g) * N * D;
    const uint8_t* Vh = V + ((int64_t)b * Hkv + g) * N * D;

    const float c2 = scale * kLog2e * descale[0] * descale[1];
    const float sv = descale[2];

    const int q0 = mb * BM;
    const int qw = q0 + 32 * wave;
    const int qrow = qw + l32;

    u32x8 qf[D / 64];
#pragma unroll
    for (int s = 0; s < D / 64; ++s) {
        u32x8 v = {};
        if (qrow < N) v = *reinterpret_cast<const u32x8*>(Qh + (int64_t)qrow * D + 64 * s + 32 * hh);
        qf[s] = v;
    }

    const int kend = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kend + BN - 1) / BN;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();
    float m = kNegBig, lsum = 0.f;

    u32x4 kreg[Cfg::kKPer];
    u32x4 vreg[4];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < Cfg::kKPer; ++i) {
            const int c = tid + i * Cfg::kThreads;
            const int row = c / (D / 16), seg = c % (D / 16);
            u32x4 v = {};
            if (k0 + row < N) v = *reinterpret_cast<const u32x4*>(Kh + (int64_t)(k0 + row) * D + 16 * seg);
            kreg[i] = v;
        }
        if (tid < Cfg::kVTasks) {
            const int rg = tid % (BN / 4), seg = tid / (BN / 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u32x4 v = {};
                const int row = k0 + 4 * rg + j;
                if (row < N) v = *reinterpret_cast<const u32x4*>(Vh + (int64_t)row * D + 16 * seg);
                vreg[j] = v;
            }
        }
    };
    auto put = [&](uint8_t* st) {
#pragma unroll
        for (int i = 0; i < Cfg::kKPer; ++i) {
            const int c = tid + i * Cfg::kThreads;
            const int row = c / (D / 16), seg = c % (D / 16);
            *reinterpret_cast<u32x4*>(st + row * KS + 16 * seg) = kreg[i];
        }
        if (tid < Cfg::kVTasks) {
            const int rg = tid % (BN / 4), seg = tid / (BN / 4);
            uint8_t* vt = st + Cfg::kKBytes;
            const int pos = fp8_vpos(4 * rg);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int w = e >> 2, sh = 8 * (e & 3);
                const uint32_t b0 = (vreg[0][w] >> sh) & 0xffu, b1 = (vreg[1][w] >> sh) & 0xffu;
                const uint32_t b2 = (vreg[2][w] >> sh) & 0xffu, b3 = (vreg[3][w] >> sh) & 0xffu;
                *reinterpret_cast<uint32_t*>(vt + (16 * seg + e) * VS + pos) = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
            }
        }
    };

    fetch(0);
    put(smem);
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
        const int k0 = j * BN;
        const bool more = j + 1 < ntiles;
        if (more) fetch(k0 + BN);
        const uint8_t* Ks = smem + (j & 1) * Cfg::kStage;
        const uint8_t* Vt = Ks + Cfg::kKBytes;

        if (!(CAUSAL && k0 > qw + 31)) {
            f32x16 sacc[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                f32x16 acc = zero16();
#pragma unroll
                for (int s = 0; s < D / 64; ++s)
                    acc = mma_fp8(*reinterpret_cast<const u32x8*>(Ks + (32 * kb + l32) * KS + 64 * s + 32 * hh),
                                  qf[s], acc);
                sacc[kb] = acc;
            }
            const bool need_mask = (CAUSAL && k0 + BN - 1 > qw) || (k0 + BN > N);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * kb + acc_row(r, hh);
                        if ((CAUSAL && key > qrow) || key >= N) sacc[kb][r] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = fmaxf(mx, other_half(mx));
            const float mnew = fmaxf(m, mx * c2);
            const float alpha = fast_exp2(m - mnew);
            float rs = 0.f;
            u32x8 pf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    float p[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        p[i] = fast_exp2(fmaf(sacc[kb][4 * r4 + i], c2, -mnew));
                        rs += p[i];
                    }
                    int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0] * 256.f, p[1] * 256.f, 0, false);
                    w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2] * 256.f, p[3] * 256.f, w, true);
                    pf[4 * kb + r4] = (uint32_t)w;
                }
            lsum = fmaf(lsum, alpha, rs);
            m = mnew;
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct) {
                oacc[ct] *= alpha;
                oacc[ct] = mma_fp8(*reinterpret_cast<const u32x8*>(Vt + (32 * ct + l32) * VS + 32 * hh), pf, oacc[ct]);
            }
        }
        if (more) put(smem + ((j + 1) & 1) * Cfg::kStage);
        __syncthreads();
    }

    const float ltot = lsum + other_half(lsum);
    if (qrow < N) {
        const float f = sv / (256.0f * ltot);
        uint16_t* Orow = O + (((int64_t)b * Hq + h) * N + qrow) * D;
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
                st4<BF16>(Orow + 32 * ct + 8 * gq + 4 * hh,
                          BF16::pack4(oacc[ct][4 * gq] * f, oacc[ct][4 * gq + 1] * f,
                                      oacc[ct][4 * gq + 2] * f, oacc[ct][4 * gq + 3] * f));
        if (hh == 0) LSE[((int64_t)b * Hq + h) * N + qrow] = (m + log2f(ltot)) * kLn2;
    }
}

hipError_t launch_fwd_fp8(int d, int causal, const void* q, const void* k, const void* v, void* o, float* lse,
                          const float* descale, int B, int Hq, int Hkv, int N, float scale, hipStream_t st) {
    const int nmb = (N + 127) / 128;
    const dim3 grid((unsigned)((int64_t)nmb * Hq * B)), block(256);
#define FA_FP8_CASE(DD)                                                                                 \
    if (d == DD) {                                                                                      \
        if (causal)                                                                                     \
            hipLaunchKernelGGL((fwd_fp8_kernel<DD, true>), grid, block, 0, st, (const uint8_t*)q,        \
                               (const uint8_t*)k, (const uint8_t*)v, (uint16_t*)o, lse, descale, Hq, Hkv, N, scale); \
        else                                                                                            \
            hipLaunchKernelGGL((fwd_fp8_kernel<DD, false>), grid, block, 0, st, (const uint8_t*)q,       \
                               (const uint8_t*)k, (const uint8_t*)v, (uint16_t*)o, lse, descale, Hq, Hkv, N, scale); \
        return hipGetLastError();                                                                       \
    }
    FA_FP8_CASE(64)
    FA_FP8_CASE(128)
#undef FA_FP8_CASE
    return hipErrorInvalidValue;
}

}  // namespace fa
