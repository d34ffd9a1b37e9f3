// bf16 forward pass of exact attention (the tuned path; float32 uses fa_fwd.hip).
//
// "flash attention io aware", sections "Flash Attention Algorithm" and "Online
// Softmax"; the FlashAttention legal glossary's online-softmax and
// FlashAttention-2 paragraphs (one workgroup per query block, head and batch;
// fewer non-matmul operations).  What differs from the pages' CUDA design is
// how the same steps map onto gfx950:
//  - K and V tiles go from HBM straight into LDS (global_load_lds, no staging
//    registers), double-buffered, in their global row-major layout;
//  - S^T = K_j Q^T puts keys down the accumulator rows, so each lane owns one
//    query and the row max / row sum need one cross-half exchange
//    (v_permlane32_swap) per tile;
//  - O^T += V_j^T P^T reads V_j^T with transposing LDS reads, and P^T is the
//    S^T accumulator itself, converted to bf16 in registers;
//  - the row sum l adds up the bf16-rounded probabilities (v_dot2 against
//    ones), the same numbers the P V product uses;
//  - the running max is only moved (and O, l rescaled) when it grows by more
//    than 2^8 for some row of the wave; otherwise exp2 is taken against the
//    stale max.  Both readings give the same softmax: exp2(s - m) / l is
//    invariant to the reference m, and the stale reference bounds each
//    exponential by 2^8, far from float overflow.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

template <int D>
struct FwdBf16Cfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BM = 32 * kWaves;            // query rows per workgroup
    static constexpr int BN = 64;                     // keys per K/V tile
    using KT = LdsTile<BN, D, kWaves>;   // read as rows
    using VT = LdsTile<BN, D, kWaves>;  // read transposed
    static constexpr int kStage = KT::kElems + VT::kElems;
    static constexpr float kTau = 8.0f;               // log2 slack before the max is moved
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(const uint16_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V,
                                                          uint16_t* __restrict__ O, float* __restrict__ LSE,
                                                          int Hq, int Hkv, int N, float c2) {
    using Cfg = FwdBf16Cfg<D>;
    using KT = typename Cfg::KT;
    using VT = typename Cfg::VT;
    constexpr int BM = Cfg::BM, BN = Cfg::BN;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * Cfg::kStage];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;

    const int nmb = (N + BM - 1) / BM;
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    const int mbi = lin % nmb, bh = lin / nmb;
    const int h = bh % Hq, b = bh / Hq;
    const int mb = CAUSAL ? nmb - 1 - mbi : mbi;      // longest causal rows first
    const int g = h / (Hq / Hkv);
    const uint16_t* Qh = Q + ((int64_t)b * Hq + h) * N * D;
    const uint16_t* Kh = K + ((int64_t)b * Hkv + g) * N * D;
    const uint16_t* Vh = V + ((int64_t)b * Hkv + g) * N * D;

    const int q0 = mb * BM;
    const int qw = q0 + 32 * wave;
    const int qrow = qw + l32;

    const int kend = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kend + BN - 1) / BN;

    // first K/V tile in flight while Q is fetched
    KT::load(Kh, N, smem, wave, lane);
    VT::load(Vh, N, smem + KT::kElems, wave, lane);

    u32x4 qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        u32x4 v = {};
        if (qrow < N) v = *reinterpret_cast<const u32x4*>(Qh + (int64_t)qrow * D + 16 * s + 8 * hh);
        qf[s] = v;
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();
    float m = kNegBig, lsum = 0.f;

    wait_dma();
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
        const int k0 = j * BN;
        if (j + 1 < ntiles) {
            uint16_t* nxt = smem + ((j + 1) & 1) * Cfg::kStage;
            KT::load(Kh + (int64_t)(k0 + BN) * D, N - (k0 + BN), nxt, wave, lane);
            VT::load(Vh + (int64_t)(k0 + BN) * D, N - (k0 + BN), nxt + KT::kElems, wave, lane);
        }
        const uint16_t* Ks = smem + (j & 1) * Cfg::kStage;
        const uint16_t* Vs = Ks + KT::kElems;

        if (!(CAUSAL && k0 > qw + 31)) {
            // ---- S^T = K_j Q^T
            f32x16 sacc[BN / 32];
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) sacc[kb] = zero16();
#pragma unroll
            for (int s = 0; s < D / 16; ++s)
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb)
                    sacc[kb] = mma_bf16(KT::row8(Ks, 32 * kb + l32, 2 * s + hh), qf[s], sacc[kb]);

            // ---- mask keys past the diagonal (causal) or past the end
            if ((CAUSAL && k0 + BN - 1 > qw) || k0 + BN > N) {
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * kb + acc_row(r, hh);
                        if ((CAUSAL && key > qrow) || key >= N) sacc[kb][r] = -INFINITY;
                    }
            }

            // ---- online softmax (base 2, scale*log2(e) folded into c2)
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            const float mnew = fmaxf(m, pair_max(mx) * c2);
            if (__any(mnew > m + Cfg::kTau)) {
                const float alpha = fast_exp2(m - mnew);
                m = mnew;
                lsum *= alpha;
#pragma unroll
                for (int ct = 0; ct < D / 32; ++ct) oacc[ct] *= alpha;
            }
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = fast_exp2(fmaf(sacc[kb][r], c2, -m));

            // ---- P^T to bf16; l sums the rounded values, so O's weights and
            // the normaliser are the same numbers
            u32x4 pf[BN / 32][2];
            float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    pf[kb][t] = pack_bf16x8(sacc[kb], 8 * t);
#pragma unroll
                    for (int i = 0; i < 4; ++i) rs[i] = dot2_bf16_sum(pf[kb][t][i], rs[i]);
                }
            lsum += (rs[0] + rs[1]) + (rs[2] + rs[3]);

            // ---- O^T += V_j^T P^T
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int ct = 0; ct < D / 32; ++ct)
                        oacc[ct] = mma_bf16(VT::tr8(Vs, 32 * kb + 16 * t, 32 * ct, lane), pf[kb][t], oacc[ct]);
        }
        wait_dma();
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l)
    const float ltot = pair_sum(lsum);
    if (qrow < N) {
        const float inv = 1.0f / ltot;
        uint16_t* Orow = O + (((int64_t)b * Hq + h) * N + qrow) * D;
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                u32x2 w;
                w[0] = pack_bf16x2(oacc[ct][4 * gq] * inv, oacc[ct][4 * gq + 1] * inv);
                w[1] = pack_bf16x2(oacc[ct][4 * gq + 2] * inv, oacc[ct][4 * gq + 3] * inv);
                *reinterpret_cast<u32x2*>(Orow + 32 * ct + 8 * gq + 4 * hh) = w;
            }
        if (hh == 0) LSE[((int64_t)b * Hq + h) * N + qrow] = (m + log2f(ltot)) * kLn2;
    }
}

template <int D, bool CAUSAL>
static hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                         int N, float scale, hipStream_t st) {
    using Cfg = FwdBf16Cfg<D>;
    const int nmb = (N + Cfg::BM - 1) / Cfg::BM;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)nmb * Hq * B)), dim3(Cfg::kThreads),
                       0, st, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, Hq,
                       Hkv, N, scale * kLog2e);
    return hipGetLastError();
}

hipError_t launch_fwd_bf16(int d, int causal, const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int N, float scale, hipStream_t st) {
    if (d == 64) return causal ? launch<64, true>(q, k, v, o, lse, B, Hq, Hkv, N, scale, st)
                               : launch<64, false>(q, k, v, o, lse, B, Hq, Hkv, N, scale, st);
    if (d == 128) return causal ? launch<128, true>(q, k, v, o, lse, B, Hq, Hkv, N, scale, st)
                                : launch<128, false>(q, k, v, o, lse, B, Hq, Hkv, N, scale, st);
    return hipErrorInvalidValue;
}

}  // namespace fa
