// bf16 forward pass of exact attention (the tuned path; float32 uses fa_fwd.hip).
//
// "flash attention io aware", sections "Flash Attention Algorithm" and "Online
// Softmax"; the FlashAttention legal glossary's online-softmax and
// FlashAttention-2 paragraphs (one workgroup per query block, head and batch;
// fewer non-matmul operations).  What differs from the pages' CUDA design is
// how the same steps map onto gfx950:
//  - K and V tiles go from HBM straight into LDS (global_load_lds, no staging
//    registers) in their global row-major layout, several tiles in flight,
//    one barrier per tile;
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

template <int D, int NW, int QB, int BN_, int NS, int MINW>
struct FwdBf16Cfg {
    static constexpr int kWaves = NW;
    static constexpr int kThreads = 64 * NW;
    static constexpr int kQB = QB;                    // 32-row query blocks per wave
    static constexpr int BM = 32 * QB * NW;           // query rows per workgroup
    static constexpr int BN = BN_;                    // keys per K/V tile
    static constexpr int kStages = NS;                // K/V tiles resident or in flight
    static constexpr int kMinWaves = MINW;            // occupancy target (waves per SIMD)
    using KT = LdsTile<BN, D, NW>;                    // read as rows
    using VT = LdsTile<BN, D, NW>;                    // read transposed
    static constexpr int kStage = KT::kElems + VT::kElems;   // elements per stage
    static constexpr int kLoads = KT::kPerWave + VT::kPerWave;
    static constexpr float kTau = 8.0f;               // log2 slack before the max is moved
};

// Tuned shape (measured on MI355X at B=4, H=32, N=4096, d=128, causal): 8 waves
// of 32 query rows share each K/V tile, 64-key tiles, two waves per SIMD;
// four stages: the tile being finished (V), the next one (K) and two in
// flight.  Two 32-row blocks per wave (each K/V fragment read feeding two
// products) needs one wave per SIMD and measured slower.
template <int D>
using FwdBf16Tuned = FwdBf16Cfg<D, 8, 1, 64, 4, 2>;

template <int D, bool CAUSAL, class Cfg>
__global__ __launch_bounds__(Cfg::kThreads, Cfg::kMinWaves) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int Hq, int Hkv, int N, float c2) {
    using KT = typename Cfg::KT;
    using VT = typename Cfg::VT;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, NS = Cfg::kStages, QB = Cfg::kQB;
    constexpr int KB = BN / 32;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * Cfg::kStage];

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
    const int qw = q0 + 32 * QB * wave;               // first query row of this wave
    int qrow[QB];                                     // this lane's query row in each block
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) qrow[qb] = qw + 32 * qb + l32;

    const int kend = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kend + BN - 1) / BN;

    // the first NS-1 K/V tiles go in flight while Q is fetched
    auto issue = [&](int t) {
        const uint16_t* st = smem + (t % NS) * Cfg::kStage;
        KT::load(Kh + (int64_t)t * BN * D, N - t * BN, st, wave, lane);
        VT::load(Vh + (int64_t)t * BN * D, N - t * BN, st + KT::kElems, wave, lane);
    };
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
        if (t < ntiles) issue(t);

    u32x4 qf[QB][D / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            u32x4 v = {};
            if (qrow[qb] < N) v = *reinterpret_cast<const u32x4*>(Qh + (int64_t)qrow[qb] * D + 16 * s + 8 * hh);
            qf[qb][s] = v;
        }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int s = 0; s < D / 16; ++s) settle(qf[qb][s]);

    f32x16 oacc[QB][D / 32];
    float m[QB], lsum[QB], mx[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[qb][i] = zero16();
        m[qb] = kNegBig;
        lsum[qb] = 0.f;
    }

    // S^T = K_t Q^T for tile t (stage t % NS): rows = keys, columns = queries.
    // Each K fragment read from LDS feeds the QB query blocks.
    auto scores = [&](int t, f32x16 (&sacc)[QB][KB]) {
        const uint16_t* Ks = smem + (t % NS) * Cfg::kStage;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sacc[qb][kb] = zero16();
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const u32x4 a = KT::row8(Ks, 32 * kb + l32, 2 * s + hh);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[qb][kb] = mma_bf16(a, qf[qb][s], sacc[qb][kb]);
            }
    };
    // mask keys past the diagonal (causal) or past the end, then the row maxima
    auto mask_max = [&](int t, f32x16 (&sacc)[QB][KB]) {
        const int k0 = t * BN;
        if ((CAUSAL && k0 + BN - 1 > qw) || k0 + BN > N) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * kb + acc_row(r, hh);
                        if ((CAUSAL && key > qrow[qb]) || key >= N) sacc[qb][kb][r] = -INFINITY;
                    }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float x = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) x = fmaxf(x, sacc[qb][kb][r]);
            mx[qb] = pair_max(x);
        }
    };
    // this wave has keys to look at in tile t
    auto active = [&](int t) { return t < ntiles && !(CAUSAL && t * BN > qw + 32 * QB - 1); };

    // One pipeline step: while the matrix cores form the scores of tile j+1,
    // the vector units exponentiate tile j; then P_j V_j runs and the row
    // maxima of tile j+1 are taken.  Tiles j and j+1 are both resident in LDS.
    auto step = [&](int j, f32x16 (&cur)[QB][KB], f32x16 (&nxt)[QB][KB]) {
        if (j + 1 < ntiles) pipe_wait<NS - 1, Cfg::kLoads>(j + 1, ntiles);
        lds_barrier();                               // tile j+1 visible, stage of tile j-1 free
        if (j + NS - 1 < ntiles) issue(j + NS - 1);
        if (!active(j)) return;
        const uint16_t* Vs = smem + (j % NS) * Cfg::kStage + KT::kElems;

        // ---- running max (base 2, scale*log2(e) in c2); moved only when some
        // row of the wave grew by more than 2^tau
        float mnew[QB];
        bool grow = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            mnew[qb] = fmaxf(m[qb], mx[qb] * c2);
            grow |= mnew[qb] > m[qb] + Cfg::kTau;
        }
        if (__any(grow)) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float alpha = fast_exp2(m[qb] - mnew[qb]);
                m[qb] = mnew[qb];
                lsum[qb] *= alpha;
#pragma unroll
                for (int ct = 0; ct < D / 32; ++ct) oacc[qb][ct] *= alpha;
            }
        }
        // ---- scores of tile j+1 (matrix cores; computed unconditionally so
        // they share a basic block with the exponentials; without a next tile
        // they read an idle stage and are discarded) ...
        scores(j + 1, nxt);
        // ---- ... while tile j is exponentiated and packed (vector units);
        // l sums the bf16-rounded values, the same numbers the product uses
        u32x4 pf[QB][KB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) cur[qb][kb][r] = fast_exp2(fmaf(cur[qb][kb][r], c2, -m[qb]));
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    pf[qb][kb][t] = pack_bf16x8(cur[qb][kb], 8 * t);
#pragma unroll
                    for (int i = 0; i < 4; ++i) rs[i] = dot2_bf16_sum(pf[qb][kb][t][i], rs[i]);
                }
            }
            lsum[qb] += (rs[0] + rs[1]) + (rs[2] + rs[3]);
        }
        // ---- O^T += V_j^T P_j^T; each V^T fragment feeds the QB blocks
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int ct = 0; ct < D / 32; ++ct) {
                    const u32x4 a = VT::tr8(Vs, 32 * kb + 16 * t, 32 * ct, lane);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) oacc[qb][ct] = mma_bf16(a, pf[qb][kb][t], oacc[qb][ct]);
                }
        if (active(j + 1)) mask_max(j + 1, nxt);
    };

    f32x16 sA[QB][KB], sB[QB][KB];
    pipe_wait<NS, Cfg::kLoads>(0, ntiles);
    lds_barrier();
    scores(0, sA);
    mask_max(0, sA);
    for (int j = 0; j < ntiles; j += 2) {
        step(j, sA, sB);
        if (j + 1 < ntiles) step(j + 1, sB, sA);
    }

    // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float ltot = pair_sum(lsum[qb]);
        if (qrow[qb] < N) {
            const float inv = 1.0f / ltot;
            uint16_t* Orow = O + (((int64_t)b * Hq + h) * N + qrow[qb]) * D;
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    u32x2 w;
                    w[0] = pack_bf16x2(oacc[qb][ct][4 * gq] * inv, oacc[qb][ct][4 * gq + 1] * inv);
                    w[1] = pack_bf16x2(oacc[qb][ct][4 * gq + 2] * inv, oacc[qb][ct][4 * gq + 3] * inv);
                    *reinterpret_cast<u32x2*>(Orow + 32 * ct + 8 * gq + 4 * hh) = w;
                }
            if (hh == 0) LSE[((int64_t)b * Hq + h) * N + qrow[qb]] = (m[qb] + log2f(ltot)) * kLn2;
        }
    }
}

template <int D, bool CAUSAL>
static hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                         int N, float scale, hipStream_t st) {
    using Cfg = FwdBf16Tuned<D>;
    const int nmb = (N + Cfg::BM - 1) / Cfg::BM;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, Cfg>), dim3((unsigned)((int64_t)nmb * Hq * B)), dim3(Cfg::kThreads),
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
