// Forward pass of exact attention: tiled, fused, online softmax (float32
// instantiation; bf16 runs the tuned kernel in fa_fwd_bf16.hip).
//
// "flash attention io aware", section "Flash Attention Algorithm": Q, K, V are
// cut into blocks held on chip; for each Q block the kernel walks the K/V
// blocks, computes the block of scores, updates the running softmax
// statistics and accumulates the output, and writes only O (and the
// statistics) back.  Section "Online Softmax" and the FlashAttention legal
// glossary's online-softmax paragraph: running max m and sum l, with the
// partial sums rescaled when the max grows.  The legal glossary's
// FlashAttention-2 paragraph: the work is split over the sequence (one
// workgroup per query block, head and batch).
//
// Shape of one workgroup: 4 waves x 32 query rows = 128 rows.  Each wave
// computes S^T = K_j Q^T for its 32 queries (keys down the rows, so each lane
// owns one query and sixteen of every 32 keys), then O^T += V_j^T P^T.  K_j is
// staged in LDS as is, V_j transposed (see fa_device.hpp), double-buffered so
// one barrier per K/V tile suffices and the next tile's global loads overlap
// the current tile's math.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

template <class ET, int D>
struct FwdCfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BM = 32 * kWaves;   // query rows per workgroup
    static constexpr int BN = 64;            // keys per K/V tile
    using KTile = NatTile<ET, BN, D, kThreads>;
    using VTile = TrTile<ET, BN, D, kThreads>;
    static constexpr int kStage = KTile::kElems + VTile::kElems;
};

template <class ET, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_kernel(const typename ET::elem* __restrict__ Q,
                                                  const typename ET::elem* __restrict__ K,
                                                  const typename ET::elem* __restrict__ V,
                                                  typename ET::elem* __restrict__ O,
                                                  float* __restrict__ LSE,
                                                  int Hq, int Hkv, int N, float c2) {
    using Cfg = FwdCfg<ET, D>;
    using elem = typename ET::elem;
    using raw8 = typename ET::raw8;
    constexpr int BM = Cfg::BM, BN = Cfg::BN;
    constexpr int KS = Cfg::KTile::kStride, VS = Cfg::VTile::kStride;
    __shared__ __attribute__((aligned(64))) elem smem[2 * Cfg::kStage];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;

    // ---- which (query block, head, batch) this workgroup owns
    const int nmb = (N + BM - 1) / BM;
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    const int mbi = lin % nmb, bh = lin / nmb;
    const int h = bh % Hq, b = bh / Hq;
    const int mb = CAUSAL ? nmb - 1 - mbi : mbi;     // longest causal rows first
    const int g = h / (Hq / Hkv);
    const elem* Qh = Q + ((int64_t)b * Hq + h) * N * D;
    const elem* Kh = K + ((int64_t)b * Hkv + g) * N * D;
    const elem* Vh = V + ((int64_t)b * Hkv + g) * N * D;

    const int q0 = mb * BM;
    const int qw = q0 + 32 * wave;     // first query row of this wave
    const int qrow = qw + l32;         // this lane's query row

    // ---- Q block as B operands (held in registers for the whole kernel)
    raw8 qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        raw8 v = {};
        if (qrow < N) v = ld8<ET>(Qh + (int64_t)qrow * D + 16 * s + 8 * hh);
        qf[s] = v;
    }

    const int kend = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kend + BN - 1) / BN;

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();
    float m = kNegBig, lsum = 0.f;

    typename Cfg::KTile kt_regs;
    typename Cfg::VTile vt_regs;
    kt_regs.load(Kh, N, tid);
    vt_regs.load(Vh, N, tid);
    kt_regs.store(smem, tid);
    vt_regs.store(smem + Cfg::KTile::kElems, tid);
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
        const int k0 = j * BN;
        const bool more = j + 1 < ntiles;
        if (more) {
            kt_regs.load(Kh + (int64_t)(k0 + BN) * D, N - (k0 + BN), tid);
            vt_regs.load(Vh + (int64_t)(k0 + BN) * D, N - (k0 + BN), tid);
        }
        const elem* Ks = smem + (j & 1) * Cfg::kStage;
        const elem* Vt = Ks + Cfg::KTile::kElems;

        if (!(CAUSAL && k0 > qw + 31)) {
            // ---- S^T = K_j Q^T : rows = keys, columns = this wave's queries
            f32x16 sacc[BN / 32];
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
                f32x16 acc = zero16();
#pragma unroll
                for (int s = 0; s < D / 16; ++s)
                    acc = ET::mma(ld8<ET>(Ks + (32 * kb + l32) * KS + 16 * s + 8 * hh), qf[s], acc);
                sacc[kb] = acc;
            }
            // ---- mask: keys past the diagonal (causal) or past the end
            const bool need_mask = (CAUSAL && k0 + BN - 1 > qw) || (k0 + BN > N);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * kb + acc_row(r, hh);
                        if ((CAUSAL && key > qrow) || key >= N) sacc[kb][r] = -INFINITY;
                    }
            }
            // ---- online softmax update (base-2, log2(e) folded into c2)
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
            mx = fmaxf(mx, other_half(mx));
            const float mnew = fmaxf(m, mx * c2);
            const float alpha = fast_exp2(m - mnew);
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(sacc[kb][r], c2, -mnew));
                    sacc[kb][r] = p;
                    rs += p;
                }
            lsum = fmaf(lsum, alpha, rs);
            m = mnew;
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct) oacc[ct] *= alpha;
            // ---- O^T += V_j^T P^T
            raw8 pf[BN / 32][2];
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
                pf[kb][0] = ET::pack8(sacc[kb], 0);
                pf[kb][1] = ET::pack8(sacc[kb], 8);
            }
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        oacc[ct] = ET::mma(ld8<ET>(Vt + (32 * ct + l32) * VS + 32 * kb + 16 * t + 8 * hh),
                                           pf[kb][t], oacc[ct]);
        }
        if (more) {
            elem* nxt = smem + ((j + 1) & 1) * Cfg::kStage;
            kt_regs.store(nxt, tid);
            vt_regs.store(nxt + Cfg::KTile::kElems, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l)
    const float ltot = lsum + other_half(lsum);
    if (qrow < N) {
        const float inv = 1.0f / ltot;
        elem* Orow = O + (((int64_t)b * Hq + h) * N + qrow) * D;
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
                st4<ET>(Orow + 32 * ct + 8 * gq + 4 * hh,
                        ET::pack4(oacc[ct][4 * gq] * inv, oacc[ct][4 * gq + 1] * inv,
                                  oacc[ct][4 * gq + 2] * inv, oacc[ct][4 * gq + 3] * inv));
        if (hh == 0) LSE[((int64_t)b * Hq + h) * N + qrow] = (m + log2f(ltot)) * kLn2;
    }
}

template <class ET, int D, bool CAUSAL>
static hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int N, float scale, hipStream_t st) {
    using Cfg = FwdCfg<ET, D>;
    using elem = typename ET::elem;
    const int nmb = (N + Cfg::BM - 1) / Cfg::BM;
    const int64_t grid = (int64_t)nmb * Hq * B;
    hipLaunchKernelGGL((fwd_kernel<ET, D, CAUSAL>), dim3((unsigned)grid), dim3(Cfg::kThreads), 0, st,
                       (const elem*)q, (const elem*)k, (const elem*)v, (elem*)o, lse, Hq, Hkv, N,
                       scale * kLog2e);
    return hipGetLastError();
}

hipError_t launch_fwd(int dtype, int d, int causal, const void* q, const void* k, const void* v,
                      void* o, float* lse, int B, int Hq, int Hkv, int N, float scale,
                      hipStream_t st) {
#define FA_FWD_CASE(ET, DD)                                                                        \
    if (d == DD) return causal ? launch<ET, DD, true>(q, k, v, o, lse, B, Hq, Hkv, N, scale, st)  \
                               : launch<ET, DD, false>(q, k, v, o, lse, B, Hq, Hkv, N, scale, st);
    if (dtype == 1) {
        return launch_fwd_bf16(d, causal, q, k, v, o, lse, B, Hq, Hkv, N, scale, st);
    } else if (dtype == 0) {
        FA_FWD_CASE(F32, 64)
        FA_FWD_CASE(F32, 128)
    }
#undef FA_FWD_CASE
    return hipErrorInvalidValue;
}

}  // namespace fa
