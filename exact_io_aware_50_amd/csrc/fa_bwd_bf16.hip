// bf16 backward pass (the tuned path; float32 uses the generic kernels in
// fa_bwd.hip).  Same arithmetic as there; what changes is the mapping onto
// gfx950: Q/dO (dK/dV kernel) and K/V (dQ kernel) tiles, and the per-row
// statistics, go from HBM straight into LDS in row-major layout with several
// tiles in flight; every transposed operand (Q^T, dO^T, K^T) is read with
// transposing LDS reads, so no tile is transposed through registers; P and dS
// are packed to bf16 by the hardware converter.
//
// FlashAttention legal glossary, backward paragraph and entry "Recomputation"
// (P is recomputed from Q, K and the stored statistics), FlashAttention-2
// paragraph (the dK/dV pass is parallel over key blocks, without atomics).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

// ------------------------------------------------------------ dK, dV
template <int D, int NW, int NS>
struct KVBf16Cfg {
    static constexpr int kWaves = NW;
    static constexpr int kThreads = 64 * NW;
    static constexpr int BNK = 32 * NW;                 // keys per workgroup (32 per wave)
    static constexpr int BMQ = D == 128 ? 32 : 64;      // query rows per step
    static constexpr int QB = BMQ / 32;
    static constexpr int kStages = NS;
    using QT = LdsTile<BMQ, D, NW>;
    static constexpr int kStatChunks = BMQ / 2;         // 16-byte chunks of (LSE*log2e, D) per step
    static constexpr int kStatPerWave = kStatChunks / NW;
    static_assert(kStatChunks % NW == 0, "statistics split evenly over the waves");
    static constexpr int kStatBytes = 8 * BMQ;
    static constexpr int kStageBytes = 2 * QT::kBytes + kStatBytes;
    static constexpr int kLoads = 2 * QT::kPerWave + 1;
};
template <int D>
using KVBf16Tuned = KVBf16Cfg<D, 8, 4>;

template <int D, bool CAUSAL, class Cfg>
__global__ __launch_bounds__(Cfg::kThreads, 2) void bwd_dkdv_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ WSd, const float* __restrict__ WSl,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Hq, int Hkv, int N, int Npad, float c2,
    float scale) {
    using QT = typename Cfg::QT;
    constexpr int BNK = Cfg::BNK, BMQ = Cfg::BMQ, QB = Cfg::QB, NS = Cfg::kStages;
    __shared__ __attribute__((aligned(1024))) char smem[NS * Cfg::kStageBytes];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;

    const int nkb = (N + BNK - 1) / BNK;
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    const int kbk = lin % nkb, bg = lin / nkb;      // ascending key blocks: causal-heavy first
    const int g = bg % Hkv, b = bg / Hkv;
    const int G = Hq / Hkv;
    const int k0 = kbk * BNK;
    const int kw = k0 + 32 * wave;
    const int krow = kw + l32;

    const uint16_t* Kg = K + ((int64_t)b * Hkv + g) * N * D;
    const uint16_t* Vg = V + ((int64_t)b * Hkv + g) * N * D;

    const int nqt = (N + BMQ - 1) / BMQ;
    const int qt0 = CAUSAL ? k0 / BMQ : 0;          // earlier query blocks see none of these keys
    const int per_head = nqt - qt0;
    const int total = G * per_head;

    // Step `it`: query head g*G + it / per_head, query block qt0 + it % per_head.
    auto issue = [&](int it) {
        const int hq = g * G + it / per_head;
        const int q0 = (qt0 + it % per_head) * BMQ;
        const int64_t bh = (int64_t)b * Hq + hq;
        const char* st = smem + (it % NS) * Cfg::kStageBytes;
        QT::load(Q + (bh * N + q0) * D, N - q0, (const uint16_t*)st, wave, lane);
        QT::load(dO + (bh * N + q0) * D, N - q0, (const uint16_t*)(st + QT::kBytes), wave, lane);
        // statistics: chunk c < BMQ/4 holds LSE*log2e rows q0+4c.., the rest D rows
        const int c = wave * Cfg::kStatPerWave + lane;
        if (lane < Cfg::kStatPerWave) {
            const float* src = c < BMQ / 4 ? WSl + bh * Npad + q0 + 4 * c : WSd + bh * Npad + q0 + 4 * (c - BMQ / 4);
            dma16(src, lds_addr(st + 2 * QT::kBytes) + 16 * wave * Cfg::kStatPerWave);
        }
    };
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
        if (t < total) issue(t);

    u32x4 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        u32x4 a = {}, c = {};
        if (krow < N) {
            a = *reinterpret_cast<const u32x4*>(Kg + (int64_t)krow * D + 16 * s + 8 * hh);
            c = *reinterpret_cast<const u32x4*>(Vg + (int64_t)krow * D + 16 * s + 8 * hh);
        }
        kf[s] = a;
        vf[s] = c;
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        settle(kf[s]);
        settle(vf[s]);
    }
    f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        dkacc[i] = zero16();
        dvacc[i] = zero16();
    }

    for (int it = 0; it < total; ++it) {
        const int q0 = (qt0 + it % per_head) * BMQ;
        pipe_wait<NS, Cfg::kLoads>(it, total);
        lds_barrier();
        if (it + NS - 1 < total) issue(it + NS - 1);
        const char* st = smem + (it % NS) * Cfg::kStageBytes;
        const uint16_t* Qs = (const uint16_t*)st;
        const uint16_t* dOs = (const uint16_t*)(st + QT::kBytes);
        const float* sl = (const float*)(st + 2 * QT::kBytes);   // LSE*log2e [BMQ], then D [BMQ]

        if (!(CAUSAL && q0 + BMQ - 1 < kw)) {
            const bool need_mask = CAUSAL && kw + 31 > q0;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                // S = Q K^T and dP = dO V^T: rows = queries, columns = this wave's keys
                f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
                for (int s = 0; s < D / 16; ++s) {
                    sacc = mma_bf16(QT::row8(Qs, 32 * qb + l32, 2 * s + hh), kf[s], sacc);
                    dpacc = mma_bf16(QT::row8(dOs, 32 * qb + l32, 2 * s + hh), vf[s], dpacc);
                }
                // P from the stored statistics.  Causal: key krow is hidden from
                // query q0 + 32*qb + row(r) iff delta > 8*(r/4) + r%4, with
                // delta = krow - q0 - 32*qb - 4*hh (forced below every row
                // when the block needs no mask): one compare and one select
                const int delta = need_mask ? krow - q0 - 32 * qb - 4 * hh : -64;
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(sl + 32 * qb + 8 * gq + 4 * hh);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(sl + BMQ + 32 * qb + 8 * gq + 4 * hh);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 4 * gq + j;
                        float p = fast_exp2(fmaf(sacc[r], c2, -l4[j]));
                        if (CAUSAL && delta > 8 * gq + j) p = 0.f;
                        sacc[r] = p;
                        dpacc[r] = p * (dpacc[r] - d4[j]);
                    }
                }
                // dV^T += dO^T P ;  dK^T += Q^T dS
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const u32x4 pb = pack_bf16x8(sacc, 8 * t);
                    const u32x4 sb = pack_bf16x8(dpacc, 8 * t);
#pragma unroll
                    for (int ct = 0; ct < D / 32; ++ct) {
                        dvacc[ct] = mma_bf16(QT::tr8(dOs, 32 * qb + 16 * t, 32 * ct, lane), pb, dvacc[ct]);
                        dkacc[ct] = mma_bf16(QT::tr8(Qs, 32 * qb + 16 * t, 32 * ct, lane), sb, dkacc[ct]);
                    }
                }
            }
        }
    }

    if (krow < N) {
        uint16_t* dKr = dK + (((int64_t)b * Hkv + g) * N + krow) * D;
        uint16_t* dVr = dV + (((int64_t)b * Hkv + g) * N + krow) * D;
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int c = 32 * ct + 8 * gq + 4 * hh;
                u32x2 wk, wv;
                wk[0] = pack_bf16x2(dkacc[ct][4 * gq] * scale, dkacc[ct][4 * gq + 1] * scale);
                wk[1] = pack_bf16x2(dkacc[ct][4 * gq + 2] * scale, dkacc[ct][4 * gq + 3] * scale);
                wv[0] = pack_bf16x2(dvacc[ct][4 * gq], dvacc[ct][4 * gq + 1]);
                wv[1] = pack_bf16x2(dvacc[ct][4 * gq + 2], dvacc[ct][4 * gq + 3]);
                *reinterpret_cast<u32x2*>(dKr + c) = wk;
                *reinterpret_cast<u32x2*>(dVr + c) = wv;
            }
    }
}

// ------------------------------------------------------------ dQ
template <int D, int NW, int NS>
struct QBf16Cfg {
    static constexpr int kWaves = NW;
    static constexpr int kThreads = 64 * NW;
    static constexpr int BM = 32 * NW;          // query rows per workgroup
    static constexpr int BNK = 64;              // keys per tile
    static constexpr int kStages = NS;
    using KT = LdsTile<BNK, D, NW>;             // read as rows and transposed
    using VT = LdsTile<BNK, D, NW>;             // read as rows
    static constexpr int kStage = KT::kElems + VT::kElems;
    static constexpr int kLoads = KT::kPerWave + VT::kPerWave;
};
template <int D>
using QBf16Tuned = QBf16Cfg<D, 8, 3>;

template <int D, bool CAUSAL, class Cfg>
__global__ __launch_bounds__(Cfg::kThreads, 2) void bwd_dq_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ WSd, const float* __restrict__ WSl,
    uint16_t* __restrict__ dQ, int Hq, int Hkv, int N, int Npad, float c2, float scale) {
    using KT = typename Cfg::KT;
    using VT = typename Cfg::VT;
    constexpr int BM = Cfg::BM, BNK = Cfg::BNK, NS = Cfg::kStages;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * Cfg::kStage];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;

    const int nmb = (N + BM - 1) / BM;
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    const int mbi = lin % nmb, bh = lin / nmb;
    const int h = bh % Hq, b = bh / Hq;
    const int mb = CAUSAL ? nmb - 1 - mbi : mbi;
    const int g = h / (Hq / Hkv);
    const int64_t rowbase = ((int64_t)b * Hq + h) * N;
    const uint16_t* Kg = K + ((int64_t)b * Hkv + g) * N * D;
    const uint16_t* Vg = V + ((int64_t)b * Hkv + g) * N * D;

    const int q0 = mb * BM;
    const int qw = q0 + 32 * wave;
    const int qrow = qw + l32;
    const int kend = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kend + BNK - 1) / BNK;

    auto issue = [&](int t) {
        const uint16_t* st = smem + (t % NS) * Cfg::kStage;
        KT::load(Kg + (int64_t)t * BNK * D, N - t * BNK, st, wave, lane);
        VT::load(Vg + (int64_t)t * BNK * D, N - t * BNK, st + KT::kElems, wave, lane);
    };
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
        if (t < ntiles) issue(t);

    u32x4 qf[D / 16], of[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        u32x4 a = {}, c = {};
        if (qrow < N) {
            a = *reinterpret_cast<const u32x4*>(Q + (rowbase + qrow) * D + 16 * s + 8 * hh);
            c = *reinterpret_cast<const u32x4*>(dO + (rowbase + qrow) * D + 16 * s + 8 * hh);
        }
        qf[s] = a;
        of[s] = c;
    }
    const int64_t srow = ((int64_t)b * Hq + h) * Npad + qrow;
    const float lse2 = qrow < N ? WSl[srow] : INFINITY;
    const float dq_d = qrow < N ? WSd[srow] : 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        settle(qf[s]);
        settle(of[s]);
    }
    settle(lse2);
    settle(dq_d);

    f32x16 dqacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) dqacc[i] = zero16();

    for (int j = 0; j < ntiles; ++j) {
        const int k0 = j * BNK;
        pipe_wait<NS, Cfg::kLoads>(j, ntiles);
        lds_barrier();
        if (j + NS - 1 < ntiles) issue(j + NS - 1);
        const uint16_t* Ks = smem + (j % NS) * Cfg::kStage;
        const uint16_t* Vs = Ks + KT::kElems;

        if (!(CAUSAL && k0 > qw + 31)) {
            // S^T = K Q^T and dP^T = V dO^T: rows = keys, columns = this wave's queries
            f32x16 sacc[BNK / 32], dpacc[BNK / 32];
#pragma unroll
            for (int kb = 0; kb < BNK / 32; ++kb) {
                sacc[kb] = zero16();
                dpacc[kb] = zero16();
            }
#pragma unroll
            for (int s = 0; s < D / 16; ++s)
#pragma unroll
                for (int kb = 0; kb < BNK / 32; ++kb) {
                    sacc[kb] = mma_bf16(KT::row8(Ks, 32 * kb + l32, 2 * s + hh), qf[s], sacc[kb]);
                    dpacc[kb] = mma_bf16(VT::row8(Vs, 32 * kb + l32, 2 * s + hh), of[s], dpacc[kb]);
                }
            // P from the stored statistics; keys after the query (causal) or
            // past the end are zeroed in one wave-uniform branch
#pragma unroll
            for (int kb = 0; kb < BNK / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = fast_exp2(fmaf(sacc[kb][r], c2, -lse2));
            if ((CAUSAL && k0 + BNK - 1 > qw) || (k0 + BNK > N)) {
#pragma unroll
                for (int kb = 0; kb < BNK / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * kb + acc_row(r, hh);
                        if ((CAUSAL && key > qrow) || key >= N) sacc[kb][r] = 0.f;
                    }
            }
#pragma unroll
            for (int kb = 0; kb < BNK / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) dpacc[kb][r] = sacc[kb][r] * (dpacc[kb][r] - dq_d);
            // dQ^T += K^T dS^T
#pragma unroll
            for (int kb = 0; kb < BNK / 32; ++kb)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const u32x4 sb = pack_bf16x8(dpacc[kb], 8 * t);
#pragma unroll
                    for (int ct = 0; ct < D / 32; ++ct)
                        dqacc[ct] = mma_bf16(KT::tr8(Ks, 32 * kb + 16 * t, 32 * ct, lane), sb, dqacc[ct]);
                }
        }
    }

    if (qrow < N) {
        uint16_t* dQr = dQ + (rowbase + qrow) * D;
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                u32x2 w;
                w[0] = pack_bf16x2(dqacc[ct][4 * gq] * scale, dqacc[ct][4 * gq + 1] * scale);
                w[1] = pack_bf16x2(dqacc[ct][4 * gq + 2] * scale, dqacc[ct][4 * gq + 3] * scale);
                *reinterpret_cast<u32x2*>(dQr + 32 * ct + 8 * gq + 4 * hh) = w;
            }
    }
}

template <int D, bool CAUSAL>
static hipError_t launch_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* ws,
                              void* dk, void* dv, int B, int Hq, int Hkv, int N, float scale, hipStream_t st) {
    using Cfg = KVBf16Tuned<D>;
    const int nkb = (N + Cfg::BNK - 1) / Cfg::BNK;
    const int Np = ws_rows(N);
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, CAUSAL, Cfg>), dim3((unsigned)((int64_t)nkb * Hkv * B)),
                       dim3(Cfg::kThreads), 0, st, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)dO, ws, ws + (int64_t)B * Hq * Np, (uint16_t*)dk, (uint16_t*)dv, Hq, Hkv,
                       N, Np, scale * kLog2e, scale);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_dq(const void* q, const void* k, const void* v, const void* dO, const float* ws, void* dq,
                            int B, int Hq, int Hkv, int N, float scale, hipStream_t st) {
    using Cfg = QBf16Tuned<D>;
    const int nmb = (N + Cfg::BM - 1) / Cfg::BM;
    const int Np = ws_rows(N);
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, CAUSAL, Cfg>), dim3((unsigned)((int64_t)nmb * Hq * B)),
                       dim3(Cfg::kThreads), 0, st, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)dO, ws, ws + (int64_t)B * Hq * Np, (uint16_t*)dq, Hq, Hkv, N, Np,
                       scale * kLog2e, scale);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(int d, int causal, const void* q, const void* k, const void* v, const void* dO,
                                const float* ws, void* dk, void* dv, int B, int Hq, int Hkv, int N, float scale,
                                hipStream_t st) {
#define ARGS q, k, v, dO, ws, dk, dv, B, Hq, Hkv, N, scale, st
    if (d == 64) return causal ? launch_dkdv<64, true>(ARGS) : launch_dkdv<64, false>(ARGS);
    if (d == 128) return causal ? launch_dkdv<128, true>(ARGS) : launch_dkdv<128, false>(ARGS);
#undef ARGS
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_bf16(int d, int causal, const void* q, const void* k, const void* v, const void* dO,
                              const float* ws, void* dq, int B, int Hq, int Hkv, int N, float scale, hipStream_t st) {
#define ARGS q, k, v, dO, ws, dq, B, Hq, Hkv, N, scale, st
    if (d == 64) return causal ? launch_dq<64, true>(ARGS) : launch_dq<64, false>(ARGS);
    if (d == 128) return causal ? launch_dq<128, true>(ARGS) : launch_dq<128, false>(ARGS);
#undef ARGS
    return hipErrorInvalidValue;
}

}  // namespace fa
