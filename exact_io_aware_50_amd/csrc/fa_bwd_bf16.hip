// bf16 backward pass (the tuned path; float32 uses the generic kernels in
// fa_bwd.hip).  Same arithmetic as there; what changes is the mapping onto
// gfx950: Q/dO (dK/dV kernel) and K/V (dQ kernel) tiles go from HBM straight
// into LDS in row-major layout, and every transposed operand (Q^T, dO^T, K^T)
// is read with transposing LDS reads, so no tile is ever transposed through
// registers.  Probabilities and dS are packed to bf16 by the hardware
// converter.
//
// FlashAttention legal glossary, backward paragraph and entry "Recomputation"
// (P is recomputed from Q, K and the stored statistics), FlashAttention-2
// paragraph (the dK/dV pass is parallel over key blocks, without atomics).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

// ------------------------------------------------------------ dK, dV
template <int D>
struct KVBf16Cfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BNK = 32 * kWaves;     // keys per workgroup (32 per wave)
    static constexpr int BMQ = 32;              // query rows per step
    using QT = LdsTile<BMQ, D, kWaves>;
    static constexpr int kStage = 2 * QT::kElems;   // Q and dO
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Hq, int Hkv, int N, float c2, float scale) {
    using Cfg = KVBf16Cfg<D>;
    using QT = typename Cfg::QT;
    constexpr int BNK = Cfg::BNK, BMQ = Cfg::BMQ;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * Cfg::kStage];
    __shared__ __attribute__((aligned(16))) float sstat[2][2][BMQ];   // [stage][lse*log2e | D][row]

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

    auto base_of = [&](int it, int& q0) {
        const int hq = g * G + it / per_head;
        q0 = (qt0 + it % per_head) * BMQ;
        return ((int64_t)b * Hq + hq) * N + q0;
    };
    float st_l = 0.f, st_d = 0.f;
    auto fetch = [&](int it, int stage) {
        int q0;
        const int64_t base = base_of(it, q0);
        uint16_t* s = smem + stage * Cfg::kStage;
        QT::load(Q + base * D, N - q0, s, wave, lane);
        QT::load(dO + base * D, N - q0, s + QT::kElems, wave, lane);
        if (tid < BMQ) {
            const bool ok = q0 + tid < N;
            st_l = ok ? LSE[base + tid] * kLog2e : INFINITY;
            st_d = ok ? Dl[base + tid] : 0.f;
        }
    };
    auto put_stats = [&](int stage) {
        if (tid < BMQ) {
            sstat[stage][0][tid] = st_l;
            sstat[stage][1][tid] = st_d;
        }
    };

    fetch(0, 0);
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
    f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        dkacc[i] = zero16();
        dvacc[i] = zero16();
    }
    put_stats(0);
    wait_dma();
    __syncthreads();

    for (int it = 0; it < total; ++it) {
        int q0;
        base_of(it, q0);
        const int stg = it & 1;
        if (it + 1 < total) fetch(it + 1, stg ^ 1);
        const uint16_t* Qs = smem + stg * Cfg::kStage;
        const uint16_t* dOs = Qs + QT::kElems;

        if (!(CAUSAL && q0 + BMQ - 1 < kw)) {
            // S = Q K^T and dP = dO V^T: rows = queries, columns = this wave's keys
            f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                sacc = mma_bf16(QT::row8(Qs, l32, 2 * s + hh), kf[s], sacc);
                dpacc = mma_bf16(QT::row8(dOs, l32, 2 * s + hh), vf[s], dpacc);
            }
            const bool need_mask = CAUSAL && kw + 31 > q0;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int rb = 8 * gq + 4 * hh;
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sstat[stg][0][rb]);
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sstat[stg][1][rb]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 4 * gq + j;
                    float p = fast_exp2(fmaf(sacc[r], c2, -l4[j]));
                    if (need_mask && krow > q0 + rb + j) p = 0.f;
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
                    dvacc[ct] = mma_bf16(QT::tr8(dOs, 16 * t, 32 * ct, lane), pb, dvacc[ct]);
                    dkacc[ct] = mma_bf16(QT::tr8(Qs, 16 * t, 32 * ct, lane), sb, dkacc[ct]);
                }
            }
        }
        if (it + 1 < total) put_stats(stg ^ 1);
        wait_dma();
        __syncthreads();
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
template <int D>
struct QBf16Cfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BM = 32 * kWaves;      // query rows per workgroup
    static constexpr int BNK = 64;              // keys per tile
    using KT = LdsTile<BNK, D, kWaves>;   // read as rows and transposed
    using VT = LdsTile<BNK, D, kWaves>;  // read as rows
    static constexpr int kStage = KT::kElems + VT::kElems;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    uint16_t* __restrict__ dQ, int Hq, int Hkv, int N, float c2, float scale) {
    using Cfg = QBf16Cfg<D>;
    using KT = typename Cfg::KT;
    using VT = typename Cfg::VT;
    constexpr int BM = Cfg::BM, BNK = Cfg::BNK;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * Cfg::kStage];

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

    KT::load(Kg, N, smem, wave, lane);
    VT::load(Vg, N, smem + KT::kElems, wave, lane);

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
    const float lse2 = qrow < N ? LSE[rowbase + qrow] * kLog2e : INFINITY;
    const float dq_d = qrow < N ? Dl[rowbase + qrow] : 0.f;

    f32x16 dqacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) dqacc[i] = zero16();
    wait_dma();
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
        const int k0 = j * BNK;
        if (j + 1 < ntiles) {
            uint16_t* nxt = smem + ((j + 1) & 1) * Cfg::kStage;
            KT::load(Kg + (int64_t)(k0 + BNK) * D, N - (k0 + BNK), nxt, wave, lane);
            VT::load(Vg + (int64_t)(k0 + BNK) * D, N - (k0 + BNK), nxt + KT::kElems, wave, lane);
        }
        const uint16_t* Ks = smem + (j & 1) * Cfg::kStage;
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
            const bool need_mask = (CAUSAL && k0 + BNK - 1 > qw) || (k0 + BNK > N);
#pragma unroll
            for (int kb = 0; kb < BNK / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p = fast_exp2(fmaf(sacc[kb][r], c2, -lse2));
                    if (need_mask) {
                        const int key = k0 + 32 * kb + acc_row(r, hh);
                        if ((CAUSAL && key > qrow) || key >= N) p = 0.f;
                    }
                    dpacc[kb][r] = p * (dpacc[kb][r] - dq_d);
                }
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
        wait_dma();
        __syncthreads();
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
static hipError_t launch_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                              const float* delta, void* dk, void* dv, int B, int Hq, int Hkv, int N, float scale,
                              hipStream_t st) {
    using Cfg = KVBf16Cfg<D>;
    const int nkb = (N + Cfg::BNK - 1) / Cfg::BNK;
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)nkb * Hkv * B)),
                       dim3(Cfg::kThreads), 0, st, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)dO, lse, delta, (uint16_t*)dk, (uint16_t*)dv, Hq, Hkv, N, scale * kLog2e,
                       scale);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                            const float* delta, void* dq, int B, int Hq, int Hkv, int N, float scale,
                            hipStream_t st) {
    using Cfg = QBf16Cfg<D>;
    const int nmb = (N + Cfg::BM - 1) / Cfg::BM;
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)nmb * Hq * B)),
                       dim3(Cfg::kThreads), 0, st, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)dO, lse, delta, (uint16_t*)dq, Hq, Hkv, N, scale * kLog2e, scale);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(int d, int causal, const void* q, const void* k, const void* v, const void* dO,
                                const float* lse, const float* delta, void* dk, void* dv, int B, int Hq, int Hkv,
                                int N, float scale, hipStream_t st) {
#define ARGS q, k, v, dO, lse, delta, dk, dv, B, Hq, Hkv, N, scale, st
    if (d == 64) return causal ? launch_dkdv<64, true>(ARGS) : launch_dkdv<64, false>(ARGS);
    if (d == 128) return causal ? launch_dkdv<128, true>(ARGS) : launch_dkdv<128, false>(ARGS);
#undef ARGS
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_bf16(int d, int causal, const void* q, const void* k, const void* v, const void* dO,
                              const float* lse, const float* delta, void* dq, int B, int Hq, int Hkv, int N,
                              float scale, hipStream_t st) {
#define ARGS q, k, v, dO, lse, delta, dq, B, Hq, Hkv, N, scale, st
    if (d == 64) return causal ? launch_dq<64, true>(ARGS) : launch_dq<64, false>(ARGS);
    if (d == 128) return causal ? launch_dq<128, true>(ARGS) : launch_dq<128, false>(ARGS);
#undef ARGS
    return hipErrorInvalidValue;
}

}  // namespace fa
