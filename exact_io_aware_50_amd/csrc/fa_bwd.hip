// Backward pass of exact attention by recomputation (generic kernels, used for
// float32; bf16 dK/dV and dQ run the tuned kernels in fa_bwd_bf16.hip).
//
// The FlashAttention legal glossary (backward paragraph, entry
// "Recomputation"): the forward keeps only the softmax statistics; the
// backward recomputes the scores and probabilities on chip from Q, K and
// those statistics instead of reading an N x N matrix.  Its FlashAttention-2
// paragraph: the backward is parallel over the column (key) dimension, which
// removes atomic adds.  Per query row i and key j, with LSE from the forward:
//   P_ij = exp(scale q_i.k_j - LSE_i),  dP_ij = dO_i.v_j,
//   D_i = sum_c dO_ic O_ic,  dS_ij = P_ij (dP_ij - D_i),
//   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,  dQ_i = scale sum_j dS_ij k_j.
// Three kernels: D (one pass over O and dO), dK/dV (a workgroup per key block
// of a K/V head, looping over the query heads of its group and all query
// blocks; no atomics), and dQ (a workgroup per query block of a query head).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

// ------------------------------------------------------------ workspace: D, LSE*log2e
// Row r of the padded [B*Hq][Np] layout: -D * keep with D = sum_c dO*O, and
// LSE*log2(e), for query rows < N; 0 and +infinity (zero probability) for
// padding rows.  -D rather than D: the bf16 dK/dV kernel starts its dP
// accumulators from it.  keep is 1, or 1 - p for the backward through dropout.
// A thread takes 8 columns of kDeltaRows rows (a workgroup, kDeltaRows runs
// of 256/(D/8) rows) and issues all their loads before the arithmetic: more
// bytes in flight per thread (7% faster than one row per thread).
constexpr int kDeltaRows = 2;

template <class ET, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const typename ET::elem* __restrict__ O,
                                                        const typename ET::elem* __restrict__ dO,
                                                        const float* __restrict__ LSE, float* __restrict__ WSd,
                                                        float* __restrict__ WSl, int N, int Np, int64_t rows,
                                                        float keep) {
    constexpr int TPR = D / 8, RPB = 256 / TPR, R = kDeltaRows;
    const int seg = threadIdx.x % TPR;
    typename ET::raw8 a[R], d[R];
    int64_t rowv[R];
    bool validv[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int64_t row = ((int64_t)blockIdx.x * R + j) * RPB + threadIdx.x / TPR;
        const int64_t bh = row / Np;
        const int i = (int)(row - bh * Np);
        const bool valid = row < rows && i < N;
        rowv[j] = row;
        validv[j] = valid;
        a[j] = d[j] = typename ET::raw8{};
        if (valid) {
            const int64_t src = (bh * N + i) * D + seg * 8;
            a[j] = ld8<ET>(O + src);
            d[j] = ld8<ET>(dO + src);
        }
    }
#pragma unroll
    for (int j = 0; j < R; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(ET::to_f32(a[j], e), ET::to_f32(d[j], e), acc);
#pragma unroll
        for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
        const int64_t row = rowv[j];
        if (seg == 0 && row < rows) {
            const int64_t bh = row / Np;
            const int i = (int)(row - bh * Np);
            WSd[row] = -acc * keep;
            WSl[row] = validv[j] ? LSE[bh * N + i] * kLog2e : INFINITY;
        }
    }
}

// ------------------------------------------------------------ dK, dV
template <class ET, int D>
struct KVCfg {
    static constexpr int kThreads = 256;
    static constexpr int BNK = 128;                          // keys per workgroup (32 per wave)
    static constexpr int BMQ = ET::kBytes == 2 ? 64 : 32;    // query rows per step
    using QTile = NatTile<ET, BMQ, D, kThreads>;
    using QtTile = TrTile<ET, BMQ, D, kThreads>;
    static constexpr int kStage = 2 * QTile::kElems + 2 * QtTile::kElems;
};

template <class ET, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(
    const typename ET::elem* __restrict__ Q, const typename ET::elem* __restrict__ K,
    const typename ET::elem* __restrict__ V, const typename ET::elem* __restrict__ dO,
    const float* __restrict__ WSd, const float* __restrict__ WSl,
    typename ET::elem* __restrict__ dK, typename ET::elem* __restrict__ dV,
    int Hq, int Hkv, int N, int Np, float c2, float scale) {
    using Cfg = KVCfg<ET, D>;
    using elem = typename ET::elem;
    using raw8 = typename ET::raw8;
    constexpr int BNK = Cfg::BNK, BMQ = Cfg::BMQ;
    constexpr int QS = Cfg::QTile::kStride, QTS = Cfg::QtTile::kStride;
    constexpr int kNat = Cfg::QTile::kElems, kTr = Cfg::QtTile::kElems;
    __shared__ __attribute__((aligned(64))) elem smem[2 * Cfg::kStage];
    __shared__ __attribute__((aligned(16))) float sstat[2][2][BMQ];   // [stage][lse2 | D][row]

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

    const elem* Kg = K + ((int64_t)b * Hkv + g) * N * D;
    const elem* Vg = V + ((int64_t)b * Hkv + g) * N * D;

    raw8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        raw8 a = {}, c = {};
        if (krow < N) {
            a = ld8<ET>(Kg + (int64_t)krow * D + 16 * s + 8 * hh);
            c = ld8<ET>(Vg + (int64_t)krow * D + 16 * s + 8 * hh);
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

    const int nqt = (N + BMQ - 1) / BMQ;
    const int qt0 = CAUSAL ? k0 / BMQ : 0;          // earlier query blocks see none of these keys
    const int per_head = nqt - qt0;
    const int total = G * per_head;

    typename Cfg::QTile q_nat, o_nat;
    typename Cfg::QtTile q_tr, o_tr;
    float st_l = 0.f, st_d = 0.f;

    auto fetch = [&](int it) {
        const int hq = g * G + it / per_head;
        const int q0 = (qt0 + it % per_head) * BMQ;
        const int64_t base = (((int64_t)b * Hq + hq) * N + q0);
        q_nat.load(Q + base * D, N - q0, tid);
        q_tr.load(Q + base * D, N - q0, tid);
        o_nat.load(dO + base * D, N - q0, tid);
        o_tr.load(dO + base * D, N - q0, tid);
        if (tid < BMQ) {
            // padded workspace rows (>= N) hold +inf and 0
            const int64_t srow = ((int64_t)b * Hq + hq) * Np + q0 + tid;
            st_l = WSl[srow];
            st_d = WSd[srow];
        }
    };
    auto put = [&](int stage) {
        elem* s = smem + stage * Cfg::kStage;
        q_nat.store(s, tid);
        o_nat.store(s + kNat, tid);
        q_tr.store(s + 2 * kNat, tid);
        o_tr.store(s + 2 * kNat + kTr, tid);
        if (tid < BMQ) {
            sstat[stage][0][tid] = st_l;
            sstat[stage][1][tid] = st_d;
        }
    };

    if (total > 0) {
        fetch(0);
        put(0);
    }
    __syncthreads();

    for (int it = 0; it < total; ++it) {
        const int q0 = (qt0 + it % per_head) * BMQ;
        const bool more = it + 1 < total;
        if (more) fetch(it + 1);
        const int stg = it & 1;
        const elem* Qs = smem + stg * Cfg::kStage;
        const elem* dOs = Qs + kNat;
        const elem* Qt = Qs + 2 * kNat;
        const elem* dOt = Qt + kTr;

        if (!(CAUSAL && q0 + BMQ - 1 < kw)) {
            f32x16 sacc[BMQ / 32], dpacc[BMQ / 32];
#pragma unroll
            for (int qb = 0; qb < BMQ / 32; ++qb) {
                f32x16 s_ = zero16(), p_ = zero16();
#pragma unroll
                for (int s = 0; s < D / 16; ++s) {
                    s_ = ET::mma(ld8<ET>(Qs + (32 * qb + l32) * QS + 16 * s + 8 * hh), kf[s], s_);
                    p_ = ET::mma(ld8<ET>(dOs + (32 * qb + l32) * QS + 16 * s + 8 * hh), vf[s], p_);
                }
                sacc[qb] = s_;
                dpacc[qb] = p_;
            }
            const bool need_mask = CAUSAL && kw + 31 > q0;
#pragma unroll
            for (int qb = 0; qb < BMQ / 32; ++qb)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int rb = 32 * qb + 8 * gq + 4 * hh;
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sstat[stg][0][rb]);
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sstat[stg][1][rb]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 4 * gq + j;
                        float p = fast_exp2(fmaf(sacc[qb][r], c2, -l4[j]));
                        if (need_mask && krow > q0 + rb + j) p = 0.f;
                        sacc[qb][r] = p;
                        dpacc[qb][r] = p * (dpacc[qb][r] + d4[j]);     // d4 = -D
                    }
                }
            // dV^T += dO^T P ;  dK^T += Q^T dS
#pragma unroll
            for (int qb = 0; qb < BMQ / 32; ++qb)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const raw8 pb = ET::pack8(sacc[qb], 8 * t);
                    const raw8 sb = ET::pack8(dpacc[qb], 8 * t);
#pragma unroll
                    for (int ct = 0; ct < D / 32; ++ct) {
                        const int off = (32 * ct + l32) * QTS + 32 * qb + 16 * t + 8 * hh;
                        dvacc[ct] = ET::mma(ld8<ET>(dOt + off), pb, dvacc[ct]);
                        dkacc[ct] = ET::mma(ld8<ET>(Qt + off), sb, dkacc[ct]);
                    }
                }
        }
        if (more) put(stg ^ 1);
        __syncthreads();
    }

    if (krow < N) {
        elem* dKr = dK + (((int64_t)b * Hkv + g) * N + krow) * D;
        elem* dVr = dV + (((int64_t)b * Hkv + g) * N + krow) * D;
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int c = 32 * ct + 8 * gq + 4 * hh;
                st4<ET>(dKr + c, ET::pack4(dkacc[ct][4 * gq] * scale, dkacc[ct][4 * gq + 1] * scale,
                                           dkacc[ct][4 * gq + 2] * scale, dkacc[ct][4 * gq + 3] * scale));
                st4<ET>(dVr + c, ET::pack4(dvacc[ct][4 * gq], dvacc[ct][4 * gq + 1],
                                           dvacc[ct][4 * gq + 2], dvacc[ct][4 * gq + 3]));
            }
    }
}

// ------------------------------------------------------------ dQ
template <class ET, int D>
struct QCfg {
    static constexpr int kThreads = 256;
    static constexpr int BM = 128;                           // query rows per workgroup
    static constexpr int BNK = ET::kBytes == 2 ? 64 : 32;    // keys per tile
    using KTile = NatTile<ET, BNK, D, kThreads>;
    using KtTile = TrTile<ET, BNK, D, kThreads>;
    static constexpr int kStage = 2 * KTile::kElems + KtTile::kElems;
};

template <class ET, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dq_kernel(
    const typename ET::elem* __restrict__ Q, const typename ET::elem* __restrict__ K,
    const typename ET::elem* __restrict__ V, const typename ET::elem* __restrict__ dO,
    const float* __restrict__ WSd, const float* __restrict__ WSl, typename ET::elem* __restrict__ dQ,
    int Hq, int Hkv, int N, int Np, float c2, float scale) {
    using Cfg = QCfg<ET, D>;
    using elem = typename ET::elem;
    using raw8 = typename ET::raw8;
    constexpr int BM = Cfg::BM, BNK = Cfg::BNK;
    constexpr int KS = Cfg::KTile::kStride, KTS = Cfg::KtTile::kStride;
    constexpr int kNat = Cfg::KTile::kElems;
    __shared__ __attribute__((aligned(64))) elem smem[2 * Cfg::kStage];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;

    const int nmb = (N + BM - 1) / BM;
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    const int mbi = lin % nmb, bh = lin / nmb;
    const int h = bh % Hq, b = bh / Hq;
    const int mb = CAUSAL ? nmb - 1 - mbi : mbi;
    const int g = h / (Hq / Hkv);
    const int64_t rowbase = ((int64_t)b * Hq + h) * N;
    const elem* Kg = K + ((int64_t)b * Hkv + g) * N * D;
    const elem* Vg = V + ((int64_t)b * Hkv + g) * N * D;

    const int q0 = mb * BM;
    const int qw = q0 + 32 * wave;
    const int qrow = qw + l32;

    raw8 qf[D / 16], of[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        raw8 a = {}, c = {};
        if (qrow < N) {
            a = ld8<ET>(Q + (rowbase + qrow) * D + 16 * s + 8 * hh);
            c = ld8<ET>(dO + (rowbase + qrow) * D + 16 * s + 8 * hh);
        }
        qf[s] = a;
        of[s] = c;
    }
    const int64_t srow = ((int64_t)b * Hq + h) * Np + qrow;
    const float lse2 = qrow < N ? WSl[srow] : INFINITY;
    const float dq_nd = qrow < N ? WSd[srow] : 0.f;     // the workspace holds -D

    f32x16 dqacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) dqacc[i] = zero16();

    const int kend = CAUSAL ? min(N, q0 + BM) : N;
    const int ntiles = (kend + BNK - 1) / BNK;

    typename Cfg::KTile k_nat, v_nat;
    typename Cfg::KtTile k_tr;
    k_nat.load(Kg, N, tid);
    v_nat.load(Vg, N, tid);
    k_tr.load(Kg, N, tid);
    k_nat.store(smem, tid);
    v_nat.store(smem + kNat, tid);
    k_tr.store(smem + 2 * kNat, tid);
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
        const int k0 = j * BNK;
        const bool more = j + 1 < ntiles;
        if (more) {
            const int64_t nb = (int64_t)(k0 + BNK) * D;
            k_nat.load(Kg + nb, N - (k0 + BNK), tid);
            v_nat.load(Vg + nb, N - (k0 + BNK), tid);
            k_tr.load(Kg + nb, N - (k0 + BNK), tid);
        }
        const elem* Ks = smem + (j & 1) * Cfg::kStage;
        const elem* Vs = Ks + kNat;
        const elem* Kt = Ks + 2 * kNat;

        if (!(CAUSAL && k0 > qw + 31)) {
            f32x16 sacc[BNK / 32], dpacc[BNK / 32];
#pragma unroll
            for (int kb = 0; kb < BNK / 32; ++kb) {
                f32x16 s_ = zero16(), p_ = zero16();
#pragma unroll
                for (int s = 0; s < D / 16; ++s) {
                    s_ = ET::mma(ld8<ET>(Ks + (32 * kb + l32) * KS + 16 * s + 8 * hh), qf[s], s_);
                    p_ = ET::mma(ld8<ET>(Vs + (32 * kb + l32) * KS + 16 * s + 8 * hh), of[s], p_);
                }
                sacc[kb] = s_;
                dpacc[kb] = p_;
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
                    dpacc[kb][r] = p * (dpacc[kb][r] + dq_nd);
                }
            // dQ^T += K^T dS^T
#pragma unroll
            for (int kb = 0; kb < BNK / 32; ++kb)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const raw8 sb = ET::pack8(dpacc[kb], 8 * t);
#pragma unroll
                    for (int ct = 0; ct < D / 32; ++ct)
                        dqacc[ct] = ET::mma(ld8<ET>(Kt + (32 * ct + l32) * KTS + 32 * kb + 16 * t + 8 * hh),
                                            sb, dqacc[ct]);
                }
        }
        if (more) {
            elem* nxt = smem + ((j + 1) & 1) * Cfg::kStage;
            k_nat.store(nxt, tid);
            v_nat.store(nxt + kNat, tid);
            k_tr.store(nxt + 2 * kNat, tid);
        }
        __syncthreads();
    }

    if (qrow < N) {
        elem* dQr = dQ + (rowbase + qrow) * D;
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
                st4<ET>(dQr + 32 * ct + 8 * gq + 4 * hh,
                        ET::pack4(dqacc[ct][4 * gq] * scale, dqacc[ct][4 * gq + 1] * scale,
                                  dqacc[ct][4 * gq + 2] * scale, dqacc[ct][4 * gq + 3] * scale));
    }
}

template <class ET, int D>
static hipError_t launch_delta(const void* o, const void* dO, const float* lse, float* ws, int B, int Hq, int N,
                               float keep, hipStream_t st) {
    using elem = typename ET::elem;
    const int Np = ws_rows(N);
    const int64_t rows = (int64_t)B * Hq * Np;
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((bwd_delta_kernel<ET, D>), dim3((unsigned)((rows + RPB * kDeltaRows - 1) / (RPB * kDeltaRows))),
                       dim3(256), 0, st,
                       (const elem*)o, (const elem*)dO, lse, ws, ws + rows, N, Np, rows, keep);
    return hipGetLastError();
}

template <class ET, int D, bool CAUSAL>
static hipError_t launch_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* ws,
                              void* dk, void* dv, int B, int Hq, int Hkv, int N, float scale, hipStream_t st) {
    using elem = typename ET::elem;
    const int nkb = (N + KVCfg<ET, D>::BNK - 1) / KVCfg<ET, D>::BNK;
    const int Np = ws_rows(N);
    hipLaunchKernelGGL((bwd_dkdv_kernel<ET, D, CAUSAL>), dim3((unsigned)((int64_t)nkb * Hkv * B)), dim3(256), 0,
                       st, (const elem*)q, (const elem*)k, (const elem*)v, (const elem*)dO, ws,
                       ws + (int64_t)B * Hq * Np, (elem*)dk, (elem*)dv, Hq, Hkv, N, Np, scale * kLog2e, scale);
    return hipGetLastError();
}

template <class ET, int D, bool CAUSAL>
static hipError_t launch_dq(const void* q, const void* k, const void* v, const void* dO, const float* ws, void* dq,
                            int B, int Hq, int Hkv, int N, float scale, hipStream_t st) {
    using elem = typename ET::elem;
    const int nmb = (N + QCfg<ET, D>::BM - 1) / QCfg<ET, D>::BM;
    const int Np = ws_rows(N);
    hipLaunchKernelGGL((bwd_dq_kernel<ET, D, CAUSAL>), dim3((unsigned)((int64_t)nmb * Hq * B)), dim3(256), 0, st,
                       (const elem*)q, (const elem*)k, (const elem*)v, (const elem*)dO, ws,
                       ws + (int64_t)B * Hq * Np, (elem*)dq, Hq, Hkv, N, Np, scale * kLog2e, scale);
    return hipGetLastError();
}

hipError_t launch_bwd_delta(int dtype, int d, const void* o, const void* dO, const float* lse, float* ws, int B,
                            int Hq, int N, hipStream_t st, float keep) {
    if (dtype == 1 && d == 64) return launch_delta<BF16, 64>(o, dO, lse, ws, B, Hq, N, keep, st);
    if (dtype == 1 && d == 128) return launch_delta<BF16, 128>(o, dO, lse, ws, B, Hq, N, keep, st);
    if (dtype == 0 && d == 64) return launch_delta<F32, 64>(o, dO, lse, ws, B, Hq, N, keep, st);
    if (dtype == 0 && d == 128) return launch_delta<F32, 128>(o, dO, lse, ws, B, Hq, N, keep, st);
    return hipErrorInvalidValue;
}

#define FA_DISPATCH(FN, ...)                                                                                  \
    if (dtype == 0 && d == 64) return causal ? FN<F32, 64, true>(__VA_ARGS__) : FN<F32, 64, false>(__VA_ARGS__);     \
    if (dtype == 0 && d == 128) return causal ? FN<F32, 128, true>(__VA_ARGS__) : FN<F32, 128, false>(__VA_ARGS__);  \
    return hipErrorInvalidValue;

hipError_t launch_bwd_dkdv(int dtype, int d, int causal, const void* q, const void* k, const void* v,
                           const void* dO, const float* ws, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                           float scale, hipStream_t st) {
    if (dtype == 1) return launch_bwd_dkdv_bf16(d, causal, q, k, v, dO, ws, dk, dv, B, Hq, Hkv, N, scale, st);
    FA_DISPATCH(launch_dkdv, q, k, v, dO, ws, dk, dv, B, Hq, Hkv, N, scale, st)
}

hipError_t launch_bwd_dq(int dtype, int d, int causal, const void* q, const void* k, const void* v,
                         const void* dO, const float* ws, void* dq, int B, int Hq, int Hkv, int N, float scale,
                         hipStream_t st) {
    if (dtype == 1) return launch_bwd_dq_bf16(d, causal, q, k, v, dO, ws, dq, B, Hq, Hkv, N, scale, st);
    FA_DISPATCH(launch_dq, q, k, v, dO, ws, dq, B, Hq, Hkv, N, scale, st)
}
#undef FA_DISPATCH

}  // namespace fa
