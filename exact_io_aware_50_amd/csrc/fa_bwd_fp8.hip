// FP8 (OCP E4M3) backward pass, d = 128: the backward of the fp8 forward.
//
// The FlashAttention legal glossary (FlashAttention-3 paragraph) and "flash
// attention io aware" (section "Flash Attention 2 and 3") name FP8 attention
// on the low-precision matrix units but give no recipe, and no backward.  The
// recipe here (the fp8 forward's, carried through the recomputation of the
// glossary's backward paragraph):
//  - Q, K, V and dO are E4M3 codes with one descale per tensor (real value =
//    code * s_X, from fa_quantize_fp8); O (bf16) and LSE are the fp8
//    forward's outputs;
//  - the two products over the head dimension, S = Q K^T and dP = dO V^T, run
//    on the fp8 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4), float32
//    accumulation;
//  - D = rowsum(dO o O) in float32; the workspace holds -D / (s_dO s_V), the
//    dP accumulators start from it, and every descale goes into the final
//    scales;
//  - dQ = scale dS K on the fp8 matrix cores: dS is rounded to E4M3 after a
//    power-of-two scale chosen per query and block of 32 keys (the block's
//    largest |dS| lands in [128, 256)), which the matrix core divides back out
//    as the block scale of its B operand (one E8M0 exponent per block of 32
//    contraction slots of a column);
//  - dK = scale dS^T Q and dV = P^T dO on the bf16 matrix cores with P and dS
//    rounded to bf16 (as the bf16 backward) and the E4M3 codes of Q and dO
//    widened to bf16, which holds every E4M3 value exactly.
// Work partition, schedules and data paths are those of the bf16 kernels
// (fa_bwd_bf16.hip): dK/dV column-parallel without atomics, dQ row-parallel,
// ping-pong wave groups, direct global -> LDS loads, persistent workgroups.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

__device__ __forceinline__ f32x16 mma_fp8s(const u32x8& a, const u32x8& b, f32x16 c, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b),
                                                           c, 0, 0,        // A and B are E4M3
                                                           0, 127,         // A block scale 2^0
                                                           0, scale_b);    // B block scale (E8M0) per lane
}

// Four E4M3 codes (bytes of w) -> two words of two bf16 each, exactly.
__device__ __forceinline__ u32x2 widen4(uint32_t w) {
    u32x2 r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true));
    return r;
}

// A tile of E4M3 rows of 128 bytes, in the row-group LDS layout of LdsTile
// (addressed in 16-bit units: 64 per row).
template <int ROWS, int NW>
using Fp8Rows = LdsTile<ROWS, 64, NW>;

// 32 bytes of row r (bytes 16 c .. 16 c + 31): an fp8 operand fragment.
template <class T>
__device__ __forceinline__ u32x8 row32(const uint16_t* tile, int r, int c) {
    const u32x4 lo = T::row8(tile, r, c), hi = T::row8(tile, r, c + 1);
    return u32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Transposed bf16 operand fragment from an E4M3 row tile: this lane gets
// column n0 + lane % 32 (bytes) for the rows kk + swap23(8 hh + e), e = 0..7
// (the "accumulator as operand" order of fa_device.hpp), widened to bf16.
// ds_read_b64_tr_b8: inside each 16-lane group, output lane i, byte j is byte
// i % 8 of what source lane 2 j + i / 8 read, so source lane t = 2 j + p reads
// row kk + swap23(8 hh + j), bytes n0 + 16 half + 8 p .. + 7.
template <class T>
__device__ __forceinline__ u32x4 tr_fp8_bf16(const uint16_t* tile, int kk, int n0, int lane) {
    const int hh = lane >> 5, half = (lane >> 4) & 1, t = lane & 15;
    const int row = kk + swap23(8 * hh + (t >> 1));
    const int col = n0 + 16 * half + 8 * (t & 1);
    const char* a = (const char*)tile + T::off(row, col >> 4) + (col & 15);
    const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(__attribute__((address_space(3))) char*)a);
    const u32x2 lo = widen4((uint32_t)w[0]), hi = widen4((uint32_t)w[1]);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// ------------------------------------------------------------ workspace: -D / (s_dO s_V), LSE*log2e
// Row r of the padded [B*Hq][Np] layout, as the bf16 delta kernel: padding
// rows hold 0 and +infinity.  D / (s_dO s_V) = sum_c dO8_c O_c / s_V.
__global__ __launch_bounds__(256) void bwd_delta_fp8_kernel(const uint16_t* __restrict__ O,
                                                          const uint8_t* __restrict__ dO,
                                                          const float* __restrict__ LSE,
                                                          const float* __restrict__ descale,
                                                          float* __restrict__ WSd, float* __restrict__ WSl, int N,
                                                          int Np, int64_t rows) {
    constexpr int D = 128, TPR = D / 8, RPB = 256 / TPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int seg = threadIdx.x % TPR;
    const int64_t bh = row / Np;
    const int i = (int)(row - bh * Np);
    const bool valid = row < rows && i < N;
    float acc = 0.f;
    if (valid) {
        const int64_t src = (bh * N + i) * D + seg * 8;
        const u32x4 o = *reinterpret_cast<const u32x4*>(O + src);
        const u32x2 d8 = *reinterpret_cast<const u32x2*>(dO + src);
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const float dv[4] = {__builtin_amdgcn_cvt_f32_fp8((int)d8[w], 0), __builtin_amdgcn_cvt_f32_fp8((int)d8[w], 1),
                                 __builtin_amdgcn_cvt_f32_fp8((int)d8[w], 2), __builtin_amdgcn_cvt_f32_fp8((int)d8[w], 3)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t ow = o[2 * w + (e >> 1)];
                acc = fmaf(dv[e], __uint_as_float(e & 1 ? (ow & 0xffff0000u) : (ow << 16)), acc);
            }
        }
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (seg == 0 && row < rows) {
        WSd[row] = -acc / descale[2];
        WSl[row] = valid ? LSE[bh * N + i] * kLog2e : INFINITY;
    }
}

// ------------------------------------------------------------ dK, dV
//
// As bwd_dkdv_bf16_kernel<128>: a workgroup holds 256 keys (32 per wave), walks
// the steps (query head of the group, block of 32 queries), waves w and w+4
// share a SIMD and alternate
//   G(i): dV^T += dO_{i-1}^T P_{i-1}, dK^T += Q_{i-1}^T dS_{i-1} (bf16, the
//         E4M3 rows widened), then S_i = Q_i K^T and dP_i = dO_i V^T (fp8)
//   X(i): P_i = exp2(c2 s - LSE log2 e), causal mask, dS_i = P_i (dP_i - D), pack
// The wave's 32 K and V rows stay in registers as fp8 operands (no V tile).
struct KVFp8Cfg {
    static constexpr int D = 128;
    static constexpr int kWaves = 8;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BNK = 32 * kWaves;             // keys per workgroup
    static constexpr int BMQ = 32;                      // query rows per step
    static constexpr int kStages = 4;
    using QT = Fp8Rows<BMQ, 4>;                         // 4 row groups: waves 0-3 load Q, 4-7 dO
    static constexpr int kStatChunks = BMQ / 2;         // 16-byte chunks of (LSE*log2e, -D) per step
    static constexpr int kStatPerWave = kStatChunks / kWaves;
    static constexpr int kStatBytes = 8 * BMQ;
    static constexpr int kStageBytes = 2 * QT::kBytes + kStatBytes;
    static constexpr int kLdsBytes = kStages * kStageBytes;
    static constexpr int kLoads = 2;                    // direct loads per wave per step
};

template <bool CAUSAL>
__global__ __launch_bounds__(KVFp8Cfg::kThreads, 2) void bwd_dkdv_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const uint8_t* __restrict__ dO, const float* __restrict__ WSd, const float* __restrict__ WSl,
    const float* __restrict__ descale, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int B, int Hq, int Hkv,
    int n_rows, int Npad, float scale) {
    using Cfg = KVFp8Cfg;
    using QT = Cfg::QT;
    constexpr int D = Cfg::D, NW = Cfg::kWaves, BNK = Cfg::BNK, BMQ = Cfg::BMQ, NS = Cfg::kStages;
    constexpr int kLoads = Cfg::kLoads;
    __shared__ __attribute__((aligned(1024))) char smem[Cfg::kLdsBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int grp = wave >> 2;
    const float c2 = scale * kLog2e * descale[0] * descale[1];        // scores are Q8 K8^T s_Q s_K
    const float sk = scale * descale[0] * descale[3] * descale[2];    // dK: scale s_Q s_dO s_V
    const float sv = descale[3];                                      // dV: s_dO

    const int nkb = (n_rows + BNK - 1) / BNK;
    const PersistentSched sched(nkb * Hkv * B);
    for (int r = 0; sched.more(r); ++r) {
        const int lin = sched.item(r);
        if (lin < 0) continue;
        int N = n_rows;
        asm volatile("" : "+s"(N));
        const int kbk = lin % nkb, bg = lin / nkb;
        const int g = bg % Hkv, b = bg / Hkv;
        const int G = Hq / Hkv;
        const int k0 = kbk * BNK;
        const int kw = k0 + 32 * wave;
        const int krow = kw + l32;
        const uint8_t* Kg = K + ((int64_t)b * Hkv + g) * N * D;
        const uint8_t* Vg = V + ((int64_t)b * Hkv + g) * N * D;

        const int nqt = (N + BMQ - 1) / BMQ;
        const int qt0 = CAUSAL ? k0 / BMQ : 0;
        const int total = G * (nqt - qt0);

        // ---- direct loads of step u, in step order, from running offsets (as
        // the bf16 kernel): waves 0-3 load the Q row group `wave`, waves 4-7
        // the dO row group `wave - 4`, and every wave two statistics chunks
        const int64_t bg0 = (int64_t)b * Hq + g * G;
        int64_t qo = (bg0 * N + qt0 * BMQ) * D;
        int64_t so = bg0 * Npad + qt0 * BMQ;
        int qrem = N - qt0 * BMQ;
        const float* Sw = (wave < NW / 2 ? WSl : WSd) + 4 * Cfg::kStatPerWave * (wave % (NW / 2));
        const uint8_t* src8 = wave < NW / 2 ? Q : dO;
        const int grpw = wave % (NW / 2);
        int u_next = 0;
        auto issue = [&](int u) __attribute__((always_inline)) {
            const uint32_t st = lds_addr(smem + (u % NS) * Cfg::kStageBytes);
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int row = grpw * QT::RG + ln % QT::RG;
            const int grow = row < qrem ? row : qrem - 1;
            const uint32_t off = (uint32_t)(grow * D + (ln / QT::RG) * 16);
            dma16s(src8 + qo, off, st + (wave < NW / 2 ? 0 : QT::kBytes) + grpw * QT::RGS);
            if (ln < Cfg::kStatPerWave)
                dma16s(Sw + so, 16u * (uint32_t)ln, st + 2 * QT::kBytes + 16 * wave * Cfg::kStatPerWave);
            qo += BMQ * D;
            so += BMQ;
            qrem -= BMQ;
            if (qrem <= 0) {
                qo += ((int64_t)N - (nqt - qt0) * BMQ) * D;
                so += Npad - (nqt - qt0) * BMQ;
                qrem = N - qt0 * BMQ;
            }
        };
#pragma unroll
        for (int t = 0; t < NS; ++t)
            if (t < total) {
                issue(u_next);
                ++u_next;
            }

        // the wave's K and V rows as fp8 B operands: bytes 64 s2 + 32 hh .. + 31
        u32x8 kf[D / 64], vf[D / 64];
        {
            const int row = min(krow, N - 1);
#pragma unroll
            for (int s2 = 0; s2 < D / 64; ++s2) {
                u32x8 a = *reinterpret_cast<const u32x8*>(Kg + (int64_t)row * D + 64 * s2 + 32 * hh);
                u32x8 c = *reinterpret_cast<const u32x8*>(Vg + (int64_t)row * D + 64 * s2 + 32 * hh);
                if (krow >= N) a = c = u32x8{};
                kf[s2] = a;
                vf[s2] = c;
            }
        }
#pragma unroll
        for (int s2 = 0; s2 < D / 64; ++s2) {
            asm volatile("" : : "v"(kf[s2]));
            asm volatile("" : : "v"(vf[s2]));
        }
        wait_vm<0>();

        f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
        for (int i = 0; i < D / 32; ++i) dkacc[i] = dvacc[i] = zero16();
        f32x16 sacc = zero16(), dpacc = zero16();
        u32x4 pb[2], sb[2];
        pb[0] = pb[1] = sb[0] = sb[1] = u32x4{};

        auto stage = [&](int i) __attribute__((always_inline)) { return smem + (i % NS) * Cfg::kStageBytes; };
        // S = Q K^T and dP = dO V^T of step i (fp8): rows = queries, columns = this wave's keys
        auto do_sdp = [&](int i) __attribute__((always_inline)) {
            const uint16_t* Qs = (const uint16_t*)stage(i);
            const uint16_t* dOs = (const uint16_t*)(stage(i) + QT::kBytes);
            sacc = zero16();
#pragma unroll
            for (int s2 = 0; s2 < D / 64; ++s2) {
                sacc = mma_fp8s(row32<QT>(Qs, l32, 4 * s2 + 2 * hh), kf[s2], sacc, 127);
                dpacc = mma_fp8s(row32<QT>(dOs, l32, 4 * s2 + 2 * hh), vf[s2], dpacc, 127);
            }
        };
        // dV^T += dO_i^T P_i ;  dK^T += Q_i^T dS_i  (bf16, E4M3 rows widened)
        auto do_dvdk = [&](int i) __attribute__((always_inline)) {
            const uint16_t* Qs = (const uint16_t*)stage(i);
            const uint16_t* dOs = (const uint16_t*)(stage(i) + QT::kBytes);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int ct = 0; ct < D / 32; ++ct) {
                    dvacc[ct] = mma_bf16(tr_fp8_bf16<QT>(dOs, 16 * t, 32 * ct, lane), pb[t], dvacc[ct]);
                    dkacc[ct] = mma_bf16(tr_fp8_bf16<QT>(Qs, 16 * t, 32 * ct, lane), sb[t], dkacc[ct]);
                }
        };
        // dP of step i starts from -D / (s_dO s_V) of its query rows
        auto init_dp = [&](int i) __attribute__((always_inline)) {
            const float* sd = (const float*)(stage(i) + 2 * QT::kBytes) + BMQ;
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(sd + 8 * gq + 4 * hh);
#pragma unroll
                for (int j = 0; j < 4; ++j) dpacc[4 * gq + j] = d4[j];
            }
        };
        // G(i), i >= 1; causal: the first nd query blocks of each head lie wholly
        // before this wave's keys, and a phase whose two steps are both such
        // blocks is skipped
        int gb = qt0;
        const int nd = CAUSAL ? 32 * wave / BMQ : 0;
        auto gemm = [&](int i) __attribute__((always_inline)) {
            if (++gb == nqt) gb = qt0;
            if (gb > qt0 && gb - qt0 < nd) return;
            init_dp(i);
            do_dvdk(i - 1);
            do_sdp(i);
        };
        // X(i)
        int xq = qt0;
        auto softmax = [&](int i, auto&& mid) __attribute__((always_inline)) {
            if (i >= total) {
                mid();
                pb[0] = pb[1] = sb[0] = sb[1] = u32x4{};
                return;
            }
            const int q0 = xq * BMQ;
            if (++xq == nqt) xq = qt0;
            const float* sl = (const float*)(stage(i) + 2 * QT::kBytes);
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const f32x4 l4 = *reinterpret_cast<const f32x4*>(sl + 8 * gq + 4 * hh);
#pragma unroll
                for (int j = 0; j < 4; ++j) sacc[4 * gq + j] = fast_exp2(fmaf(sacc[4 * gq + j], c2, -l4[j]));
            }
            settle(sacc);
            mid();
            if (CAUSAL && kw + 31 > q0) {
                const int delta = krow - q0 - 4 * hh;
#pragma unroll
                for (int r2 = 0; r2 < 16; ++r2)
                    if (delta > 8 * (r2 / 4) + r2 % 4) sacc[r2] = 0.f;
            }
#pragma unroll
            for (int r2 = 0; r2 < 16; ++r2) dpacc[r2] = sacc[r2] * dpacc[r2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                pb[t] = pack_bf16x8(sacc, 8 * t);
                sb[t] = pack_bf16x8(dpacc, 8 * t);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                settle(pb[t]);
                settle(sb[t]);
            }
        };

        // ---- phases, as the bf16 kernel: in loop round i both groups load step
        // i+NS-2 in their vector phase; before the barrier ending odd slot s,
        // step (s+1)/2 has landed
        static_assert((NS - 3) * kLoads <= 63, "vmcnt range");
        auto refill = [&](int i) __attribute__((always_inline)) {
            if (i >= 2 && i + NS - 2 < total) {
                issue(u_next);
                ++u_next;
            }
        };
        auto tail_odd = [&](int s) __attribute__((always_inline)) {
            const int tv = (s + 1) / 2;
            if (tv >= NS && tv < total) {
                const int later = min(NS - 3, total - 1 - tv);
                wait_vm_dyn<kLoads, NS - 3>(later);
            }
            lds_barrier();
        };
        lds_barrier();
        if (grp == 0) {
            init_dp(0);
            do_sdp(0);
            lds_barrier();
            softmax(0, [] {});
            tail_odd(1);
            for (int i = 1; i <= total; ++i) {
                gemm(i);
                lds_barrier();
                softmax(i, [&] { refill(i); });
                tail_odd(2 * i + 1);
            }
        } else {
            lds_barrier();
            init_dp(0);
            do_sdp(0);
            tail_odd(1);
            for (int i = 1; i <= total; ++i) {
                softmax(i - 1, [&] { refill(i); });
                lds_barrier();
                gemm(i);
                tail_odd(2 * i + 1);
            }
        }

        if (krow < N) {
            int le = lane;
            asm volatile("" : "+v"(le));
            const int64_t row = ((int64_t)b * Hkv + g) * N + kw + (le & 31);
            uint16_t* dKr = dK + row * D;
            uint16_t* dVr = dV + row * D;
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int c = 32 * ct + 8 * gq + 4 * (le >> 5);
                    u32x2 wk, wv;
                    wk[0] = pack_bf16x2(dkacc[ct][4 * gq] * sk, dkacc[ct][4 * gq + 1] * sk);
                    wk[1] = pack_bf16x2(dkacc[ct][4 * gq + 2] * sk, dkacc[ct][4 * gq + 3] * sk);
                    wv[0] = pack_bf16x2(dvacc[ct][4 * gq] * sv, dvacc[ct][4 * gq + 1] * sv);
                    wv[1] = pack_bf16x2(dvacc[ct][4 * gq + 2] * sv, dvacc[ct][4 * gq + 3] * sv);
                    *reinterpret_cast<u32x2*>(dKr + c) = wk;
                    *reinterpret_cast<u32x2*>(dVr + c) = wv;
                }
        }
    }
}

// ------------------------------------------------------------ dQ
//
// As bwd_dq_bf16_kernel<128>: waves w and w+4 share a SIMD and alternate
//   G(t): dQ^T += K_{t-1}^T dS_{t-1}^T, then S_t^T = K_t Q^T, dP_t^T = V_t dO^T
//   X(t): P_t, mask, dS_t = P_t (dP_t - D), scaled and rounded to E4M3
// all three products on the fp8 matrix cores.  dS^T is the B operand of the dQ
// product: byte e of this lane's operand is dS of key 32 (e / 16) +
// row(e % 16, hh) (the fp8 forward's P layout); the 32 keys of key block kb
// of a query (16 bytes in each lane half) share the block scale 2^-E with
// 2^E |dS|max in [128, 256).
struct QFp8Cfg {
    static constexpr int D = 128;
    static constexpr int kWaves = 8;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BM = 32 * kWaves;
    static constexpr int BNK = 64;
    static constexpr int kStages = 4;
    using KT = Fp8Rows<BNK, kWaves>;            // K rows (scores, transposed for dQ), V rows
    static constexpr int kStage = 2 * KT::kElems;
    static constexpr int kLoads = 2 * KT::kPerWave;
};

template <bool CAUSAL>
__global__ __launch_bounds__(QFp8Cfg::kThreads, 2) void bwd_dq_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const uint8_t* __restrict__ dO, const float* __restrict__ WSd, const float* __restrict__ WSl,
    const float* __restrict__ descale, uint16_t* __restrict__ dQ, int B, int Hq, int Hkv, int n_rows, int Npad,
    float scale) {
    using Cfg = QFp8Cfg;
    using KT = Cfg::KT;
    constexpr int D = Cfg::D, BM = Cfg::BM, BNK = Cfg::BNK, NS = Cfg::kStages, KB = BNK / 32;
    constexpr int kStage = Cfg::kStage, kLoads = Cfg::kLoads;
    static_assert(KT::kPerWave == 1, "one row group per wave per tile");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * kStage];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int grp = wave >> 2;
    const float c2 = scale * kLog2e * descale[0] * descale[1];
    const float sq = scale * descale[1] * descale[3] * descale[2];    // dQ: scale s_K s_dO s_V

    const int nmb = (n_rows + BM - 1) / BM;
    const PersistentSched sched(nmb * Hq * B);
    for (int r = 0; sched.more(r); ++r) {
        const int lin = sched.item(r);
        if (lin < 0) continue;
        int N = n_rows;
        asm volatile("" : "+s"(N));
        const int mbi = lin % nmb, bh = lin / nmb;
        const int h = bh % Hq, b = bh / Hq;
        const int mb = CAUSAL ? nmb - 1 - mbi : mbi;
        const int g = h / (Hq / Hkv);
        const int64_t rowbase = ((int64_t)b * Hq + h) * N;
        const uint8_t* Kg = K + ((int64_t)b * Hkv + g) * N * D;
        const uint8_t* Vg = V + ((int64_t)b * Hkv + g) * N * D;

        const int q0 = mb * BM;
        const int qw = q0 + 32 * wave;
        const int qrow = qw + l32;
        const int kend = CAUSAL ? min(N, q0 + BM) : N;
        const int ntiles = (kend + BNK - 1) / BNK;
        const int ntw = qw >= N ? 0 : CAUSAL ? (min(N, qw + 32) + BNK - 1) / BNK : ntiles;

        auto stage = [&](int t) __attribute__((always_inline)) { return smem + (t % NS) * kStage; };
        auto issue = [&](int t) __attribute__((always_inline)) {
            const uint32_t st = lds_addr(stage(t));
            const uint8_t* kb = Kg + (int64_t)t * BNK * D;
            const uint8_t* vb = Vg + (int64_t)t * BNK * D;
            const int rows_valid = N - t * BNK;
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int row = wave * KT::RG + ln % KT::RG;
            const int grow = row < rows_valid ? row : rows_valid - 1;
            const uint32_t off = (uint32_t)(grow * D + (ln / KT::RG) * 16);
            dma16s(kb, off, st + wave * KT::RGS);
            dma16s(vb, off, st + KT::kBytes + wave * KT::RGS);
        };
#pragma unroll
        for (int t = 0; t < NS; ++t)
            if (t < ntiles) issue(t);

        // Q and dO rows as fp8 B operands (rows past the end read the last row;
        // those queries are never stored)
        u32x8 qf[D / 64], of[D / 64];
        {
            const int row = min(qrow, N - 1);
#pragma unroll
            for (int s2 = 0; s2 < D / 64; ++s2) {
                qf[s2] = *reinterpret_cast<const u32x8*>(Q + (rowbase + row) * D + 64 * s2 + 32 * hh);
                of[s2] = *reinterpret_cast<const u32x8*>(dO + (rowbase + row) * D + 64 * s2 + 32 * hh);
            }
        }
        const int64_t srow = ((int64_t)b * Hq + h) * Npad + qrow;
        const float lse2 = qrow < N ? WSl[srow] : INFINITY;
        const float dq_nd = qrow < N ? WSd[srow] : 0.f;     // -D / (s_dO s_V)
#pragma unroll
        for (int s2 = 0; s2 < D / 64; ++s2) {
            asm volatile("" : : "v"(qf[s2]));
            asm volatile("" : : "v"(of[s2]));
        }
        settle(lse2);
        settle(dq_nd);
        wait_vm<0>();

        f32x16 dqacc[D / 32];
#pragma unroll
        for (int i = 0; i < D / 32; ++i) dqacc[i] = zero16();
        f32x16 sacc[KB], dpacc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sacc[kb] = dpacc[kb] = zero16();
        u32x8 dsf = {};
        int dss = 127;                                  // E8M0 block scale of dsf (this lane's)

        auto do_sdp = [&](int t) __attribute__((always_inline)) {
            const uint16_t* Ks = stage(t);
            const uint16_t* Vs = Ks + KT::kElems;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sacc[kb] = dpacc[kb] = zero16();
#pragma unroll
            for (int s2 = 0; s2 < D / 64; ++s2)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    sacc[kb] = mma_fp8s(row32<KT>(Ks, 32 * kb + l32, 4 * s2 + 2 * hh), qf[s2], sacc[kb], 127);
                    dpacc[kb] = mma_fp8s(row32<KT>(Vs, 32 * kb + l32, 4 * s2 + 2 * hh), of[s2], dpacc[kb], 127);
                }
        };
        // dQ^T += K_t^T dS_t^T: read p (0..3) of a fragment gives this lane the
        // keys 32(p/2) + 16(p%2) + 8(j/4) + 4hh + j%4, j = 0..7 (byte 8p + j of dsf)
        const int g16 = lane >> 4, s16 = lane & 15, jj = s16 >> 1, qq = s16 & 1;
        auto do_dq = [&](int t) __attribute__((always_inline)) {
            const char* Kb = (const char*)stage(t);
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct) {
                u32x8 a;
#pragma unroll
                for (int pq = 0; pq < 4; ++pq) {
                    const int key = 32 * (pq >> 1) + 16 * (pq & 1) + 8 * (jj >> 2) + 4 * (g16 >> 1) + (jj & 3);
                    const int col = 32 * ct + 16 * (g16 & 1) + 8 * qq;
                    const char* ad = Kb + KT::off(key, col >> 4) + (col & 15);
                    const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (lds_i32x2*)(__attribute__((address_space(3))) char*)ad);
                    a[2 * pq] = (uint32_t)w[0];
                    a[2 * pq + 1] = (uint32_t)w[1];
                }
                dqacc[ct] = mma_fp8s(a, dsf, dqacc[ct], dss);
            }
        };
        auto gemm = [&](int t) __attribute__((always_inline)) {
            do_dq(t - 1);
            do_sdp(t);
        };
        auto softmax = [&](int t) __attribute__((always_inline)) {
            if (t >= ntw) {
                dsf = u32x8{};
                dss = 127;
                return;
            }
            const int k0 = t * BNK;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r2 = 0; r2 < 16; ++r2) sacc[kb][r2] = fast_exp2(fmaf(sacc[kb][r2], c2, -lse2));
            if ((CAUSAL && k0 + BNK - 1 > qw) || (k0 + BNK > N)) {
                int hm = hh;
                asm volatile("" : "+v"(hm));
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r2 = 0; r2 < 16; ++r2) {
                        const int key = k0 + 32 * kb + acc_row(r2, hm);
                        if ((CAUSAL && key > qrow) || key >= N) sacc[kb][r2] = 0.f;
                    }
            }
            float amax[KB] = {0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r2 = 0; r2 < 16; ++r2) {
                    dpacc[kb][r2] = sacc[kb][r2] * (dpacc[kb][r2] + dq_nd);
                    amax[kb] = fmaxf(amax[kb], fabsf(dpacc[kb][r2]));
                }
            // Block scales.  The matrix core groups a column's 64 contraction
            // slots into two blocks of 32: block kb is bytes 16 kb .. 16 kb + 15 of
            // lane l and of lane l ^ 32 (here: key block kb of the query, both
            // lane halves), scaled by the exponent in lane l (kb = 0) or l + 32
            // (kb = 1).  Block kb gets 2^E |dS|max in [128, 256), E = 134 - (biased
            // exponent of its |dS|max).
            int se[KB];
            float psc[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const float bm = pair_max(amax[kb]);
                se[kb] = max((int)((__float_as_uint(bm) >> 23) & 0xffu) - 7, 1);   // E8M0 of 2^-E
                psc[kb] = __uint_as_float((uint32_t)se[kb] << 23);
            }
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const f32x16& v = dpacc[w >> 2];
                const int o = 4 * (w & 3);
                s16x2 lo;
                asm("" : "=v"(lo) : "v"(v[o]));               // any value: both halves are written
                lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, v[o], v[o + 1], psc[w >> 2], false);
                lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, v[o + 2], v[o + 3], psc[w >> 2], true);
                dsf[w] = __builtin_bit_cast(uint32_t, lo);
            }
            dss = hh ? se[1] : se[0];
            asm volatile("" : : "v"(dsf));
        };

        // In loop round t each group refills the stage of tile t+2 (its previous
        // tile, t-2, was last read in slot 2t-1) at the start of its matrix
        // phase (slot 2t for the first group, 2t+1 for the second): with fp8
        // products that phase is the shorter one (2-3% faster for the whole
        // backward than refilling in the vector phase, as the bf16 kernel
        // does).  Before the barrier ending odd slot s, tile (s+1)/2 has landed.
        auto refill = [&](int t) __attribute__((always_inline)) {
            if (t + 2 >= NS && t + 2 < ntiles) issue(t + 2);
        };
        auto tail_odd = [&](int s) __attribute__((always_inline)) {
            const int tv = (s + 1) / 2;
            if (tv >= NS && tv < ntiles) {
                if (tv + 1 < ntiles) wait_vm<kLoads>();
                else wait_vm<0>();
            }
            lds_barrier();
        };
        lds_barrier();
        if (grp == 0) {
            do_sdp(0);
            lds_barrier();
            softmax(0);
            tail_odd(1);
            for (int t = 1; t <= ntiles; ++t) {
                refill(t);
                gemm(t);
                lds_barrier();
                softmax(t);
                tail_odd(2 * t + 1);
            }
        } else {
            lds_barrier();
            do_sdp(0);
            tail_odd(1);
            for (int t = 1; t <= ntiles; ++t) {
                softmax(t - 1);
                lds_barrier();
                refill(t);
                gemm(t);
                tail_odd(2 * t + 1);
            }
        }

        if (qrow < N) {
            int le = lane;
            asm volatile("" : "+v"(le));
            uint16_t* dQr = dQ + (rowbase + qw + (le & 31)) * D + 4 * (le >> 5);
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    u32x2 w;
                    w[0] = pack_bf16x2(dqacc[ct][4 * gq] * sq, dqacc[ct][4 * gq + 1] * sq);
                    w[1] = pack_bf16x2(dqacc[ct][4 * gq + 2] * sq, dqacc[ct][4 * gq + 3] * sq);
                    *reinterpret_cast<u32x2*>(dQr + 32 * ct + 8 * gq) = w;
                }
        }
    }
}

hipError_t launch_bwd_fp8(int causal, const void* q, const void* k, const void* v, const void* o, const void* dO,
                          const float* lse, const float* descale, float* ws, void* dq, void* dk, void* dv, int B,
                          int Hq, int Hkv, int N, float scale, hipStream_t st) {
    const int Np = ws_rows(N);
    const int64_t rows = (int64_t)B * Hq * Np;
    float* wsd = ws;
    float* wsl = ws + rows;
    constexpr int RPB = 256 / (128 / 8);
    hipLaunchKernelGGL(bwd_delta_fp8_kernel, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st,
                       (const uint16_t*)o, (const uint8_t*)dO, lse, descale, wsd, wsl, N, Np, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        using Cfg = KVFp8Cfg;
        const int nkb = (N + Cfg::BNK - 1) / Cfg::BNK;
        static PerDevice slots_c, slots_n;
        const void* kern = causal ? (const void*)bwd_dkdv_fp8_kernel<true> : (const void*)bwd_dkdv_fp8_kernel<false>;
        const int grid = persistent_grid(kern, Cfg::kThreads, nkb * Hkv * B, causal ? slots_c : slots_n);
        if (causal)
            hipLaunchKernelGGL(bwd_dkdv_fp8_kernel<true>, dim3((unsigned)grid), dim3(Cfg::kThreads), 0, st,
                               (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, (const uint8_t*)dO, wsd, wsl,
                               descale, (uint16_t*)dk, (uint16_t*)dv, B, Hq, Hkv, N, Np, scale);
        else
            hipLaunchKernelGGL(bwd_dkdv_fp8_kernel<false>, dim3((unsigned)grid), dim3(Cfg::kThreads), 0, st,
                               (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, (const uint8_t*)dO, wsd, wsl,
                               descale, (uint16_t*)dk, (uint16_t*)dv, B, Hq, Hkv, N, Np, scale);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    {
        using Cfg = QFp8Cfg;
        const int nmb = (N + Cfg::BM - 1) / Cfg::BM;
        static PerDevice slots_c, slots_n;
        const void* kern = causal ? (const void*)bwd_dq_fp8_kernel<true> : (const void*)bwd_dq_fp8_kernel<false>;
        const int grid = persistent_grid(kern, Cfg::kThreads, nmb * Hq * B, causal ? slots_c : slots_n);
        if (causal)
            hipLaunchKernelGGL(bwd_dq_fp8_kernel<true>, dim3((unsigned)grid), dim3(Cfg::kThreads), 0, st,
                               (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, (const uint8_t*)dO, wsd, wsl,
                               descale, (uint16_t*)dq, B, Hq, Hkv, N, Np, scale);
        else
            hipLaunchKernelGGL(bwd_dq_fp8_kernel<false>, dim3((unsigned)grid), dim3(Cfg::kThreads), 0, st,
                               (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, (const uint8_t*)dO, wsd, wsl,
                               descale, (uint16_t*)dq, B, Hq, Hkv, N, Np, scale);
    }
    return hipGetLastError();
}

}  // namespace fa
