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
//
// A workgroup holds 256 keys (32 per wave: K as MFMA operands in registers,
// V in LDS, dK and dV accumulators) and walks the steps (query head of the
// group, query block).  Ping-pong schedule as in the forward: waves w and w+4
// share a SIMD, each wave alternates
//   G(i): dV^T += dO_{i-1}^T P_{i-1}, dK^T += Q_{i-1}^T dS_{i-1}, then
//         S_i = Q_i K^T and dP_i = dO_i V^T
//   X(i): P_i = exp2(c2 s - LSE log2 e), causal mask, dS_i = P_i (dP_i - D), pack
// and the two wave groups run one phase apart, a barrier after every phase.
template <int D>
struct KVBf16Cfg {
    static constexpr int kWaves = 8;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BNK = 32 * kWaves;             // keys per workgroup (32 per wave)
    static constexpr int BMQ = D == 128 ? 32 : 64;      // query rows per step
    static constexpr int QB = BMQ / 32;
    static constexpr int kStages = 4;
    using QT = LdsTile<BMQ, D, kWaves>;
    using VT = LdsTile<BNK, D, kWaves>;                 // the workgroup's V rows, read as B operands of dP
    static constexpr int kStatChunks = BMQ / 2;         // 16-byte chunks of (LSE*log2e, D) per step
    static constexpr int kStatPerWave = kStatChunks / kWaves;
    static_assert(kStatChunks % kWaves == 0, "statistics split evenly over the waves");
    static constexpr int kStatBytes = 8 * BMQ;
    static constexpr int kStageBytes = 2 * QT::kBytes + kStatBytes;
    static constexpr int kLdsBytes = VT::kBytes + kStages * kStageBytes;
    static constexpr int kLoads = 2 * QT::kPerWave + 1;
};

// G phase order: the NSTAT reads of the statistics that start dP and L
// fragment reads ahead; the dV/dK products (two transposed reads per
// fragment) first, then the S products (one read: Q) alternating with the dP
// products (dO and V rows).
template <int L, int NSTAT>
__device__ __forceinline__ void sched_dkdv_phase() {
#pragma unroll
    for (int i = 0; i < L + NSTAT; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    static_assert(L % 4 == 0, "whole (S, dP) pairs");
#pragma unroll
    for (int i = 0; i < 8 - L / 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < L / 2; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// LOCAL (with CAUSAL): sliding window with S global tokens, key j visible to
// query i iff j <= i and (i - W < j or j < S); a key block's steps end at the
// last query block that sees one of its keys (every later one when the block
// holds global tokens).
// BSP: block-sparse, key block kbk is seen by the query blocks bidx[bptr[kbk]
// .. bptr[kbk+1]) (ascending, BNK rows each, BNK / BMQ steps per block; the
// mask's column layout), clamped so that any layout stays in bounds.
// DROP: the backward through attention dropout (the FlashAttention page of the
// self-hosted LLM glossary: dropout is fused into the kernel; its mask is
// regenerated here from the same counter-based generator, not stored).  With
// Z the keep mask, p the drop probability (thr / 256) and r = 1/(1 - p),
// O = (Z o P) r V, so dV = r (Z o P)^T dO
// and dS = P o (Z o dP r - D).  The workspace then holds -D (1 - p), the dP
// accumulator starts from it, and dS = r P o (Z ? acc : -D (1 - p)); the
// factor r goes into the final scales of dK and dV.
template <int D, bool CAUSAL, bool LOCAL = false, bool BSP = false, bool DROP = false, bool SPLIT = false>
__global__ __launch_bounds__(KVBf16Cfg<D>::kThreads, 2) void bwd_dkdv_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ WSd, const float* __restrict__ WSl,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int B, int Hq, int Hkv, int n_rows, int Npad, float c2,
    float scale, int W, int S, const int* __restrict__ bptr, const int* __restrict__ bidx, int nnz, DropArgs drop,
    BspSplit sp) {
    static_assert(!(LOCAL && BSP), "one sparsity pattern at a time");
    static_assert(!(DROP && (LOCAL || BSP)), "dropout with the dense masks only");
    using Cfg = KVBf16Cfg<D>;
    using QT = typename Cfg::QT;
    constexpr int NW = Cfg::kWaves, BNK = Cfg::BNK, BMQ = Cfg::BMQ, QB = Cfg::QB, NS = Cfg::kStages;
    constexpr int kLoads = Cfg::kLoads;
    static_assert(QB * D == 128, "16 + 16 products per G phase");
    __shared__ __attribute__((aligned(1024))) char lds[Cfg::kLdsBytes];
    using VT = typename Cfg::VT;
    // stages first: their fragment offsets stay inside the 16-bit immediate of
    // the LDS reads (the V rows sit above them)
    char* smem = lds;                                   // Q / dO / statistics stages
    const uint16_t* Vl = (const uint16_t*)(lds + NS * Cfg::kStageBytes);   // V rows k0 .. k0+255

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int grp = wave >> 2;                      // waves w and w+4 share a SIMD

    const int nkb = (n_rows + BNK - 1) / BNK;
    constexpr bool split = BSP && SPLIT;               // work items from sp.chunks
    const int nit = split ? sp.nchunks : nkb;            // work items per (batch, K/V head)
    const PersistentSched sched(nit * Hkv * B);
    for (int r = 0; sched.more(r); ++r) {
        const int lin = sched.item(r);
        if (lin < 0) continue;
        // the sequence length as an opaque per-item value: whatever derives
        // from it (tail clamps and masks) is computed per item, not hoisted
        // out of the item loop into registers for the whole kernel
        int N = n_rows;
        asm volatile("" : "+s"(N));
        const int kbi = lin % nit, bg = lin / nit;
        int kbk = kbi;                                  // ascending key blocks: causal-heavy first
        // (block-sparse) the item's entries (row blocks) bbeg .. bbeg+bcnt-1
        int bbeg = 0, bcnt = 0;
        if constexpr (BSP) {
            if (split) {
                const int* c = sp.chunks + 4 * kbi;
                kbk = min(max(c[0], 0), nkb - 1);
                bbeg = min(max(c[1], 0), nnz);
                bcnt = min(max(c[2], bbeg), nnz) - bbeg;
            } else {
                bbeg = min(max(bptr[kbk], 0), nnz);
                bcnt = min(max(bptr[kbk + 1], bbeg), nnz) - bbeg;
            }
        }
        const int g = bg % Hkv, b = bg / Hkv;
        const int G = Hq / Hkv;
        const int k0 = kbk * BNK;
        const int kw = k0 + 32 * wave;
        const int krow = kw + l32;

        const uint16_t* Kg = K + ((int64_t)b * Hkv + g) * N * D;
        const uint16_t* Vg = V + ((int64_t)b * Hkv + g) * N * D;

        const int nqt = (N + BMQ - 1) / BMQ;
        const int qt0 = CAUSAL && !BSP ? k0 / BMQ : 0;  // earlier query blocks see none of these keys
        // (local) later query blocks than qt1 - 1 see none of them either
        const int qt1 = LOCAL && k0 >= S ? min(nqt, (min(N, k0 + BNK) - 2 + W) / BMQ + 1) : nqt;
        // (block-sparse) the listed row blocks bbeg .. bbeg+bcnt-1, SPB steps
        // each (fewer for a last block that ends past N): nsh steps per head
        constexpr int SPB = BNK / BMQ;
        int nsh = 0;
        if constexpr (BSP) {
            if (bcnt) nsh = SPB * (bcnt - 1) + min(SPB, nqt - min(max(bidx[bbeg + bcnt - 1], 0), nkb - 1) * SPB);
        }
        // query block (of BMQ rows) of a head's j-th step
        auto qblk = [&](int j) __attribute__((always_inline)) {
            return min(min(max(bidx[bbeg + j / SPB], 0), nkb - 1) * SPB + j % SPB, nqt - 1);
        };
        // steps: (head g*G + i / (qt1-qt0), block qt0 + i % (qt1-qt0)); block-sparse:
        // (head g*G + i / nsh, block qblk(i % nsh))
        const int total = BSP ? G * nsh : G * (qt1 - qt0);

        // ---- direct loads of step u, issued in step order.  The next step's
        // rows are kept as running element offsets: one for Q and dO (the two
        // share a layout) and one for the statistics rows; both move on by a
        // block per step and to the next head of the group after the last block.
        // The per-lane offsets are recomputed at every issue from an opaque copy
        // of the lane index: kept live across the loop they would be spilled, and
        // a scratch reload is a vector-memory load whose wait would also drain
        // the tile loads in flight.
        const int64_t bg0 = (int64_t)b * Hq + g * G;    // first query head of the group
        int64_t qo = (bg0 * N + qt0 * BMQ) * D;
        int64_t so = bg0 * Npad + qt0 * BMQ;
        int qrem = N - qt0 * BMQ;                       // rows from the next step's first row to the head's end
        int bq = qt0;                                   // (local) query block of the next step
        int ji = 0, hi = 0;                             // (block-sparse) step and head of the next issue
        // statistics: chunk c < BMQ/4 of a stage holds LSE*log2e rows 4c.., the
        // rest -D rows; chunk c is loaded by wave c / kStatPerWave, so the first
        // half of the waves loads LSE rows and the second half -D rows
        const float* Sw = (wave < NW / 2 ? WSl : WSd) + 4 * Cfg::kStatPerWave * (wave % (NW / 2));
        int u_next = 0;
        auto issue = [&](int u) __attribute__((always_inline)) {
            const uint32_t st = lds_addr(smem + (u % NS) * Cfg::kStageBytes);
            if constexpr (BSP) {
                const int qb = qblk(ji);
                qo = ((bg0 + hi) * N + (int64_t)qb * BMQ) * D;
                so = (bg0 + hi) * Npad + qb * BMQ;
                qrem = N - qb * BMQ;
                if (++ji == nsh) {
                    ji = 0;
                    ++hi;
                }
            }
            int ln = lane;
            asm volatile("" : "+v"(ln));
#pragma unroll
            for (int i = 0; i < QT::kPerWave; ++i) {
                const int row = (i * NW + wave) * QT::RG + ln % QT::RG;
                const int grow = row < qrem ? row : qrem - 1;
                const uint32_t off = (uint32_t)(grow * D + (ln / QT::RG) * 8) * 2u;
                dma16s(Q + qo, off, st + (i * NW + wave) * QT::RGS);
                dma16s(dO + qo, off, st + QT::kBytes + (i * NW + wave) * QT::RGS);
            }
            if (ln < Cfg::kStatPerWave) dma16s(Sw + so, 16u * (uint32_t)ln, st + 2 * QT::kBytes + 16 * wave * Cfg::kStatPerWave);
            if constexpr (!BSP) {
                qo += BMQ * D;
                so += BMQ;
                qrem -= BMQ;
                if (LOCAL ? ++bq == qt1 : qrem <= 0) {     // past the head's last block: the next head, block qt0
                    qo += ((int64_t)N - (qt1 - qt0) * BMQ) * D;
                    so += Npad - (qt1 - qt0) * BMQ;
                    qrem = N - qt0 * BMQ;
                    if (LOCAL) bq = qt0;
                }
            }
        };
        VT::load(Vg + (int64_t)k0 * D, N - k0, Vl, wave, lane);
#pragma unroll
        for (int t = 0; t < NS; ++t)
            if (t < total) {
                issue(u_next);
                ++u_next;
            }

        u32x4 kf[D / 16];
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            u32x4 a = {};
            if (krow < N) a = *reinterpret_cast<const u32x4*>(Kg + (int64_t)krow * D + 16 * s + 8 * hh);
            kf[s] = a;
        }
#pragma unroll
        for (int s = 0; s < D / 16; ++s) settle(kf[s]);
        wait_vm<0>();

        f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
        for (int i = 0; i < D / 32; ++i) dkacc[i] = dvacc[i] = zero16();
        f32x16 sacc[QB], dpacc[QB];
        u32x4 pb[QB][2], sb[QB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            sacc[qb] = dpacc[qb] = zero16();
            pb[qb][0] = pb[qb][1] = sb[qb][0] = sb[qb][1] = u32x4{};
        }

        // S = Q K^T and dP = dO V^T of step i: rows = queries, columns = this wave's keys
        auto do_sdp = [&](int i) __attribute__((always_inline)) {
            const char* st = smem + (i % NS) * Cfg::kStageBytes;
            const uint16_t* Qs = (const uint16_t*)st;
            const uint16_t* dOs = (const uint16_t*)(st + QT::kBytes);
            // the V fragments are the same every step; an opaque zero offset keeps
            // their reads here instead of hoisted (and held) outside the loop
            int vz = 0;
            asm volatile("" : "+s"(vz));
            const uint16_t* Vw = Vl + vz;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sacc[qb] = zero16();
#pragma unroll
            for (int s = 0; s < D / 16; ++s)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    sacc[qb] = mma_bf16(QT::row8(Qs, 32 * qb + l32, 2 * s + hh), kf[s], sacc[qb]);
                    dpacc[qb] = mma_bf16(QT::row8(dOs, 32 * qb + l32, 2 * s + hh),
                                         VT::row8(Vw, 32 * wave + l32, 2 * s + hh), dpacc[qb]);
                }
        };
        // dV^T += dO_i^T P_i ;  dK^T += Q_i^T dS_i
        auto do_dvdk = [&](int i) __attribute__((always_inline)) {
            const char* st = smem + (i % NS) * Cfg::kStageBytes;
            const uint16_t* Qs = (const uint16_t*)st;
            const uint16_t* dOs = (const uint16_t*)(st + QT::kBytes);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int ct = 0; ct < D / 32; ++ct) {
                        dvacc[ct] = mma_bf16(QT::tr8(dOs, 32 * qb + 16 * t, 32 * ct, lane), pb[qb][t], dvacc[ct]);
                        dkacc[ct] = mma_bf16(QT::tr8(Qs, 32 * qb + 16 * t, 32 * ct, lane), sb[qb][t], dkacc[ct]);
                    }
        };
        // dP of step i starts from -D of its query rows (the workspace holds
        // -D), so the accumulator ends as dP - D and dS = P (dP - D) is one
        // multiply in the vector phase
        auto init_dp = [&](int i) __attribute__((always_inline)) {
            const float* sd = (const float*)(smem + (i % NS) * Cfg::kStageBytes + 2 * QT::kBytes) + BMQ;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(sd + 32 * qb + 8 * gq + 4 * hh);
#pragma unroll
                    for (int j = 0; j < 4; ++j) dpacc[qb][4 * gq + j] = d4[j];
                }
        };
        // G(i), i >= 1 (i == total: the products of the last step only).  gb is
        // the query block of step i.  Causal: the first nd blocks of each head
        // lie wholly before this wave's keys (P = dS = 0); a phase whose two
        // steps are both such blocks is void and skipped (the slot takes as
        // long, but the matrix cores spend no power on it)
        int gb = qt0;
        const int nd = CAUSAL && !BSP ? 32 * wave / BMQ : 0;
        auto gemm = [&](int i) __attribute__((always_inline)) {
            if (++gb == qt1) gb = qt0;
            if (gb > qt0 && gb - qt0 < nd) return;
            init_dp(i);
            do_dvdk(i - 1);
            do_sdp(i);
            // 8 fragments ahead at d = 128 causal; the non-causal kernel has 4
            // (with 8 it needs more than 256 registers and the scheduler drops
            // the read-ahead altogether)
            sched_dkdv_phase<D == 128 && CAUSAL ? 8 : 4, 4 * QB>();
        };
        // X(i): step i's query block is xq.  `mid` (the phase's loads) is
        // issued after the first query block's exponentials, whose results it
        // waits for
        int xq = qt0, jx = 0, hx = 0;                   // (dropout) hx: the step's head within the group
        auto softmax = [&](int i, auto&& mid) __attribute__((always_inline)) {
            if (i >= total) {
                mid();
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) pb[qb][0] = pb[qb][1] = sb[qb][0] = sb[qb][1] = u32x4{};
                return;
            }
            int q0;
            if constexpr (BSP) {
                q0 = qblk(jx) * BMQ;
                if (++jx == nsh) jx = 0;
            } else {
                q0 = xq * BMQ;
                if (++xq == qt1) xq = qt0;
            }
            const int hstep = hx;
            if constexpr (DROP) hx += xq == qt0;
            const float* sl = (const float*)(smem + (i % NS) * Cfg::kStageBytes + 2 * QT::kBytes);
            // causal: key krow is hidden from query q0 + 32*qb + row(r) iff
            // delta > 8*(r/4) + r%4, delta = krow - q0 - 32*qb - 4*hh; steps whose
            // queries all follow this wave's keys skip the test (uniform branch)
            const bool need_mask = CAUSAL && kw + 31 > q0;
            // local: query q0 + 32*qb + row(r) is past the window of key krow iff
            // 8*(r/4) + r%4 + dw >= W, dw = q0 + 32*qb + 4*hh - krow, unless the
            // key is a global token
            const bool need_wmask = LOCAL && q0 + BMQ - 1 >= kw + W;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const f32x4 l4 = *reinterpret_cast<const f32x4*>(sl + 32 * qb + 8 * gq + 4 * hh);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 4 * gq + j;
                        sacc[qb][r] = fast_exp2(fmaf(sacc[qb][r], c2, -l4[j]));
                    }
                }
                if (qb == 0) {
                    settle(sacc[qb]);                    // the exponentials stay above the loads
                    mid();
                }
                if (need_mask) {
                    const int delta = krow - q0 - 32 * qb - 4 * hh;
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (delta > 8 * (r / 4) + r % 4) sacc[qb][r] = 0.f;
                }
                if (need_wmask) {
                    const int dw = krow >= S ? q0 + 32 * qb + 4 * hh - krow : -(1 << 30);
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (dw + 8 * (r / 4) + r % 4 >= W) sacc[qb][r] = 0.f;
                }
                if constexpr (DROP) {
                    // keep bytes of this lane's key krow for the queries
                    // q0 + 32 qb + 8 gq + 4 hh + e (element 4 gq + e): one Philox
                    // call per lane and 32-query block, shared by the quad
                    int ln = lane;
                    asm volatile("" : "+v"(ln));
                    const uint32_t bhq = (uint32_t)(b * Hq + g * G + hstep);
                    uint32_t zw[4];
                    drop_words_krow(zw, q0 + 32 * qb, krow, ln >> 5, ln & 3, bhq, drop);
                    const float* sd = sl + BMQ;       // -D (1 - p) of the step's rows: the dP accumulator's start
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const f32x4 d4 = *reinterpret_cast<const f32x4*>(sd + 32 * qb + 8 * gq + 4 * hh);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 4 * gq + e;
                            const bool keep = drop_keep(zw[gq], e, drop.thr);
                            dpacc[qb][r] = sacc[qb][r] * (keep ? dpacc[qb][r] : d4[e]);
                            sacc[qb][r] = keep ? sacc[qb][r] : 0.f;
                        }
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) dpacc[qb][r] = sacc[qb][r] * dpacc[qb][r];
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    pb[qb][t] = pack_bf16x8(sacc[qb], 8 * t);
                    sb[qb][t] = pack_bf16x8(dpacc[qb], 8 * t);
                }
                // one query block at a time (its statistics reads are not hoisted
                // above the previous block's arithmetic)
                __builtin_amdgcn_sched_barrier(0);
            }
            // the packed operands are finished here, inside this phase (not sunk
            // past the barrier into the next matrix phase)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    settle(pb[qb][t]);
                    settle(sb[qb][t]);
                }
        };

        // ---- phases (slot s ends with a barrier).  In loop round i both groups
        // load step i+NS-2 (that stage held step i-2, last read in slot 2i-1) in
        // their vector phase (slot 2i+1 for the first group, 2i for the
        // second); before the barrier ending odd slot s, step tv = (s+1)/2
        // has landed, while up to NS-3 later steps may still be in flight.
        static_assert(NS >= 4 && (NS - 3) * kLoads <= 63, "vmcnt range");
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
            // G(i) in slot 2i, X(i) in slot 2i + 1
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
            // X(i-1) in slot 2i, G(i) in slot 2i + 1
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

        // (split column) the partial slot, read here rather than kept live
        int slot = -1;
        if (split) slot = sp.chunks[4 * kbi + 3] < sp.nslots ? sp.chunks[4 * kbi + 3] : -1;
        if (BSP && slot >= 0 && krow < N) {
            // (split column) this item's shares of dK and dV, float32, for the
            // merge; row pointers from an opaque lane, as below
            int le = lane;
            asm volatile("" : "+v"(le));
            const int64_t prow = ((int64_t)slot * B * Hkv + bg) * BNK + 32 * wave + (le & 31);
            float* Pk = sp.part + prow * D + 4 * (le >> 5);
            float* Pv = sp.part + ((int64_t)sp.nslots * B * Hkv * BNK + prow) * D + 4 * (le >> 5);
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    f32x4 wk, wv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        wk[e] = dkacc[ct][4 * gq + e] * scale;
                        wv[e] = dvacc[ct][4 * gq + e];
                    }
                    *reinterpret_cast<f32x4*>(Pk + 32 * ct + 8 * gq) = wk;
                    *reinterpret_cast<f32x4*>(Pv + 32 * ct + 8 * gq) = wv;
                }
        } else if (krow < N) {
            // per-lane row pointers from an opaque lane: hoisted out of the
            // item loop they would be spilled
            int le = lane;
            asm volatile("" : "+v"(le));
            const int64_t row = ((int64_t)b * Hkv + g) * N + kw + (le & 31);
            uint16_t* dKr = dK + row * D;
            uint16_t* dVr = dV + row * D;
            const float sk = DROP ? scale * drop.rkeep : scale;     // (dropout) r = 1/(1 - p) into both
            const float sv = DROP ? drop.rkeep : 1.f;
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int c = 32 * ct + 8 * gq + 4 * (le >> 5);
                    u32x2 wk, wv;
                    wk[0] = pack_bf16x2(dkacc[ct][4 * gq] * sk, dkacc[ct][4 * gq + 1] * sk);
                    wk[1] = pack_bf16x2(dkacc[ct][4 * gq + 2] * sk, dkacc[ct][4 * gq + 3] * sk);
                    if constexpr (DROP) {
                        wv[0] = pack_bf16x2(dvacc[ct][4 * gq] * sv, dvacc[ct][4 * gq + 1] * sv);
                        wv[1] = pack_bf16x2(dvacc[ct][4 * gq + 2] * sv, dvacc[ct][4 * gq + 3] * sv);
                    } else {
                        wv[0] = pack_bf16x2(dvacc[ct][4 * gq], dvacc[ct][4 * gq + 1]);
                        wv[1] = pack_bf16x2(dvacc[ct][4 * gq + 2], dvacc[ct][4 * gq + 3]);
                    }
                    *reinterpret_cast<u32x2*>(dKr + c) = wk;
                    *reinterpret_cast<u32x2*>(dVr + c) = wv;
                }
        }
    }
}

// ------------------------------------------------------------ dQ
//
// Same ping-pong schedule as the bf16 forward: waves w and w+4 share a SIMD,
// each wave alternates
//   G(t): dQ^T += K_{t-1}^T dS_{t-1}^T, then S_t^T = K_t Q^T, dP_t^T = V_t dO^T
//   X(t): P_t = exp2(c2 s - LSE log2 e), mask, dS_t = P_t (dP_t - D), pack
// and the two wave groups run one phase apart, a barrier after every phase.
template <int D>
struct QBf16Cfg {
    static constexpr int kWaves = 8;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BM = 32 * kWaves;      // query rows per workgroup
    static constexpr int BNK = 64;              // keys per tile
    static constexpr int kStages = 4;
    using KT = LdsTile<BNK, D, kWaves>;         // K (rows and transposed), V (rows)
    static constexpr int kStage = 2 * KT::kElems;
    static constexpr int kLoads = 2 * KT::kPerWave;
};

// G phase order: L = d/16 reads ahead; the dQ products (two transposed
// reads per fragment) first, then the S and dP products (one read each).
template <int D>
__device__ __forceinline__ void sched_dq_phase() {
    constexpr int L = D / 16;
#pragma unroll
    for (int i = 0; i < L; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < D / 4 - L; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < L; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// LOCAL (with CAUSAL): sliding window with S global tokens, key j visible to
// query i iff j <= i and (i - W < j or j < S); a query block's key tiles are
// the ns tiles holding global tokens left of its window, then the tiles from
// the first one its first row can see.
// BSP: block-sparse, row block mb sees the key blocks bidx[bptr[mb] ..
// bptr[mb+1]) (ascending, BM keys each), clamped as in the forward.
// DROP: through attention dropout, as in the dK/dV kernel: the workspace holds
// -D (1 - p), dS = r P o (Z ? dP + (-D (1 - p)) : -D (1 - p)) with the mask
// regenerated per element, and r = 1/(1 - p) goes into dQ's final scale.
template <int D, bool CAUSAL, bool LOCAL = false, bool BSP = false, bool DROP = false, bool SPLIT = false>
__global__ __launch_bounds__(QBf16Cfg<D>::kThreads, 2) void bwd_dq_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ WSd, const float* __restrict__ WSl,
    uint16_t* __restrict__ dQ, int B, int Hq, int Hkv, int n_rows, int Npad, float c2, float scale, int W,
    int S, const int* __restrict__ bptr, const int* __restrict__ bidx, int nnz, DropArgs drop, BspSplit sp) {
    static_assert(!(LOCAL && BSP), "one sparsity pattern at a time");
    static_assert(!(DROP && (LOCAL || BSP)), "dropout with the dense masks only");
    using Cfg = QBf16Cfg<D>;
    using KT = typename Cfg::KT;
    constexpr int NW = Cfg::kWaves, BM = Cfg::BM, BNK = Cfg::BNK, NS = Cfg::kStages, KB = BNK / 32;
    constexpr int kStage = Cfg::kStage, kLoads = Cfg::kLoads;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * kStage];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int grp = wave >> 2;                  // waves w and w+4 share a SIMD

    const int nmb = (n_rows + BM - 1) / BM;
    constexpr bool split = BSP && SPLIT;               // work items from sp.chunks
    const int nit = split ? sp.nchunks : nmb;            // work items per (batch, head)
    const PersistentSched sched(nit * Hq * B);
    for (int r = 0; sched.more(r); ++r) {
        const int lin = sched.item(r);
        if (lin < 0) continue;
        // the sequence length as an opaque per-item value: whatever derives
        // from it (tail clamps and masks) is computed per item, not hoisted
        // out of the item loop into registers for the whole kernel
        int N = n_rows;
        asm volatile("" : "+s"(N));
        const int mbi = lin % nit, bh = lin / nit;
        const int h = bh % Hq, b = bh / Hq;
        int mb = CAUSAL ? nmb - 1 - mbi : mbi;
        // (block-sparse) the item's entries bbeg .. bbeg+bcnt-1
        int bbeg = 0, bcnt = 0;
        if constexpr (BSP) {
            if (split) {
                const int* c = sp.chunks + 4 * mbi;
                mb = min(max(c[0], 0), nmb - 1);
                bbeg = min(max(c[1], 0), nnz);
                bcnt = min(max(c[2], bbeg), nnz) - bbeg;
            } else {
                bbeg = min(max(bptr[mb], 0), nnz);
                bcnt = min(max(bptr[mb + 1], bbeg), nnz) - bbeg;
            }
        }
        const int g = h / (Hq / Hkv);
        const int64_t rowbase = ((int64_t)b * Hq + h) * N;
        const uint16_t* Kg = K + ((int64_t)b * Hkv + g) * N * D;
        const uint16_t* Vg = V + ((int64_t)b * Hkv + g) * N * D;

        const int q0 = mb * BM;
        const int qw = q0 + 32 * wave;
        const int qrow = qw + l32;
        const int kend = CAUSAL ? min(N, q0 + BM) : N;
        const int ts = LOCAL ? max(0, q0 - W + 1) / BNK : 0;   // first window key tile
        const int ns = LOCAL ? min((S + BNK - 1) / BNK, ts) : 0;  // global-token tiles before it
        constexpr int TPB = BM / BNK;               // key tiles per mask block
        const int ntk = (N + BNK - 1) / BNK;
        auto bcol = [&](int e) __attribute__((always_inline)) { return min(max(bidx[bbeg + e], 0), nmb - 1); };
        auto tile_of = [&](int t) __attribute__((always_inline)) {
            return BSP ? min(bcol(t / TPB) * TPB + t % TPB, ntk - 1) : LOCAL ? (t < ns ? t : t - ns + ts) : t;
        };
        const int ntiles = BSP ? (bcnt ? TPB * (bcnt - 1) + min(TPB, ntk - bcol(bcnt - 1) * TPB) : 0)
                               : ns + (kend + BNK - 1) / BNK - ts;
        const int ntw = qw >= N ? 0 : CAUSAL && !BSP ? ns + (min(N, qw + 32) + BNK - 1) / BNK - ts : ntiles;

        // direct loads of tile t; the per-lane offsets are recomputed at every
        // issue from an opaque copy of the lane index (kept live across the
        // loop they would take registers the products need)
        auto issue = [&](int t) __attribute__((always_inline)) {
            const uint32_t st = lds_addr(smem + (t % NS) * kStage);
            const uint16_t* kb = Kg + (int64_t)tile_of(t) * BNK * D;
            const uint16_t* vb = Vg + (int64_t)tile_of(t) * BNK * D;
            const int rows_valid = N - tile_of(t) * BNK;
            int ln = lane;
            asm volatile("" : "+v"(ln));
#pragma unroll
            for (int i = 0; i < KT::kPerWave; ++i) {
                const int row = (i * NW + wave) * KT::RG + ln % KT::RG;
                const int grow = row < rows_valid ? row : rows_valid - 1;
                const uint32_t off = (uint32_t)(grow * D + (ln / KT::RG) * 8) * 2u;
                dma16s(kb, off, st + (i * NW + wave) * KT::RGS);
                dma16s(vb, off, st + KT::kBytes + (i * NW + wave) * KT::RGS);
            }
        };
#pragma unroll
        for (int t = 0; t < NS; ++t)
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
        const float dq_nd = qrow < N ? WSd[srow] : 0.f;     // the workspace holds -D
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            settle(qf[s]);
            settle(of[s]);
        }
        settle(lse2);
        settle(dq_nd);
        wait_vm<0>();

        f32x16 dqacc[D / 32];
#pragma unroll
        for (int i = 0; i < D / 32; ++i) dqacc[i] = zero16();
        f32x16 sacc[KB], dpacc[KB];
        u32x4 dsf[KB][2];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            sacc[kb] = dpacc[kb] = zero16();
            dsf[kb][0] = dsf[kb][1] = u32x4{};
        }

        // S^T = K_t Q^T and dP^T = V_t dO^T: rows = keys, columns = this wave's queries
        auto do_sdp = [&](int t) __attribute__((always_inline)) {
            const uint16_t* Ks = smem + (t % NS) * kStage;
            const uint16_t* Vs = Ks + KT::kElems;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sacc[kb] = dpacc[kb] = zero16();
#pragma unroll
            for (int s = 0; s < D / 16; ++s)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    sacc[kb] = mma_bf16(KT::row8(Ks, 32 * kb + l32, 2 * s + hh), qf[s], sacc[kb]);
                    dpacc[kb] = mma_bf16(KT::row8(Vs, 32 * kb + l32, 2 * s + hh), of[s], dpacc[kb]);
                }
        };
        // dQ^T += K_t^T dS_t^T
        auto do_dq = [&](int t) __attribute__((always_inline)) {
            const uint16_t* Ks = smem + (t % NS) * kStage;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                    for (int ct = 0; ct < D / 32; ++ct)
                        dqacc[ct] = mma_bf16(KT::tr8(Ks, 32 * kb + 16 * t2, 32 * ct, lane), dsf[kb][t2], dqacc[ct]);
        };
        // G(t), t >= 1 (past this wave's last tile the scores are discarded and
        // dS is zero)
        auto gemm = [&](int t) __attribute__((always_inline)) {
            do_dq(t - 1);
            do_sdp(t);
            sched_dq_phase<D>();
        };
        // X(t): P from the stored statistics; keys after the query (causal) or
        // past the end zeroed in one wave-uniform branch; dS packed to bf16
        auto softmax = [&](int t) __attribute__((always_inline)) {
            if (t >= ntw) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) dsf[kb][0] = dsf[kb][1] = u32x4{};
                return;
            }
            const int k0 = tile_of(t) * BNK;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = fast_exp2(fmaf(sacc[kb][r], c2, -lse2));
            if ((CAUSAL && k0 + BNK - 1 > qw) || (k0 + BNK > N) || (LOCAL && k0 < qw + 32 - W && k0 + BNK > S)) {
                // row indices from an opaque copy of the lane half: hoisted
                // out of the item loop, they and the masks derived from them
                // would stay live in registers
                int hm = hh;
                asm volatile("" : "+v"(hm));
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 32 * kb + acc_row(r, hm);
                        if ((CAUSAL && key > qrow) || key >= N || (LOCAL && key <= qrow - W && key >= S))
                            sacc[kb][r] = 0.f;
                    }
            }
            // (dropout) keys k0 + 32 kb + 8 gq + 4 hh + e (element 4 gq + e of
            // block kb): one Philox call per lane and 32-key block, shared by the quad
            uint32_t zw[DROP ? KB : 1][4];
            if constexpr (DROP) {
                int ln = lane;
                asm volatile("" : "+v"(ln));
                drop_words_qrow(zw, k0, qrow, ln >> 5, ln & 3, (uint32_t)(b * Hq + h), drop);
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                if constexpr (DROP) {
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 4 * gq + e;
                            const float x = dpacc[kb][r] + dq_nd;
                            dpacc[kb][r] = sacc[kb][r] * (drop_keep(zw[kb][gq], e, drop.thr) ? x : dq_nd);
                        }
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) dpacc[kb][r] = sacc[kb][r] * (dpacc[kb][r] + dq_nd);
                }
                dsf[kb][0] = pack_bf16x8(dpacc[kb], 0);
                dsf[kb][1] = pack_bf16x8(dpacc[kb], 8);
            }
            // dS is finished inside this phase (not sunk into the next matrix phase)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                settle(dsf[kb][0]);
                settle(dsf[kb][1]);
            }
        };

        // ---- phases (slot s ends with a barrier).  In loop round t both groups
        // refill the stage of tile t+2 (its previous tile, t-2, was last read in
        // slot 2t-1) at the start of their vector phase (slot 2t+1 for the first
        // group, 2t for the second; at its end, or in the matrix phase, is 0.5-2%
        // and 3-6% slower); before the barrier ending odd slot s, tile (s+1)/2
        // has landed (one later tile may still be in flight).
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
            // G(t) in slot 2t, X(t) in slot 2t + 1
            do_sdp(0);
            lds_barrier();
            softmax(0);
            tail_odd(1);
            for (int t = 1; t <= ntiles; ++t) {
                gemm(t);
                lds_barrier();
                refill(t);
                softmax(t);
                tail_odd(2 * t + 1);
            }
        } else {
            // X(t-1) in slot 2t, G(t) in slot 2t + 1
            lds_barrier();
            do_sdp(0);
            tail_odd(1);
            for (int t = 1; t <= ntiles; ++t) {
                refill(t);
                softmax(t - 1);
                lds_barrier();
                gemm(t);
                tail_odd(2 * t + 1);
            }
        }

        // (split row) the partial slot, read here rather than kept live
        int slot = -1;
        if (split) slot = sp.chunks[4 * mbi + 3] < sp.nslots ? sp.chunks[4 * mbi + 3] : -1;
        if (BSP && slot >= 0 && qrow < N) {
            // (split row) this item's share of dQ, float32, for the merge; row
            // pointer from an opaque lane, as below
            int le = lane;
            asm volatile("" : "+v"(le));
            float* P = sp.part + (((int64_t)slot * B * Hq + bh) * BM + 32 * wave + (le & 31)) * D + 4 * (le >> 5);
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    f32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = dqacc[ct][4 * gq + e] * scale;
                    *reinterpret_cast<f32x4*>(P + 32 * ct + 8 * gq) = w;
                }
        } else if (qrow < N) {
            // per-lane row pointer from an opaque lane: hoisted out of the
            // item loop it would be spilled
            int le = lane;
            asm volatile("" : "+v"(le));
            uint16_t* dQr = dQ + (rowbase + qw + (le & 31)) * D + 4 * (le >> 5);
            const float sq = DROP ? scale * drop.rkeep : scale;     // (dropout) r = 1/(1 - p)
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

template <int D, bool CAUSAL, bool LOCAL = false, bool BSP = false, bool DROP = false, bool SPLIT = false>
static hipError_t launch_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* ws,
                              void* dk, void* dv, int B, int Hq, int Hkv, int N, float scale, hipStream_t st,
                              int W = 0, int S = 0, const int* bptr = nullptr, const int* bidx = nullptr,
                              int nnz = 0, DropArgs drop = {0u, 0u, 0u, 1.f},
                              BspSplit sp = {nullptr, 0, 0, nullptr}) {
    using Cfg = KVBf16Cfg<D>;
    const int nkb = (N + Cfg::BNK - 1) / Cfg::BNK;
    const int nit = BSP && SPLIT ? sp.nchunks : nkb;
    const int Np = ws_rows(N);
    static PerDevice slots;
    const int grid = persistent_grid((const void*)bwd_dkdv_bf16_kernel<D, CAUSAL, LOCAL, BSP, DROP, SPLIT>,
                                     Cfg::kThreads, nit * Hkv * B, slots);
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, CAUSAL, LOCAL, BSP, DROP, SPLIT>), dim3((unsigned)grid),
                       dim3(Cfg::kThreads), 0, st, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)dO, ws, ws + (int64_t)B * Hq * Np, (uint16_t*)dk, (uint16_t*)dv, B, Hq, Hkv, N,
                       Np, scale * kLog2e, scale, W, S, bptr, bidx, nnz, drop, sp);
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool LOCAL = false, bool BSP = false, bool DROP = false, bool SPLIT = false>
static hipError_t launch_dq(const void* q, const void* k, const void* v, const void* dO, const float* ws, void* dq,
                            int B, int Hq, int Hkv, int N, float scale, hipStream_t st, int W = 0, int S = 0,
                            const int* bptr = nullptr, const int* bidx = nullptr, int nnz = 0,
                            DropArgs drop = {0u, 0u, 0u, 1.f}, BspSplit sp = {nullptr, 0, 0, nullptr}) {
    using Cfg = QBf16Cfg<D>;
    const int nmb = (N + Cfg::BM - 1) / Cfg::BM;
    const int nit = BSP && SPLIT ? sp.nchunks : nmb;
    const int Np = ws_rows(N);
    static PerDevice slots;
    const int grid = persistent_grid((const void*)bwd_dq_bf16_kernel<D, CAUSAL, LOCAL, BSP, DROP, SPLIT>, Cfg::kThreads,
                                     nit * Hq * B, slots);
    hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, CAUSAL, LOCAL, BSP, DROP, SPLIT>), dim3((unsigned)grid),
                       dim3(Cfg::kThreads), 0, st, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)dO, ws, ws + (int64_t)B * Hq * Np, (uint16_t*)dq, B, Hq, Hkv, N, Np,
                       scale * kLog2e, scale, W, S, bptr, bidx, nnz, drop, sp);
    return hipGetLastError();
}

// Sum of a split block's float32 partials into a bf16 output (block-sparse
// backward): merge m = merges[4m .. 4m+2] = (block r, first slot s0, slot
// count ns); rows r * 256 .. of each of the nh heads (the query heads for dQ,
// the K/V heads for dK and dV) get sum_s part[s0 + s][head][row].  One
// workgroup per (merge, head, run of 256 / (D/8) rows); a thread per 8
// columns of a row.
template <int D>
__global__ __launch_bounds__(256) void bsp_merge_sum_kernel(const int* __restrict__ merges, int nmerge,
                                                            const float* __restrict__ part, int nslots,
                                                            uint16_t* __restrict__ out, int nh, int N) {
    constexpr int BR = 256, CPR = D / 8, RB = 256 / CPR;
    const int mi = blockIdx.x % nmerge, hd = (blockIdx.x / nmerge) % nh, rb = blockIdx.x / nmerge / nh;
    const int nb = (N + BR - 1) / BR;
    const int r = min(max(merges[4 * mi], 0), nb - 1);
    const int s0 = min(max(merges[4 * mi + 1], 0), nslots);
    const int ns = min(max(merges[4 * mi + 2], 0), nslots - s0);
    {
        const int row = rb * RB + threadIdx.x / CPR, c8 = (threadIdx.x % CPR) * 8;
        const int i = r * BR + row;
        if (i >= N) return;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < ns; ++s) {
            const float* p = part + (((int64_t)(s0 + s) * nh + hd) * BR + row) * D + c8;
            const f32x4 a = *reinterpret_cast<const f32x4*>(p), c = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] += a[e];
                acc[4 + e] += c[e];
            }
        }
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
        *reinterpret_cast<u32x4*>(out + ((int64_t)hd * N + i) * D + c8) = w;
    }
}

static hipError_t launch_merge_sum(int d, const int* merges, int nmerge, const float* part, int nslots, void* out,
                                   int nh, int N, hipStream_t st) {
    if (nmerge <= 0) return hipSuccess;
    // 256 rows per block, 256 / (d/8) rows per workgroup
    if (d == 64)
        hipLaunchKernelGGL(bsp_merge_sum_kernel<64>, dim3((unsigned)(nmerge * nh * 8)), dim3(256), 0, st, merges,
                           nmerge, part, nslots, (uint16_t*)out, nh, N);
    else
        hipLaunchKernelGGL(bsp_merge_sum_kernel<128>, dim3((unsigned)(nmerge * nh * 16)), dim3(256), 0, st, merges,
                           nmerge, part, nslots, (uint16_t*)out, nh, N);
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

hipError_t launch_bwd_dkdv_bf16_local(int d, const void* q, const void* k, const void* v, const void* dO,
                                      const float* ws, void* dk, void* dv, int B, int Hq, int Hkv, int N, int W,
                                      int S, float scale, hipStream_t st) {
    if (d == 64) return launch_dkdv<64, true, true>(q, k, v, dO, ws, dk, dv, B, Hq, Hkv, N, scale, st, W, S);
    if (d == 128) return launch_dkdv<128, true, true>(q, k, v, dO, ws, dk, dv, B, Hq, Hkv, N, scale, st, W, S);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_bf16_bsparse(int d, int causal, const void* q, const void* k, const void* v, const void* dO,
                                   const float* ws, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                                   const int* row_ptr, const int* col_idx, const int* col_ptr, const int* row_idx,
                                   int nnz, float scale, hipStream_t st) {
#define KV q, k, v, dO, ws, dk, dv, B, Hq, Hkv, N, scale, st, 0, 0, col_ptr, row_idx, nnz
#define QA q, k, v, dO, ws, dq, B, Hq, Hkv, N, scale, st, 0, 0, row_ptr, col_idx, nnz
    hipError_t e = hipErrorInvalidValue;
    if (d == 64) e = causal ? launch_dkdv<64, true, false, true>(KV) : launch_dkdv<64, false, false, true>(KV);
    if (d == 128) e = causal ? launch_dkdv<128, true, false, true>(KV) : launch_dkdv<128, false, false, true>(KV);
    if (e != hipSuccess) return e;
    if (d == 64) return causal ? launch_dq<64, true, false, true>(QA) : launch_dq<64, false, false, true>(QA);
    return causal ? launch_dq<128, true, false, true>(QA) : launch_dq<128, false, false, true>(QA);
#undef KV
#undef QA
}

hipError_t launch_bwd_bf16_bsparse_split(int d, int causal, const void* q, const void* k, const void* v,
                                         const void* dO, const float* ws, void* dq, void* dk, void* dv, int B, int Hq,
                                         int Hkv, int N, const int* col_idx, const int* row_idx, int nnz,
                                         const int* row_chunks, int n_row_chunks, const int* row_merges,
                                         int n_row_merges, int n_row_slots, const int* col_chunks, int n_col_chunks,
                                         const int* col_merges, int n_col_merges, int n_col_slots, float* part,
                                         float scale, hipStream_t st) {
    // partials: dQ [n_row_slots][B Hq][256][d], then dK and dV [n_col_slots][B Hkv][256][d] each
    float* pq = part;
    float* pkv = part + (int64_t)n_row_slots * B * Hq * 256 * d;
    const BspSplit sq{row_chunks, n_row_chunks, n_row_slots, pq}, skv{col_chunks, n_col_chunks, n_col_slots, pkv};
    const DropArgs nd{0u, 0u, 0u, 1.f};
#define KV q, k, v, dO, ws, dk, dv, B, Hq, Hkv, N, scale, st, 0, 0, nullptr, row_idx, nnz, nd, skv
#define QA q, k, v, dO, ws, dq, B, Hq, Hkv, N, scale, st, 0, 0, nullptr, col_idx, nnz, nd, sq
    hipError_t e = hipErrorInvalidValue;
    if (d == 64)
        e = causal ? launch_dkdv<64, true, false, true, false, true>(KV)
                   : launch_dkdv<64, false, false, true, false, true>(KV);
    if (d == 128)
        e = causal ? launch_dkdv<128, true, false, true, false, true>(KV)
                   : launch_dkdv<128, false, false, true, false, true>(KV);
    if (e == hipSuccess) e = launch_merge_sum(d, col_merges, n_col_merges, pkv, n_col_slots, dk, B * Hkv, N, st);
    if (e == hipSuccess)
        e = launch_merge_sum(d, col_merges, n_col_merges, pkv + (int64_t)n_col_slots * B * Hkv * 256 * d, n_col_slots,
                             dv, B * Hkv, N, st);
    if (e != hipSuccess) return e;
    if (d == 64)
        e = causal ? launch_dq<64, true, false, true, false, true>(QA) : launch_dq<64, false, false, true, false, true>(QA);
    else
        e = causal ? launch_dq<128, true, false, true, false, true>(QA)
                   : launch_dq<128, false, false, true, false, true>(QA);
    if (e == hipSuccess) e = launch_merge_sum(d, row_merges, n_row_merges, pq, n_row_slots, dq, B * Hq, N, st);
    return e;
#undef KV
#undef QA
}

hipError_t launch_bwd_dq_bf16_local(int d, const void* q, const void* k, const void* v, const void* dO,
                                    const float* ws, void* dq, int B, int Hq, int Hkv, int N, int W, int S,
                                    float scale, hipStream_t st) {
    if (d == 64) return launch_dq<64, true, true>(q, k, v, dO, ws, dq, B, Hq, Hkv, N, scale, st, W, S);
    if (d == 128) return launch_dq<128, true, true>(q, k, v, dO, ws, dq, B, Hq, Hkv, N, scale, st, W, S);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_bf16_dropout(int d, int causal, const void* q, const void* k, const void* v, const void* dO,
                                   const float* ws, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                                   uint32_t thr, uint64_t seed, float rkeep, float scale, hipStream_t st) {
    const DropArgs dr{thr, (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32), rkeep};
#define KV q, k, v, dO, ws, dk, dv, B, Hq, Hkv, N, scale, st, 0, 0, nullptr, nullptr, 0, dr
#define QA q, k, v, dO, ws, dq, B, Hq, Hkv, N, scale, st, 0, 0, nullptr, nullptr, 0, dr
    hipError_t e = hipErrorInvalidValue;
    if (d == 64) e = causal ? launch_dkdv<64, true, false, false, true>(KV) : launch_dkdv<64, false, false, false, true>(KV);
    if (d == 128)
        e = causal ? launch_dkdv<128, true, false, false, true>(KV) : launch_dkdv<128, false, false, false, true>(KV);
    if (e != hipSuccess) return e;
    if (d == 64) return causal ? launch_dq<64, true, false, false, true>(QA) : launch_dq<64, false, false, false, true>(QA);
    return causal ? launch_dq<128, true, false, false, true>(QA) : launch_dq<128, false, false, false, true>(QA);
#undef KV
#undef QA
}

}  // namespace fa
