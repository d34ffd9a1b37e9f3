// bf16 forward pass of exact attention (the tuned path; float32 uses fa_fwd.hip).
//
// "flash attention io aware", sections "Flash Attention Algorithm" and "Online
// Softmax"; the FlashAttention legal glossary's online-softmax and
// FlashAttention-2 paragraphs (one workgroup per query block, head and batch;
// fewer non-matmul operations).  What differs from the pages' CUDA design is
// how the same steps map onto gfx950:
//  - K and V tiles go from HBM straight into LDS (global_load_lds, no staging
//    registers) in their global row-major layout, four tiles resident or in
//    flight;
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
//
// Schedule ("ping-pong").  A gfx950 SIMD runs the matrix instructions of one
// wave and the vector instructions of another side by side, but a single wave
// issues a vector instruction only about every 8 cycles, so a wave that
// interleaves its own exponentials with its own products leaves one of the
// two units idle much of the time.  Each wave therefore alternates two phases:
//   G(t): S_t = K_t Q^T and O += P_{t-1} V_{t-1}   (32 products at d = 128)
//   X(t): mask, row max, rescale, P_t = exp2(...), pack, row sum (vector only)
// and the workgroup's two wave groups (waves w and w+4 share a SIMD) run one
// phase apart with a barrier after every phase: on each SIMD one wave feeds
// the matrix core while the other does the softmax of its previous tile.
// Inside G the LDS fragment reads are scheduled about d/16 fragments ahead of
// the products that consume them.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

template <int D>
struct FwdBf16Cfg {
    static constexpr int kWaves = 8;                  // two groups of four, one wave of each per SIMD
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BM = 32 * kWaves;            // query rows per workgroup (32 per wave)
    static constexpr int BN = 64;                     // keys per K/V tile
    static constexpr int kStages = 4;                 // K/V tiles resident or in flight
    using KT = LdsTile<BN, D, kWaves>;                // K read as rows, V read transposed
    static constexpr int kStage = 2 * KT::kElems;     // elements per stage (K then V)
    static constexpr int kLoads = 2 * KT::kPerWave;   // direct loads per wave per tile
    static constexpr float kTau = 8.0f;               // log2 slack before the max is moved
};

// Order of one G phase for the instruction scheduler: L = d/16 K fragments
// read ahead of the score products, then V^T fragments (two reads each) about
// L fragments ahead of theirs.
template <int D>
__device__ __forceinline__ void sched_gemm_phase() {
    constexpr int L = D / 16;
#pragma unroll
    for (int i = 0; i < L; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // LDS read
#pragma unroll
    for (int i = 0; i < L; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < 2 * L; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < L; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// LOCAL (with CAUSAL): sliding-window attention with S global tokens, key j
// visible to query i iff j <= i and (i - W < j or j < S) (the FlashAttention
// legal glossary, entry "Block-sparse": sliding-window local attention and
// global tokens, whole tiles outside the pattern skipped).  A workgroup's
// tiles are the ns tiles holding global tokens left of its window, then the
// tiles from ts, the first one holding a key its first query row can see;
// other keys left of a row's window are masked like those past the diagonal.
//
// BSP: block-sparse attention (same glossary entry: a mask over BM x BM blocks
// of the score matrix, the blocks that are off never computed).  Row block mb
// sees the key blocks bidx[bptr[mb] .. bptr[mb+1]), ascending, BM / BN tiles
// each; with CAUSAL the keys past the diagonal are masked as well.  Offsets are
// clamped to [0, nnz) and block indices to the block count, so any layout keeps
// every access in bounds.  A row that sees no key gets O = 0 and LSE = -inf.
// DROP: attention dropout on the normalised probabilities (the FlashAttention
// page of the self-hosted LLM glossary: dropout is one of the operations fused
// into the kernel).  The normaliser and LSE are those of the undropped softmax;
// kept probabilities are scaled by 1 / (1 - p), p = thr / 256 (DropArgs).
template <int D, bool CAUSAL, bool LOCAL = false, bool BSP = false, bool DROP = false, bool SPLIT = false>
__global__ __launch_bounds__(FwdBf16Cfg<D>::kThreads, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int N, float c2, int W,
    int S, const int* __restrict__ bptr, const int* __restrict__ bidx, int nnz, DropArgs drop, BspSplit sp) {
    static_assert(!(LOCAL && BSP), "one sparsity pattern at a time");
    using Cfg = FwdBf16Cfg<D>;
    using KT = typename Cfg::KT;
    constexpr int NW = Cfg::kWaves, BM = Cfg::BM, BN = Cfg::BN, NS = Cfg::kStages, KB = BN / 32;
    constexpr int kStage = Cfg::kStage;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * kStage];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: phase branches stay scalar
    const int grp = wave >> 2;                                           // waves w and w+4 share a SIMD

    const int nmb = (N + BM - 1) / BM;
    constexpr bool split = BSP && SPLIT;               // work items from sp.chunks
    const int nit = split ? sp.nchunks : nmb;            // work items per (batch, head)
    const PersistentSched sched(nit * Hq * B);
    for (int r = 0; sched.more(r); ++r) {
        const int lin = sched.item(r);
        if (lin < 0) continue;
        const int lane = threadIdx.x & 63;
        const int l32 = lane & 31, hh = lane >> 5;
        const int mbi = lin % nit, bh = lin / nit;
        const int h = bh % Hq, b = bh / Hq;
        int mb = CAUSAL ? nmb - 1 - mbi : mbi;            // longest causal rows first
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
        const uint16_t* Qh = Q + ((int64_t)b * Hq + h) * N * D;
        const uint16_t* Kh = K + ((int64_t)b * Hkv + g) * N * D;
        const uint16_t* Vh = V + ((int64_t)b * Hkv + g) * N * D;

        const int q0 = mb * BM;
        const int qw = q0 + 32 * wave;                    // first query row of this wave
        const int qrow = qw + l32;                        // this lane's query row
        const int kend = CAUSAL ? min(N, q0 + BM) : N;
        const int ts = LOCAL ? max(0, q0 - W + 1) / BN : 0;   // first window tile of the workgroup
        const int ns = LOCAL ? min((S + BN - 1) / BN, ts) : 0;    // global-token tiles before it
        constexpr int TPB = BM / BN;                      // tiles per mask block
        const int ntk = (N + BN - 1) / BN;
        auto bcol = [&](int e) __attribute__((always_inline)) { return min(max(bidx[bbeg + e], 0), nmb - 1); };
        // the workgroup's t-th tile: tiles 0 .. ns-1, then ts, ts+1, ... (local);
        // tile t % TPB of the (t / TPB)-th listed block (block-sparse)
        auto tile_of = [&](int t) __attribute__((always_inline)) {
            return BSP ? min(bcol(t / TPB) * TPB + t % TPB, ntk - 1) : LOCAL ? (t < ns ? t : t - ns + ts) : t;
        };
        const int ntiles = BSP ? (bcnt ? TPB * (bcnt - 1) + min(TPB, ntk - bcol(bcnt - 1) * TPB) : 0)
                               : ns + (kend + BN - 1) / BN - ts;    // tiles of the workgroup
        const int ntw = qw >= N ? 0 : CAUSAL && !BSP ? ns + (min(N, qw + 32) + BN - 1) / BN - ts : ntiles;   // tiles of this wave

        // ---- direct loads: this wave's row groups of a K/V tile, as byte offsets
        // from the tile's first row (rows past the end re-read the last row)
        uint32_t voff[KT::kPerWave];
#pragma unroll
        for (int i = 0; i < KT::kPerWave; ++i) {
            const int row = (i * NW + wave) * KT::RG + lane % KT::RG;
            voff[i] = (uint32_t)(row * D + (lane / KT::RG) * 8) * 2u;
        }
        // half = 0: the K rows of tile t, 1: its V rows
        auto issue_half = [&](int t, const int half) __attribute__((always_inline)) {
            const uint32_t st = lds_addr(smem + (t % NS) * kStage) + half * KT::kBytes;
            const uint16_t* src = (half ? Vh : Kh) + (int64_t)tile_of(t) * BN * D;
            const int rows_valid = N - tile_of(t) * BN;
            if (rows_valid >= BN) {
#pragma unroll
                for (int i = 0; i < KT::kPerWave; ++i) dma16s(src, voff[i], st + (i * NW + wave) * KT::RGS);
            } else {
#pragma unroll
                for (int i = 0; i < KT::kPerWave; ++i) {
                    const int row = (i * NW + wave) * KT::RG + lane % KT::RG;
                    const int grow = row < rows_valid ? row : rows_valid - 1;
                    const uint32_t off = (uint32_t)(grow * D + (lane / KT::RG) * 8) * 2u;
                    dma16s(src, off, st + (i * NW + wave) * KT::RGS);
                }
            }
        };
        auto issue = [&](int t) __attribute__((always_inline)) {
            issue_half(t, 0);
            issue_half(t, 1);
        };
        // the same half tile for this wave's row groups and its partner's (the
        // other wave on this SIMD, four waves away: four row groups further)
        auto issue_half_pair = [&](int t, const int half) __attribute__((always_inline)) {
            const uint32_t st = lds_addr(smem + (t % NS) * kStage) + half * KT::kBytes;
            const uint16_t* src = (half ? Vh : Kh) + (int64_t)tile_of(t) * BN * D;
            const int rows_valid = N - tile_of(t) * BN;
            const int w0 = wave & 3;
            if (rows_valid >= BN) {
#pragma unroll
                for (int i = 0; i < KT::kPerWave; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int w = w0 + 4 * j;
                        dma16s(src, voff[i] + (uint32_t)((w - wave) * KT::RG * D * 2), st + (i * NW + w) * KT::RGS);
                    }
            } else {
#pragma unroll
                for (int i = 0; i < KT::kPerWave; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int w = w0 + 4 * j;
                        const int row = (i * NW + w) * KT::RG + lane % KT::RG;
                        const int grow = row < rows_valid ? row : rows_valid - 1;
                        const uint32_t off = (uint32_t)(grow * D + (lane / KT::RG) * 8) * 2u;
                        dma16s(src, off, st + (i * NW + w) * KT::RGS);
                    }
            }
        };
        // the first NS tiles go in flight while Q is fetched
#pragma unroll
        for (int t = 0; t < NS; ++t)
            if (t < ntiles) issue(t);

        u32x4 qf[D / 16];                                 // Q block as B operands, for the whole kernel
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            u32x4 v = {};
            if (qrow < N) v = *reinterpret_cast<const u32x4*>(Qh + (int64_t)qrow * D + 16 * s + 8 * hh);
            qf[s] = v;
        }
#pragma unroll
        for (int s = 0; s < D / 16; ++s) settle(qf[s]);
        wait_vm<0>();

        f32x16 oacc[D / 32];
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();
        float m = kNegBig, lsum = 0.f;
        f32x16 sacc[KB];
        u32x4 pf[KB][2];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            sacc[kb] = zero16();
            pf[kb][0] = pf[kb][1] = u32x4{};
        }

        // S^T = K_t Q^T (stage t % NS): rows = keys, columns = this wave's queries
        auto do_s = [&](int t) __attribute__((always_inline)) {
            const uint16_t* Ks = smem + (t % NS) * kStage;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sacc[kb] = zero16();
#pragma unroll
            for (int s = 0; s < D / 16; ++s)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) sacc[kb] = mma_bf16(KT::row8(Ks, 32 * kb + l32, 2 * s + hh), qf[s], sacc[kb]);
        };
        // O^T += V_t^T P_t^T
        auto do_pv = [&](int t) __attribute__((always_inline)) {
            const uint16_t* Vs = smem + (t % NS) * kStage + KT::kElems;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                    for (int ct = 0; ct < D / 32; ++ct)
                        oacc[ct] = mma_bf16(KT::tr8(Vs, 32 * kb + 16 * t2, 32 * ct, lane), pf[kb][t2], oacc[ct]);
        };
        // G(t), t >= 1: scores of tile t (past this wave's last tile they are
        // discarded) and the product of tile t-1 (P is zero past the last
        // tile).  Causal: past t = ntw both are void and the wave skips the
        // phase; the slot takes as long, but the matrix cores spend no power
        // on it.
        auto gemm = [&](int t) __attribute__((always_inline)) {
            if (CAUSAL && t > ntw) return;
            do_s(t);
            do_pv(t - 1);
            sched_gemm_phase<D>();
        };
        // X(t)
        auto softmax = [&](int t) __attribute__((always_inline)) {
            if (t >= ntw) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) pf[kb][0] = pf[kb][1] = u32x4{};
                return;
            }
            const int k0 = tile_of(t) * BN;
            // ---- keys past the diagonal (causal), past the end, or (local)
            // left of some row's window and not global
            if ((CAUSAL && k0 + BN - 1 > qw) || k0 + BN > N || (LOCAL && k0 < qw + 32 - W && k0 + BN > S)) {
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
                            sacc[kb][r] = -INFINITY;
                    }
            }
            // ---- running max (base 2, scale*log2(e) in c2); moved only when some
            // row of the wave grew by more than 2^tau
            float x = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) x = fmaxf(x, sacc[kb][r]);
            x = pair_max(x);
            const float mnew = fmaxf(m, x * c2);
            if (__any(mnew > m + Cfg::kTau)) {
                const float alpha = fast_exp2(m - mnew);
                m = mnew;
                lsum *= alpha;
#pragma unroll
                for (int ct = 0; ct < D / 32; ++ct) oacc[ct] *= alpha;
            }
            // ---- P = exp2(c2 s - m), packed to bf16; l sums the rounded values
            float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][r] = fast_exp2(fmaf(sacc[kb][r], c2, -m));
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2) {
                    pf[kb][t2] = pack_bf16x8(sacc[kb], 8 * t2);
#pragma unroll
                    for (int i = 0; i < 4; ++i) rs[i] = dot2_bf16_sum(pf[kb][t2][i], rs[i]);
                }
            }
            lsum += (rs[0] + rs[1]) + (rs[2] + rs[3]);
            if constexpr (DROP) {
                // one Philox call per lane and 32-key block, shared by the quad
                const uint32_t bhq = (uint32_t)(b * Hq + h);
                int ln = lane;
                asm volatile("" : "+v"(ln));
                uint32_t zw[KB][4];
                drop_words_qrow(zw, k0, qrow, hh, ln & 3, bhq, drop);
                // the packed pair of elements 2c, 2c + 1 is cleared half by half:
                // bytes e, e + 1 of the keep word zero-extended to 16 bits, minus
                // thr, are negative exactly where dropped; the sign spread over
                // the half is the clearing mask (packed 16-bit integer arithmetic)
                const s16x2 thr2 = {(short)drop.thr, (short)drop.thr};
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const uint32_t w = zw[kb][c >> 1];
                        const uint32_t x = __builtin_amdgcn_perm(0u, w, (c & 1) ? 0x0c030c02u : 0x0c010c00u);
                        const s16x2 y = __builtin_bit_cast(s16x2, x) - thr2;
                        const uint32_t m = __builtin_bit_cast(uint32_t, (s16x2)(y >> (short)15));
                        pf[kb][c >> 2][c & 3] &= ~m;
                    }
            }
            // P is finished inside this phase (not sunk into the next matrix phase)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                settle(pf[kb][0]);
                settle(pf[kb][1]);
            }
        };

        // ---- phases.  Slot s ends with a barrier.  For tile u >= NS the K rows
        // are loaded at the start of slot 2u - 4 and the V rows at the start of
        // slot 2u - 3 (the stage's previous tile, u - NS, was last read as K in
        // slot 2u - 7 and as V in slot 2u - 5), so every slot carries half a
        // tile of loads.  They are issued by the wave group that starts its
        // vector phase in that slot (the second group the K rows in even
        // slots, the first group the V rows in odd slots), each wave for its
        // partner too, so that no load waits for the load path in the matrix
        // phase (6% faster at the causal 4096 workload than every wave issuing
        // its own rows in both phases).  Before the barrier ending odd slot
        // 2tv - 1, K_tv and V_tv-1 have landed: the second group waits for its
        // K_tv (K_tv+1 may still be in flight), the first for its V_tv-1 (V_tv
        // and V_tv+1 may be); the V rows of the last tile are waited for before
        // the barrier ending slot 2 ntiles - 1, ahead of their one read.
        auto head = [&](int s) __attribute__((always_inline)) {
            const int u = (s >> 1) + 2;
            if (s >= 4 && u < ntiles && grp != (s & 1)) issue_half_pair(u, s & 1);
        };
        auto tail_odd = [&](int s) __attribute__((always_inline)) {
            const int tv = (s + 1) / 2;
            if (tv >= NS && tv < ntiles) {
                if (grp == 1) {
                    if (tv + 1 < ntiles) wait_vm<2 * KT::kPerWave>();
                    else wait_vm<0>();
                } else {
                    if (tv + 1 < ntiles) wait_vm<4 * KT::kPerWave>();
                    else wait_vm<2 * KT::kPerWave>();
                }
            } else if (tv == ntiles && ntiles > NS) {
                wait_vm<0>();                         // V of the last tile (read in G(ntiles))
            }
            lds_barrier();
        };
        lds_barrier();
        if (grp == 0) {
            // G(t) in slot 2t, X(t) in slot 2t + 1
            do_s(0);
            lds_barrier();
            softmax(0);
            tail_odd(1);
            for (int t = 1; t <= ntiles; ++t) {
                head(2 * t);
                gemm(t);
                lds_barrier();
                head(2 * t + 1);
                softmax(t);                               // t == ntiles: past every wave's last tile
                tail_odd(2 * t + 1);
            }
        } else {
            // X(t-1) in slot 2t, G(t) in slot 2t + 1
            lds_barrier();
            do_s(0);
            tail_odd(1);
            for (int t = 1; t <= ntiles; ++t) {
                head(2 * t);
                softmax(t - 1);
                lds_barrier();
                head(2 * t + 1);
                gemm(t);
                tail_odd(2 * t + 1);
            }
        }

        // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l)
        const float ltot = pair_sum(lsum);
        // (split row) the partial slot, read here rather than kept live
        int slot = -1;
        if (split) slot = sp.chunks[4 * mbi + 3] < sp.nslots ? sp.chunks[4 * mbi + 3] : -1;
        if (BSP && slot >= 0 && qrow < N) {
            // (split row) this item's O and base-2 log-sum-exp, float32, for the merge
            const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
            const int64_t prow = ((int64_t)slot * B * Hq + bh) * BM + (qrow - q0);
            float* Op = sp.part + prow * D;
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    f32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = oacc[ct][4 * gq + e] * inv;
                    *reinterpret_cast<f32x4*>(Op + 32 * ct + 8 * gq + 4 * hh) = w;
                }
            if (hh == 0) sp.part[(int64_t)sp.nslots * B * Hq * BM * D + prow] = ltot > 0.f ? m + log2f(ltot) : -INFINITY;
        } else if (qrow < N) {
            float inv = BSP && !(ltot > 0.f) ? 0.f : 1.0f / ltot;   // (block-sparse) a row with no key: O = 0
            if constexpr (DROP) inv *= drop.rkeep;
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
            if (hh == 0)
                LSE[((int64_t)b * Hq + h) * N + qrow] = BSP && !(ltot > 0.f) ? -INFINITY : (m + log2f(ltot)) * kLn2;
        }
    }
}

template <int D, bool CAUSAL, bool LOCAL = false, bool BSP = false, bool DROP = false, bool SPLIT = false>
static hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                         int N, float scale, hipStream_t st, int W = 0, int S = 0, const int* bptr = nullptr,
                         const int* bidx = nullptr, int nnz = 0, DropArgs drop = {0u, 0u, 0u, 1.f},
                         BspSplit sp = {nullptr, 0, 0, nullptr}) {
    using Cfg = FwdBf16Cfg<D>;
    const int nmb = (N + Cfg::BM - 1) / Cfg::BM;
    const int nit = BSP && SPLIT ? sp.nchunks : nmb;
    static PerDevice slots;
    const int grid = persistent_grid((const void*)fwd_bf16_kernel<D, CAUSAL, LOCAL, BSP, DROP, SPLIT>, Cfg::kThreads,
                                     nit * Hq * B, slots);
    hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, LOCAL, BSP, DROP, SPLIT>), dim3((unsigned)grid), dim3(Cfg::kThreads), 0,
                       st, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)o, lse, B, Hq, Hkv,
                       N, scale * kLog2e, W, S, bptr, bidx, nnz, drop, sp);
    return hipGetLastError();
}

// Merge of a split row block's partials (block-sparse forward): merge m =
// merges[4m .. 4m+2] = (row block r, first slot s0, slot count ns).  With
// L_s the base-2 log-sum-exp and O_s the output of slot s over its keys:
// L = log2 sum_s 2^L_s, O = sum_s 2^(L_s - L) O_s, LSE = L ln 2 (the online
// softmax's rescale, applied once per slot).  A row no slot saw: O = 0,
// LSE = -inf.  One workgroup per (merge, batch x head, run of 256 / (D/8)
// rows); a thread per 8 columns of a row.
template <int D>
__global__ __launch_bounds__(256) void bsp_merge_fwd_kernel(const int* __restrict__ merges, int nmerge,
                                                            const float* __restrict__ part, int nslots,
                                                            uint16_t* __restrict__ O, float* __restrict__ LSE, int BH,
                                                            int N) {
    constexpr int BM = FwdBf16Cfg<D>::BM, CPR = D / 8, RB = 256 / CPR, NRB = BM / RB;
    const int mi = blockIdx.x % nmerge, bh = (blockIdx.x / nmerge) % BH, rb = blockIdx.x / nmerge / BH;
    const int nmb = (N + BM - 1) / BM;
    const int r = min(max(merges[4 * mi], 0), nmb - 1);
    const int s0 = min(max(merges[4 * mi + 1], 0), nslots);
    const int ns = min(max(merges[4 * mi + 2], 0), nslots - s0);
    const float* Lp = part + (int64_t)nslots * BH * BM * D;
    static_assert(NRB * RB == BM, "rows split evenly over the workgroups");
    {
        const int row = rb * RB + threadIdx.x / CPR, c8 = (threadIdx.x % CPR) * 8;
        const int i = r * BM + row;
        if (i >= N) return;
        float lmax = -INFINITY;
        for (int s = 0; s < ns; ++s) lmax = fmaxf(lmax, Lp[((int64_t)(s0 + s) * BH + bh) * BM + row]);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, wsum = 0.f;
        if (lmax > -INFINITY) {
            for (int s = 0; s < ns; ++s) {
                const int64_t prow = ((int64_t)(s0 + s) * BH + bh) * BM + row;
                const float wgt = exp2f(Lp[prow] - lmax);
                const f32x4 a = *reinterpret_cast<const f32x4*>(part + prow * D + c8);
                const f32x4 c = *reinterpret_cast<const f32x4*>(part + prow * D + c8 + 4);
                wsum += wgt;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[e] += wgt * a[e];
                    acc[4 + e] += wgt * c[e];
                }
            }
        }
        const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
        *reinterpret_cast<u32x4*>(O + ((int64_t)bh * N + i) * D + c8) = w;
        if (c8 == 0) LSE[(int64_t)bh * N + i] = wsum > 0.f ? (lmax + log2f(wsum)) * kLn2 : -INFINITY;
    }
}

template <int D>
static hipError_t launch_merge_fwd(const int* merges, int nmerge, const float* part, int nslots, void* o, float* lse,
                                   int BH, int N, hipStream_t st) {
    if (nmerge <= 0) return hipSuccess;
    constexpr int NRB = FwdBf16Cfg<D>::BM / (256 / (D / 8));
    hipLaunchKernelGGL(bsp_merge_fwd_kernel<D>, dim3((unsigned)(nmerge * BH * NRB)), dim3(256), 0, st, merges,
                       nmerge, part, nslots, (uint16_t*)o, lse, BH, N);
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

hipError_t launch_fwd_bf16_local(int d, const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                 int Hq, int Hkv, int N, int W, int S, float scale, hipStream_t st) {
    if (d == 64) return launch<64, true, true>(q, k, v, o, lse, B, Hq, Hkv, N, scale, st, W, S);
    if (d == 128) return launch<128, true, true>(q, k, v, o, lse, B, Hq, Hkv, N, scale, st, W, S);
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_bf16_bsparse(int d, int causal, const void* q, const void* k, const void* v, void* o,
                                   float* lse, int B, int Hq, int Hkv, int N, const int* row_ptr,
                                   const int* col_idx, int nnz, float scale, hipStream_t st) {
#define ARGS q, k, v, o, lse, B, Hq, Hkv, N, scale, st, 0, 0, row_ptr, col_idx, nnz
    if (d == 64) return causal ? launch<64, true, false, true>(ARGS) : launch<64, false, false, true>(ARGS);
    if (d == 128) return causal ? launch<128, true, false, true>(ARGS) : launch<128, false, false, true>(ARGS);
#undef ARGS
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_bf16_bsparse_split(int d, int causal, const void* q, const void* k, const void* v, void* o,
                                         float* lse, int B, int Hq, int Hkv, int N, const int* col_idx, int nnz,
                                         const int* chunks, int nchunks, const int* merges, int nmerge, int nslots,
                                         float* part, float scale, hipStream_t st) {
    const BspSplit sp{chunks, nchunks, nslots, part};
    const DropArgs nd{0u, 0u, 0u, 1.f};
    hipError_t e = hipErrorInvalidValue;
#define ARGS q, k, v, o, lse, B, Hq, Hkv, N, scale, st, 0, 0, nullptr, col_idx, nnz, nd, sp
    if (d == 64)
        e = causal ? launch<64, true, false, true, false, true>(ARGS) : launch<64, false, false, true, false, true>(ARGS);
    if (d == 128)
        e = causal ? launch<128, true, false, true, false, true>(ARGS)
                   : launch<128, false, false, true, false, true>(ARGS);
#undef ARGS
    if (e != hipSuccess) return e;
    return d == 64 ? launch_merge_fwd<64>(merges, nmerge, part, nslots, o, lse, B * Hq, N, st)
                   : launch_merge_fwd<128>(merges, nmerge, part, nslots, o, lse, B * Hq, N, st);
}

hipError_t launch_fwd_bf16_dropout(int d, int causal, const void* q, const void* k, const void* v, void* o,
                                   float* lse, int B, int Hq, int Hkv, int N, uint32_t thr, uint64_t seed, float rkeep,
                                   float scale, hipStream_t st) {
    const DropArgs dr{thr, (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32), rkeep};
#define ARGS q, k, v, o, lse, B, Hq, Hkv, N, scale, st, 0, 0, nullptr, nullptr, 0, dr
    if (d == 64) return causal ? launch<64, true, false, false, true>(ARGS) : launch<64, false, false, false, true>(ARGS);
    if (d == 128)
        return causal ? launch<128, true, false, false, true>(ARGS) : launch<128, false, false, false, true>(ARGS);
#undef ARGS
    return hipErrorInvalidValue;
}

}  // namespace fa
