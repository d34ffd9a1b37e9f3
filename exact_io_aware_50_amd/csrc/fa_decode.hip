// Attention of a few new query rows against a long key/value cache (decode),
// split over the keys.
//
// "Paper digest: FlashAttention", section "Limits": attention at decode time
// reads a large KV cache for few new queries and has a bottleneck of its own;
// the self-hosted LLM glossary, entries "KV Cache" (the keys and values of all
// earlier tokens, read again for every new token) and "Grouped-Query
// Attention" (query heads in groups share one key/value head).  The result is
// the same exact softmax attention: new query row i (of Nq) attends to every
// cache key j <= Nk - Nq + i when causal (the new rows are the last Nq
// positions of the sequence), to all Nk keys otherwise.
//
// What bounds it on gfx950 is the one pass over the cache at HBM bandwidth;
// the products are small.  So:
//  - the query rows of the G heads that share a K/V head are packed into the
//    32 columns of one matrix-core block (packed row r = head-in-group * Nq +
//    i), so K and V are read once per group, not once per query head;
//  - the keys are cut into chunks; every wave takes one (batch, K/V head, row
//    block, chunk) unit on its own, streams the chunk through a private
//    four-stage LDS ring with direct global->LDS loads, and runs the forward
//    pass's online softmax on it (S^T = K Q^T, P packed to bf16, O^T += V^T
//    P^T with transposing LDS reads of V);
//  - each unit writes its chunk's normalised O and log-sum-exp to a float32
//    workspace, and a second kernel merges the chunks of every row with the
//    rescale of the online softmax ("flash attention io aware", section
//    "Online Softmax": partial results taken against different maxima are
//    combined after scaling each by exp(m_s - m)).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

template <int D>
struct DecCfg {
    // Independent waves per workgroup: one workgroup fills the LDS (136 KiB),
    // so these are the waves of a CU.  The cache read needs bytes in flight
    // more than it needs waves: each wave keeps kStages - 1 tiles in flight.
    static constexpr int kWaves = D == 128 ? 2 : 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BN = 32;                     // keys per tile
    static constexpr int kStages = 4;
    using KT = LdsTile<BN, D, 1>;                     // one wave fills a whole tile
    static constexpr int kStage = 2 * KT::kElems;     // elements per stage (K then V)
    static constexpr float kTau = 8.0f;               // log2 slack before the running max is moved
};

// Paged cache: the pool [nblk][Hkv][bs][D], the block table [B][maxb] and the
// lengths [B]; `seq` receives the chunk plan for the merge: seq[b] = (first
// chunk, chunk count) of sequence b.
struct PagedArgs {
    const int* table;
    const int* lens;
    int* seq;
    int maxb, bs, nblk, T;
};

// The chunks of a paged decode, from the sequence lengths: a nonempty sequence
// of n keys (clamped to [0, maxb * bs]) gets 1 + floor(n (T - B) / L) chunks
// of equal size rounded up to 32 keys, L being the total length, so that
// every chunk slot holds about the same number of keys whatever the lengths
// (T >= 2B makes the counts add up to at most T); the chunks are numbered
// sequence by sequence.  Every wave works this out for its own chunk slot `cid`
// (the lengths read once per 64 sequences, a wave-wide sum and prefix sum of
// the counts): sequence, first and end key, and length of the chunk, or
// b = -1 for an unused slot.  With `write`, the wave also stores every
// sequence's (first chunk, count) in pg.seq.
__device__ __forceinline__ int64_t wave_sum64(int64_t x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}
__device__ __forceinline__ int paged_plan(const PagedArgs& pg, int B, int cid, int lane, bool write, int& kbeg,
                                          int& kend, int& nlen) {
    const int cap = pg.maxb * pg.bs;
    int64_t part = 0;
    for (int b0 = 0; b0 < B; b0 += 64)
        if (b0 + lane < B) part += min(max(pg.lens[b0 + lane], 0), cap);
    int64_t L = wave_sum64(part);
    if (L <= 0) L = 1;
    int found = -1;
    int base = 0;                                     // chunks of the sequences before this pass
    for (int b0 = 0; b0 < B; b0 += 64) {
        const int bb = b0 + lane;
        int n = 0, c = 0, cs = 0;
        if (bb < B) {
            n = min(max(pg.lens[bb], 0), cap);
            if (n > 0) {
                c = 1 + (int)((int64_t)n * (pg.T - B) / L);
                cs = ((n + c - 1) / c + 31) / 32 * 32;
                c = (n + cs - 1) / cs;
            }
        }
        const int incl = wave_incl_scan(c, lane);
        const int off = base + incl - c;
        if (write && bb < B) {
            pg.seq[2 * bb] = off;
            pg.seq[2 * bb + 1] = c;
        }
        const uint64_t hit = __ballot(c > 0 && cid >= off && cid < off + c);
        if (found < 0 && hit) {
            const int l = __ffsll((unsigned long long)hit) - 1;
            found = b0 + l;
            const int j = cid - __shfl(off, l);
            const int csl = __shfl(cs, l);
            nlen = __shfl(n, l);
            kbeg = j * csl;
            kend = min(nlen, (j + 1) * csl);
            if (!write) break;
        }
        base += __shfl(incl, 63);
    }
    return found;
}

// PAGED: the cache is a pool of blocks [nblk][Hkv][bs][D] and sequence b's
// key j sits in block table[b][j / bs], row j % bs; sequence b has lens[b]
// keys (the self-hosted LLM glossary, entry "PagedAttention": the KV cache in
// fixed-size, non-contiguous blocks; the digest's "Limits": batch-varying
// lengths at decode time).  bs is a multiple of the 32-key tile, so a tile
// never straddles two blocks.  Lengths are clamped to [0, maxb * bs] and
// block ids to [0, nblk): a bad table reads wrong rows, never outside the pool.
// A wave's unit is (chunk of the plan, K/V head, row block); the chunk's
// partial result for query row (h, i) goes to slot (chunk * Hq + h) * Nq + i.
template <int D, bool CAUSAL, bool PAGED = false>
__global__ __launch_bounds__(DecCfg<D>::kThreads) void decode_split_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    float* __restrict__ Wo, float* __restrict__ Wl, int B, int Hq, int Hkv, int Nq, int Nk, int chunk, int nsplit,
    float c2, PagedArgs pg = PagedArgs{}) {
    using Cfg = DecCfg<D>;
    using KT = typename Cfg::KT;
    constexpr int BN = Cfg::BN, kStage = Cfg::kStage, KP = KT::kPerWave, NS = Cfg::kStages;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[Cfg::kWaves * Cfg::kStages * kStage];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = Hq / Hkv, R = G * Nq, nrb = (R + 31) / 32;
    const int64_t u = (int64_t)blockIdx.x * Cfg::kWaves + wave;    // this wave's unit
    int s, rb, g, b, cid = 0;
    int pkbeg = 0, pkend = 0, pnb = 0;                // (paged) this chunk's keys and its sequence's length
    if constexpr (PAGED) {
        if (u >= (int64_t)pg.T * Hkv * nrb) return;                 // wave-uniform; no barriers below
        rb = (int)(u % nrb);
        g = (int)((u / nrb) % Hkv);
        cid = (int)(u / nrb / Hkv);
        const int lane0 = threadIdx.x & 63;
        b = paged_plan(pg, B, cid, lane0, u == 0, pkbeg, pkend, pnb);
        if (b < 0) return;                                           // an unused chunk slot
        s = 0;
    } else {
        if (u >= (int64_t)B * Hkv * nrb * nsplit) return;
        s = (int)(u % nsplit);
        const int64_t rest = u / nsplit;
        rb = (int)(rest % nrb);
        g = (int)((rest / nrb) % Hkv);
        b = (int)(rest / nrb / Hkv);
    }

    const int lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
    const int r = rb * 32 + l32;                      // this lane's packed query row
    const bool rv = r < R;
    const int hq = g * G + (rv ? r / Nq : 0), qi = rv ? r % Nq : 0;
    const int Nb = PAGED ? pnb : Nk;                  // this sequence's keys
    const int lim = CAUSAL ? Nb - Nq + qi : Nb - 1;   // last key the row sees
    const int kbeg = PAGED ? pkbeg : s * chunk;
    const int kend = PAGED ? pkend : min(Nb, kbeg + chunk);
    const int nt = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;

    uint16_t* ring = smem + wave * Cfg::kStages * kStage;
    const uint16_t* Kg = K + ((int64_t)b * Hkv + g) * Nk * D;
    const uint16_t* Vg = V + ((int64_t)b * Hkv + g) * Nk * D;
    // (paged) the unit's block ids, one per lane: table entries kbeg / bs .. + 63,
    // read once before the ring starts.  Read per tile inside the loop, the
    // entry is a vector load whose wait also drains the ring's tile loads.
    int tab = 0, tab0 = 0;
    if constexpr (PAGED) {
        tab0 = kbeg / pg.bs;
        if (tab0 + lane < pg.maxb) tab = pg.table[(int64_t)b * pg.maxb + tab0 + lane];
    }
    // K and V rows of tile t into stage t % NS (rows past the chunk re-read its last row)
    auto issue = [&](int t) __attribute__((always_inline)) {
        const uint16_t* st = ring + (t % NS) * kStage;
        const int k0 = kbeg + t * BN;
        const uint16_t *ks = Kg + (int64_t)k0 * D, *vs = Vg + (int64_t)k0 * D;
        if constexpr (PAGED) {
            const int jb = k0 / pg.bs - tab0;           // uniform
            const int raw = jb < 64 ? __builtin_amdgcn_readlane(tab, jb) : pg.table[(int64_t)b * pg.maxb + k0 / pg.bs];
            const int blk = min(max(raw, 0), pg.nblk - 1);
            const int64_t off = (((int64_t)blk * Hkv + g) * pg.bs + k0 % pg.bs) * D;
            ks = K + off;
            vs = V + off;
        }
        KT::load(ks, kend - k0, st, 0, lane);
        KT::load(vs, kend - k0, st + KT::kElems, 0, lane);
    };
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
        if (t < nt) issue(t);
    u32x4 qf[D / 16];                                 // this lane's query row as B operands
    {
        const uint16_t* qp = Q + (((int64_t)b * Hq + hq) * Nq + qi) * D + 8 * hh;
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
            u32x4 v = {};
            if (rv) v = *reinterpret_cast<const u32x4*>(qp + 16 * j);
            qf[j] = v;
        }
#pragma unroll
        for (int j = 0; j < D / 16; ++j) settle(qf[j]);
    }
    wait_vm<0>();

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();
    float m = kNegBig, lsum = 0.f;
    for (int t = 0; t < nt; ++t) {
        // tile t + NS - 1 goes into the stage of tile t - 1, whose reads all
        // fed products of the previous iteration; tile t has landed once at
        // most the loads of the tiles issued after it are outstanding
        if (t + NS - 1 < nt) issue(t + NS - 1);
        wait_vm_dyn<2 * KP, NS - 1>(min(NS - 1, nt - 1 - t));
        const uint16_t* Ks = ring + (t % NS) * kStage;
        const uint16_t* Vs = Ks + KT::kElems;
        // S^T = K_t Q^T: rows = 32 keys, columns = the packed query rows
        f32x16 sacc = zero16();
#pragma unroll
        for (int j = 0; j < D / 16; ++j) sacc = mma_bf16(KT::row8(Ks, l32, 2 * j + hh), qf[j], sacc);
        const int k0 = kbeg + t * BN;
        if (k0 + BN > kend || (CAUSAL && k0 + BN - 1 > Nb - Nq)) {
#pragma unroll
            for (int r2 = 0; r2 < 16; ++r2) {
                const int key = k0 + acc_row(r2, hh);
                if (key >= kend || key > lim) sacc[r2] = -INFINITY;
            }
        }
        // online softmax in base 2 (scale * log2 e in c2); the running max is
        // moved only when some row of the wave grew by more than 2^tau
        float x = -INFINITY;
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) x = fmaxf(x, sacc[r2]);
        x = pair_max(x);
        const float mnew = fmaxf(m, x * c2);
        if (__any(mnew > m + Cfg::kTau)) {
            const float alpha = fast_exp2(m - mnew);
            m = mnew;
            lsum *= alpha;
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct) oacc[ct] *= alpha;
        }
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) sacc[r2] = fast_exp2(fmaf(sacc[r2], c2, -m));
        u32x4 pf[2];
        float rs[2] = {0.f, 0.f};
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
            pf[t2] = pack_bf16x8(sacc, 8 * t2);
#pragma unroll
            for (int i = 0; i < 4; ++i) rs[i & 1] = dot2_bf16_sum(pf[t2][i], rs[i & 1]);
        }
        lsum += rs[0] + rs[1];
        // O^T += V_t^T P^T
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct)
                oacc[ct] = mma_bf16(KT::tr8(Vs, 16 * t2, 32 * ct, lane), pf[t2], oacc[ct]);
    }

    // this chunk's O (normalised) and log-sum-exp; a row that sees no key of
    // the chunk gets weight zero (LSE = -inf, O = 0)
    const float lt = pair_sum(lsum);
    if (rv) {
        const int64_t row = ((int64_t)b * Hq + hq) * Nq + qi;
        const int64_t slot = PAGED ? ((int64_t)cid * Hq + hq) * Nq + qi : row * nsplit + s;
        float* wo = Wo + slot * D;
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
        for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                f32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = oacc[ct][4 * gq + e] * inv;
                *reinterpret_cast<f32x4*>(wo + 32 * ct + 8 * gq + 4 * hh) = w;
            }
        if (hh == 0) Wl[slot] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
    }
}

// One wave per query row: LSE = L + ln(sum_s exp(LSE_s - L)) with L the
// largest chunk LSE, O = sum_s exp(LSE_s - LSE) O_s.  The chunks of row r are
// slots r * nsplit + s (contiguous cache) or, with a paged plan `seq`, slots
// (first + j) * HqNq + r % HqNq for the row's sequence's chunks j.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ Wo,
                                                           const float* __restrict__ Wl, uint16_t* __restrict__ O,
                                                           float* __restrict__ LSE, int64_t rows, int nsplit,
                                                           const int* __restrict__ seq = nullptr, int HqNq = 0) {
    constexpr int PER = D / 64;                       // d values per lane
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    int64_t first = row * nsplit, stride = 1;
    int cnt = nsplit;
    if (seq) {
        const int b = (int)(row / HqNq);
        first = (int64_t)seq[2 * b] * HqNq + row % HqNq;
        stride = HqNq;
        cnt = seq[2 * b + 1];
    }
    float L = -INFINITY;
    for (int s = lane; s < cnt; s += 64) L = fmaxf(L, Wl[first + s * stride]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) L = fmaxf(L, __shfl_xor(L, off));
    float acc[PER], wsum = 0.f;
#pragma unroll
    for (int p = 0; p < PER; ++p) acc[p] = 0.f;
#pragma unroll 4
    for (int s = 0; s < cnt; ++s) {
        const float ls = Wl[first + s * stride];
        const float w = ls == -INFINITY ? 0.f : fast_exp2((ls - L) * kLog2e);
        wsum += w;
        const float* wo = Wo + (first + s * stride) * D + lane * PER;
#pragma unroll
        for (int p = 0; p < PER; ++p) acc[p] = fmaf(w, wo[p], acc[p]);
    }
    // a row that sees no key at all (paged: an empty sequence, or a causal
    // row before its sequence's first key) gets O = 0 and LSE = -inf
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    uint16_t* orow = O + row * D + lane * PER;
    if constexpr (PER == 2) {
        *reinterpret_cast<uint32_t*>(orow) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    } else {
        orow[0] = (uint16_t)(pack_bf16x2(acc[0] * inv, 0.f) & 0xffffu);
    }
    if (lane == 0) LSE[row] = wsum > 0.f ? L + logf(wsum) : -INFINITY;
}

DecodePlan decode_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d, int per_slot, int cus) {
    DecodePlan p;
    const int G = Hq / Hkv;
    p.nrb = (G * Nq + 31) / 32;
    const int64_t base = (int64_t)B * Hkv * p.nrb;
    // per_slot wave units per resident wave of the device's CUs (each unit streams
    // its chunk with its own ring, so fewer, longer units pay the ring's
    // start-up latency less often); chunks of at least 256 keys
    const int64_t slots = (int64_t)per_slot * cus * (d == 128 ? DecCfg<128>::kWaves : DecCfg<64>::kWaves);
    const int64_t want = (slots + base - 1) / base;
    const int64_t most = ((int64_t)Nk + 255) / 256;
    int64_t ns = want < most ? want : most;
    if (ns < 1) ns = 1;
    int64_t chunk = ((int64_t)Nk + ns - 1) / ns;
    chunk = (chunk + 31) / 32 * 32;
    p.chunk = (int)chunk;
    p.nsplit = (int)(((int64_t)Nk + chunk - 1) / chunk);
    return p;
}

template <int D, bool CAUSAL>
static hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, float* ws, int B,
                         int Hq, int Hkv, int Nq, int Nk, float scale, hipStream_t st) {
    using Cfg = DecCfg<D>;
    const DecodePlan p = decode_plan(B, Hq, Hkv, Nq, Nk, D, 1, device_cus());
    const int64_t rows = (int64_t)B * Hq * Nq;
    float* wo = ws;
    float* wl = ws + rows * p.nsplit * D;
    const int64_t units = (int64_t)B * Hkv * p.nrb * p.nsplit;
    const unsigned g1 = (unsigned)((units + Cfg::kWaves - 1) / Cfg::kWaves);
    hipLaunchKernelGGL((decode_split_kernel<D, CAUSAL, false>), dim3(g1), dim3(Cfg::kThreads), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, wo, wl, B, Hq, Hkv, Nq, Nk, p.chunk,
                       p.nsplit, scale * kLog2e, PagedArgs{});
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, wo, wl,
                       (uint16_t*)o, lse, rows, p.nsplit, (const int*)nullptr, 0);
    return hipGetLastError();
}

int paged_chunks(int B, int Hq, int Hkv, int Nq, int d, int cus) {
    // about two wave units (chunk x K/V head x row block) per resident wave
    // of the device's CUs, and at least two chunk slots per sequence.  Two per wave
    // measured best on the 16-sequence 16K workload with mixed lengths: 0.124
    // ms against 0.136 for one and 0.134 for four (the rounding of each
    // sequence's chunk count leaves some slots empty; a second round of units
    // fills the waves those free)
    const int nrb = (Hq / Hkv * Nq + 31) / 32;
    const int64_t slots = (int64_t)cus * (d == 128 ? DecCfg<128>::kWaves : DecCfg<64>::kWaves);
    const int64_t per = (int64_t)Hkv * nrb;
    const int64_t T = (2 * slots + per - 1) / per;
    return (int)(T > 2 * (int64_t)B ? T : 2 * (int64_t)B);
}

size_t paged_ws_bytes(int B, int Hq, int Hkv, int Nq, int d) {
    const int64_t T = paged_chunks(B, Hq, Hkv, Nq, d, device_cus());
    const int64_t ints = ((4 * (int64_t)B + 3 * T) * 4 + 15) / 16 * 16;
    return (size_t)(ints + 4 * T * Hq * Nq * (int64_t)(d + 1));
}

template <int D, bool CAUSAL>
static hipError_t launch_paged(const void* q, const void* kc, const void* vc, const int* table, const int* lens,
                               void* o, float* lse, float* ws, int B, int Hq, int Hkv, int Nq, int maxb, int bs,
                               int nblk, float scale, hipStream_t st) {
    using Cfg = DecCfg<D>;
    const int T = paged_chunks(B, Hq, Hkv, Nq, D, device_cus());
    const int nrb = (Hq / Hkv * Nq + 31) / 32;
    // (first chunk, count) per sequence, written by the split kernel for the merge
    int* seq = reinterpret_cast<int*>(ws);
    const int64_t ints = ((4 * (int64_t)B + 3 * (int64_t)T) * 4 + 15) / 16 * 16;
    float* wo = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + ints);
    float* wl = wo + (int64_t)T * Hq * Nq * D;
    const PagedArgs pg{table, lens, seq, maxb, bs, nblk, T};
    const int64_t units = (int64_t)T * Hkv * nrb;
    const unsigned g1 = (unsigned)((units + Cfg::kWaves - 1) / Cfg::kWaves);
    hipLaunchKernelGGL((decode_split_kernel<D, CAUSAL, true>), dim3(g1), dim3(Cfg::kThreads), 0, st,
                       (const uint16_t*)q, (const uint16_t*)kc, (const uint16_t*)vc, wo, wl, B, Hq, Hkv, Nq,
                       maxb * bs, 0, 0, scale * kLog2e, pg);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)B * Hq * Nq;
    hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, wo, wl,
                       (uint16_t*)o, lse, rows, 0, (const int*)seq, Hq * Nq);
    return hipGetLastError();
}

hipError_t launch_decode(int d, int causal, const void* q, const void* k, const void* v, void* o, float* lse,
                         float* ws, int B, int Hq, int Hkv, int Nq, int Nk, float scale, hipStream_t st) {
    if (d == 64) return causal ? launch<64, true>(q, k, v, o, lse, ws, B, Hq, Hkv, Nq, Nk, scale, st)
                               : launch<64, false>(q, k, v, o, lse, ws, B, Hq, Hkv, Nq, Nk, scale, st);
    if (d == 128) return causal ? launch<128, true>(q, k, v, o, lse, ws, B, Hq, Hkv, Nq, Nk, scale, st)
                                : launch<128, false>(q, k, v, o, lse, ws, B, Hq, Hkv, Nq, Nk, scale, st);
    return hipErrorInvalidValue;
}

hipError_t launch_decode_paged(int d, int causal, const void* q, const void* kc, const void* vc, const int* table,
                               const int* lens, void* o, float* lse, float* ws, int B, int Hq, int Hkv, int Nq,
                               int maxb, int bs, int nblk, float scale, hipStream_t st) {
#define PARGS q, kc, vc, table, lens, o, lse, ws, B, Hq, Hkv, Nq, maxb, bs, nblk, scale, st
    if (d == 64) return causal ? launch_paged<64, true>(PARGS) : launch_paged<64, false>(PARGS);
    if (d == 128) return causal ? launch_paged<128, true>(PARGS) : launch_paged<128, false>(PARGS);
#undef PARGS
    return hipErrorInvalidValue;
}

}  // namespace fa
