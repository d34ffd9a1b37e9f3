// FP8 (OCP E4M3) forward pass and the per-tensor quantiser that feeds it.
//
// The FlashAttention legal glossary (FlashAttention-3 paragraph) and "flash
// attention io aware" (section "Flash Attention 2 and 3") name FP8 attention
// on low-precision matrix units without a recipe.  Here: one descale per
// tensor (real value = code * s_X), both products on the fp8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales) with float32
// accumulation, the softmax in float32, and P multiplied by 256 before its
// E4M3 rounding so that small probabilities stay out of the E4M3 subnormal
// range (the factor is a power of two and is divided out exactly with l).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// empty asms consuming a value: its computation stays before this point
__device__ __forceinline__ void settle8(const u32x8& x) { asm volatile("" : : "v"(x)); }
__device__ __forceinline__ void settle16(const f32x16& x) { asm volatile("" : : "v"(x)); }

// ------------------------------------------------------------ quantiser
__global__ void q8_clear_kernel(float* descale) {
    if (threadIdx.x == 0) descale[0] = 0.f;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__global__ __launch_bounds__(256) void q8_absmax_kernel(const uint16_t* __restrict__ x, size_t n,
                                                       float* __restrict__ descale) {
    float m = 0.f;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        m = fmaxf(m, fabsf(bf16_to_f32(x[i])));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __shared__ float wmax[4];
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        // non-negative floats order like their bit patterns
        atomicMax(reinterpret_cast<unsigned int*>(descale), __float_as_uint(m));
    }
}

__device__ __forceinline__ float q8_scale(float absmax) {
    return fmaxf(absmax, 0x1p-120f) / 448.0f;   // IEEE division, as the format recipe states
}

// float32 -> E4M3 code, round to nearest even, saturating at +-448.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    uint32_t code;
    if (a >= 0x43e00000u) {                    // |f| >= 448
        code = 0x7e;
    } else if (a < 0x3c800000u) {              // |f| < 2^-6: multiples of 2^-9
        code = (uint32_t)rintf(__uint_as_float(a) * 512.0f);
    } else {
        uint32_t base = a >> 20;               // biased exponent and top 3 mantissa bits
        const uint32_t rem = a & 0xfffffu, half = 0x80000u;
        base += (rem > half || (rem == half && (base & 1u))) ? 1u : 0u;
        code = base - (120u << 3);             // rebias 127 -> 7
        if (code > 0x7e) code = 0x7e;
    }
    return sign | code;
}

__global__ __launch_bounds__(256) void q8_cast_kernel(const uint16_t* __restrict__ x, size_t n,
                                                     uint8_t* __restrict__ out,
                                                     const float* __restrict__ descale) {
    const float s = q8_scale(descale[0]);
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        out[i] = (uint8_t)e4m3_rne_sat(bf16_to_f32(x[i]) / s);
}

__global__ void q8_finalize_kernel(float* descale) {
    if (threadIdx.x == 0) descale[0] = q8_scale(descale[0]);
}

hipError_t launch_quantize_fp8(const void* x, size_t n, void* out, float* descale, hipStream_t st) {
    hipLaunchKernelGGL(q8_clear_kernel, dim3(1), dim3(64), 0, st, descale);
    if (n > 0) {
        size_t blocks = (n + 1023) / 1024;
        if (blocks > 2048) blocks = 2048;
        hipLaunchKernelGGL(q8_absmax_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint16_t*)x, n,
                           descale);
        hipLaunchKernelGGL(q8_cast_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const uint16_t*)x, n,
                           (uint8_t*)out, (const float*)descale);
    }
    hipLaunchKernelGGL(q8_finalize_kernel, dim3(1), dim3(64), 0, st, descale);
    return hipGetLastError();
}

// ------------------------------------------------------------ fp8 products
//
// Operands are 32 bytes per lane: lane l supplies row (A) or column (B) l % 32
// and 32 contraction slots (half hh = l / 32 of the 64).  The block scales are
// E8M0 exponents (127 = 2^0).
__device__ __forceinline__ f32x16 mma_fp8s(const u32x8& a, const u32x8& b, f32x16 c, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b),
                                                           c, 0, 0, 0, 127, 0, scale_b);
}
__device__ __forceinline__ f32x16 mma_fp8(const u32x8& a, const u32x8& b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a),
                                                           __builtin_bit_cast(i32x8, b), c,
                                                           0, 0,        // A and B are E4M3
                                                           0, 127,      // A block scale 2^0
                                                           0, 127);     // B block scale 2^0
}

// ------------------------------------------------------------ fp8 forward (d = 64 and 128)
//
// The schedule of the bf16 forward (two wave groups one phase apart, K and V
// tiles loaded straight into a ring of four LDS stages in their row-major
// layout, persistent workgroups) with E4M3 operands and 128-key tiles (twice
// the bf16 kernel's: an E4M3 tile is half the bytes, and the per-phase costs
// that do not grow with the tile -- the row max exchange, the scale exponent,
// the barrier -- are paid half as often; 2.5-7% faster than 64-key tiles):
//  - a 128-key tile of E4M3 codes is 16 row groups of 8 rows at d = 128 (two
//    per wave) and 8 groups of 16 rows at d = 64 (one per wave);
//  - S^T = K_t Q^T: per 32-key block, d/64 fp8 products whose K fragment is
//    two 16-byte row reads;
//  - O^T += V_t^T P^T: one fp8 product per 32 d-columns and 64 keys.
//    Its V^T fragment comes from four transposing byte reads of the
//    row-major V tile (ds_read_b64_tr_b8: within a 16-lane group, output lane
//    i, byte j is byte i % 8 of what source lane 2j + i/8 read).  Source lanes
//    2j and 2j + 1 read 8 columns each of the same key, so every lane receives
//    one column over eight keys, in the order its P bytes hold the keys.
//  - P is scaled before its E4M3 rounding, per query row and tile, by the
//    power of two 2^e that puts the tile's largest P of the row just below
//    2^8.5 (below the largest E4M3 value 448, with all of the format's binades
//    under it), and the P V and row-sum products divide it back out with the
//    instruction's B-operand block scale 2^-e (free).  The scaled P never
//    overflows however stale the running max is, so the max is moved only past
//    2^8 growth, as in the bf16 kernel (float32 range), not past 2^1 growth:
//    6-8% faster at the 4096-token causal workload.
//  - l is the sum of the rounded P that the P V product weighs V with, formed
//    on the matrix cores: one more fp8 product per tile, of a ones operand
//    with P under the same block scale (every output row is the key sum of its
//    query column), instead of 32 vector additions per lane.
template <int D>
struct FwdFp8Cfg {
    static constexpr int kWaves = 8;                  // two groups of four, one wave of each per SIMD
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BM = 32 * kWaves;            // query rows per workgroup
    static constexpr int kSub = 2;                    // 64-key sub-tiles per tile (one P operand each)
    static constexpr int BN = 64 * kSub;              // keys per K/V tile
    static constexpr int kStages = 4;
    using KT = LdsTile<BN, D / 2, kWaves>;            // byte rows, in 16-bit units
    static constexpr int kStage = 2 * KT::kElems;     // 16-bit units per stage (K then V)
    static constexpr float kTau = 8.0f;               // log2 slack before the max is moved
    static constexpr float kPTop = 8.5f;              // log2 of the largest scaled P of a tile, at most
};

// G phase order: the K fragments (two reads) of the NSM score products, then
// the V^T fragments (four reads) of the NPV P V products, each read three
// products ahead; the NR row-sum products (no reads) while the first reads
// are in flight.
template <int NSM, int NPV, int NR>
__device__ __forceinline__ void sched_fp8_phase() {
    constexpr int NT = NSM + NPV, A = 3;
#pragma unroll
    for (int f = 0; f < A; ++f) {
        if (f < NSM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (j + A < NSM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else if (j + A < NT) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(FwdFp8Cfg<D>::kThreads, 2) void fwd_fp8_pp_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, const float* __restrict__ descale, int B, int Hq, int Hkv,
    int n_rows, float scale) {
    using Cfg = FwdFp8Cfg<D>;
    using KT = typename Cfg::KT;
    constexpr int NW = Cfg::kWaves, BM = Cfg::BM, BN = Cfg::BN, NS = Cfg::kStages, KB = BN / 32;
    constexpr int kStage = Cfg::kStage, SUB = Cfg::kSub, PW = KT::kPerWave;
    static_assert((NS & (NS - 1)) == 0, "stage index by mask");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * kStage];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2;
    const float c2 = scale * kLog2e * descale[0] * descale[1];
    const float sv = descale[2];

    const int nmb = (n_rows + BM - 1) / BM;
    const PersistentSched sched(nmb * Hq * B);
    for (int r = 0; sched.more(r); ++r) {
        const int lin = sched.item(r);
        if (lin < 0) continue;
        // the sequence length as an opaque per-item value: whatever derives
        // from it (tail clamps and masks) is computed per item, not hoisted
        // out of the item loop into registers for the whole kernel
        int N = n_rows;
        asm volatile("" : "+s"(N));
        const int lane = threadIdx.x & 63;
        const int l32 = lane & 31, hh = lane >> 5;
        const int mbi = lin % nmb, bh = lin / nmb;
        const int h = bh % Hq, b = bh / Hq;
        const int mb = CAUSAL ? nmb - 1 - mbi : mbi;      // longest causal rows first
        const int g = h / (Hq / Hkv);
        const uint8_t* Qh = Q + ((int64_t)b * Hq + h) * N * D;
        const uint8_t* Kh = K + ((int64_t)b * Hkv + g) * N * D;
        const uint8_t* Vh = V + ((int64_t)b * Hkv + g) * N * D;

        const int q0 = mb * BM;
        const int qw = q0 + 32 * wave;
        const int qrow = qw + l32;
        const int kend = CAUSAL ? min(N, q0 + BM) : N;
        const int ntiles = (kend + BN - 1) / BN;
        const int ntw = qw >= N ? 0 : CAUSAL ? (min(N, qw + 32) + BN - 1) / BN : ntiles;
        auto stage = [&](int t) __attribute__((always_inline)) { return smem + (t & (NS - 1)) * kStage; };

        // ---- direct loads: this wave's PW row groups of a K/V tile (rows past
        // the end re-read the last row)
        uint32_t voff[PW];
#pragma unroll
        for (int i = 0; i < PW; ++i) voff[i] = (uint32_t)(((i * NW + wave) * KT::RG + lane % KT::RG) * D + (lane / KT::RG) * 16);
        auto issue_half = [&](int t, const int half) __attribute__((always_inline)) {
            const uint32_t st = lds_addr(stage(t)) + half * KT::kBytes;
            const uint8_t* src = (half ? Vh : Kh) + (int64_t)t * BN * D;
            const int rows_valid = N - t * BN;
            if (rows_valid >= BN) {
#pragma unroll
                for (int i = 0; i < PW; ++i) dma16s(src, voff[i], st + (i * NW + wave) * KT::RGS);
            } else {
                int ln = lane;
                asm volatile("" : "+v"(ln));
#pragma unroll
                for (int i = 0; i < PW; ++i) {
                    const int row = (i * NW + wave) * KT::RG + ln % KT::RG;
                    const int grow = row < rows_valid ? row : rows_valid - 1;
                    dma16s(src, (uint32_t)(grow * D + (ln / KT::RG) * 16), st + (i * NW + wave) * KT::RGS);
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
            const uint32_t st = lds_addr(stage(t)) + half * KT::kBytes;
            const uint8_t* src = (half ? Vh : Kh) + (int64_t)t * BN * D;
            const int rows_valid = N - t * BN;
            const int w0 = wave & 3;
            if (rows_valid >= BN) {
#pragma unroll
                for (int i = 0; i < PW; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int w = w0 + 4 * j;
                        dma16s(src, voff[i] + (uint32_t)((w - wave) * KT::RG * D), st + (i * NW + w) * KT::RGS);
                    }
            } else {
                int ln = lane;
                asm volatile("" : "+v"(ln));
#pragma unroll
                for (int i = 0; i < PW; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int w = w0 + 4 * j;
                        const int row = (i * NW + w) * KT::RG + ln % KT::RG;
                        const int grow = row < rows_valid ? row : rows_valid - 1;
                        dma16s(src, (uint32_t)(grow * D + (ln / KT::RG) * 16), st + (i * NW + w) * KT::RGS);
                    }
            }
        };
#pragma unroll
        for (int t = 0; t < NS; ++t)
            if (t < ntiles) issue(t);

        // Q rows as B operands: 32 bytes per lane and product (rows past the
        // end read the last row; those queries are never stored)
        u32x8 qf[D / 64];
        {
            const int row = min(qrow, N - 1);
#pragma unroll
            for (int s2 = 0; s2 < D / 64; ++s2) qf[s2] = *reinterpret_cast<const u32x8*>(Qh + (int64_t)row * D + 64 * s2 + 32 * hh);
        }
#pragma unroll
        for (int s2 = 0; s2 < D / 64; ++s2) settle8(qf[s2]);
        wait_vm<0>();

        f32x16 oacc[D / 32];
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();
        float m = kNegBig;
        f32x16 lacc = zero16();                           // row sums of the rounded P (all rows alike)
        u32x8 ones;
#pragma unroll
        for (int i = 0; i < 8; ++i) ones[i] = 0x38383838u;   // E4M3 1.0 in every byte
        f32x16 sacc[KB];
        u32x8 pf[SUB];                                    // P of each 64-key sub-tile, E4M3
#pragma unroll
        for (int p = 0; p < SUB; ++p) pf[p] = u32x8{};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) sacc[kb] = zero16();

        // S^T = K_t Q^T: rows = keys, columns = this wave's queries
        auto do_s = [&](int t) __attribute__((always_inline)) {
            const uint16_t* Ks = stage(t);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) sacc[kb] = zero16();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int s2 = 0; s2 < D / 64; ++s2) {
                    const u32x4 lo = KT::row8(Ks, 32 * kb + l32, 4 * s2 + 2 * hh);
                    const u32x4 hi = KT::row8(Ks, 32 * kb + l32, 4 * s2 + 2 * hh + 1);
                    const u32x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    sacc[kb] = mma_fp8(a, qf[s2], sacc[kb]);
                }
        };
        // O^T += V_t^T P^T, one product per 32 d-columns and 64-key sub-tile
        // sb.  Read p (0..3) of a fragment gives this lane the keys
        // 64 sb + 32(p/2) + 16(p%2) + 8(j/4) + 4hh + j%4, j = 0..7: key of byte
        // e = 8p + j of P.
        const int g16 = lane >> 4, s16 = lane & 15, jj = s16 >> 1, qq = s16 & 1;
        int pscale = 127;                                 // E8M0 block scale of pf: 2^-e
        auto do_pv = [&](int t) __attribute__((always_inline)) {
            const char* Vb = (const char*)(stage(t) + KT::kElems);
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
                for (int sb = 0; sb < SUB; ++sb) {
                    u32x8 a;
#pragma unroll
                    for (int pq = 0; pq < 4; ++pq) {
                        const int key = 64 * sb + 32 * (pq >> 1) + 16 * (pq & 1) + 8 * (jj >> 2) + 4 * (g16 >> 1) + (jj & 3);
                        const int col = 32 * ct + 16 * (g16 & 1) + 8 * qq;
                        const char* ad = Vb + KT::off(key, col >> 4) + (col & 15);
                        const auto w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                            (__attribute__((address_space(3))) i32x2*)(__attribute__((address_space(3))) char*)ad);
                        a[2 * pq] = (uint32_t)w[0];
                        a[2 * pq + 1] = (uint32_t)w[1];
                    }
                    oacc[ct] = mma_fp8s(a, pf[sb], oacc[ct], pscale);
                }
        };
        auto do_rowsum = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int sb = 0; sb < SUB; ++sb) lacc = mma_fp8s(ones, pf[sb], lacc, pscale);
        };
        // The scaled fp8 products are not held in their phase by the ordering
        // hints alone: consuming their results at the end of the phase keeps
        // them (and their completion) before the barrier.  The matrix phase is
        // much shorter than the vector phase here, so the wait costs nothing.
        auto gemm = [&](int t) __attribute__((always_inline)) {
            // causal: past t = ntw the scores are unused and P is zero; the
            // phase is skipped (no time saved in the slot, power saved)
            if (CAUSAL && t > ntw) return;
            do_rowsum();
            do_s(t);
            do_pv(t - 1);
            sched_fp8_phase<KB * (D / 64), (D / 32) * SUB, SUB>();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) settle16(sacc[kb]);
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct) settle16(oacc[ct]);
            settle16(lacc);
        };
        // X(t)
        auto softmax = [&](int t) __attribute__((always_inline)) {
            if (t >= ntw) {
#pragma unroll
                for (int sb = 0; sb < SUB; ++sb) pf[sb] = u32x8{};
                return;
            }
            const int k0 = t * BN;
            if ((CAUSAL && k0 + BN - 1 > qw) || k0 + BN > N) {
                int hm = hh;
                asm volatile("" : "+v"(hm));
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                    for (int r2 = 0; r2 < 16; ++r2) {
                        const int key = k0 + 32 * kb + acc_row(r2, hm);
                        if ((CAUSAL && key > qrow) || key >= N) sacc[kb][r2] = -INFINITY;
                    }
                    // one key block at a time: the compares' lane masks are not all held at once
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            float x = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r2 = 0; r2 < 16; ++r2) x = fmaxf(x, sacc[kb][r2]);
            x = pair_max(x);
            const float mnew = fmaxf(m, x * c2);
            if (__any(mnew > m + Cfg::kTau)) {
                const float alpha = fast_exp2(m - mnew);
                m = mnew;
                lacc *= alpha;
#pragma unroll
                for (int ct = 0; ct < D / 32; ++ct) oacc[ct] *= alpha;
            }
            // P 2^e = exp2(c2 s - m + e), packed to E4M3 (byte e of pf[sb] is
            // register e % 16 of key block 2 sb + e / 16), with
            // e = floor(kPTop - (c2 x - m)) the exponent that puts the tile's
            // largest P of this row just below 2^kPTop (x = -inf, a row with no
            // key in the tile: e = 126, P = 0)
            const int e = (int)fminf(fmaf(-x, c2, Cfg::kPTop + m), 126.0f);
            pscale = 127 - e;
            const float base = (float)e - m;
#pragma unroll
            for (int sb = 0; sb < SUB; ++sb) {
#pragma unroll
                for (int w = 0; w < 8; ++w) {
                    float p[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        p[i] = fast_exp2(fmaf(sacc[2 * sb + (w >> 2)][4 * (w & 3) + i], c2, base));
                    int pk;
                    asm("" : "=v"(pk) : "v"(p[0]));       // any value: both halves are written
                    pk = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pk, false);
                    pk = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], pk, true);
                    pf[sb][w] = (uint32_t)pk;
                }
                settle8(pf[sb]);
            }
        };

        // ---- phases: as in the bf16 forward (K rows of tile u >= NS at the
        // start of slot 2u - 4, V rows at the start of slot 2u - 3), except
        // that the loads of a slot are issued by the group that starts its
        // matrix phase there (the first group the K rows, the second the V
        // rows), each wave for its partner too: here the vector phase is the
        // longer one (3% faster at the causal 4096 workload than every wave
        // issuing in both phases, 1.5% faster than the vector-phase group
        // issuing).  Before the barrier ending odd slot 2tv - 1 the first group
        // has its K_tv (K_tv+1 may be in flight), the second its V_tv-1 (V_tv
        // and V_tv+1 may be).
        auto head = [&](int s2) __attribute__((always_inline)) {
            const int u = (s2 >> 1) + 2;
            if (s2 >= 4 && u < ntiles && grp == (s2 & 1)) issue_half_pair(u, s2 & 1);
        };
        auto tail_odd = [&](int s2) __attribute__((always_inline)) {
            const int tv = (s2 + 1) / 2;
            if (tv >= NS && tv < ntiles) {
                if (grp == 0) {
                    if (tv + 1 < ntiles) wait_vm<2 * PW>();
                    else wait_vm<0>();
                } else {
                    if (tv + 1 < ntiles) wait_vm<4 * PW>();
                    else wait_vm<2 * PW>();
                }
            } else if (tv == ntiles && ntiles > NS) {
                wait_vm<0>();                         // V of the last tile
            }
            lds_barrier();
        };
        lds_barrier();
        if (grp == 0) {
            do_s(0);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) settle16(sacc[kb]);
            lds_barrier();
            softmax(0);
            tail_odd(1);
            for (int t = 1; t <= ntiles; ++t) {
                head(2 * t);
                gemm(t);
                lds_barrier();
                head(2 * t + 1);
                softmax(t);
                tail_odd(2 * t + 1);
            }
        } else {
            lds_barrier();
            do_s(0);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) settle16(sacc[kb]);
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

        // ---- epilogue: O = s_V O_acc / l, LSE = ln2 (m + log2 l)
        // (G(t) adds the row sums of P_{t-1}, so G(ntiles) added the last tile's)
        const float ltot = lacc[0];
        if (qrow < N) {
            const float f = sv / ltot;
            int le = lane;
            asm volatile("" : "+v"(le));
            uint16_t* Orow = O + (((int64_t)b * Hq + h) * N + qw + (le & 31)) * D + 4 * (le >> 5);
#pragma unroll
            for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    u32x2 w;
                    w[0] = pack_bf16x2(oacc[ct][4 * gq] * f, oacc[ct][4 * gq + 1] * f);
                    w[1] = pack_bf16x2(oacc[ct][4 * gq + 2] * f, oacc[ct][4 * gq + 3] * f);
                    *reinterpret_cast<u32x2*>(Orow + 32 * ct + 8 * gq) = w;
                }
            if (hh == 0) LSE[((int64_t)b * Hq + h) * N + qrow] = (m + log2f(ltot)) * kLn2;
        }
    }
}

template <int D, bool CAUSAL>
static hipError_t launch_fp8_pp(const void* q, const void* k, const void* v, void* o, float* lse,
                                const float* descale, int B, int Hq, int Hkv, int N, float scale, hipStream_t st) {
    using Cfg = FwdFp8Cfg<D>;
    const int nmb = (N + Cfg::BM - 1) / Cfg::BM;
    static PerDevice slots;
    const int grid = persistent_grid((const void*)fwd_fp8_pp_kernel<D, CAUSAL>, Cfg::kThreads, nmb * Hq * B, slots);
    hipLaunchKernelGGL((fwd_fp8_pp_kernel<D, CAUSAL>), dim3((unsigned)grid), dim3(Cfg::kThreads), 0, st,
                       (const uint8_t*)q, (const uint8_t*)k, (const uint8_t*)v, (uint16_t*)o, lse, descale, B, Hq,
                       Hkv, N, scale);
    return hipGetLastError();
}

hipError_t launch_fwd_fp8(int d, int causal, const void* q, const void* k, const void* v, void* o, float* lse,
                          const float* descale, int B, int Hq, int Hkv, int N, float scale, hipStream_t st) {
    if (d == 128) return causal ? launch_fp8_pp<128, true>(q, k, v, o, lse, descale, B, Hq, Hkv, N, scale, st)
                                : launch_fp8_pp<128, false>(q, k, v, o, lse, descale, B, Hq, Hkv, N, scale, st);
    if (d == 64) return causal ? launch_fp8_pp<64, true>(q, k, v, o, lse, descale, B, Hq, Hkv, N, scale, st)
                               : launch_fp8_pp<64, false>(q, k, v, o, lse, descale, B, Hq, Hkv, N, scale, st);
    return hipErrorInvalidValue;
}

}  // namespace fa
