// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Matrix-core convention used everywhere.  One 32x32 output block comes from
// v_mfma_f32_32x32x16_bf16 (bf16) or eight chained v_mfma_f32_32x32x2f32
// (float32).  Lane l of a wave64 owns column n = l % 32 of the output and the
// sixteen rows  row(r, hh) = 8*(r/4) + 4*hh + (r%4),  r = 0..15, hh = l / 32.
// For the A operand (M x 16) lane l supplies row l % 32, for the B operand
// (16 x N) column l % 32; in both, lane l supplies the eight contraction
// slots 8*hh + e, e = 0..7.  Which hardware k each slot is does not matter:
// A and B use the same slot order, and a contraction is order-free.
//
// "Accumulator as operand": registers r = 8t..8t+7 of an accumulator hold rows
// 16t + 8*(e/4) + 4*hh + (e%4).  Fed back as the B operand of a product that
// contracts over those rows, slot 8*hh + e must therefore meet row
// 16t + swap23(8*hh + e) of the other operand, where swap23 exchanges bits 2
// and 3 of an index.  Tiles that are read as "transposed" A operands store the
// contraction index at position swap23(index) (within aligned groups of 16),
// so that each lane reads eight contiguous elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite "minus infinity" for the running maximum: exp2(kNegBig - m) is 0 for
// any finite m, and kNegBig - kNegBig = 0 never produces NaN.
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ int swap23(int p) {
    return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of the same lane in the other half of the wave (lane l <-> l ^ 32).
__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    // float32 -> bfloat16, round to nearest even (inputs here are never NaN).
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// ----------------------------------------------------------------------------
// Element types.  A "raw8" holds 8 consecutive elements as opaque bits (one
// operand fragment or one staging chunk); "raw4" holds 4.
// ----------------------------------------------------------------------------
struct BF16 {
    using elem = uint16_t;
    using raw8 = u32x4;
    using raw4 = u32x2;
    static constexpr int kBytes = 2;

    static __device__ __forceinline__ f32x16 mma(raw8 a, raw8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // 8 accumulator registers (floats) -> one operand fragment.
    static __device__ __forceinline__ raw8 pack8(const f32x16& v, int base) {
        raw8 r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r[i] = bf16_bits_rne(v[base + 2 * i]) | (bf16_bits_rne(v[base + 2 * i + 1]) << 16);
        return r;
    }
    static __device__ __forceinline__ raw8 pack8_scaled(const f32x16& v, int base, float s) {
        raw8 r;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r[i] = bf16_bits_rne(v[base + 2 * i] * s) | (bf16_bits_rne(v[base + 2 * i + 1] * s) << 16);
        return r;
    }
    static __device__ __forceinline__ raw4 pack4(float a, float b, float c, float d) {
        raw4 r;
        r[0] = bf16_bits_rne(a) | (bf16_bits_rne(b) << 16);
        r[1] = bf16_bits_rne(c) | (bf16_bits_rne(d) << 16);
        return r;
    }
    // element e of a raw8 as its 16 bits in the low half of a word
    static __device__ __forceinline__ uint32_t get(const raw8& r, int e) {
        return (e & 1) ? (r[e >> 1] >> 16) : (r[e >> 1] & 0xffffu);
    }
    static __device__ __forceinline__ raw4 join4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
        raw4 r;
        r[0] = a | (b << 16);
        r[1] = c | (d << 16);
        return r;
    }
    static __device__ __forceinline__ float to_f32(const raw8& r, int e) {
        return __uint_as_float(get(r, e) << 16);
    }
};

struct F32 {
    using elem = float;
    using raw8 = u32x8;
    using raw4 = u32x4;
    static constexpr int kBytes = 4;

    static __device__ __forceinline__ f32x16 mma(raw8 a, raw8 b, f32x16 c) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ raw8 pack8(const f32x16& v, int base) {
        raw8 r;
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = __float_as_uint(v[base + i]);
        return r;
    }
    static __device__ __forceinline__ raw8 pack8_scaled(const f32x16& v, int base, float s) {
        raw8 r;
#pragma unroll
        for (int i = 0; i < 8; ++i) r[i] = __float_as_uint(v[base + i] * s);
        return r;
    }
    static __device__ __forceinline__ raw4 pack4(float a, float b, float c, float d) {
        raw4 r;
        r[0] = __float_as_uint(a); r[1] = __float_as_uint(b);
        r[2] = __float_as_uint(c); r[3] = __float_as_uint(d);
        return r;
    }
    static __device__ __forceinline__ uint32_t get(const raw8& r, int e) { return r[e]; }
    static __device__ __forceinline__ raw4 join4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
        raw4 r;
        r[0] = a; r[1] = b; r[2] = c; r[3] = d;
        return r;
    }
    static __device__ __forceinline__ float to_f32(const raw8& r, int e) { return __uint_as_float(r[e]); }
};

template <class ET>
__device__ __forceinline__ typename ET::raw8 ld8(const typename ET::elem* p) {
    return *reinterpret_cast<const typename ET::raw8*>(p);
}
template <class ET>
__device__ __forceinline__ void st8(typename ET::elem* p, const typename ET::raw8& v) {
    *reinterpret_cast<typename ET::raw8*>(p) = v;
}
template <class ET>
__device__ __forceinline__ void st4(typename ET::elem* p, const typename ET::raw4& v) {
    *reinterpret_cast<typename ET::raw4*>(p) = v;
}

// ----------------------------------------------------------------------------
// Global -> LDS staging of one ROWS x COLS tile (row-major in global memory,
// COLS elements per row, rows past `rows_valid` read as zero).  Loads go to
// registers first so that the next tile's loads overlap the current compute.
//
// NatTile: LDS copy keeps the layout, row stride COLS + 8 elements.
// TrTile : LDS copy is transposed, [COLS][ROWS + 8], with the row index
//          stored at position swap23(row) -- the "transposed A operand" form.
// ----------------------------------------------------------------------------
template <class ET, int ROWS, int COLS, int NT>
struct NatTile {
    using elem = typename ET::elem;
    using raw8 = typename ET::raw8;
    static constexpr int kSegs = COLS / 8;
    static constexpr int kChunks = ROWS * kSegs;
    static constexpr int kPer = (kChunks + NT - 1) / NT;
    static constexpr int kStride = COLS + 8;
    static constexpr int kElems = ROWS * kStride;
    raw8 r[kPer];

    __device__ __forceinline__ void load(const elem* src, int rows_valid, int tid) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = tid + i * NT;
            const int row = c / kSegs, seg = c % kSegs;
            raw8 v = {};
            if ((kChunks % NT == 0 || c < kChunks) && row < rows_valid)
                v = ld8<ET>(src + (int64_t)row * COLS + seg * 8);
            r[i] = v;
        }
    }
    __device__ __forceinline__ void store(elem* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = tid + i * NT;
            if (kChunks % NT == 0 || c < kChunks) {
                const int row = c / kSegs, seg = c % kSegs;
                st8<ET>(lds + row * kStride + seg * 8, r[i]);
            }
        }
    }
};

template <class ET, int ROWS, int COLS, int NT>
struct TrTile {
    using elem = typename ET::elem;
    using raw8 = typename ET::raw8;
    static constexpr int kGroups = ROWS / 4;          // groups of 4 source rows
    static constexpr int kSegs = COLS / 8;            // 8-column segments
    static constexpr int kTasks = kGroups * kSegs;    // one 4 x 8 block per task
    static constexpr int kPer = (kTasks + NT - 1) / NT;
    static constexpr int kStride = ROWS + 8;
    static constexpr int kElems = COLS * kStride;
    static_assert(ROWS % 16 == 0, "transposed tiles hold whole groups of 16 rows");
    raw8 r[kPer][4];

    __device__ __forceinline__ void load(const elem* src, int rows_valid, int tid) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int t = tid + i * NT;
            const int rg = t % kGroups, seg = t / kGroups;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                raw8 v = {};
                const int row = 4 * rg + j;
                if ((kTasks % NT == 0 || t < kTasks) && row < rows_valid)
                    v = ld8<ET>(src + (int64_t)row * COLS + seg * 8);
                r[i][j] = v;
            }
        }
    }
    __device__ __forceinline__ void store(elem* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int t = tid + i * NT;
            if (kTasks % NT == 0 || t < kTasks) {
                const int rg = t % kGroups, seg = t / kGroups;
                const int pos = swap23(4 * rg);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    st4<ET>(lds + (8 * seg + e) * kStride + pos,
                            ET::join4(ET::get(r[i][0], e), ET::get(r[i][1], e),
                                      ET::get(r[i][2], e), ET::get(r[i][3], e)));
            }
        }
    }
};

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own L2.
// Give every XCD one contiguous range of logical tiles, so that the tiles of a
// head (which share K and V) run on the same XCD.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
    constexpr int kXcd = 8;
    const int per = total / kXcd, rem = total % kXcd;
    const int x = bid % kXcd, i = bid / kXcd;
    return x * per + (x < rem ? x : rem) + i;
}

// Persistent launches: one workgroup per resident slot, each looping over
// work items.  The hardware dispatches workgroups in order, so with items of
// unequal length (causal row blocks) a non-persistent grid leaves CUs idle
// while a busy XCD holds up the dispatch of the next workgroups.
//
// Items [0, total) are split into 8 contiguous ranges, one per XCD (workgroup
// w runs on XCD w % 8), so that the items sharing K and V stay on one L2.
// The Cx workgroups of an XCD take its items in rounds of Cx, alternating
// direction every round: with items listed long-to-short inside each run of
// row blocks, a workgroup that drew a long item in one round draws a short
// one in the next.  With total <= gridDim.x every workgroup gets at most one
// item, the mapping of xcd_remap.
struct PersistentSched {
    int first, cnt, c, cx;
    __device__ __forceinline__ explicit PersistentSched(int total) {
        constexpr int kXcd = 8;
        const int x = blockIdx.x % kXcd, w = gridDim.x;
        c = blockIdx.x / kXcd;
        cx = w / kXcd + (x < w % kXcd ? 1 : 0);
        const int per = total / kXcd, rem = total % kXcd;
        first = x * per + (x < rem ? x : rem);
        cnt = per + (x < rem ? 1 : 0);
    }
    // round r has items left for this XCD
    __device__ __forceinline__ bool more(int r) const { return r * cx < cnt; }
    // this workgroup's item in round r, or -1 (the last, partial round)
    __device__ __forceinline__ int item(int r) const {
        const int j = r * cx + ((r & 1) ? cx - 1 - c : c);
        return j < cnt ? first + j : -1;
    }
};

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Row index (within a 32-row block) held by register r of lane half hh.
__device__ __forceinline__ constexpr int acc_row(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }


// ----------------------------------------------------------------------------
// bf16 tiles kept in LDS in their global (row-major) layout, filled by direct
// global -> LDS loads and read either as rows (16-byte reads, the operand of a
// product that contracts over the row's columns) or transposed (the operand
// of a product that contracts over rows).
//
// Transposed read (ds_read_b64_tr_b16): inside each 16-lane group, output
// lane i, element j receives element (i % 4) of what source lane 4*j + i/4
// loaded.  Source lane t therefore reads row kbase + t/4, columns
// n0 + 4*(t%4) .. +3, and output lane i ends up holding the column n0 + i for
// rows kbase .. kbase+3: four consecutive contraction slots of one row of the
// transposed operand.  Two such reads fill the eight slots of a lane.
// ----------------------------------------------------------------------------
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef const __attribute__((address_space(1))) void gbl_void;

// Pack two floats into two bf16 (hardware round-to-nearest-even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ u32x4 pack_bf16x8(const f32x16& v, int base) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(v[base + 2 * i], v[base + 2 * i + 1]);
    return r;
}

// acc + (lo + hi) of the two bf16 values packed in w, in float32.
__device__ __forceinline__ float dot2_bf16_sum(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                           acc, false);
}

// Both halves of the wave: (x of lane l%32, x of lane l%32 + 32).
__device__ __forceinline__ float pair_max(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// ----------------------------------------------------------------------------
// Direct global -> LDS loads are issued from inline assembly, so the compiler
// does not see their LDS writes and never inserts its own conservative
// "wait for every outstanding load" before an LDS read.  Completion is managed
// explicitly: a tile is ready once this wave's loads for it are done
// (s_waitcnt vmcnt) and every wave has passed the next s_barrier.
// ----------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
// 16 bytes per lane from `gptr` to LDS address m0 + 16 * lane (m0 must be
// wave-uniform; it is moved to a scalar register here).  M0 is written inside
// the statement; these kernels use M0 for nothing else.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(m0))
                 : "memory");
}
// Same copy from a wave-uniform base plus a 32-bit per-lane byte offset (the
// scalar-base form of the instruction: no per-lane 64-bit address arithmetic).
// (readfirstlane returns int: each half goes through uint32_t before it is
// widened, or the low half would be sign-extended into the high one.)
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t m0) {
    const uint64_t p = (uint64_t)(uintptr_t)sbase;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
    const uint64_t ps = ((uint64_t)hi << 32) | (uint64_t)lo;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(ps), "s"(__builtin_amdgcn_readfirstlane(m0))
                 : "memory");
}
// Make the compiler finish its own pending loads into these registers here
// (an empty statement that reads them), so that its waits are not placed in a
// later pipelined loop, where they would also drain the asm-issued loads.
__device__ __forceinline__ void settle(const u32x4& x) { asm volatile("" : : "v"(x)); }
__device__ __forceinline__ void settle(float x) { asm volatile("" : : "v"(x)); }
__device__ __forceinline__ void settle(const f32x16& x) { asm volatile("" : : "v"(x)); }

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// vmcnt(later * L) for a run-time later in [0, MAXL] (the count is an
// immediate of the instruction).
template <int L, int MAXL>
__device__ __forceinline__ void wait_vm_dyn(int later) {
    if constexpr (MAXL >= 5) { if (later >= 5) { wait_vm<5 * L>(); return; } }
    if constexpr (MAXL >= 4) { if (later == 4) { wait_vm<4 * L>(); return; } }
    if constexpr (MAXL >= 3) { if (later == 3) { wait_vm<3 * L>(); return; } }
    if constexpr (MAXL >= 2) { if (later == 2) { wait_vm<2 * L>(); return; } }
    if constexpr (MAXL >= 1) { if (later == 1) { wait_vm<L>(); return; } }
    wait_vm<0>();
}
// Workgroup barrier that does not drain outstanding global loads; LDS reads
// of the previous tile are completed first.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory"); }

// Wait until this wave's loads for tile j have landed, with a pipeline of NS
// stages (tiles j+1 .. j+NS-2, when they exist, may still be in flight) and L
// load instructions per wave per tile.
template <int NS, int L>
__device__ __forceinline__ void pipe_wait(int j, int total) {
    static_assert(NS >= 2 && NS <= 4 && L * (NS - 2) <= 63, "vmcnt range");
    const int later = total - 1 - j;
    if constexpr (NS == 2) {
        wait_vm<0>();
    } else if constexpr (NS == 3) {
        if (later >= 1) wait_vm<L>(); else wait_vm<0>();
    } else {
        if (later >= 2) wait_vm<2 * L>(); else if (later == 1) wait_vm<L>(); else wait_vm<0>();
    }
}

// Tile layout in LDS ("row groups"): rows are taken in groups of RG, where RG
// rows hold exactly 64 chunks (1 KB, the bytes one wave moves with one direct
// load).  Inside a group, chunk c of row r sits at 16 * (c * RG + r % RG);
// groups are RGS = 1 KB + 64 bytes apart.  Consequences:
//  - one wave fills one group with one global_load_lds, reading 1 KB of
//    contiguous global memory;
//  - a row read (16 consecutive lanes: 16 rows, one chunk) touches
//    16 * 16 bytes spread over groups offset by 64 bytes: no bank collision;
//  - a transposed read touches, per 16 lanes, 4 rows of 2 neighbouring chunks:
//    128 contiguous bytes;
//  - every fragment address is one per-lane base plus a compile-time offset.
// RG is 4 rows of 256 bytes (bf16, d = 128), 8 rows of 128 bytes (bf16 d = 64,
// or E4M3 codes at d = 128) or 16 rows of 64 bytes (E4M3 codes at d = 64).
template <int ROWS, int COLS, int NW>
struct LdsTile {
    static constexpr int CPR = COLS / 8;                 // 16-byte chunks per row
    static constexpr int RG = 64 / CPR;                  // rows per group
    static constexpr int RGS = 1024 + 64;                // bytes between groups
    static constexpr int kGroups = ROWS / RG;
    static constexpr int kBytes = kGroups * RGS;
    static constexpr int kElems = kBytes / 2;
    static constexpr int kPerWave = kGroups / NW;
    static_assert(CPR == 4 || CPR == 8 || CPR == 16, "32, 64 or 128 columns");
    static_assert(kGroups % NW == 0, "the waves cover the tile in whole groups");

    // Direct global -> LDS copy of rows [0, ROWS) of `src` (row stride COLS).
    // Rows at or past rows_valid re-read the last valid row: finite values the
    // caller masks out.
    static __device__ __forceinline__ void load(const uint16_t* src, int rows_valid, const uint16_t* tile,
                                                int wave, int lane) {
        const int c = lane / RG, r = lane % RG;
        const uint32_t base = lds_addr(tile);
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            const int grp = i * NW + wave;
            const int row = grp * RG + r;
            const int grow = row < rows_valid ? row : rows_valid - 1;
            dma16(src + (int64_t)grow * COLS + c * 8, base + grp * RGS);
        }
    }
    // Byte offset of (row, chunk).
    static __device__ __forceinline__ constexpr int off(int row, int c) {
        return (row / RG) * RGS + (c * RG + row % RG) * 16;
    }
    // 8 consecutive elements (chunk c) of row r.
    static __device__ __forceinline__ u32x4 row8(const uint16_t* tile, int r, int c) {
        return *reinterpret_cast<const u32x4*>((const char*)tile + off(r, c));
    }
    // Transposed operand fragment: this lane gets column n0 + lane%32 (n0 a
    // multiple of 32) for rows kk + swap23(8*hh + e), e = 0..7 (kk a multiple of 16).
    static __device__ __forceinline__ u32x4 tr8(const uint16_t* tile, int kk, int n0, int lane) {
        const int hh = lane >> 5, half = (lane >> 4) & 1, t = lane & 15;
        const int col = n0 + 16 * half + 4 * (t & 3);
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = kk + 8 * i + 4 * hh + (t >> 2);
            const char* a = (const char*)tile + off(row, col >> 3) + 2 * (col & 7);
            const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a);
            const u32x2 w = __builtin_bit_cast(u32x2, v);
            r[2 * i] = w[0];
            r[2 * i + 1] = w[1];
        }
        return r;
    }
};

// ----------------------------------------------------------------------------
// Attention dropout.  Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011):
// a four-word counter and a two-word key; each of ten rounds forms two 32 x 32
// -> 64-bit products of counter words 0 and 2, builds the new counter from
// their halves, the other two words and the key, and bumps the key by the
// Weyl constants.  The 64-bit product form compiles to one v_mad_u64_u32 per
// product.  Returns the four output words in c.
// ----------------------------------------------------------------------------
// NC counters under one key, their rounds interleaved: each round key is
// formed once for all of them.
template <int NC>
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[NC][4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
#pragma unroll
        for (int n = 0; n < NC; ++n) {
            const uint64_t p0 = (uint64_t)0xD2511F53u * c[n][0];
            const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[n][2];
            // three-input xor in one v_bitop3_b32 (truth table 0x96)
            const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c[n][1], k0, 0x96);
            const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c[n][3], k1, 0x96);
            c[n][1] = (uint32_t)p1;
            c[n][3] = (uint32_t)p0;
            c[n][0] = n0;
            c[n][2] = n2;
        }
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

// A work split of a block mask (block-sparse kernels): work item c covers the
// entries e0 .. e1-1 of row (or column) block r of the compressed layout,
// chunks[4c .. 4c+3] = (r, e0, e1, slot).  slot < 0: the item is the whole
// row (column) and writes the outputs; slot >= 0: it writes a float32 partial
// into that slot of `part`, and a merge pass combines a block's partials.
// chunks == nullptr: one item per block row (column), the plain layout.
struct BspSplit {
    const int* chunks;
    int nchunks, nslots;
    float* part;
};

// Dropout parameters.  One Philox call serves a 4 x 4 block of the score
// matrix, one byte per element: element (query i, key j) of (batch b, query
// head h) takes byte 4 (i % 4) + j % 4 of Philox((j / 4, i / 4, b * Hq + h,
// 0), (key0, key1)) -- byte e of output word i % 4 -- and is kept iff that
// byte is >= thr = floor(256 p).  Kept probabilities are scaled by
// rkeep = 256 / (256 - thr), one over the keep probability.
struct DropArgs {
    uint32_t thr, key0, key1;
    float rkeep;
};

__device__ __forceinline__ bool drop_keep(uint32_t w, int e, uint32_t thr) { return ((w >> (8 * e)) & 0xffu) >= thr; }

// 4 x 4 transpose of 32-bit words inside each quad of lanes: lane x of a quad
// holds a[0..3]; afterwards lane y holds (a[y] of lane 0, ..., a[y] of lane 3).
// Two butterfly stages (partners x ^ 1, then x ^ 2), each lane sending the
// words whose index bit differs from its own lane bit.
__device__ __forceinline__ void quad_transpose(uint32_t a[4], int x) {
    const bool b0 = x & 1, b1 = x & 2;
#pragma unroll
    for (int k = 0; k < 4; k += 2) {
        const uint32_t s = b0 ? a[k] : a[k + 1];
        const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)s, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
        a[k] = b0 ? r : a[k];
        a[k + 1] = b0 ? a[k + 1] : r;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t s = b1 ? a[k] : a[k + 2];
        const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)s, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
        a[k] = b1 ? r : a[k];
        a[k + 2] = b1 ? a[k + 2] : r;
    }
}

// Keep bytes of KB 32-key blocks for an accumulator that holds a query per
// lane (forward, dQ): lane query qrow, element 4 t + e of block kb the key
// k0 + 32 kb + 8 t + 4 hh + e (k0 a multiple of 32).  The quad's lanes hold
// four consecutive queries (qrow % 4 = x, the lane in the quad), so each call
// serves the whole quad: lane x makes the calls of the keys k0 + 32 kb + 8 x +
// 4 hh .. + 3, and the quad transpose gives lane y word y of each block's four
// calls.  On return byte e of w[kb][t] decides element 4 t + e of block kb.
template <int KB>
__device__ __forceinline__ void drop_words_qrow(uint32_t (&w)[KB][4], int k0, int qrow, int hh, int x,
                                                uint32_t bhq, const DropArgs& d) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        w[kb][0] = (uint32_t)((k0 + 32 * kb) >> 2) + (uint32_t)(2 * x + hh);
        w[kb][1] = (uint32_t)qrow >> 2;
        w[kb][2] = bhq;
        w[kb][3] = 0u;
    }
    philox4x32_10(w, d.key0, d.key1);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) quad_transpose(w[kb], x);
}

// Keep bytes of one 32-query block for an accumulator that holds a key per
// lane (dK/dV): lane key krow, element 4 g + e the query qb0 + 8 g + 4 hh + e
// (qb0 a multiple of 32).  The quad's lanes hold four consecutive keys
// (krow % 4 = x): lane x makes the call of the queries qb0 + 8 x + 4 hh .. + 3,
// gathers byte y of its four words into word y (word e of a call belongs to
// query offset e, byte y to key offset y), and the quad transpose gives lane y
// word y of each call.  On return byte e of w[g] decides element 4 g + e.
__device__ __forceinline__ void drop_words_krow(uint32_t w[4], int qb0, int krow, int hh, int x, uint32_t bhq,
                                                const DropArgs& d) {
    uint32_t c[1][4] = {{(uint32_t)krow >> 2, (uint32_t)(qb0 >> 2) + (uint32_t)(2 * x + hh), bhq, 0u}};
    philox4x32_10(c, d.key0, d.key1);
#pragma unroll
    for (int y = 0; y < 4; ++y)
        w[y] = ((c[0][0] >> (8 * y)) & 0xffu) | (((c[0][1] >> (8 * y)) & 0xffu) << 8) |
               (((c[0][2] >> (8 * y)) & 0xffu) << 16) | (((c[0][3] >> (8 * y)) & 0xffu) << 24);
    quad_transpose(w, x);
}

__device__ __forceinline__ f32x16 mma_bf16(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

}  // namespace fa
