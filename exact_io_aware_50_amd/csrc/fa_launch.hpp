// Internal launchers (C++ linkage) called by the C entry points in fa_api.hip.
// Arguments are already validated; each returns the launch's hipError_t.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <atomic>

namespace fa {

// Values fixed by the device and the code object (the CU count, a kernel's
// resident workgroups per CU), queried on a device's first use and kept per
// device for the process.  0 = not yet known.
constexpr int kMaxDevices = 64;
struct PerDevice {
    std::atomic<int> v[kMaxDevices];
};

// The current device, or -1 if it cannot be queried or is past kMaxDevices.
inline int current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    return dev;
}

// CUs of the current device (256 on MI355X; 256 also if the query fails).
inline int device_cus() {
    static PerDevice cache;
    const int dev = current_device();
    if (dev < 0) return 256;
    int cus = cache.v[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return 256;
        cache.v[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

// Workgroups of a persistent launch: every resident slot of the current
// device (CUs x workgroups per CU), at most `items`.  The slot count is kept
// per device in `cache`; if a query fails the grid is `items`, one item per
// workgroup, which the kernels' schedule also handles.
inline int persistent_grid(const void* kernel, int threads, int items, PerDevice& cache) {
    const int dev = current_device();
    int slots = dev < 0 ? 0 : cache.v[dev].load(std::memory_order_relaxed);
    if (slots == 0) {
        int per = 0;
        const int cus = device_cus();
        if (dev < 0 || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, threads, 0) != hipSuccess ||
            per <= 0)
            return items;
        slots = cus * per;
        cache.v[dev].store(slots, std::memory_order_relaxed);
    }
    return items < slots ? items : slots;
}

// dtype: 0 = float32, 1 = bfloat16 (fp8 goes through launch_fwd_fp8)
hipError_t launch_fwd(int dtype, int d, int causal, const void* q, const void* k, const void* v,
                      void* o, float* lse, int B, int Hq, int Hkv, int N, float scale,
                      hipStream_t st);

hipError_t launch_fwd_bf16(int d, int causal, const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int N, float scale, hipStream_t st);

hipError_t launch_fwd_fp8(int d, int causal, const void* q, const void* k, const void* v,
                          void* o, float* lse, const float* descale, int B, int Hq, int Hkv, int N,
                          float scale, hipStream_t st);

// Rows per (batch, head) in the backward workspace: N rounded up to 64.
inline int ws_rows(int N) { return (N + 63) / 64 * 64; }

// keep: the factor on -D in the workspace (1, or 1 - p through dropout)
hipError_t launch_bwd_delta(int dtype, int d, const void* o, const void* dO, const float* lse, float* ws, int B,
                            int Hq, int N, hipStream_t st, float keep = 1.f);

hipError_t launch_bwd_dkdv(int dtype, int d, int causal, const void* q, const void* k, const void* v,
                           const void* dO, const float* ws, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                           float scale, hipStream_t st);

hipError_t launch_bwd_dq(int dtype, int d, int causal, const void* q, const void* k, const void* v,
                         const void* dO, const float* ws, void* dq, int B, int Hq, int Hkv, int N, float scale,
                         hipStream_t st);

hipError_t launch_bwd_dkdv_bf16(int d, int causal, const void* q, const void* k, const void* v, const void* dO,
                                const float* ws, void* dk, void* dv, int B, int Hq, int Hkv, int N, float scale,
                                hipStream_t st);

hipError_t launch_bwd_dq_bf16(int d, int causal, const void* q, const void* k, const void* v, const void* dO,
                              const float* ws, void* dq, int B, int Hq, int Hkv, int N, float scale, hipStream_t st);

// Causal sliding-window (local) attention with S global tokens, bf16: key j
// visible to query i iff j <= i and (i - W < j or j < S).
hipError_t launch_fwd_bf16_local(int d, const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                 int Hq, int Hkv, int N, int W, int S, float scale, hipStream_t st);
hipError_t launch_bwd_dkdv_bf16_local(int d, const void* q, const void* k, const void* v, const void* dO,
                                      const float* ws, void* dk, void* dv, int B, int Hq, int Hkv, int N, int W,
                                      int S, float scale, hipStream_t st);
hipError_t launch_bwd_dq_bf16_local(int d, const void* q, const void* k, const void* v, const void* dO,
                                    const float* ws, void* dq, int B, int Hq, int Hkv, int N, int W, int S,
                                    float scale, hipStream_t st);

// Block-sparse attention, bf16: key j visible to query i iff block
// (i / 256, j / 256) is on (and j <= i with causal).  The forward and dQ read
// the mask by rows (row_ptr / col_idx), dK / dV by columns (col_ptr / row_idx).
hipError_t launch_fwd_bf16_bsparse(int d, int causal, const void* q, const void* k, const void* v, void* o,
                                   float* lse, int B, int Hq, int Hkv, int N, const int* row_ptr,
                                   const int* col_idx, int nnz, float scale, hipStream_t st);
hipError_t launch_bwd_bf16_bsparse(int d, int causal, const void* q, const void* k, const void* v, const void* dO,
                                   const float* ws, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                                   const int* row_ptr, const int* col_idx, const int* col_ptr, const int* row_idx,
                                   int nnz, float scale, hipStream_t st);

// Forward with attention dropout, bf16: element (i, j) of (b, h) kept iff word
// j % 4 of Philox4x32-10((j / 4, i, b * Hq + h, 0), seed halves) >= thr; kept
// probabilities scaled by rkeep.
hipError_t launch_fwd_bf16_dropout(int d, int causal, const void* q, const void* k, const void* v, void* o,
                                   float* lse, int B, int Hq, int Hkv, int N, uint32_t thr, uint64_t seed, float rkeep,
                                   float scale, hipStream_t st);

// Backward through that dropout (the same mask regenerated), bf16: dK/dV then
// dQ, from a workspace written by launch_bwd_delta with keep = 1 - p.
// Block-sparse with a work split (heavy block rows / columns cut into several
// items): the attention kernels write float32 partials of split blocks into
// `part`, merge passes combine them (the LSE merge forward, sums backward).
hipError_t launch_fwd_bf16_bsparse_split(int d, int causal, const void* q, const void* k, const void* v, void* o,
                                         float* lse, int B, int Hq, int Hkv, int N, const int* col_idx, int nnz,
                                         const int* chunks, int nchunks, const int* merges, int nmerge, int nslots,
                                         float* part, float scale, hipStream_t st);
hipError_t launch_bwd_bf16_bsparse_split(int d, int causal, const void* q, const void* k, const void* v,
                                         const void* dO, const float* ws, void* dq, void* dk, void* dv, int B, int Hq,
                                         int Hkv, int N, const int* col_idx, const int* row_idx, int nnz,
                                         const int* row_chunks, int n_row_chunks, const int* row_merges,
                                         int n_row_merges, int n_row_slots, const int* col_chunks, int n_col_chunks,
                                         const int* col_merges, int n_col_merges, int n_col_slots, float* part,
                                         float scale, hipStream_t st);

hipError_t launch_bwd_bf16_dropout(int d, int causal, const void* q, const void* k, const void* v, const void* dO,
                                   const float* ws, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                                   uint32_t thr, uint64_t seed, float rkeep, float scale, hipStream_t st);

// FP8 backward (d = 128): delta, dK/dV and dQ kernels; descale = (s_Q, s_K, s_V, s_dO).
hipError_t launch_bwd_fp8(int causal, const void* q, const void* k, const void* v, const void* o, const void* dO,
                          const float* lse, const float* descale, float* ws, void* dq, void* dk, void* dv, int B,
                          int Hq, int Hkv, int N, float scale, hipStream_t st);

hipError_t launch_quantize_fp8(const void* x, size_t n, void* out, float* descale, hipStream_t st);

// Decode split over the keys: nrb blocks of 32 packed query rows per K/V head,
// nsplit chunks of `chunk` keys (a multiple of 32).
struct DecodePlan {
    int nrb, nsplit, chunk;
};
// `cus` is the CU count the split is sized for (the current device's at a
// launch and in the workspace size).
DecodePlan decode_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d, int per_slot, int cus);
// Paged decode: chunk slots of the device-side plan, and the workspace
// (plan ints [B][4] + [T][3], 16-byte aligned, then float32 O [T][Hq][Nq][d]
// and LSE [T][Hq][Nq]), both for the current device's CU count.
int paged_chunks(int B, int Hq, int Hkv, int Nq, int d, int cus);
size_t paged_ws_bytes(int B, int Hq, int Hkv, int Nq, int d);

// Upper bound on the CU count used when sizes are checked before any HIP call.
constexpr int kCuBound = 1024;

// Workspace of fa_decode: float32 O per (row, chunk) [rows][nsplit][d], then
// the chunk LSEs [rows][nsplit], rows = B * Hq * Nq.
inline size_t decode_ws_bytes(const DecodePlan& p, int B, int Hq, int Nq, int d) {
    return (size_t)4 * (size_t)B * (size_t)Hq * (size_t)Nq * (size_t)p.nsplit * (size_t)(d + 1);
}

// Paged cache [nblk][Hkv][bs][d], block table [B][maxb], lengths [B] (device).
hipError_t launch_decode_paged(int d, int causal, const void* q, const void* kc, const void* vc, const int* table,
                               const int* lens, void* o, float* lse, float* ws, int B, int Hq, int Hkv, int Nq,
                               int maxb, int bs, int nblk, float scale, hipStream_t st);

hipError_t launch_decode(int d, int causal, const void* q, const void* k, const void* v, void* o, float* lse,
                         float* ws, int B, int Hq, int Hkv, int Nq, int Nk, float scale, hipStream_t st);

}  // namespace fa
