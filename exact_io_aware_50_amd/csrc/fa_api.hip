// C entry points declared in include/fa.h: argument validation (host only,
// before any HIP call), then dispatch to the kernel launchers.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <initializer_list>
#include <mutex>

#include "fa.h"
#include "fa_launch.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Common shape checks.  Returns FA_OK and sets *empty for an empty problem.
fa_status_t check_shape(int B, int Hq, int Hkv, int N, int d, int causal, float scale, bool* empty) {
    if (B < 0 || Hq < 0 || Hkv < 0 || N < 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_UNSUPPORTED;
    *empty = (B == 0 || Hq == 0 || N == 0);
    if (*empty) return FA_OK;
    if (Hkv == 0 || Hq % Hkv != 0) return FA_ERR_SHAPE;
    // grids are one-dimensional: (query or key blocks) x heads x batch must fit
    const int64_t blocks = ((int64_t)N + 31) / 32 * (int64_t)Hq * (int64_t)B;
    if (blocks > INT32_MAX) return FA_ERR_SHAPE;
    return FA_OK;
}

fa_status_t launch_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

}  // namespace

extern "C" {

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                   int N, int d, int causal, float softmax_scale, fa_dtype_t dtype, const float* descale_qkv,
                   hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP8_E4M3) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_shape(B, Hq, Hkv, N, d, causal, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
    const bool fp8 = dtype == FA_DTYPE_FP8_E4M3;
    if (fp8 != (descale_qkv != nullptr)) return fp8 ? FA_ERR_NULL : FA_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return FA_ERR_ALIGN;
    if (fp8 && !aligned(descale_qkv, 4)) return FA_ERR_ALIGN;
    if (o == q || o == k || o == v || (void*)lse == q || (void*)lse == k || (void*)lse == v || (void*)lse == o)
        return FA_ERR_ALIAS;
    if (fp8)
        return launch_status(fa::launch_fwd_fp8(d, causal, q, k, v, o, lse, descale_qkv, B, Hq, Hkv, N,
                                                softmax_scale, stream));
    return launch_status(fa::launch_fwd(dtype, d, causal, q, k, v, o, lse, B, Hq, Hkv, N, softmax_scale, stream));
}

}  // extern "C"

namespace {

// Pointer checks shared by the backward entry points: non-NULL, aligned (float
// arrays to 4 bytes, tensors to 16), and no output equal to an input or to
// another output.
fa_status_t check_ptrs(std::initializer_list<const void*> in, std::initializer_list<const void*> in_f32,
                       std::initializer_list<const void*> out, std::initializer_list<const void*> out_f32) {
    for (auto l : {in, in_f32, out, out_f32})
        for (const void* p : l)
            if (!p) return FA_ERR_NULL;
    for (const void* p : in)
        if (!aligned(p, 16)) return FA_ERR_ALIGN;
    for (const void* p : out)
        if (!aligned(p, 16)) return FA_ERR_ALIGN;
    for (const void* p : in_f32)
        if (!aligned(p, 4)) return FA_ERR_ALIGN;
    for (const void* p : out_f32)
        if (!aligned(p, 4)) return FA_ERR_ALIGN;
    for (auto lo : {out, out_f32})
        for (const void* a : lo) {
            for (auto li : {in, in_f32})
                for (const void* b : li)
                    if (a == b) return FA_ERR_ALIAS;
            int same = 0;
            for (auto lo2 : {out, out_f32})
                for (const void* b : lo2) same += (a == b);
            if (same > 1) return FA_ERR_ALIAS;
        }
    return FA_OK;
}

}  // namespace

extern "C" {

fa_status_t fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv, float* delta_ws, int B, int Hq, int Hkv, int N, int d,
                   int causal, float softmax_scale, fa_dtype_t dtype, hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_shape(B, Hq, Hkv, N, d, causal, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    s = check_ptrs({q, k, v, o, dO, delta_ws}, {lse}, {dq, dk, dv}, {});
    if (s != FA_OK) return s;
    hipError_t e = fa::launch_bwd_delta(dtype, d, o, dO, lse, delta_ws, B, Hq, N, stream);
    if (e == hipSuccess)
        e = fa::launch_bwd_dkdv(dtype, d, causal, q, k, v, dO, delta_ws, dk, dv, B, Hq, Hkv, N, softmax_scale,
                                stream);
    if (e == hipSuccess)
        e = fa::launch_bwd_dq(dtype, d, causal, q, k, v, dO, delta_ws, dq, B, Hq, Hkv, N, softmax_scale, stream);
    return launch_status(e);
}

}  // extern "C"

// ---------------------------------------------------------------- scratch-free backward
// The workspace of fa_bwd_noalloc: a library-owned device array, one copy per
// device.  In host code `scratch` only names the symbol; its address on a
// device comes from hipGetSymbolAddress with that device current, and only
// that address is ever passed to a kernel.
static __device__ __align__(256) float scratch[FA_BWD_NOALLOC_MAX_BYTES / 4];

namespace {

std::atomic<float*> g_scratch[fa::kMaxDevices];
std::mutex g_scratch_mu;

// Address of `scratch` on the current device, looked up once per device
// (nullptr if the device or the lookup fails).
float* scratch_on_current_device() {
    const int dev = fa::current_device();
    if (dev < 0) return nullptr;
    float* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        void* a = nullptr;
        if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return nullptr;
        p = static_cast<float*>(a);
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

fa_status_t fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                           const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
                           int causal, float softmax_scale, fa_dtype_t dtype, hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_shape(B, Hq, Hkv, N, d, causal, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    if ((uint64_t)8 * (uint64_t)B * (uint64_t)Hq * (uint64_t)fa::ws_rows(N) > FA_BWD_NOALLOC_MAX_BYTES)
        return FA_ERR_SHAPE;
    s = check_ptrs({q, k, v, o, dO}, {lse}, {dq, dk, dv}, {});
    if (s != FA_OK) return s;
    float* ws = scratch_on_current_device();
    if (!ws) return FA_ERR_LAUNCH;
    // the three kernels of fa_bwd: the delta kernel writes every workspace row
    // (padding included) before the other two read it, so nothing is cleared
    hipError_t e = fa::launch_bwd_delta(dtype, d, o, dO, lse, ws, B, Hq, N, stream);
    if (e == hipSuccess)
        e = fa::launch_bwd_dkdv(dtype, d, causal, q, k, v, dO, ws, dk, dv, B, Hq, Hkv, N, softmax_scale, stream);
    if (e == hipSuccess)
        e = fa::launch_bwd_dq(dtype, d, causal, q, k, v, dO, ws, dq, B, Hq, Hkv, N, softmax_scale, stream);
    return launch_status(e);
}

fa_status_t fa_bwd_delta(const void* o, const void* dO, const float* lse, float* ws, int B, int Hq, int N, int d,
                         fa_dtype_t dtype, hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_shape(B, Hq, 1, N, d, 0, 1.0f, &empty);
    if (s != FA_OK || empty) return s;
    s = check_ptrs({o, dO}, {lse}, {ws}, {});
    if (s != FA_OK) return s;
    return launch_status(fa::launch_bwd_delta(dtype, d, o, dO, lse, ws, B, Hq, N, stream));
}

fa_status_t fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* ws, void* dk,
                        void* dv, int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                        fa_dtype_t dtype, hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_shape(B, Hq, Hkv, N, d, causal, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    s = check_ptrs({q, k, v, dO, ws}, {}, {dk, dv}, {});
    if (s != FA_OK) return s;
    return launch_status(fa::launch_bwd_dkdv(dtype, d, causal, q, k, v, dO, ws, dk, dv, B, Hq, Hkv, N,
                                             softmax_scale, stream));
}

fa_status_t fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const float* ws, void* dq, int B,
                      int Hq, int Hkv, int N, int d, int causal, float softmax_scale, fa_dtype_t dtype,
                      hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_shape(B, Hq, Hkv, N, d, causal, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    s = check_ptrs({q, k, v, dO, ws}, {}, {dq}, {});
    if (s != FA_OK) return s;
    return launch_status(fa::launch_bwd_dq(dtype, d, causal, q, k, v, dO, ws, dq, B, Hq, Hkv, N, softmax_scale,
                                           stream));
}

// Sliding window: W >= N, or S >= N, sees exactly the causal keys, so the
// causal kernels run.
fa_status_t fa_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                         int N, int d, int window, int sink, float softmax_scale, fa_dtype_t dtype,
                         hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    if (window < 1 || sink < 0) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_shape(B, Hq, Hkv, N, d, 1, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    s = check_ptrs({q, k, v}, {}, {o}, {lse});
    if (s != FA_OK) return s;
    if (window >= N || sink >= N)
        return launch_status(fa::launch_fwd(dtype, d, 1, q, k, v, o, lse, B, Hq, Hkv, N, softmax_scale, stream));
    return launch_status(
        fa::launch_fwd_bf16_local(d, q, k, v, o, lse, B, Hq, Hkv, N, window, sink, softmax_scale, stream));
}

fa_status_t fa_bwd_local(const void* q, const void* k, const void* v, const void* o, const void* dO,
                         const float* lse, void* dq, void* dk, void* dv, float* delta_ws, int B, int Hq, int Hkv,
                         int N, int d, int window, int sink, float softmax_scale, fa_dtype_t dtype,
                         hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    if (window < 1 || sink < 0) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_shape(B, Hq, Hkv, N, d, 1, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    s = check_ptrs({q, k, v, o, dO, delta_ws}, {lse}, {dq, dk, dv}, {});
    if (s != FA_OK) return s;
    if (window >= N || sink >= N)
        return fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, delta_ws, B, Hq, Hkv, N, d, 1, softmax_scale, dtype, stream);
    hipError_t e = fa::launch_bwd_delta(dtype, d, o, dO, lse, delta_ws, B, Hq, N, stream);
    if (e == hipSuccess)
        e = fa::launch_bwd_dkdv_bf16_local(d, q, k, v, dO, delta_ws, dk, dv, B, Hq, Hkv, N, window, sink,
                                           softmax_scale, stream);
    if (e == hipSuccess)
        e = fa::launch_bwd_dq_bf16_local(d, q, k, v, dO, delta_ws, dq, B, Hq, Hkv, N, window, sink, softmax_scale,
                                         stream);
    return launch_status(e);
}

// The keep threshold of a drop probability 0 <= p < 1: a score element is
// kept iff its random byte is >= floor(256 p).
static uint32_t drop_threshold(double p) { return (uint32_t)floor(p * 256.0); }

fa_status_t fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                           int N, int d, int causal, double dropout_p, uint64_t seed, float softmax_scale,
                           fa_dtype_t dtype, hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    if (!(dropout_p >= 0.0 && dropout_p < 1.0)) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_shape(B, Hq, Hkv, N, d, causal, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    s = check_ptrs({q, k, v}, {}, {o}, {lse});
    if (s != FA_OK) return s;
    const uint32_t thr = drop_threshold(dropout_p);
    const float rkeep = 256.f / (float)(256u - thr);
    return launch_status(fa::launch_fwd_bf16_dropout(d, causal, q, k, v, o, lse, B, Hq, Hkv, N, thr, seed, rkeep,
                                                     softmax_scale, stream));
}

fa_status_t fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dO,
                           const float* lse, void* dq, void* dk, void* dv, float* delta_ws, int B, int Hq, int Hkv,
                           int N, int d, int causal, double dropout_p, uint64_t seed, float softmax_scale,
                           fa_dtype_t dtype, hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    if (!(dropout_p >= 0.0 && dropout_p < 1.0)) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_shape(B, Hq, Hkv, N, d, causal, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    s = check_ptrs({q, k, v, o, dO, delta_ws}, {lse}, {dq, dk, dv}, {});
    if (s != FA_OK) return s;
    const uint32_t thr = drop_threshold(dropout_p);
    const float rkeep = 256.f / (float)(256u - thr);
    // the keep probability (256 - thr) / 256 is exact in float32
    hipError_t e = fa::launch_bwd_delta(dtype, d, o, dO, lse, delta_ws, B, Hq, N, stream, (float)(256u - thr) / 256.f);
    if (e == hipSuccess)
        e = fa::launch_bwd_bf16_dropout(d, causal, q, k, v, dO, delta_ws, dq, dk, dv, B, Hq, Hkv, N, thr, seed, rkeep,
                                        softmax_scale, stream);
    return launch_status(e);
}

fa_status_t fa_bwd_fp8(const void* q8, const void* k8, const void* v8, const void* o, const void* do8,
                       const float* lse, const float* descale, void* dq, void* dk, void* dv, float* delta_ws, int B,
                       int Hq, int Hkv, int N, int d, int causal, float softmax_scale, hipStream_t stream) {
    bool empty = false;
    fa_status_t s = check_shape(B, Hq, Hkv, N, d, causal, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    if (d != 128) return FA_ERR_UNSUPPORTED;
    s = check_ptrs({q8, k8, v8, o, do8, delta_ws}, {lse, descale}, {dq, dk, dv}, {});
    if (s != FA_OK) return s;
    return launch_status(fa::launch_bwd_fp8(causal, q8, k8, v8, o, do8, lse, descale, delta_ws, dq, dk, dv, B, Hq,
                                            Hkv, N, softmax_scale, stream));
}

// Mask arrays of the block-sparse entry points (device int arrays).
static fa_status_t check_bsparse(int N, const int* ptr, const int* idx, int nnz) {
    const int64_t nb = ((int64_t)N + FA_BSPARSE_BLOCK - 1) / FA_BSPARSE_BLOCK;
    if (nnz < 0 || nnz > nb * nb) return FA_ERR_SHAPE;
    if (!ptr || (nnz > 0 && !idx)) return FA_ERR_NULL;
    if (!aligned(ptr, 4) || (idx && !aligned(idx, 4))) return FA_ERR_ALIGN;
    return FA_OK;
}

fa_status_t fa_fwd_bsparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                           int Hkv, int N, int d, int causal, const int* row_ptr, const int* col_idx, int nnz,
                           float softmax_scale, fa_dtype_t dtype, hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_shape(B, Hq, Hkv, N, d, causal, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    s = check_bsparse(N, row_ptr, col_idx, nnz);
    if (s != FA_OK) return s;
    s = check_ptrs({q, k, v}, {}, {o}, {lse});
    if (s != FA_OK) return s;
    return launch_status(fa::launch_fwd_bf16_bsparse(d, causal, q, k, v, o, lse, B, Hq, Hkv, N, row_ptr, col_idx,
                                                     nnz, softmax_scale, stream));
}

fa_status_t fa_bwd_bsparse(const void* q, const void* k, const void* v, const void* o, const void* dO,
                           const float* lse, void* dq, void* dk, void* dv, float* delta_ws, int B, int Hq, int Hkv,
                           int N, int d, int causal, const int* row_ptr, const int* col_idx, const int* col_ptr,
                           const int* row_idx, int nnz, float softmax_scale, fa_dtype_t dtype, hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_shape(B, Hq, Hkv, N, d, causal, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    s = check_bsparse(N, row_ptr, col_idx, nnz);
    if (s == FA_OK) s = check_bsparse(N, col_ptr, row_idx, nnz);
    if (s != FA_OK) return s;
    s = check_ptrs({q, k, v, o, dO, delta_ws}, {lse}, {dq, dk, dv}, {});
    if (s != FA_OK) return s;
    hipError_t e = fa::launch_bwd_delta(dtype, d, o, dO, lse, delta_ws, B, Hq, N, stream);
    if (e == hipSuccess)
        e = fa::launch_bwd_bf16_bsparse(d, causal, q, k, v, dO, delta_ws, dq, dk, dv, B, Hq, Hkv, N, row_ptr,
                                        col_idx, col_ptr, row_idx, nnz, softmax_scale, stream);
    return launch_status(e);
}

// Work split of the block-sparse entry points: chunk and merge tables (device
// int4 arrays) and the float32 partial buffer.
static fa_status_t check_split(int N, int nnz, const int* chunks, int nchunks, const int* merges, int nmerges,
                               int nslots, const float* part, int64_t heads) {
    const int64_t nb = ((int64_t)N + FA_BSPARSE_BLOCK - 1) / FA_BSPARSE_BLOCK;
    if (nchunks < 1 || nchunks > nb + nnz || nmerges < 0 || nmerges > nb || nslots < 0 || nslots > nnz)
        return FA_ERR_SHAPE;
    if ((int64_t)nchunks * heads > INT32_MAX || (int64_t)nmerges * heads > INT32_MAX) return FA_ERR_SHAPE;
    if (!chunks || (nmerges > 0 && !merges) || (nslots > 0 && !part)) return FA_ERR_NULL;
    if (!aligned(chunks, 16) || (merges && !aligned(merges, 16)) || (part && !aligned(part, 16))) return FA_ERR_ALIGN;
    return FA_OK;
}

fa_status_t fa_fwd_bsparse_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                                 int Hkv, int N, int d, int causal, const int* col_idx, int nnz,
                                 const int* row_chunks, int n_row_chunks, const int* row_merges, int n_row_merges,
                                 int n_row_slots, float* part_ws, float softmax_scale, fa_dtype_t dtype,
                                 hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_shape(B, Hq, Hkv, N, d, causal, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    const int64_t nb = ((int64_t)N + FA_BSPARSE_BLOCK - 1) / FA_BSPARSE_BLOCK;
    if (nnz < 0 || nnz > nb * nb) return FA_ERR_SHAPE;
    if (nnz > 0 && !col_idx) return FA_ERR_NULL;
    if (col_idx && !aligned(col_idx, 4)) return FA_ERR_ALIGN;
    s = check_split(N, nnz, row_chunks, n_row_chunks, row_merges, n_row_merges, n_row_slots, part_ws,
                    (int64_t)B * Hq);
    if (s != FA_OK) return s;
    s = n_row_slots > 0 ? check_ptrs({q, k, v}, {}, {o}, {lse, part_ws}) : check_ptrs({q, k, v}, {}, {o}, {lse});
    if (s != FA_OK) return s;
    return launch_status(fa::launch_fwd_bf16_bsparse_split(d, causal, q, k, v, o, lse, B, Hq, Hkv, N, col_idx, nnz,
                                                           row_chunks, n_row_chunks, row_merges, n_row_merges,
                                                           n_row_slots, part_ws, softmax_scale, stream));
}

fa_status_t fa_bwd_bsparse_split(const void* q, const void* k, const void* v, const void* o, const void* dO,
                                 const float* lse, void* dq, void* dk, void* dv, float* delta_ws, int B, int Hq,
                                 int Hkv, int N, int d, int causal, const int* col_idx, const int* row_idx, int nnz,
                                 const int* row_chunks, int n_row_chunks, const int* row_merges, int n_row_merges,
                                 int n_row_slots, const int* col_chunks, int n_col_chunks, const int* col_merges,
                                 int n_col_merges, int n_col_slots, float* part_ws, float softmax_scale,
                                 fa_dtype_t dtype, hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_shape(B, Hq, Hkv, N, d, causal, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    const int64_t nb = ((int64_t)N + FA_BSPARSE_BLOCK - 1) / FA_BSPARSE_BLOCK;
    if (nnz < 0 || nnz > nb * nb) return FA_ERR_SHAPE;
    if (nnz > 0 && (!col_idx || !row_idx)) return FA_ERR_NULL;
    if ((col_idx && !aligned(col_idx, 4)) || (row_idx && !aligned(row_idx, 4))) return FA_ERR_ALIGN;
    const int slots = n_row_slots + n_col_slots;
    s = check_split(N, nnz, row_chunks, n_row_chunks, row_merges, n_row_merges, n_row_slots, slots ? part_ws : nullptr,
                    (int64_t)B * Hq);
    if (s == FA_OK)
        s = check_split(N, nnz, col_chunks, n_col_chunks, col_merges, n_col_merges, n_col_slots,
                        slots ? part_ws : nullptr, (int64_t)B * Hkv);
    if (s != FA_OK) return s;
    s = slots > 0 ? check_ptrs({q, k, v, o, dO, delta_ws}, {lse}, {dq, dk, dv}, {part_ws})
                  : check_ptrs({q, k, v, o, dO, delta_ws}, {lse}, {dq, dk, dv}, {});
    if (s != FA_OK) return s;
    hipError_t e = fa::launch_bwd_delta(dtype, d, o, dO, lse, delta_ws, B, Hq, N, stream);
    if (e == hipSuccess)
        e = fa::launch_bwd_bf16_bsparse_split(d, causal, q, k, v, dO, delta_ws, dq, dk, dv, B, Hq, Hkv, N, col_idx,
                                              row_idx, nnz, row_chunks, n_row_chunks, row_merges, n_row_merges,
                                              n_row_slots, col_chunks, n_col_chunks, col_merges, n_col_merges,
                                              n_col_slots, part_ws, softmax_scale, stream);
    return launch_status(e);
}

size_t fa_fwd_bsparse_split_workspace_bytes(int B, int Hq, int d, int n_row_slots) {
    if (B < 0 || Hq < 0 || (d != 64 && d != 128) || n_row_slots < 0) return 0;
    return (size_t)n_row_slots * B * Hq * FA_BSPARSE_BLOCK * (d + 1) * sizeof(float);
}

size_t fa_bwd_bsparse_split_workspace_bytes(int B, int Hq, int Hkv, int d, int n_row_slots, int n_col_slots) {
    if (B < 0 || Hq < 0 || Hkv < 0 || (d != 64 && d != 128) || n_row_slots < 0 || n_col_slots < 0) return 0;
    return ((size_t)n_row_slots * B * Hq + 2 * (size_t)n_col_slots * B * Hkv) * FA_BSPARSE_BLOCK * d * sizeof(float);
}

// Shape checks of the decode entry points; sets *empty for an empty problem.
static fa_status_t check_decode(int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                                bool* empty) {
    if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
    if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_UNSUPPORTED;
    *empty = (B == 0 || Hq == 0 || Nq == 0);
    if (*empty) return FA_OK;
    if (Hkv == 0 || Hq % Hkv != 0) return FA_ERR_SHAPE;
    // every query row must see at least one key
    if (Nk == 0 || (causal && Nq > Nk)) return FA_ERR_SHAPE;
    const fa::DecodePlan p = fa::decode_plan(B, Hq, Hkv, Nq, Nk, d, 1, fa::kCuBound);
    const int64_t units = (int64_t)B * Hkv * p.nrb * p.nsplit;
    const int64_t rows = (int64_t)B * Hq * Nq;
    if (units / 4 + 1 > INT32_MAX || rows / 4 + 1 > INT32_MAX) return FA_ERR_SHAPE;
    return FA_OK;
}

size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    bool empty = false;
    if (check_decode(B, Hq, Hkv, Nq, Nk, d, 0, 1.0f, &empty) != FA_OK || empty) return 0;
    return fa::decode_ws_bytes(fa::decode_plan(B, Hq, Hkv, Nq, Nk, d, 1, fa::device_cus()), B, Hq, Nq, d);
}

fa_status_t fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, float* ws, int B, int Hq,
                      int Hkv, int Nq, int Nk, int d, int causal, float softmax_scale, fa_dtype_t dtype,
                      hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_decode(B, Hq, Hkv, Nq, Nk, d, causal, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    s = check_ptrs({q, k, v}, {}, {o, ws}, {lse});
    if (s != FA_OK) return s;
    return launch_status(fa::launch_decode(d, causal, q, k, v, o, lse, ws, B, Hq, Hkv, Nq, Nk, softmax_scale,
                                           stream));
}

// Paged decode: the host checks the pool and table shapes; the sequence
// lengths and block ids live on the device and are clamped by the kernel.
static fa_status_t check_paged(int B, int Hq, int Hkv, int Nq, int maxb, int bs, int nblk, int d, int causal,
                               float scale, bool* empty) {
    if (maxb < 0 || bs < 0 || nblk < 0) return FA_ERR_SHAPE;
    if (bs == 0 || bs % 32 != 0) return FA_ERR_UNSUPPORTED;
    if ((int64_t)maxb * bs > INT32_MAX / 2) return FA_ERR_SHAPE;
    fa_status_t s = check_decode(B, Hq, Hkv, Nq, maxb * bs, d, 0, scale, empty);
    if (s != FA_OK || *empty) return s;
    if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
    if (nblk == 0) return FA_ERR_SHAPE;
    const int64_t units =
        (int64_t)fa::paged_chunks(B, Hq, Hkv, Nq, d, fa::kCuBound) * Hkv * ((Hq / Hkv * (int64_t)Nq + 31) / 32);
    if (units / 4 + 1 > INT32_MAX) return FA_ERR_SHAPE;
    return FA_OK;
}

size_t fa_decode_paged_workspace_bytes(int B, int Hq, int Hkv, int Nq, int max_blocks, int block_size, int d) {
    bool empty = false;
    if (check_paged(B, Hq, Hkv, Nq, max_blocks, block_size, 1, d, 0, 1.0f, &empty) != FA_OK || empty) return 0;
    return fa::paged_ws_bytes(B, Hq, Hkv, Nq, d);
}

fa_status_t fa_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                            const int* seq_lens, void* o, float* lse, float* ws, int B, int Hq, int Hkv, int Nq,
                            int max_blocks, int block_size, int num_blocks, int d, int causal, float softmax_scale,
                            fa_dtype_t dtype, hipStream_t stream) {
    bool empty = false;
    if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    fa_status_t s = check_paged(B, Hq, Hkv, Nq, max_blocks, block_size, num_blocks, d, causal, softmax_scale, &empty);
    if (s != FA_OK || empty) return s;
    s = check_ptrs({q, k_cache, v_cache}, {block_table, seq_lens}, {o, ws}, {lse});
    if (s != FA_OK) return s;
    return launch_status(fa::launch_decode_paged(d, causal, q, k_cache, v_cache, block_table, seq_lens, o, lse, ws,
                                                 B, Hq, Hkv, Nq, max_blocks, block_size, num_blocks, softmax_scale,
                                                 stream));
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int N) {
    if (B <= 0 || Hq <= 0 || N <= 0) return 0;
    return (size_t)8 * (size_t)B * (size_t)Hq * (size_t)fa::ws_rows(N);
}

fa_status_t fa_quantize_fp8(const void* x_bf16, size_t n, void* x_e4m3, float* descale, hipStream_t stream) {
    if (!descale || (n > 0 && (!x_bf16 || !x_e4m3))) return FA_ERR_NULL;
    if (!aligned(descale, 4) || (n > 0 && !aligned(x_bf16, 2))) return FA_ERR_ALIGN;
    if (n > 0 && ((const void*)x_e4m3 == x_bf16 || (const void*)descale == x_bf16 ||
                  (const void*)descale == (const void*)x_e4m3))
        return FA_ERR_ALIAS;
    return launch_status(fa::launch_quantize_fp8(x_bf16, n, x_e4m3, descale, stream));
}

const char* fa_status_string(fa_status_t s) {
    switch (s) {
        case FA_OK: return "ok";
        case FA_ERR_NULL: return "a required pointer is NULL";
        case FA_ERR_SHAPE: return "invalid shape (negative size, Hkv == 0 or Hq % Hkv != 0, or too large)";
        case FA_ERR_UNSUPPORTED: return "unsupported head dim, dtype, causal flag or softmax scale";
        case FA_ERR_ALIGN: return "pointer misaligned (tensors need 16 bytes, float arrays 4)";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        case FA_ERR_ALIAS: return "an output aliases an input";
        default: return "unknown status";
    }
}

int fa_abi_version(void) { return FA_ABI_VERSION; }

}  // extern "C"
