/*
 * fa.h -- exact, tiled, fused softmax attention on AMD MI355X (gfx950).
 *
 * The operation (all pages; "flash attention io aware", section "The Memory
 * Bandwidth Bottleneck", steps 1-3): for every batch b and query head h,
 *     S = scale * Q[b,h] K[b,g]^T        (N x N, never stored)
 *     causal: S[i,j] = -inf for j > i    ("Paper digest: FlashAttention",
 *                                        section "Limits", names causal masks)
 *     P = softmax(S) over keys,  O[b,h] = P V[b,g],
 *     LSE[b,h,i] = ln sum_j exp(S[i,j])  (natural log; the log-sum-exp of the
 *                                        FA-LLM glossary's third paragraph)
 * where g = h / (Hq / Hkv) is the key/value head of the query head's group
 * ("Flash Attention" self-hosted-LLM glossary, entry "Grouped-Query Attention":
 * query heads are split into contiguous groups sharing one K/V head).
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates, frees or synchronises, and enqueues all work on
 *    `stream` (NULL = the default stream).  Its only mutable global state is
 *    a per-device cache of values fixed by the device and the code object
 *    (CU count, resident workgroups per CU of each kernel), filled on a
 *    device's first call, and the workspace array of fa_bwd_noalloc; no
 *    argument or result of a call is kept.
 *  - Layouts are contiguous, row-major, head dimension fastest:
 *    Q, O, dO, dQ are [B, Hq, N, d]; K, V, dK, dV are [B, Hkv, N, d];
 *    LSE and the backward workspace are [B, Hq, N] float32.
 *  - Element types: FA_DTYPE_F32 = IEEE float32, FA_DTYPE_BF16 = bfloat16
 *    bits, FA_DTYPE_FP8_E4M3 = OCP E4M3 ("e4m3fn") codes.  O and the
 *    gradients take the input type, except that an FP8 forward writes bf16 O.
 *  - Supported: d in {64, 128}; Hkv >= 1 and Hq % Hkv == 0; causal in {0, 1};
 *    0 < softmax_scale < inf.  B == 0, Hq == 0 or N == 0 is an empty problem:
 *    FA_OK is returned and nothing is read or written.
 *  - Tensor base pointers must be 16-byte aligned, float pointers 4-byte.
 *    Outputs must not alias inputs.
 *  - Errors: every argument is validated on the host before any HIP call;
 *    a bad argument returns a nonzero fa_status_t and enqueues nothing.  A
 *    failed launch returns FA_ERR_LAUNCH.  Device faults surface at the
 *    caller's next synchronisation of `stream`.
 *  - No atomics in attention: results are bitwise reproducible run to run.
 *  - Graph capture: a call enqueues kernel launches only (no memset, copy,
 *    allocation or wait), so it can be recorded into a HIP graph by stream
 *    capture and replayed; a replay reads the buffers' contents at replay
 *    time.  The first call on a device should run outside a capture, so that
 *    the per-device cache above is filled by then.
 *  - Calls on different streams are independent and thread-safe.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum {
    FA_DTYPE_F32 = 0,
    FA_DTYPE_BF16 = 1,
    FA_DTYPE_FP8_E4M3 = 2
} fa_dtype_t;

typedef int fa_status_t;
enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,          /* a required pointer is NULL                  */
    FA_ERR_SHAPE = 2,         /* negative size, Hkv == 0, Hq % Hkv != 0, ... */
    FA_ERR_UNSUPPORTED = 3,   /* d, dtype, causal flag or scale not supported */
    FA_ERR_ALIGN = 4,         /* pointer misaligned                          */
    FA_ERR_LAUNCH = 5,        /* the HIP launch failed                       */
    FA_ERR_ALIAS = 6          /* an output aliases an input                  */
};

#define FA_ABI_VERSION 2

/*
 * Forward pass.  "flash attention io aware", section "Flash Attention
 * Algorithm" (tiles of Q, K, V in on-chip memory; online softmax; write only
 * O) and section "Online Softmax"; "FlashAttention" legal-glossary paragraph
 * on FlashAttention-2 (parallel over the sequence).
 *   q, k, v     : inputs, dtype `dtype` (FP8: E4M3 codes from fa_quantize_fp8)
 *   o           : output [B,Hq,N,d]; dtype `dtype` (bf16 when dtype is FP8)
 *   lse         : output [B,Hq,N] float32, natural-log log-sum-exp of the
 *                 scaled scores of each query row
 *   descale_qkv : FP8 only, device float[3] = (s_Q, s_K, s_V) with real value
 *                 = code value * s_X; must be NULL for other dtypes
 * Returns FA_OK once the kernel is enqueued.
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v,
                   void* o, float* lse,
                   int B, int Hq, int Hkv, int N, int d,
                   int causal, float softmax_scale,
                   fa_dtype_t dtype, const float* descale_qkv,
                   hipStream_t stream);

/*
 * Backward pass by recomputation: "FlashAttention" legal glossary, backward
 * paragraph and entry "Recomputation" (only the softmax statistics are kept;
 * S and P are recomputed on chip); FlashAttention-2 paragraph (the backward
 * is parallel over the key (column) blocks, without atomic adds).
 * Three kernels run in order on `stream`: D = rowsum(dO * O) and LSE*log2(e)
 * into `delta_ws`, then dK/dV (one workgroup per key block and K/V head,
 * looping over the query heads of its group) and dQ (one workgroup per query
 * block and query head).
 *   q, k, v, o, dO, lse : as produced/consumed by fa_fwd (same dtype, F32 or
 *                         BF16 only)
 *   dq [B,Hq,N,d], dk, dv [B,Hkv,N,d] : outputs, overwritten (not accumulated)
 *   delta_ws : caller-owned device workspace of fa_bwd_workspace_bytes() bytes,
 *              16-byte aligned; see fa_bwd_workspace_bytes for its contents
 */
fa_status_t fa_bwd(const void* q, const void* k, const void* v,
                   const void* o, const void* dO, const float* lse,
                   void* dq, void* dk, void* dv,
                   float* delta_ws,
                   int B, int Hq, int Hkv, int N, int d,
                   int causal, float softmax_scale, fa_dtype_t dtype,
                   hipStream_t stream);

/*
 * The three stages of fa_bwd as separate calls, for callers that schedule or
 * time them one by one; fa_bwd is exactly these three in order.  Same
 * validation, dtypes and tensor layouts as fa_bwd.
 *   fa_bwd_delta : fills the workspace `ws` from O, dO and LSE: the negated
 *                  row term of the softmax gradient, -D[b,h,i] with
 *                  D[b,h,i] = sum_c dO[b,h,i,c] O[b,h,i,c] (which equals
 *                  sum_j P_ij dP_ij), and LSE[b,h,i] * log2(e)
 *   fa_bwd_dkdv  : dK, dV from the workspace, parallel over key blocks
 *                  ("FlashAttention" legal glossary, FlashAttention-2
 *                  paragraph: column-parallel backward without atomic adds);
 *                  a workgroup owns one key block of one K/V head and sums
 *                  over its group's query heads
 *   fa_bwd_dq    : dQ from the workspace, parallel over query blocks
 * fa_bwd_dkdv and fa_bwd_dq only read `ws` and do not depend on each other.
 */
fa_status_t fa_bwd_delta(const void* o, const void* dO, const float* lse, float* ws,
                         int B, int Hq, int N, int d, fa_dtype_t dtype,
                         hipStream_t stream);

fa_status_t fa_bwd_dkdv(const void* q, const void* k, const void* v,
                        const void* dO, const float* ws,
                        void* dk, void* dv,
                        int B, int Hq, int Hkv, int N, int d,
                        int causal, float softmax_scale, fa_dtype_t dtype,
                        hipStream_t stream);

fa_status_t fa_bwd_dq(const void* q, const void* k, const void* v,
                      const void* dO, const float* ws,
                      void* dq,
                      int B, int Hq, int Hkv, int N, int d,
                      int causal, float softmax_scale, fa_dtype_t dtype,
                      hipStream_t stream);

/*
 * fa_bwd without a caller workspace, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, validation, kernels and results as
 * fa_bwd, minus `delta_ws`: the workspace lives in a library-owned device
 * array of FA_BWD_NOALLOC_MAX_BYTES (one copy on each device the library runs
 * on, held until the process ends).  No call allocates or frees anything.
 *  - fa_bwd_workspace_bytes(B, Hq, N) must be <= FA_BWD_NOALLOC_MAX_BYTES
 *    (B * Hq * Np <= 2^21 rows), else FA_ERR_SHAPE before any HIP call.
 *  - Every call on one device shares that device's array, and each call
 *    rewrites every byte it reads: calls that overlap on one device (other
 *    streams, other threads) race and must be serialised by the caller.
 *  - The array's device address is looked up on the first call on each
 *    device; if that fails the call returns FA_ERR_LAUNCH.
 */
#define FA_BWD_NOALLOC_MAX_BYTES (16u << 20)

fa_status_t fa_bwd_noalloc(const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           void* dq, void* dk, void* dv,
                           int B, int Hq, int Hkv, int N, int d,
                           int causal, float softmax_scale, fa_dtype_t dtype,
                           hipStream_t stream);

/*
 * Bytes of the backward workspace: 8 * B * Hq * Np with Np = N rounded up to
 * a multiple of 64 (0 for an empty problem).  Layout: float32 -D[B*Hq][Np]
 * followed by float32 LSE*log2(e)[B*Hq][Np]; rows i >= N hold 0 and
 * +infinity, so padded query rows carry zero probability.
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int N);

/*
 * FP8 backward: dQ, dK, dV of the FP8 forward (fa_fwd with FA_DTYPE_FP8_E4M3).
 * The FlashAttention legal glossary (FlashAttention-3 paragraph) and "flash
 * attention io aware" (section "Flash Attention 2 and 3") name FP8 attention
 * without a recipe; this one carries the forward's through the recomputation
 * of the glossary's backward paragraph.  S = Q K^T and dP = dO V^T run on the
 * fp8 matrix cores; dQ = scale dS K too, dS rounded to E4M3 after a power-of-
 * two scale per query and block of 32 keys that the matrix core divides back
 * out; dK = scale dS^T Q and dV = P^T dO run on the bf16 matrix cores (P, dS
 * rounded to bf16, the E4M3 codes of Q and dO widened exactly).  float32
 * accumulation; D = rowsum(dO o O).
 *   q8, k8, v8, do8 : E4M3 codes, [B,Hq,N,d], [B,Hkv,N,d], [B,Hkv,N,d],
 *                     [B,Hq,N,d] (fa_quantize_fp8 of the bf16 tensors)
 *   o, lse          : the FP8 forward's outputs (o bf16)
 *   descale         : device float[4] = (s_Q, s_K, s_V, s_dO)
 *   dq, dk, dv      : bf16 outputs, [B,Hq,N,d], [B,Hkv,N,d] x 2
 *   delta_ws        : as fa_bwd (fa_bwd_workspace_bytes bytes); it holds
 *                     -D / (s_dO s_V) and LSE * log2(e)
 * d must be 128 (else FA_ERR_UNSUPPORTED); other checks as fa_bwd.
 */
fa_status_t fa_bwd_fp8(const void* q8, const void* k8, const void* v8,
                       const void* o, const void* do8, const float* lse,
                       const float* descale,
                       void* dq, void* dk, void* dv,
                       float* delta_ws,
                       int B, int Hq, int Hkv, int N, int d,
                       int causal, float softmax_scale,
                       hipStream_t stream);

/*
 * Per-tensor FP8 quantisation for the FP8 forward ("FlashAttention" legal
 * glossary, FlashAttention-3 paragraph, and "flash attention io aware",
 * section "Flash Attention 2 and 3", name FP8 attention but give no recipe;
 * this is the plainest one): s = max(absmax(x), 2^-120) / 448 in float32 and
 * code_i = E4M3 round-to-nearest-even, saturating at +-448, of x_i / s.
 *   x_bf16  : n bf16 values (device)        x_e4m3 : n output codes (device)
 *   descale : device float[1] receiving s (it is also used as the absmax
 *             scratch while the call runs)
 * Four small kernels are enqueued; n == 0 writes s = 2^-120 / 448.
 */
fa_status_t fa_quantize_fp8(const void* x_bf16, size_t n, void* x_e4m3,
                            float* descale, hipStream_t stream);

/*
 * Causal sliding-window (local) attention with global tokens: key j is
 * visible to query i iff j <= i and (i - window < j or j < sink).  The
 * FlashAttention legal glossary, entry "Block-sparse": a sparsity mask picks
 * the blocks of the attention matrix worth computing, sliding-window (local)
 * attention and global tokens being common patterns, and whole tiles outside
 * it are skipped.  Same arguments, layouts and outputs as fa_fwd / fa_bwd with
 * causal = 1, plus `window` (>= 1) and `sink` (>= 0, the number of leading
 * tokens every later query sees; 0 for none).  A window or sink of N or more
 * is plain causal attention.  bf16 only.  The backward reads the LSE of
 * fa_fwd_local with the same window and sink.
 */
fa_status_t fa_fwd_local(const void* q, const void* k, const void* v,
                         void* o, float* lse,
                         int B, int Hq, int Hkv, int N, int d,
                         int window, int sink, float softmax_scale, fa_dtype_t dtype,
                         hipStream_t stream);

fa_status_t fa_bwd_local(const void* q, const void* k, const void* v,
                         const void* o, const void* dO, const float* lse,
                         void* dq, void* dk, void* dv,
                         float* delta_ws,
                         int B, int Hq, int Hkv, int N, int d,
                         int window, int sink, float softmax_scale, fa_dtype_t dtype,
                         hipStream_t stream);

/*
 * Forward with attention dropout on the normalised probabilities: the
 * FlashAttention page of the self-hosted LLM glossary (opening paragraphs:
 * matrix products, masking, softmax and dropout fused in one kernel) and the
 * FlashAttention digest, section "Limits" (dropout among the features a
 * kernel must handle).  The pages fix no generator; this library uses
 * Philox4x32-10 (Salmon et al., SC 2011), one call per 4 x 4 block of the
 * score matrix and one byte per element: element (query i, key j) of batch
 * entry b and query head h takes byte j % 4 of word i % 4 of
 * Philox((j / 4, i / 4, b * Hq + h, 0), (seed % 2^32, seed / 2^32)) (byte e =
 * bits 8e .. 8e+7) and is kept iff that byte is >= t = floor(256 dropout_p).
 * The drop probability is therefore p' = t / 256, dropout_p rounded down to a
 * multiple of 1/256 (no dropout below 1/256), and O = ((Z o P) / (1 - p')) V.
 * LSE is that of the undropped softmax.  Same arguments, layouts and errors
 * as fa_fwd (bf16 only) plus dropout_p in [0, 1) (else FA_ERR_UNSUPPORTED)
 * and the 64-bit seed.
 */
fa_status_t fa_fwd_dropout(const void* q, const void* k, const void* v,
                           void* o, float* lse,
                           int B, int Hq, int Hkv, int N, int d, int causal,
                           double dropout_p, uint64_t seed,
                           float softmax_scale, fa_dtype_t dtype, hipStream_t stream);

/*
 * Backward through the dropout of fa_fwd_dropout (same pages).  The keep mask
 * Z is regenerated from (dropout_p, seed), never stored.  With r = 1/(1 - p')
 * (p' as in fa_fwd_dropout) and P the undropped softmax: dV = r (Z o P)^T dO, dP = r Z o (dO V^T),
 * D = rowsum(dO o O) (= rowsum(P o dP), O the dropped output), dS = P o (dP - D),
 * dQ = scale dS K, dK = scale dS^T Q, K/V gradients summed over each group.
 * Same arguments, layouts, workspace and errors as fa_bwd (bf16 only) plus the
 * dropout_p and seed given to fa_fwd_dropout; o and lse are its outputs.  The
 * workspace holds -D (1 - p') instead of -D.
 */
fa_status_t fa_bwd_dropout(const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           void* dq, void* dk, void* dv,
                           float* delta_ws,
                           int B, int Hq, int Hkv, int N, int d, int causal,
                           double dropout_p, uint64_t seed,
                           float softmax_scale, fa_dtype_t dtype, hipStream_t stream);

/*
 * Block-sparse attention: key j is visible to query i iff block
 * (i / FA_BSPARSE_BLOCK, j / FA_BSPARSE_BLOCK) of the mask is on (and, with
 * causal = 1, j <= i).  The FlashAttention legal glossary, entry
 * "Block-sparse": a mask over the blocks of the attention matrix says which
 * blocks are computed; the blocks that are off are skipped whole.  Same
 * arguments, layouts and outputs as fa_fwd / fa_bwd plus the mask, one
 * pattern for every batch entry and head, in device memory (the library
 * neither copies nor frees it):
 *   nb      = ceil(N / FA_BSPARSE_BLOCK) blocks per side
 *   row_ptr : int[nb + 1], col_idx : int[nnz] — the blocks that are on, by
 *             rows: row block r sees the key blocks col_idx[row_ptr[r] ..
 *             row_ptr[r+1]), strictly ascending (compressed sparse rows)
 *   col_ptr : int[nb + 1], row_idx : int[nnz] — the same mask by columns
 *             (the backward's dK / dV pass reads it that way)
 * A query row that sees no key gets O = 0 and LSE = -inf, and contributes
 * nothing to the gradients; a key seen by no row gets dK = dV = 0.  With
 * causal = 1, blocks above the diagonal may be listed (their keys are masked)
 * but cost time.  The kernels clamp every offset and block index to the
 * arrays, so a malformed layout reads nothing out of bounds, but its results
 * are unspecified.  bf16 only, d in {64, 128}.  Errors: FA_ERR_SHAPE for
 * nnz < 0 or nnz > nb * nb, FA_ERR_NULL for a null row_ptr / col_ptr or a
 * null index array with nnz > 0, FA_ERR_ALIGN for a misaligned mask array,
 * others as fa_fwd / fa_bwd.  The backward reads
 * the LSE of fa_fwd_bsparse with the same mask.
 */
#define FA_BSPARSE_BLOCK 256

fa_status_t fa_fwd_bsparse(const void* q, const void* k, const void* v,
                           void* o, float* lse,
                           int B, int Hq, int Hkv, int N, int d, int causal,
                           const int* row_ptr, const int* col_idx, int nnz,
                           float softmax_scale, fa_dtype_t dtype, hipStream_t stream);

fa_status_t fa_bwd_bsparse(const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           void* dq, void* dk, void* dv,
                           float* delta_ws,
                           int B, int Hq, int Hkv, int N, int d, int causal,
                           const int* row_ptr, const int* col_idx,
                           const int* col_ptr, const int* row_idx, int nnz,
                           float softmax_scale, fa_dtype_t dtype, hipStream_t stream);

/*
 * Block-sparse attention with a work split, for masks whose block rows or
 * columns differ widely in length (a global block row or column sees every
 * block): the same results as fa_fwd_bsparse / fa_bwd_bsparse up to float32
 * summation order (same pages; the split is the split-KV rescale of the
 * "Online Softmax" section of "flash attention io aware" applied to key
 * chunks).  A work item is a run of consecutive entries of one block row (for
 * the forward and dQ) or one block column (for dK/dV); a long row or column
 * is cut into several items, run in parallel, that write float32 partials,
 * and a merge pass combines them: the log-sum-exp merge for O and LSE, sums
 * for dQ, dK and dV.  Tables (device int32, 16-byte aligned, four ints per
 * entry; the library neither copies nor frees them):
 *   row_chunks[4c..4c+3] = (r, e0, e1, slot): entries e0 .. e1-1 of the
 *       compressed rows (col_idx) of row block r; slot = -1 when the item is
 *       all of row r, else the partial slot it writes (0 <= slot < n_row_slots).
 *       Every row block needs at least one item (an empty row: e0 = e1).
 *   row_merges[4m..4m+3] = (r, s0, ns, 0): row block r is the merge of slots
 *       s0 .. s0+ns-1 (its split items).
 *   col_chunks, col_merges: the same over the compressed columns (row_idx)
 *       and the key blocks, with n_col_slots slots.
 * 1 <= n_*_chunks <= nb + nnz, 0 <= n_*_merges <= nb, 0 <= n_*_slots <= nnz.
 * part_ws (float, 16-byte aligned; NULL allowed when no slot is used) holds
 * the partials: fa_fwd_bsparse_split_workspace_bytes() and
 * fa_bwd_bsparse_split_workspace_bytes() bytes.  Table entries are clamped on
 * the device, so malformed tables read and write nothing out of bounds, but
 * then the results are unspecified.  Other arguments, layouts and errors as
 * fa_fwd_bsparse / fa_bwd_bsparse (row_ptr and col_ptr are not needed: the
 * items carry their ranges); delta_ws as fa_bwd.
 */
fa_status_t fa_fwd_bsparse_split(const void* q, const void* k, const void* v,
                                 void* o, float* lse,
                                 int B, int Hq, int Hkv, int N, int d, int causal,
                                 const int* col_idx, int nnz,
                                 const int* row_chunks, int n_row_chunks,
                                 const int* row_merges, int n_row_merges, int n_row_slots,
                                 float* part_ws,
                                 float softmax_scale, fa_dtype_t dtype, hipStream_t stream);

fa_status_t fa_bwd_bsparse_split(const void* q, const void* k, const void* v,
                                 const void* o, const void* dO, const float* lse,
                                 void* dq, void* dk, void* dv,
                                 float* delta_ws,
                                 int B, int Hq, int Hkv, int N, int d, int causal,
                                 const int* col_idx, const int* row_idx, int nnz,
                                 const int* row_chunks, int n_row_chunks,
                                 const int* row_merges, int n_row_merges, int n_row_slots,
                                 const int* col_chunks, int n_col_chunks,
                                 const int* col_merges, int n_col_merges, int n_col_slots,
                                 float* part_ws,
                                 float softmax_scale, fa_dtype_t dtype, hipStream_t stream);

/* Bytes of part_ws: n_row_slots * B * Hq * 256 * (d + 1) * 4 for the forward;
 * (n_row_slots * B * Hq + 2 * n_col_slots * B * Hkv) * 256 * d * 4 for the
 * backward (0 for invalid arguments). */
size_t fa_fwd_bsparse_split_workspace_bytes(int B, int Hq, int d, int n_row_slots);
size_t fa_bwd_bsparse_split_workspace_bytes(int B, int Hq, int Hkv, int d, int n_row_slots, int n_col_slots);

/*
 * Decode: attention of Nq new query rows against a key/value cache of Nk
 * rows.  "Paper digest: FlashAttention", section "Limits" (decode-time
 * attention reads a large KV cache for few queries); self-hosted LLM
 * glossary, entries "KV Cache" (the keys and values of all earlier tokens,
 * read for every new token) and "Grouped-Query Attention".  Exact softmax
 * attention as in fa_fwd; with causal = 1 the new rows are the last Nq
 * positions: row i sees cache keys j <= Nk - Nq + i (so Nq <= Nk is
 * required); with causal = 0 every row sees all Nk keys.
 *   q    : [B,Hq,Nq,d] bf16        k, v : [B,Hkv,Nk,d] bf16 (the cache)
 *   o    : output [B,Hq,Nq,d] bf16
 *   lse  : output [B,Hq,Nq] float32, natural-log log-sum-exp of the scaled
 *          scores of each row
 *   ws   : caller-owned device workspace of fa_decode_workspace_bytes()
 *          bytes, 16-byte aligned (per-chunk partial results; overwritten)
 * Two kernels are enqueued: a split over key chunks (one wave per batch, K/V
 * head, block of 32 packed query rows and chunk) and a merge of the chunks.
 * dtype must be FA_DTYPE_BF16, d 64 or 128.  Nk == 0, or causal with
 * Nq > Nk, returns FA_ERR_SHAPE (a row with no visible key); B, Hq or Nq == 0
 * returns FA_OK and touches nothing.
 */
fa_status_t fa_decode(const void* q, const void* k, const void* v,
                      void* o, float* lse, float* ws,
                      int B, int Hq, int Hkv, int Nq, int Nk, int d,
                      int causal, float softmax_scale, fa_dtype_t dtype,
                      hipStream_t stream);

/*
 * Bytes of the decode workspace for these sizes (0 for an empty or invalid
 * problem): 4 * B * Hq * Nq * nsplit * (d + 1), nsplit being the number of
 * key chunks the library chooses for the shape.
 */
size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d);

/*
 * Decode against a paged KV cache with per-sequence lengths.  Self-hosted LLM
 * glossary, entry "PagedAttention" (the KV cache split into fixed-size,
 * non-contiguous blocks, like pages of virtual memory); "Paper digest:
 * FlashAttention", section "Limits" (decode-time attention over batch-varying
 * lengths).  Same attention as fa_decode, per sequence b of seq_lens[b] keys.
 *   k_cache, v_cache : the block pool, [num_blocks, Hkv, block_size, d] bf16
 *   block_table      : device int32 [B, max_blocks]; key j of sequence b is
 *                      row j % block_size of block block_table[b][j / block_size]
 *   seq_lens         : device int32 [B]
 *   q, o, lse        : as fa_decode ([B,Hq,Nq,d], [B,Hq,Nq,d], [B,Hq,Nq])
 *   ws               : fa_decode_paged_workspace_bytes() bytes, 16-byte aligned
 * block_size must be a positive multiple of 32.  The lengths and block ids are
 * read on the device: lengths are clamped to [0, max_blocks * block_size] and
 * block ids to [0, num_blocks), so a bad table reads wrong rows but never
 * outside the pool.  A row that sees no key (an empty sequence, or with
 * causal = 1 a row i with seq_lens[b] - Nq + i < 0) gets O = 0 and
 * LSE = -infinity.
 */
fa_status_t fa_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                            const int* block_table, const int* seq_lens,
                            void* o, float* lse, float* ws,
                            int B, int Hq, int Hkv, int Nq,
                            int max_blocks, int block_size, int num_blocks, int d,
                            int causal, float softmax_scale, fa_dtype_t dtype,
                            hipStream_t stream);

/* Bytes of the paged decode workspace (0 for an empty or invalid problem). */
size_t fa_decode_paged_workspace_bytes(int B, int Hq, int Hkv, int Nq,
                                       int max_blocks, int block_size, int d);

/* Static text for a status code ("unknown status" for other values). */
const char* fa_status_string(fa_status_t s);

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
