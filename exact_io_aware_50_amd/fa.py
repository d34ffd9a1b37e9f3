"""Python binding of libfa.so (the C ABI in include/fa.h).

Argument marshalling only: every step of attention runs in the HIP kernels
behind the C entry points.  The raw entry points keep their C names
(``fa_fwd``, ``fa_bwd``, ...) and take integer device addresses; the tensor
helpers ``fwd``, ``bwd`` and ``quantize_fp8`` allocate outputs with torch and
pass its current HIP stream.

Importing this module fails loudly if the library has not been built
(``python -m exact_io_aware_50_amd.build``); there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m exact_io_aware_50_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

FA_DTYPE_F32, FA_DTYPE_BF16, FA_DTYPE_FP8_E4M3 = 0, 1, 2
FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_LAUNCH, FA_ERR_ALIAS = range(7)

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float

_lib.fa_fwd.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p, _p]
_lib.fa_fwd.restype = _i
_lib.fa_bwd.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p]
_lib.fa_bwd.restype = _i
_lib.fa_bwd_noalloc.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p]
_lib.fa_bwd_noalloc.restype = _i
_lib.fa_bwd_delta.argtypes = [_p, _p, _p, _p, _i, _i, _i, _i, _i, _p]
_lib.fa_bwd_delta.restype = _i
_lib.fa_bwd_dkdv.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p]
_lib.fa_bwd_dkdv.restype = _i
_lib.fa_bwd_dq.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p]
_lib.fa_bwd_dq.restype = _i
_lib.fa_bwd_workspace_bytes.argtypes = [_i, _i, _i]
_lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
_lib.fa_quantize_fp8.argtypes = [_p, ctypes.c_size_t, _p, _p, _p]
_lib.fa_quantize_fp8.restype = _i
_lib.fa_fwd_local.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i, _p]
_lib.fa_fwd_local.restype = _i
_lib.fa_bwd_local.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i, _p]
_lib.fa_bwd_local.restype = _i
_d = ctypes.c_double
_lib.fa_fwd_dropout.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _d, ctypes.c_uint64, _f, _i, _p]
_lib.fa_fwd_dropout.restype = _i
_lib.fa_bwd_dropout.argtypes = [_p] * 10 + [_i] * 6 + [_d, ctypes.c_uint64, _f, _i, _p]
_lib.fa_bwd_dropout.restype = _i
_lib.fa_bwd_fp8.argtypes = [_p] * 11 + [_i] * 6 + [_f, _p]
_lib.fa_bwd_fp8.restype = _i
_lib.fa_fwd_bsparse.argtypes = [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _i, _f, _i, _p]
_lib.fa_fwd_bsparse.restype = _i
_lib.fa_bwd_bsparse.argtypes = ([_p] * 10 + [_i] * 6 + [_p] * 4 + [_i, _f, _i, _p])
_lib.fa_bwd_bsparse.restype = _i
_lib.fa_fwd_bsparse_split.argtypes = [_p] * 5 + [_i] * 6 + [_p, _i, _p, _i, _p, _i, _i, _p, _f, _i, _p]
_lib.fa_fwd_bsparse_split.restype = _i
_lib.fa_bwd_bsparse_split.argtypes = ([_p] * 10 + [_i] * 6 + [_p, _p, _i] + [_p, _i, _p, _i, _i] * 2 +
                                      [_p, _f, _i, _p])
_lib.fa_bwd_bsparse_split.restype = _i
_lib.fa_fwd_bsparse_split_workspace_bytes.argtypes = [_i] * 4
_lib.fa_fwd_bsparse_split_workspace_bytes.restype = ctypes.c_size_t
_lib.fa_bwd_bsparse_split_workspace_bytes.argtypes = [_i] * 6
_lib.fa_bwd_bsparse_split_workspace_bytes.restype = ctypes.c_size_t
_lib.fa_decode.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _i, _p]
_lib.fa_decode.restype = _i
_lib.fa_decode_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
_lib.fa_decode_workspace_bytes.restype = ctypes.c_size_t
_lib.fa_decode_paged.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p] + [_i] * 9 + [_f, _i, _p]
_lib.fa_decode_paged.restype = _i
_lib.fa_decode_paged_workspace_bytes.argtypes = [_i] * 7
_lib.fa_decode_paged_workspace_bytes.restype = ctypes.c_size_t
_lib.fa_status_string.argtypes = [_i]
_lib.fa_status_string.restype = ctypes.c_char_p
_lib.fa_abi_version.argtypes = []
_lib.fa_abi_version.restype = _i

EXPORTS = ("fa_fwd", "fa_bwd", "fa_bwd_noalloc", "fa_bwd_delta", "fa_bwd_dkdv", "fa_bwd_dq",
           "fa_bwd_workspace_bytes",
           "fa_quantize_fp8", "fa_fwd_local", "fa_bwd_local", "fa_fwd_bsparse", "fa_bwd_bsparse",
           "fa_fwd_bsparse_split", "fa_bwd_bsparse_split", "fa_fwd_bsparse_split_workspace_bytes",
           "fa_bwd_bsparse_split_workspace_bytes", "fa_fwd_dropout", "fa_bwd_dropout", "fa_bwd_fp8", "fa_decode",
           "fa_decode_workspace_bytes", "fa_decode_paged", "fa_decode_paged_workspace_bytes",
           "fa_status_string", "fa_abi_version")


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({fa_status_string(status)})")
        self.status = status


# ------------------------------------------------------------------ raw C entry points

def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, softmax_scale, dtype, descale_qkv, stream) -> int:
    return _lib.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, int(causal), float(softmax_scale), dtype,
                       descale_qkv, stream)


def fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, delta_ws, B, Hq, Hkv, N, d, causal, softmax_scale, dtype,
           stream) -> int:
    return _lib.fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, delta_ws, B, Hq, Hkv, N, d, int(causal),
                       float(softmax_scale), dtype, stream)


def fa_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, N, d, causal, softmax_scale, dtype, stream) -> int:
    return _lib.fa_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, B, Hq, Hkv, N, d, int(causal), float(softmax_scale),
                               dtype, stream)


# bytes of the library-owned workspace behind fa_bwd_noalloc (FA_BWD_NOALLOC_MAX_BYTES)
BWD_NOALLOC_MAX_BYTES = 16 << 20


def fa_bwd_delta(o, dO, lse, ws, B, Hq, N, d, dtype, stream) -> int:
    return _lib.fa_bwd_delta(o, dO, lse, ws, B, Hq, N, d, dtype, stream)


def fa_bwd_dkdv(q, k, v, dO, ws, dk, dv, B, Hq, Hkv, N, d, causal, softmax_scale, dtype, stream) -> int:
    return _lib.fa_bwd_dkdv(q, k, v, dO, ws, dk, dv, B, Hq, Hkv, N, d, int(causal), float(softmax_scale),
                            dtype, stream)


def fa_bwd_dq(q, k, v, dO, ws, dq, B, Hq, Hkv, N, d, causal, softmax_scale, dtype, stream) -> int:
    return _lib.fa_bwd_dq(q, k, v, dO, ws, dq, B, Hq, Hkv, N, d, int(causal), float(softmax_scale),
                          dtype, stream)


def fa_bwd_workspace_bytes(B, Hq, N) -> int:
    return int(_lib.fa_bwd_workspace_bytes(B, Hq, N))


def fa_quantize_fp8(x_bf16, n, x_e4m3, descale, stream) -> int:
    return _lib.fa_quantize_fp8(x_bf16, n, x_e4m3, descale, stream)


def fa_fwd_local(q, k, v, o, lse, B, Hq, Hkv, N, d, window, sink, softmax_scale, dtype, stream) -> int:
    return _lib.fa_fwd_local(q, k, v, o, lse, B, Hq, Hkv, N, d, window, sink, float(softmax_scale), dtype, stream)


def fa_bwd_local(q, k, v, o, dO, lse, dq, dk, dv, delta_ws, B, Hq, Hkv, N, d, window, sink, softmax_scale, dtype,
                 stream) -> int:
    return _lib.fa_bwd_local(q, k, v, o, dO, lse, dq, dk, dv, delta_ws, B, Hq, Hkv, N, d, window, sink,
                             float(softmax_scale), dtype, stream)


def fa_decode(q, k, v, o, lse, ws, B, Hq, Hkv, Nq, Nk, d, causal, softmax_scale, dtype, stream) -> int:
    return _lib.fa_decode(q, k, v, o, lse, ws, B, Hq, Hkv, Nq, Nk, d, int(causal), float(softmax_scale), dtype,
                          stream)


def fa_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, d) -> int:
    return int(_lib.fa_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, d))


def fa_decode_paged(q, k_cache, v_cache, block_table, seq_lens, o, lse, ws, B, Hq, Hkv, Nq, max_blocks, block_size,
                    num_blocks, d, causal, softmax_scale, dtype, stream) -> int:
    return _lib.fa_decode_paged(q, k_cache, v_cache, block_table, seq_lens, o, lse, ws, B, Hq, Hkv, Nq, max_blocks,
                                block_size, num_blocks, d, int(causal), float(softmax_scale), dtype, stream)


def fa_decode_paged_workspace_bytes(B, Hq, Hkv, Nq, max_blocks, block_size, d) -> int:
    return int(_lib.fa_decode_paged_workspace_bytes(B, Hq, Hkv, Nq, max_blocks, block_size, d))


def fa_status_string(status: int) -> str:
    return _lib.fa_status_string(status).decode()


def fa_abi_version() -> int:
    return int(_lib.fa_abi_version())


# ------------------------------------------------------------------ torch tensor helpers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.uint8:
        return FA_DTYPE_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_handle(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(status: int, where: str):
    if status != FA_OK:
        raise FAError(status, where)


def _shape(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    for t in (q, k):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")
    B, Hq, N, d = q.shape
    return B, Hq, k.shape[1], N, d


def fwd(q, k, v, causal: bool, scale: float, descale=None, stream=None):
    """(o, lse) for q [B,Hq,N,d], k, v [B,Hkv,N,d] (fp32, bf16, or E4M3 codes as uint8 + descale[3])."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shape(q, k)
    if v.shape != k.shape or not v.is_contiguous() or q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("v must match k in shape and all of q, k, v in dtype")
    code = _dtype_code(q)
    odt = torch.bfloat16 if code == FA_DTYPE_FP8_E4M3 else q.dtype
    o = torch.empty((B, Hq, N, d), dtype=odt, device=q.device)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    dptr = None if descale is None else descale.data_ptr()
    _check(fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d,
                  causal, scale, code, dptr, _stream_handle(stream)), "fa_fwd")
    return o, lse


def bwd(q, k, v, o, do, lse, causal: bool, scale: float, stream=None, workspace=None):
    """(dq, dk, dv, workspace) for the forward's inputs and outputs and the output gradient do.

    The workspace (float32) holds D = rowsum(dO * O) for [B*Hq][Np] rows, then
    LSE*log2(e) for the same rows; Np = N rounded up to 64."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shape(q, k)
    code = _dtype_code(q)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if workspace is None:
        workspace = torch.empty(fa_bwd_workspace_bytes(B, Hq, N) // 4, dtype=torch.float32, device=q.device)
    _check(fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                  dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), B, Hq, Hkv, N, d, causal,
                  scale, code, _stream_handle(stream)), "fa_bwd")
    return dq, dk, dv, workspace


def fa_fwd_bsparse(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, row_ptr, col_idx, nnz, softmax_scale, dtype,
                   stream) -> int:
    return _lib.fa_fwd_bsparse(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, row_ptr, col_idx, nnz,
                               float(softmax_scale), dtype, stream)


def fa_bwd_bsparse(q, k, v, o, dO, lse, dq, dk, dv, delta_ws, B, Hq, Hkv, N, d, causal, row_ptr, col_idx, col_ptr,
                   row_idx, nnz, softmax_scale, dtype, stream) -> int:
    return _lib.fa_bwd_bsparse(q, k, v, o, dO, lse, dq, dk, dv, delta_ws, B, Hq, Hkv, N, d, causal, row_ptr,
                               col_idx, col_ptr, row_idx, nnz, float(softmax_scale), dtype, stream)


def fa_fwd_bsparse_split(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, col_idx, nnz, row_chunks, n_row_chunks,
                         row_merges, n_row_merges, n_row_slots, part_ws, softmax_scale, dtype, stream) -> int:
    return _lib.fa_fwd_bsparse_split(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, col_idx, nnz, row_chunks,
                                     n_row_chunks, row_merges, n_row_merges, n_row_slots, part_ws,
                                     float(softmax_scale), dtype, stream)


def fa_bwd_bsparse_split(q, k, v, o, dO, lse, dq, dk, dv, delta_ws, B, Hq, Hkv, N, d, causal, col_idx, row_idx, nnz,
                         row_chunks, n_row_chunks, row_merges, n_row_merges, n_row_slots, col_chunks, n_col_chunks,
                         col_merges, n_col_merges, n_col_slots, part_ws, softmax_scale, dtype, stream) -> int:
    return _lib.fa_bwd_bsparse_split(q, k, v, o, dO, lse, dq, dk, dv, delta_ws, B, Hq, Hkv, N, d, causal, col_idx,
                                     row_idx, nnz, row_chunks, n_row_chunks, row_merges, n_row_merges, n_row_slots,
                                     col_chunks, n_col_chunks, col_merges, n_col_merges, n_col_slots, part_ws,
                                     float(softmax_scale), dtype, stream)


def fa_fwd_bsparse_split_workspace_bytes(B, Hq, d, n_row_slots) -> int:
    return _lib.fa_fwd_bsparse_split_workspace_bytes(B, Hq, d, n_row_slots)


def fa_bwd_bsparse_split_workspace_bytes(B, Hq, Hkv, d, n_row_slots, n_col_slots) -> int:
    return _lib.fa_bwd_bsparse_split_workspace_bytes(B, Hq, Hkv, d, n_row_slots, n_col_slots)


def fa_fwd_dropout(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, dropout_p, seed, softmax_scale, dtype, stream) -> int:
    return _lib.fa_fwd_dropout(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, float(dropout_p), int(seed),
                               float(softmax_scale), dtype, stream)


def fa_bwd_dropout(q, k, v, o, dO, lse, dq, dk, dv, delta_ws, B, Hq, Hkv, N, d, causal, dropout_p, seed,
                   softmax_scale, dtype, stream) -> int:
    return _lib.fa_bwd_dropout(q, k, v, o, dO, lse, dq, dk, dv, delta_ws, B, Hq, Hkv, N, d, causal,
                               float(dropout_p), int(seed), float(softmax_scale), dtype, stream)


def bwd_dropout(q, k, v, o, do, lse, causal: bool, scale: float, dropout_p: float, seed: int, stream=None,
                workspace=None):
    """(dq, dk, dv, workspace) through the dropout of ``fwd_dropout`` (same p and seed; o, lse its outputs)."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shape(q, k)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        workspace = torch.empty(fa_bwd_workspace_bytes(B, Hq, N) // 4, dtype=torch.float32, device=q.device)
    _check(fa_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), B, Hq, Hkv, N, d,
                          int(causal), dropout_p, seed, scale, _dtype_code(q), _stream_handle(stream)),
           "fa_bwd_dropout")
    return dq, dk, dv, workspace


def fwd_dropout(q, k, v, causal: bool, scale: float, dropout_p: float, seed: int, stream=None):
    """(o, lse) of attention with dropout on P (Philox4x32-10 keep mask, see fa_fwd_dropout), bf16."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shape(q, k)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check(fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d,
                          int(causal), dropout_p, seed, scale, _dtype_code(q), _stream_handle(stream)),
           "fa_fwd_dropout")
    return o, lse


BSPARSE_BLOCK = 256   # side of a mask block (FA_BSPARSE_BLOCK)


class BlockSparseLayout:
    """A block mask [nb, nb] (nb = ceil(N / 256)) as the two int32 layouts the kernels read.

    ``row_ptr``/``col_idx``: the blocks that are on, row by row (columns ascending);
    ``col_ptr``/``row_idx``: the same blocks column by column.  With ``causal``
    the blocks above the diagonal are dropped (their keys are masked anyway).

    Work split: a block row (column) with more than ``split`` blocks is cut
    into ceil(n / split) work items of nearly equal length whose partials are
    merged (``row_chunks``/``row_merges``, ``col_chunks``/``col_merges``, the
    tables of fa_fwd_bsparse_split / fa_bwd_bsparse_split; items listed longest
    first).  ``split`` defaults to 1.5 times the mean blocks per row, rounded
    up (at least 4), so only rows and columns far longer than the rest are cut
    (on a 64-block mask with one global row and column, about 7 blocks per
    row, splits of 10 and 14 blocks ran the forward at 715 and 702 TFLOP/s,
    7 at 671, 5 at 521, no split at 264)."""

    def __init__(self, mask, causal: bool = False, device=None, split=None):
        torch = _torch()
        m = torch.as_tensor(mask, dtype=torch.bool).cpu()
        if m.dim() != 2 or m.shape[0] != m.shape[1]:
            raise ValueError("the block mask must be square [nb, nb]")
        if causal:
            m = torch.tril(m)
        self.mask, self.nb = m, m.shape[0]
        rows = m.to(torch.int32)
        self.nnz = int(rows.sum())
        cnt_r, cnt_c = rows.sum(1), rows.sum(0)
        zero = torch.zeros(1, dtype=torch.int64)
        rp = torch.cat([zero, torch.cumsum(cnt_r, 0)]).to(torch.int32)
        cp = torch.cat([zero, torch.cumsum(cnt_c, 0)]).to(torch.int32)
        ci = torch.nonzero(m, as_tuple=False)[:, 1].to(torch.int32)           # row-major: columns ascending per row
        ri = torch.nonzero(m.t().contiguous(), as_tuple=False)[:, 1].to(torch.int32)
        pad = lambda t: t if t.numel() else torch.zeros(1, dtype=torch.int32)
        self.row_ptr, self.col_ptr = rp.to(device), cp.to(device)
        self.col_idx, self.row_idx = pad(ci).to(device), pad(ri).to(device)
        if split is None:
            split = max(4, -(-3 * self.nnz // (2 * max(self.nb, 1))))
        if int(split) < 1:
            raise ValueError("split must be at least one block")
        self.split = int(split)
        tab = lambda rows: torch.tensor(rows if rows else [[0, 0, 0, 0]], dtype=torch.int32).to(device)
        rc, rm, self.n_row_slots = split_plan(rp.tolist(), self.split)
        cc, cm, self.n_col_slots = split_plan(cp.tolist(), self.split)
        self.row_chunks, self.row_merges, self.n_row_chunks, self.n_row_merges = tab(rc), tab(rm), len(rc), len(rm)
        self.col_chunks, self.col_merges, self.n_col_chunks, self.n_col_merges = tab(cc), tab(cm), len(cc), len(cm)


def split_plan(ptr, split: int):
    """Work items of a compressed block layout (``ptr``: nb + 1 offsets): a block row with n <= split entries is
    one item (slot -1), a longer one ceil(n / split) items of nearly equal length with consecutive partial slots
    and one merge entry.  Returns (chunks [(r, e0, e1, slot)] longest first, merges [(r, s0, ns, 0)], slots)."""
    chunks, merges, slots = [], [], 0
    for r in range(len(ptr) - 1):
        e0, e1 = int(ptr[r]), int(ptr[r + 1])
        n = e1 - e0
        if n <= split:
            chunks.append([r, e0, e1, -1])
            continue
        parts = -(-n // split)
        merges.append([r, slots, parts, 0])
        for i in range(parts):
            chunks.append([r, e0 + n * i // parts, e0 + n * (i + 1) // parts, slots])
            slots += 1
    chunks.sort(key=lambda c: c[1] - c[2])           # longest first (stable)
    return chunks, merges, slots


def _layout(layout, N, q):
    nb = (N + BSPARSE_BLOCK - 1) // BSPARSE_BLOCK
    if layout.nb != nb:
        raise ValueError(f"the block mask is {layout.nb} blocks per side, N = {N} needs {nb}")
    if layout.row_ptr.device != q.device:
        raise ValueError("the block-sparse layout must be on the tensors' device")


def fwd_bsparse(q, k, v, layout: BlockSparseLayout, causal: bool, scale: float, stream=None):
    """(o, lse) of block-sparse attention, bf16: key j is visible to query i iff
    ``layout.mask[i // 256, j // 256]`` (and j <= i with ``causal``)."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shape(q, k)
    _layout(layout, N, q)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if layout.n_row_slots:
        part = torch.empty(fa_fwd_bsparse_split_workspace_bytes(B, Hq, d, layout.n_row_slots) // 4,
                           dtype=torch.float32, device=q.device)
        _check(fa_fwd_bsparse_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq,
                                    Hkv, N, d, int(causal), layout.col_idx.data_ptr(), layout.nnz,
                                    layout.row_chunks.data_ptr(), layout.n_row_chunks, layout.row_merges.data_ptr(),
                                    layout.n_row_merges, layout.n_row_slots, part.data_ptr(), scale, _dtype_code(q),
                                    _stream_handle(stream)), "fa_fwd_bsparse_split")
        return o, lse
    _check(fa_fwd_bsparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d,
                          int(causal), layout.row_ptr.data_ptr(), layout.col_idx.data_ptr(), layout.nnz, scale,
                          _dtype_code(q), _stream_handle(stream)), "fa_fwd_bsparse")
    return o, lse


def bwd_bsparse(q, k, v, o, do, lse, layout: BlockSparseLayout, causal: bool, scale: float, stream=None,
                workspace=None):
    """(dq, dk, dv, workspace) of block-sparse attention (the mask of ``fwd_bsparse``)."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shape(q, k)
    _layout(layout, N, q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        workspace = torch.empty(fa_bwd_workspace_bytes(B, Hq, N) // 4, dtype=torch.float32, device=q.device)
    if layout.n_row_slots or layout.n_col_slots:
        part = torch.empty(fa_bwd_bsparse_split_workspace_bytes(B, Hq, Hkv, d, layout.n_row_slots,
                                                                layout.n_col_slots) // 4,
                           dtype=torch.float32, device=q.device)
        L = layout
        _check(fa_bwd_bsparse_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                                    B, Hq, Hkv, N, d, int(causal), L.col_idx.data_ptr(), L.row_idx.data_ptr(), L.nnz,
                                    L.row_chunks.data_ptr(), L.n_row_chunks, L.row_merges.data_ptr(), L.n_row_merges,
                                    L.n_row_slots, L.col_chunks.data_ptr(), L.n_col_chunks, L.col_merges.data_ptr(),
                                    L.n_col_merges, L.n_col_slots, part.data_ptr(), scale, _dtype_code(q),
                                    _stream_handle(stream)), "fa_bwd_bsparse_split")
        return dq, dk, dv, workspace
    _check(fa_bwd_bsparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), B, Hq, Hkv, N, d,
                          int(causal), layout.row_ptr.data_ptr(), layout.col_idx.data_ptr(),
                          layout.col_ptr.data_ptr(), layout.row_idx.data_ptr(), layout.nnz, scale, _dtype_code(q),
                          _stream_handle(stream)), "fa_bwd_bsparse")
    return dq, dk, dv, workspace


def fwd_local(q, k, v, window: int, scale: float, stream=None, sink: int = 0):
    """(o, lse) of causal sliding-window attention with `sink` global tokens, bf16.

    Key j is visible to query i iff j <= i and (i - window < j or j < sink)."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shape(q, k)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check(fa_fwd_local(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, d,
                        window, sink, scale, _dtype_code(q), _stream_handle(stream)), "fa_fwd_local")
    return o, lse


def bwd_local(q, k, v, o, do, lse, window: int, scale: float, stream=None, workspace=None, sink: int = 0):
    """(dq, dk, dv, workspace) of causal sliding-window attention with `sink` global tokens."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shape(q, k)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        workspace = torch.empty(fa_bwd_workspace_bytes(B, Hq, N) // 4, dtype=torch.float32, device=q.device)
    _check(fa_bwd_local(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), B, Hq, Hkv, N, d, window,
                        sink, scale, _dtype_code(q), _stream_handle(stream)), "fa_bwd_local")
    return dq, dk, dv, workspace


def decode(q, k, v, causal: bool, scale: float, stream=None, workspace=None):
    """(o, lse) for new query rows q [B,Hq,Nq,d] against a bf16 cache k, v [B,Hkv,Nk,d].

    Causal: the rows are the last Nq positions (row i sees keys j <= Nk - Nq + i)."""
    torch = _torch()
    for t in (q, k, v):
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous [B, H, N, d] tensors")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if v.shape != k.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must be [B, Hkv, Nk, d] with q's B and d")
    code = _dtype_code(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = fa_decode_workspace_bytes(B, Hq, Hkv, Nq, Nk, d) // 4
        workspace = torch.empty(max(n, 4), dtype=torch.float32, device=q.device)
    _check(fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                     B, Hq, Hkv, Nq, Nk, d, causal, scale, code, _stream_handle(stream)), "fa_decode")
    return o, lse


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, causal: bool, scale: float, stream=None, workspace=None):
    """(o, lse) for q [B,Hq,Nq,d] against a paged bf16 cache [num_blocks,Hkv,block_size,d].

    block_table: int32 [B, max_blocks]; seq_lens: int32 [B] (both on the device)."""
    torch = _torch()
    B, Hq, Nq, d = q.shape
    nblk, Hkv, bs = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    maxb = block_table.shape[1]
    for t in (block_table, seq_lens):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("block_table and seq_lens must be contiguous int32 tensors")
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = fa_decode_paged_workspace_bytes(B, Hq, Hkv, Nq, maxb, bs, d) // 4
        workspace = torch.empty(max(n, 4), dtype=torch.float32, device=q.device)
    _check(fa_decode_paged(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                           seq_lens.data_ptr(), o.data_ptr(), lse.data_ptr(), workspace.data_ptr(), B, Hq, Hkv, Nq,
                           maxb, bs, nblk, d, causal, scale, _dtype_code(q), _stream_handle(stream)),
           "fa_decode_paged")
    return o, lse


def fa_bwd_fp8(q8, k8, v8, o, dO8, lse, descale, dq, dk, dv, delta_ws, B, Hq, Hkv, N, d, causal, softmax_scale,
               stream) -> int:
    return _lib.fa_bwd_fp8(q8, k8, v8, o, dO8, lse, descale, dq, dk, dv, delta_ws, B, Hq, Hkv, N, d, int(causal),
                           float(softmax_scale), stream)


def bwd_fp8(q8, k8, v8, o, do8, lse, descale, causal: bool, scale: float, stream=None, workspace=None):
    """(dq, dk, dv, workspace), bf16, through the FP8 forward: q8, k8, v8, do8 E4M3 codes (uint8), o and lse the
    FP8 forward's outputs, descale float32[4] = (s_Q, s_K, s_V, s_dO) on the device."""
    torch = _torch()
    B, Hq, Hkv, N, d = _shape(q8, k8)
    dq = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    dk = torch.empty(k8.shape, dtype=torch.bfloat16, device=q8.device)
    dv = torch.empty(v8.shape, dtype=torch.bfloat16, device=q8.device)
    if workspace is None:
        workspace = torch.empty(fa_bwd_workspace_bytes(B, Hq, N) // 4, dtype=torch.float32, device=q8.device)
    _check(fa_bwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), do8.data_ptr(), lse.data_ptr(),
                      descale.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), B, Hq,
                      Hkv, N, d, int(causal), scale, _stream_handle(stream)), "fa_bwd_fp8")
    return dq, dk, dv, workspace


def quantize_fp8(x, stream=None):
    """(codes uint8 like x, descale float32[1]) for a contiguous bf16 device tensor x."""
    torch = _torch()
    if x.dtype != torch.bfloat16 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("x must be a contiguous bf16 device tensor")
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    ds = torch.empty(1, dtype=torch.float32, device=x.device)
    _check(fa_quantize_fp8(x.data_ptr(), x.numel(), out.data_ptr(), ds.data_ptr(), _stream_handle(stream)),
           "fa_quantize_fp8")
    return out, ds
