"""Seeded synthetic inputs for exact attention.

This module only draws random numbers and arranges them into tensors; it holds
none of the attention arithmetic.  It is the one module that both the CPU
oracle side (tests, bench's CPU leg) and the GPU side use, so that both see the
same inputs.

Each (tensor, batch, head) slice has its own counter-free stream,
``PCG64(SeedSequence([seed, tensor_id, b, h]))``, so any single head can be
regenerated without building the whole tensor.  Tensor ids: Q=0, K=1, V=2,
dO=3.  K and V heads are indexed by the key/value head.

The workloads are the five shapes of the attention pages' regimes: a tiny fp32
check, a short non-causal bf16 batch, the N=4096 causal headline shape, a 16K
grouped-query shape (with an fp8 forward), and a 64K long-context stress shape
whose Q and K have standard deviation 3 (a wide score range).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

Q_ID, K_ID, V_ID, DO_ID = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    dtype: str          # "f32" or "bf16"
    qk_sigma: float = 1.0
    fp8_fwd: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32 (B=1 H=2 N=256 d=64, non-causal, fp32)", 1, 1, 2, 2, 256, 64, False, "f32"),
    "mha_bf16_n1024": Workload("mha_bf16_n1024 (B=8 H=16 N=1024 d=64, non-causal, bf16)", 2, 8, 16, 16, 1024, 64, False, "bf16"),
    "causal_bf16_n4096": Workload("causal_bf16_n4096 (B=4 H=32 N=4096 d=128, causal, bf16)", 3, 4, 32, 32, 4096, 128, True, "bf16"),
    "gqa_bf16_n16384": Workload("gqa_bf16_n16384 (B=1 Hq=64 Hkv=8 N=16384 d=128, causal, bf16 + fp8 fwd)", 4, 1, 64, 8, 16384, 128, True, "bf16", fp8_fwd=True),
    "long_bf16_n65536": Workload("long_bf16_n65536 (B=1 H=8 N=65536 d=128, causal, bf16, Q,K sigma=3)", 5, 1, 8, 8, 65536, 128, True, "bf16", qk_sigma=3.0),
}


@dataclass(frozen=True)
class DecodeWorkload:
    """New query rows [B, Hq, Nq, d] against a key/value cache [B, Hkv, Nk, d]."""
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


# The grouped-query shape of the 16K-token workload as a serving step: one new
# token (and a four-token chunk, causal) per sequence for a batch of 16 against
# a 16384-token cache; the cache is 1 GiB of bf16.
DECODE_WORKLOADS = {
    "decode_gqa_bf16_n16384": DecodeWorkload(
        "decode_gqa_bf16_n16384 (B=16 Hq=64 Hkv=8 Nq=1 Nk=16384 d=128, bf16)", 6, 16, 64, 8, 1, 16384, 128, False),
    "decode_gqa_bf16_n16384_q4": DecodeWorkload(
        "decode_gqa_bf16_n16384_q4 (B=16 Hq=64 Hkv=8 Nq=4 Nk=16384 d=128, causal, bf16)", 7, 16, 64, 8, 4, 16384,
        128, True),
}


# Sliding-window (local) attention at the 64K-token shape: a 4096-key causal
# window, inputs as the long-context workload (Q, K with sigma 3).
LOCAL_WORKLOADS = {
    "local_bf16_n65536_w4096": (WORKLOADS["long_bf16_n65536"], 4096),
}


def block_pattern(nb: int, band: int = 1, n_global: int = 0, n_random: int = 2, seed: int = 0) -> np.ndarray:
    """A [nb, nb] boolean block mask: a band of |r - c| <= band blocks, the first
    n_global block rows and columns, and n_random seeded random permutations
    (block (r, perm(r)) on), so that every block row and every block column
    gets about the same number of blocks."""
    r = np.arange(nb)
    m = np.abs(r[:, None] - r[None, :]) <= band
    m[:n_global, :] = True
    m[:, :n_global] = True
    rng = np.random.default_rng(seed)
    for _ in range(n_random):
        m[r, rng.permutation(nb)] = True
    return m


# Block-sparse workload: tensors of a Workload and the block mask's parameters.
BSPARSE_WORKLOADS = {
    "bsparse_bf16_n16384": (
        Workload("bsparse_bf16_n16384 (B=1 Hq=32 Hkv=8 N=16384 d=128, non-causal, 256-blocks: 3-block band "
                 "and 2 random permutations, bf16)", 8, 1, 32, 8, 16384, 128, False, "bf16"),
        dict(band=1, n_global=0, n_random=2, seed=8)),
    # the same with one global block row and column (a row that sees every
    # block and a key block every row sees): 64 blocks against about 6
    "bsparse_global_bf16_n16384": (
        Workload("bsparse_global_bf16_n16384 (B=1 Hq=32 Hkv=8 N=16384 d=128, non-causal, 256-blocks: 3-block "
                 "band, 2 random permutations, 1 global block row and column, bf16)", 8, 1, 32, 8, 16384, 128, False,
                 "bf16"),
        dict(band=1, n_global=1, n_random=2, seed=8)),
}


def decode_tensor(w: DecodeWorkload, tensor_id: int, device="cpu"):
    """Q ([B, Hq, Nq, d]) or the K / V cache ([B, Hkv, Nk, d]) of a decode workload, bf16."""
    import torch
    heads, n = (w.Hq, w.Nq) if tensor_id == Q_ID else (w.Hkv, w.Nk)
    out = torch.empty((w.B, heads, n, w.d), dtype=torch.bfloat16, device=device)
    for b in range(w.B):
        for h in range(heads):
            out[b, h].copy_(torch.from_numpy(slice_normal(w.seed, tensor_id, b, h, n, w.d)).to(torch.bfloat16))
    return out


def slice_normal(seed: int, tensor_id: int, b: int, h: int, n: int, d: int,
                 sigma: float = 1.0) -> np.ndarray:
    """One [n, d] float32 slice of i.i.d. N(0, sigma^2) from its own stream."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, b, h])))
    x = rng.standard_normal((n, d), dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return x


def head_slice(w: Workload, tensor_id: int, b: int, h: int, n: int | None = None):
    """A slice as a CPU torch tensor in the workload's dtype (bf16 by RNE cast)."""
    import torch
    n = w.N if n is None else n
    sigma = w.qk_sigma if tensor_id in (Q_ID, K_ID) else 1.0
    x = torch.from_numpy(slice_normal(w.seed, tensor_id, b, h, n, w.d, sigma))
    return x.to(torch.bfloat16) if w.dtype == "bf16" else x


def full_tensor(w: Workload, tensor_id: int, n: int | None = None, device="cpu"):
    """The whole [B, H, N, d] tensor; H is Hkv for K and V, Hq otherwise."""
    import torch
    n = w.N if n is None else n
    heads = w.Hkv if tensor_id in (K_ID, V_ID) else w.Hq
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = torch.empty((w.B, heads, n, w.d), dtype=dt, device=device)
    for b in range(w.B):
        for h in range(heads):
            out[b, h].copy_(head_slice(w, tensor_id, b, h, n))
    return out


def random_tensor(seed: int, shape, dtype="bf16", sigma: float = 1.0, tensor_id: int = 0):
    """A small free-shape tensor for edge-case tests ([B, H, N, d])."""
    import torch
    B, H, N, d = shape
    out = np.empty(shape, dtype=np.float32)
    for b in range(B):
        for h in range(H):
            out[b, h] = slice_normal(seed, tensor_id, b, h, N, d, sigma)
    t = torch.from_numpy(out)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def sample_heads(w: Workload, count_random: int = 2, rng_seed: int = 12345):
    """Sampled (b, q-head) pairs: first, last, group-straddling and random ones."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([rng_seed, w.seed])))
    heads = {(0, 0), (w.B - 1, w.Hq - 1)}
    G = w.Hq // w.Hkv
    if G > 1:
        heads |= {(0, G - 1), (0, G)}
    while len(heads) < 2 + (2 if G > 1 else 0) + count_random:
        heads.add((int(rng.integers(w.B)), int(rng.integers(w.Hq))))
    return sorted(heads)


def sample_rows(n: int, count_random: int = 54, rng_seed: int = 777):
    """Sampled row (or column) indices: tile edges, the middle, the tail, random."""
    fixed = [0, 1, 63, 64, 127, 128, n // 2 - 1, n // 2, n - 2, n - 1]
    rows = {r for r in fixed if 0 <= r < n}
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([rng_seed, n])))
    target = min(n, len(rows) + count_random)
    while len(rows) < target:
        rows.add(int(rng.integers(n)))
    return np.array(sorted(rows), dtype=np.int64)
