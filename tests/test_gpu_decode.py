"""GPU parity of the decode path (fa_decode through the C ABI) against the CPU float64 oracle.

Decode is exact softmax attention of Nq new query rows against a key/value
cache of Nk rows; causal rows are the last Nq positions (row i sees keys
j <= Nk - Nq + i).  Tolerances are the bf16 ones: max |err| <= 2e-2 on O,
<= 1e-2 on LSE.  Small shapes (ragged cache lengths, several 32-row blocks of
packed query rows, one key, Nq = Nk) are compared element by element; the
16-sequence, 16384-token grouped-query workload is compared on every row.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_50_amd import inputs as I

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL = 2e-2, 1e-2


@pytest.fixture(scope="module")
def fa():
    from exact_io_aware_50_amd import fa as _fa
    return _fa


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check(o, lse, O, L, tag):
    o, lse = (f64(x) if isinstance(x, torch.Tensor) else x for x in (o, lse))
    eo = float(np.max(np.abs(o - O)))
    el = float(np.max(np.abs(lse - L)))
    print(f"[{tag}] O max|err| {eo:.3e}  LSE max|err| {el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL, (tag, eo, el)


SMALL = [
    # B, Hq, Hkv, Nq, Nk, d, causal
    (1, 8, 1, 1, 1, 128, False),
    (2, 8, 2, 1, 100, 64, False),
    (1, 4, 4, 3, 257, 128, True),
    (2, 16, 2, 4, 1000, 128, True),
    (1, 16, 2, 5, 777, 64, True),
    (1, 2, 2, 17, 17, 128, True),
    (3, 32, 8, 1, 5000, 128, False),
    (1, 64, 8, 2, 3000, 128, True),
    (1, 1, 1, 40, 300, 64, False),
    (2, 8, 8, 1, 33, 64, True),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}H{}x{}q{}k{}d{}{}".format(*s[:6], "c" if s[6] else ""))
def test_decode_small_shapes(fa, dev, shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    scale = 1.0 / np.sqrt(d)
    seed = 3000 + Nq + Nk + d
    q = I.random_tensor(seed, (B, Hq, Nq, d), "bf16", tensor_id=0)
    k = I.random_tensor(seed, (B, Hkv, Nk, d), "bf16", tensor_id=1)
    v = I.random_tensor(seed, (B, Hkv, Nk, d), "bf16", tensor_id=2)
    print(f"case {shape}", flush=True)
    o, lse = fa.decode(q.to(dev), k.to(dev), v.to(dev), causal, scale)
    torch.cuda.synchronize()
    O, L = oracle.decode_forward(f64(q), f64(k), f64(v), causal, scale)
    check(o, lse, O, L, str(shape))


def test_decode_all_rows_equals_causal_forward(fa, dev):
    """Nq = Nk: decoding every row is the causal forward pass; both are held to the oracle."""
    B, Hq, Hkv, N, d = 1, 8, 2, 300, 128
    scale = 1.0 / np.sqrt(d)
    q = I.random_tensor(41, (B, Hq, N, d), "bf16", tensor_id=0).to(dev)
    k = I.random_tensor(41, (B, Hkv, N, d), "bf16", tensor_id=1).to(dev)
    v = I.random_tensor(41, (B, Hkv, N, d), "bf16", tensor_id=2).to(dev)
    o, lse = fa.decode(q, k, v, True, scale)
    of, lf = fa.fwd(q, k, v, True, scale)
    torch.cuda.synchronize()
    O, L = oracle.forward(f64(q), f64(k), f64(v), True, scale)
    check(o, lse, O, L, "decode Nq=Nk")
    check(of, lf, O, L, "forward")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", list(I.DECODE_WORKLOADS))
def test_decode_workload_every_row(fa, dev, name):
    w = I.DECODE_WORKLOADS[name]
    q, k, v = (I.decode_tensor(w, t) for t in range(3))
    print(f"workload {w.name}: inputs ready", flush=True)
    o, lse = fa.decode(q.to(dev), k.to(dev), v.to(dev), w.causal, w.scale)
    o2, lse2 = fa.decode(q.to(dev), k.to(dev), v.to(dev), w.causal, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)          # no atomics: bitwise repeatable
    o, lse = o.cpu(), lse.cpu()
    eo = el = 0.0
    for b in range(w.B):
        O, L = oracle.decode_forward(f64(q[b:b + 1]), f64(k[b:b + 1]), f64(v[b:b + 1]), w.causal, w.scale)
        eo = max(eo, float(np.max(np.abs(f64(o[b:b + 1]) - O))))
        el = max(el, float(np.max(np.abs(f64(lse[b:b + 1]) - L))))
    print(f"[{name}] every row: O max|err| {eo:.3e}  LSE max|err| {el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL


# ---------------------------------------------------------------- paged cache, per-sequence lengths

def paged_case(seed, B, Hq, Hkv, Nq, lens, d, bs, spare=3):
    """A shuffled block pool holding each sequence's keys, its block table and lengths (CPU tensors)."""
    maxb = max((n + bs - 1) // bs for n in lens) if max(lens) > 0 else 1
    nblk = B * maxb + spare
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    perm = rng.permutation(nblk)
    kc = I.random_tensor(seed, (nblk, Hkv, bs, d), "bf16", tensor_id=1)
    vc = I.random_tensor(seed, (nblk, Hkv, bs, d), "bf16", tensor_id=2)
    table = torch.tensor(perm[:B * maxb].reshape(B, maxb), dtype=torch.int32)
    q = I.random_tensor(seed, (B, Hq, Nq, d), "bf16", tensor_id=0)
    return q, kc, vc, table, torch.tensor(lens, dtype=torch.int32)


PAGED = [
    # B, Hq, Hkv, Nq, lens, d, block size, causal
    (3, 8, 1, 1, [1, 100, 257], 128, 32, False),
    (2, 16, 2, 4, [1000, 64], 128, 64, True),
    (4, 8, 8, 1, [33, 0, 500, 2048], 64, 256, False),
    (2, 64, 8, 2, [3000, 1], 128, 128, True),
    (2, 4, 2, 5, [3, 70], 64, 32, True),            # causal rows before sequence 0's first key
    # more sequences than a wave has lanes: the chunk plan is worked out in five passes of 64
    (300, 2, 1, 1, [int(x) for x in np.random.Generator(np.random.PCG64(31)).integers(0, 200, 300)], 64, 32, False),
    # 128 K/V heads leave 8 chunk slots on a 256-CU device: chunks of 2528 keys span 79 blocks of 32, past the
    # 64 block ids a wave holds in registers (the rest are read from the table)
    (1, 128, 128, 1, [20000], 128, 32, False),
]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("case", PAGED, ids=lambda c: "B{}H{}x{}q{}d{}bs{}{}".format(*c[:4], *c[5:7], "c" if c[7] else ""))
def test_decode_paged(fa, dev, case):
    B, Hq, Hkv, Nq, lens, d, bs, causal = case
    scale = 1.0 / np.sqrt(d)
    q, kc, vc, table, sl = paged_case(4000 + sum(lens), B, Hq, Hkv, Nq, lens, d, bs)
    tag = f"B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} lens[{len(lens)}] max {max(lens)} d={d} bs={bs} causal={causal}"
    print(f"case {tag}", flush=True)
    o, lse = fa.decode_paged(q.to(dev), kc.to(dev), vc.to(dev), table.to(dev), sl.to(dev), causal, scale)
    torch.cuda.synchronize()
    O, L = oracle.decode_paged_forward(f64(q), f64(kc), f64(vc), table.numpy(), lens, causal, scale)
    none = np.isneginf(L)                                    # rows that see no key: O = 0, LSE = -inf exactly
    assert np.array_equal(np.isneginf(f64(lse)), none) and np.all(f64(o)[none] == 0)
    keep = ~none
    check(f64(o)[keep], f64(lse)[keep], O[keep], L[keep], tag)


@pytest.mark.timeout(300)
def test_decode_paged_workload_mixed_lengths(fa, dev):
    """The 16-sequence 16K-token cache as shuffled 256-key blocks, lengths in [Nk/4, Nk]: every row against the oracle."""
    w = I.DECODE_WORKLOADS["decode_gqa_bf16_n16384"]
    q, k, v = (I.decode_tensor(w, t) for t in range(3))
    bs = 256
    maxb = w.Nk // bs
    g = torch.Generator().manual_seed(5)
    perm = torch.randperm(w.B * maxb, generator=g)
    lens = torch.randint(w.Nk // 4, w.Nk + 1, (w.B,), generator=g, dtype=torch.int32)
    table = perm.view(w.B, maxb).to(torch.int32)
    blk = lambda t: t.view(w.B, w.Hkv, maxb, bs, w.d).permute(0, 2, 1, 3, 4).reshape(w.B * maxb, w.Hkv, bs, w.d)
    kc, vc = torch.empty_like(blk(k)), torch.empty_like(blk(v))
    kc[perm] = blk(k)
    vc[perm] = blk(v)
    o, lse = fa.decode_paged(q.to(dev), kc.to(dev), vc.to(dev), table.to(dev), lens.to(dev), w.causal, w.scale)
    o2, lse2 = fa.decode_paged(q.to(dev), kc.to(dev), vc.to(dev), table.to(dev), lens.to(dev), w.causal, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    o, lse = o.cpu(), lse.cpu()
    eo = el = 0.0
    for b in range(w.B):
        n = int(lens[b])
        O, L = oracle.decode_forward(f64(q[b:b + 1]), f64(k[b:b + 1, :, :n]), f64(v[b:b + 1, :, :n]), w.causal,
                                     w.scale)
        eo = max(eo, float(np.max(np.abs(f64(o[b:b + 1]) - O))))
        el = max(el, float(np.max(np.abs(f64(lse[b:b + 1]) - L))))
    print(f"[paged 16K mixed lengths] every row: O max|err| {eo:.3e}  LSE max|err| {el:.3e}", flush=True)
    assert eo <= O_TOL and el <= LSE_TOL
