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
    eo = float(np.max(np.abs(f64(o) - O)))
    el = float(np.max(np.abs(f64(lse) - L)))
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
