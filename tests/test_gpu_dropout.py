"""GPU parity of the forward with attention dropout (fa_fwd_dropout) with the float64 oracle.

The keep mask is integer work (Philox4x32-10 words against a threshold), so the
kernel and the oracle drop exactly the same elements; O is compared to the
bf16 tolerance (max |err| <= 2e-2) and LSE (the undropped softmax statistic,
<= 1e-2).  p = 0 is bit for bit the plain forward.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_50_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    from exact_io_aware_50_amd import fa as _fa
    return _fa


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


CASES = [
    # B, Hq, Hkv, N, d, causal, p, seed
    (1, 2, 2, 300, 128, False, 0.25, 1),
    (1, 4, 2, 513, 64, True, 0.5, (5 << 32) + 77),
    (2, 2, 1, 1000, 128, True, 0.125, 2 ** 63 + 9),
    (1, 3, 3, 129, 64, False, 0.75, 123456789),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}x{}N{}d{}c{}p{}s{}".format(*c))
def test_dropout_forward_small(fa, case):
    B, Hq, Hkv, N, d, causal, p, seed = case
    dev = torch.device("cuda:0")
    scale = 1.0 / np.sqrt(d)
    q, k, v = (I.random_tensor(7000 + N, (B, H, N, d), "bf16", tensor_id=t) for t, H in enumerate((Hq, Hkv, Hkv)))
    print(f"case {case}", flush=True)
    o, lse = fa.fwd_dropout(q.to(dev), k.to(dev), v.to(dev), causal, scale, p, seed)
    torch.cuda.synchronize()
    O, L = oracle.forward_dropout(f64(q), f64(k), f64(v), causal, scale, p, seed)
    eo, el = float(np.max(np.abs(f64(o) - O))), float(np.max(np.abs(f64(lse) - L)))
    print(f"[{case}] O max|err| {eo:.3e}  LSE max|err| {el:.3e}", flush=True)
    assert eo <= 2e-2 and el <= 1e-2


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_p_zero_is_plain_forward(fa, causal):
    dev = torch.device("cuda:0")
    q, k, v = (I.random_tensor(71, (1, H, 700, 128), "bf16", tensor_id=t).to(dev) for t, H in enumerate((4, 2, 2)))
    o, lse = fa.fwd_dropout(q, k, v, causal, 0.1, 0.0, 5)
    oc, lc = fa.fwd(q, k, v, causal, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(lse, lc)


def test_dropout_forward_headline_shape(fa):
    """B=4 H=32 N=4096 d=128 causal, p = 0.125: sampled rows of two heads against the oracle, and the time."""
    w = I.WORKLOADS["causal_bf16_n4096"]
    dev = torch.device("cuda:0")
    q, k, v = (I.full_tensor(w, t) for t in range(3))
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    p, seed = 0.125, 2024
    for _ in range(3):
        o, lse = fa.fwd_dropout(qd, kd, vd, True, w.scale, p, seed)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    st = torch.cuda.current_stream()
    ev[0].record(st)
    for _ in range(10):
        fa.fwd_dropout(qd, kd, vd, True, w.scale, p, seed, stream=st)
    ev[1].record(st)
    for _ in range(10):
        fa.fwd(qd, kd, vd, True, w.scale, stream=st)
    ev[2].record(st)
    torch.cuda.synchronize()
    td, tp = ev[0].elapsed_time(ev[1]) / 10, ev[1].elapsed_time(ev[2]) / 10
    print(f"dropout forward {td:.4f} ms, plain forward {tp:.4f} ms", flush=True)
    rows = I.sample_rows(w.N)
    for b, h in ((0, 0), (w.B - 1, w.Hq - 1)):
        _, P, m, l = oracle.probabilities(f64(q[b, h]), f64(k[b, h]), w.scale, True, rows=rows)
        Z = oracle.keep_mask(b, h, w.Hq, rows, w.N, p, seed)
        Oref = (np.where(Z, P, 0.0) / (1 - p)) @ f64(v[b, h])
        eo = float(np.max(np.abs(f64(o[b, h, rows]) - Oref)))
        el = float(np.max(np.abs(f64(lse[b, h, rows]) - (m + np.log(l)))))
        print(f"head ({b}, {h}) O max|err| {eo:.3e} LSE max|err| {el:.3e}", flush=True)
        assert eo <= 2e-2 and el <= 1e-2
