"""GPU parity of the forward with attention dropout (fa_fwd_dropout) with the float64 oracle.

The keep mask is integer work (Philox4x32-10 words against a threshold): the
kernel's mask is recovered element by element and compared with the oracle's
bit for bit (test_dropout_keep_mask_bit_exact).  O is compared to the bf16
tolerance (max |err| <= 2e-2) and LSE (the undropped softmax statistic,
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


def one_hot_chunk(B, H, N, d, c):
    """[B, H, N, d] bf16: row j = e_{j - d c} for the keys j of chunk c (d c <= j < d (c + 1)), 0 elsewhere."""
    x = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    j = torch.arange(c * d, min(N, (c + 1) * d))
    x[:, :, j, j - c * d] = 1.0
    return x


MASK_CASES = [
    # B, Hq, Hkv, N, d, causal, p, seeds
    (2, 3, 1, 600, 128, False, 0.5, (11, (7 << 32) + 3)),
    (1, 2, 2, 700, 64, True, 0.3, (2 ** 63 + 5,)),
    (1, 4, 2, 300, 128, True, 0.1, (99,)),
]


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: "B{}H{}x{}N{}d{}c{}p{}".format(*c[:7]))
def test_dropout_keep_mask_bit_exact(fa, case):
    """Q = 0 makes every score 0, so P is uniform over the visible keys (1/N; causal 1/(i+1)).  V one-hot over
    the d keys of chunk c (V[j] = e_{j - d c}) gives O[i, m] = Z[i, d c + m] P_i / (1 - p): nonzero exactly
    where key d c + m is kept and visible.  Every chunk of every row of every (batch, head) is compared with
    oracle.keep_mask bit for bit (ragged last chunk, rows past one 256-row block, grouped heads, seeds with a
    nonzero high word, p off the float32 grid)."""
    B, Hq, Hkv, N, d, causal, p, seeds = case
    dev = torch.device("cuda:0")
    q = torch.zeros((B, Hq, N, d), dtype=torch.bfloat16, device=dev)
    k = I.random_tensor(5100 + N, (B, Hkv, N, d), "bf16", tensor_id=1).to(dev)
    rows = np.arange(N)
    vis = np.tril(np.ones((N, N), bool)) if causal else np.ones((N, N), bool)
    for seed in seeds:
        ref = {(b, h): oracle.keep_mask(b, h, Hq, rows, N, p, seed) & vis for b in range(B) for h in range(Hq)}
        for c in range((N + d - 1) // d):
            v = one_hot_chunk(B, Hkv, N, d, c).to(dev)
            print(f"case {case} seed {seed} chunk {c}", flush=True)
            o, _ = fa.fwd_dropout(q, k, v, causal, 1.0 / np.sqrt(d), p, seed)
            torch.cuda.synchronize()
            got = (o != 0).cpu().numpy()
            w = min(N, (c + 1) * d) - c * d
            for (b, h), z in ref.items():
                bad = int(np.sum(got[b, h, :, :w] != z[:, c * d:c * d + w]))
                assert bad == 0, (case, seed, c, b, h, bad)
                assert not got[b, h, :, w:].any()
        kept = np.mean([z[vis].mean() for z in ref.values()])
        print(f"[{case}] seed {seed}: every mask bit equal; kept fraction {kept:.4f}", flush=True)
