"""GPU parity of attention with dropout (fa_fwd_dropout, fa_bwd_dropout) with the float64 oracle.

The keep mask is integer work (Philox4x32-10 bytes against a threshold): the
mask each kernel regenerates is recovered element by element and compared
with the oracle's bit for bit -- the forward's through O, the dK/dV kernel's
through dV, the dQ kernel's through the sign of dQ.  O is compared to the
bf16 tolerance (max |err| <= 2e-2) and LSE (the undropped softmax statistic,
<= 1e-2); dQ, dK and dV to relative L2 <= 2e-2.  p = 0 is bit for bit the
plain forward and backward.
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
        Oref = (np.where(Z, P, 0.0) / (1 - oracle.drop_probability(p))) @ f64(v[b, h])
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
    the d keys of chunk c (V[j] = e_{j - d c}) gives O[i, m] = Z[i, d c + m] P_i / (1 - p'): nonzero exactly
    where key d c + m is kept and visible.  Every chunk of every row of every (batch, head) is compared with
    oracle.keep_mask bit for bit (ragged last chunk, rows past one 256-row block, grouped heads, seeds with a
    nonzero high word, p off the 1/256 grid)."""
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


def rel_l2(x, y):
    return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}x{}N{}d{}c{}p{}s{}".format(*c))
def test_dropout_backward_small(fa, case):
    """fa_fwd_dropout then fa_bwd_dropout against oracle.backward_dropout, every element."""
    B, Hq, Hkv, N, d, causal, p, seed = case
    dev = torch.device("cuda:0")
    scale = 1.0 / np.sqrt(d)
    q, k, v, do = (I.random_tensor(7100 + N, (B, H, N, d), "bf16", tensor_id=t)
                   for t, H in enumerate((Hq, Hkv, Hkv, Hq)))
    print(f"case {case}", flush=True)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.fwd_dropout(qd, kd, vd, causal, scale, p, seed)
    dq, dk, dv, _ = fa.bwd_dropout(qd, kd, vd, o, dod, lse, causal, scale, p, seed)
    torch.cuda.synchronize()
    rq, rk, rv, O = oracle.backward_dropout(f64(q), f64(k), f64(v), f64(do), causal, scale, p, seed)
    eo = float(np.max(np.abs(f64(o) - O)))
    errs = [rel_l2(f64(g), r) for g, r in ((dq, rq), (dk, rk), (dv, rv))]
    print(f"[{case}] O max|err| {eo:.3e}  dQ dK dV rel-L2 {errs}", flush=True)
    assert eo <= 2e-2 and max(errs) <= 2e-2


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_backward_p_zero_is_plain_backward(fa, causal):
    dev = torch.device("cuda:0")
    q, k, v, do = (I.random_tensor(72, (1, H, 700, 128), "bf16", tensor_id=t).to(dev)
                   for t, H in enumerate((4, 2, 2, 4)))
    o, lse = fa.fwd_dropout(q, k, v, causal, 0.1, 0.0, 5)
    g = fa.bwd_dropout(q, k, v, o, do, lse, causal, 0.1, 0.0, 5)[:3]
    gc = fa.bwd(q, k, v, o, do, lse, causal, 0.1)[:3]
    torch.cuda.synchronize()
    for a, b in zip(g, gc):
        assert torch.equal(a, b)


BWD_MASK_CASES = [
    # B, Hq, Hkv, N, d, causal, p, seed
    (2, 2, 2, 600, 128, False, 0.5, (3 << 32) + 17),
    (1, 2, 2, 700, 64, True, 0.3, 2 ** 63 + 5),
    (1, 4, 2, 300, 128, True, 0.25, 41),
]


@pytest.mark.parametrize("case", BWD_MASK_CASES, ids=lambda c: "B{}H{}x{}N{}d{}c{}p{}".format(*c[:7]))
def test_dropout_backward_dkdv_mask_bit_exact(fa, case):
    """The dK/dV kernel's mask, read through dV.  Q = 0 (P uniform over the visible keys) and dO one-hot over the
    d queries of chunk c (dO[i] = e_{i - d c}) give dV[j, m] = sum over the group's heads of
    Z_h[d c + m, j] P / (1 - p'): nonzero exactly where some head of the group keeps (visible) element
    (d c + m, j).  Compared with the oracle's masks for every chunk and key."""
    B, Hq, Hkv, N, d, causal, p, seed = case
    G = Hq // Hkv
    dev = torch.device("cuda:0")
    q = torch.zeros((B, Hq, N, d), dtype=torch.bfloat16, device=dev)
    k = I.random_tensor(5200 + N, (B, Hkv, N, d), "bf16", tensor_id=1).to(dev)
    v = I.random_tensor(5200 + N, (B, Hkv, N, d), "bf16", tensor_id=2).to(dev)
    rows = np.arange(N)
    vis = np.tril(np.ones((N, N), bool)) if causal else np.ones((N, N), bool)
    Z = {(b, h): oracle.keep_mask(b, h, Hq, rows, N, p, seed) & vis for b in range(B) for h in range(Hq)}
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.fwd_dropout(q, k, v, causal, scale, p, seed)
    for c in range((N + d - 1) // d):
        do = one_hot_chunk(B, Hq, N, d, c).to(dev)
        print(f"case {case} chunk {c}", flush=True)
        _, _, dv, _ = fa.bwd_dropout(q, k, v, o, do, lse, causal, scale, p, seed)
        torch.cuda.synchronize()
        got = (dv != 0).cpu().numpy()                       # [B, Hkv, N keys, d]
        w = min(N, (c + 1) * d) - c * d
        for b in range(B):
            for g in range(Hkv):
                ref = np.zeros((N, w), bool)
                for h in range(g * G, (g + 1) * G):
                    ref |= Z[(b, h)][c * d:c * d + w, :].T
                bad = int(np.sum(got[b, g, :, :w] != ref))
                assert bad == 0, (case, c, b, g, bad)
                assert not got[b, g, :, w:].any()
    print(f"[{case}] dK/dV kernel: every mask bit equal", flush=True)


@pytest.mark.parametrize("case", [(2, 2, 1, 600, 128, 0.5, 9), (1, 3, 3, 700, 64, 0.3, (1 << 40) + 1)],
                         ids=lambda c: "B{}H{}x{}N{}d{}p{}".format(*c[:6]))
def test_dropout_backward_dq_mask_bit_exact(fa, case):
    """The dQ kernel's mask, read through the sign of dQ (non-causal).  Q = 0 (P = 1/N), K one-hot over the d keys
    of chunk c, dO[i] = e_0 and V[j] = e_0 for the keys of chunk c (0 elsewhere): dP[i, j] = Z r for j in the chunk,
    D_i = r P (kept keys of the chunk), and dQ[i, m] = scale dS[i, d c + m] = scale P (Z r - D_i): positive where
    kept (D_i < r, the chunk being shorter than N), negative where dropped (some key of the chunk is kept)."""
    B, Hq, Hkv, N, d, p, seed = case
    dev = torch.device("cuda:0")
    q = torch.zeros((B, Hq, N, d), dtype=torch.bfloat16, device=dev)
    do = torch.zeros((B, Hq, N, d), dtype=torch.bfloat16)
    do[..., 0] = 1.0
    do = do.to(dev)
    rows = np.arange(N)
    Z = {(b, h): oracle.keep_mask(b, h, Hq, rows, N, p, seed) for b in range(B) for h in range(Hq)}
    scale = 1.0 / np.sqrt(d)
    for c in range((N + d - 1) // d):
        w = min(N, (c + 1) * d) - c * d
        k = one_hot_chunk(B, Hkv, N, d, c).to(dev)
        v = torch.zeros((B, Hkv, N, d), dtype=torch.bfloat16)
        v[:, :, c * d:c * d + w, 0] = 1.0
        v = v.to(dev)
        print(f"case {case} chunk {c}", flush=True)
        o, lse = fa.fwd_dropout(q, k, v, False, scale, p, seed)
        dq, _, _, _ = fa.bwd_dropout(q, k, v, o, do, lse, False, scale, p, seed)
        torch.cuda.synchronize()
        dqh = dq.float().cpu().numpy()
        for (b, h), z in Z.items():
            zc = z[:, c * d:c * d + w]
            assert zc.any(axis=1).all()                      # every row keeps some key of the chunk
            got = dqh[b, h, :, :w]
            assert np.all(got != 0), (case, c, b, h)
            bad = int(np.sum((got > 0) != zc))
            assert bad == 0, (case, c, b, h, bad)
    print(f"[{case}] dQ kernel: every mask bit equal", flush=True)


def test_dropout_backward_headline_shape(fa):
    """B=4 H=32 N=4096 d=128 causal, p = 0.125: the whole of two heads (O, dQ, dK, dV) against the oracle, and
    the time of the dropout backward beside the plain one."""
    w = I.WORKLOADS["causal_bf16_n4096"]
    dev = torch.device("cuda:0")
    q, k, v, do = (I.full_tensor(w, t) for t in range(4))
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    p, seed = 0.125, 2025
    o, lse = fa.fwd_dropout(qd, kd, vd, True, w.scale, p, seed)
    for _ in range(2):
        dq, dk, dv, ws = fa.bwd_dropout(qd, kd, vd, o, dod, lse, True, w.scale, p, seed)
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(st)
    for _ in range(5):
        fa.bwd_dropout(qd, kd, vd, o, dod, lse, True, w.scale, p, seed, stream=st, workspace=ws)
    ev[1].record(st)
    for _ in range(5):
        fa.bwd(qd, kd, vd, o, dod, lse, True, w.scale, stream=st, workspace=ws)
    ev[2].record(st)
    torch.cuda.synchronize()
    print(f"dropout backward {ev[0].elapsed_time(ev[1]) / 5:.4f} ms, plain backward "
          f"{ev[1].elapsed_time(ev[2]) / 5:.4f} ms", flush=True)
    dq, dk, dv, _ = fa.bwd_dropout(qd, kd, vd, o, dod, lse, True, w.scale, p, seed)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (w.B - 1, w.Hq - 1)):          # one query head per K/V head: dK, dV are that head's
        rq, rk, rv, O = oracle.head_backward_dropout(f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), f64(do[b, h]),
                                                     b, h, w.Hq, True, w.scale, p, seed)
        eo = float(np.max(np.abs(f64(o[b, h]) - O)))
        errs = [rel_l2(f64(g[b, h]), r) for g, r in ((dq, rq), (dk, rk), (dv, rv))]
        print(f"head ({b}, {h}) O max|err| {eo:.3e}  dQ dK dV rel-L2 {errs}", flush=True)
        assert eo <= 2e-2 and max(errs) <= 2e-2
