"""GPU parity of block-sparse attention (fa_fwd_bsparse / fa_bwd_bsparse) with the float64 oracle.

Key j is visible to query i iff block (i // 256, j // 256) of the mask is on
(and j <= i when causal).  A row that sees no key has O = 0 and LSE = -inf
(compared exactly); everything else to the bf16 tolerances: max |err| <= 2e-2
on O, <= 1e-2 on LSE, relative L2 <= 2e-2 on dQ, dK, dV.  Small shapes with
random masks (empty block rows and columns included, ragged N, grouped heads,
d = 64 and 128, causal and not) are compared element by element; the
16K-token workload bench.py times is compared on sampled rows and key columns.
Masks with global block rows and columns go through the work split (long rows
and columns cut into items whose float32 partials are merged): small shapes
against the oracle, the split against the unsplit path, and the 16K-token
global-row-and-column workload on sampled rows and key columns.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_50_amd import inputs as I

pytestmark = pytest.mark.gpu

O_TOL, LSE_TOL, REL_TOL = 2e-2, 1e-2, 2e-2
BS = 256


@pytest.fixture(scope="module")
def fa():
    from exact_io_aware_50_amd import fa as _fa
    return _fa


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel_l2(x, y):
    return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300))


def check(o, lse, grads, O, L, ref_grads, tag):
    empty = np.isneginf(L)
    assert np.array_equal(np.isneginf(lse), empty), (tag, "rows with no key")
    assert np.all(o[empty] == 0), (tag, "O of rows with no key")
    eo = float(np.max(np.abs(o - O))) if o.size else 0.0
    el = float(np.max(np.abs(lse[~empty] - L[~empty]))) if np.any(~empty) else 0.0
    msg = f"[{tag}] O max|err| {eo:.3e}  LSE max|err| {el:.3e}  empty rows {int(empty.sum())}"
    errs = []
    for name, g, r in zip(("dQ", "dK", "dV"), grads, ref_grads):
        if not np.any(r):
            errs.append((name, float(np.max(np.abs(g))), 0.0))     # an exactly zero gradient stays zero
        else:
            errs.append((name, rel_l2(g, r), REL_TOL))
        msg += f"  {name} {errs[-1][1]:.3e}"
    print(msg, flush=True)
    assert eo <= O_TOL and el <= LSE_TOL, (tag, eo, el)
    for name, e, tol in errs:
        assert e <= tol, (tag, name, e)


def random_mask(nb, density, seed):
    m = np.random.default_rng(seed).random((nb, nb)) < density
    if nb >= 3:
        m[1, :] = False          # a block row that sees no key
        m[:, 2] = False          # a key block no row sees
    return m


SMALL = [
    # B, Hq, Hkv, N, d, causal, density
    (1, 2, 2, 1024, 128, False, 0.5),
    (1, 4, 2, 1000, 64, False, 0.4),
    (2, 2, 1, 777, 128, True, 0.6),
    (1, 3, 3, 1300, 64, True, 0.5),
    (1, 2, 2, 300, 128, False, 1.0),
    (1, 4, 4, 2048, 128, False, 0.3),
    (1, 2, 1, 1537, 128, True, 0.7),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}H{}x{}N{}d{}c{}p{}".format(*s))
def test_bsparse_small_shapes(fa, dev, shape):
    B, Hq, Hkv, N, d, causal, density = shape
    nb = (N + BS - 1) // BS
    mask = random_mask(nb, density, 900 + N)
    scale = 1.0 / np.sqrt(d)
    seed = 6000 + N
    q = I.random_tensor(seed, (B, Hq, N, d), "bf16", tensor_id=0)
    k = I.random_tensor(seed, (B, Hkv, N, d), "bf16", tensor_id=1)
    v = I.random_tensor(seed, (B, Hkv, N, d), "bf16", tensor_id=2)
    do = I.random_tensor(seed, (B, Hq, N, d), "bf16", tensor_id=3)
    print(f"case {shape}", flush=True)
    layout = fa.BlockSparseLayout(mask, causal=causal, device=dev)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.fwd_bsparse(qd, kd, vd, layout, causal, scale)
    dq, dk, dv, _ = fa.bwd_bsparse(qd, kd, vd, o, dod, lse, layout, causal, scale)
    torch.cuda.synchronize()
    Q, K, V, dO = (f64(t) for t in (q, k, v, do))
    bm = oracle.BlockMask(mask, BS)
    O, L = oracle.forward(Q, K, V, causal, scale, window=bm)
    rq, rk, rv, _ = oracle.backward(Q, K, V, dO, causal, scale, window=bm)
    check(f64(o), f64(lse), [f64(x) for x in (dq, dk, dv)], O, L, [rq, rk, rv], str(shape))


@pytest.mark.parametrize("d", [64, 128])
def test_bsparse_dilated_block_window(fa, dev, d):
    """A dilated causal window at block granularity: row block r sees key blocks r, r-2, r-4, r-6 (and within
    the diagonal block only keys j <= i)."""
    B, Hq, Hkv, N = 1, 4, 2, 2000
    nb = (N + BS - 1) // BS
    r = np.arange(nb)
    off = r[:, None] - r[None, :]
    mask = (off >= 0) & (off < 8) & (off % 2 == 0)
    scale = 1.0 / np.sqrt(d)
    q, k, v, do = (I.random_tensor(93 + d, (B, H, N, d), "bf16", tensor_id=t) for t, H in enumerate((Hq, Hkv, Hkv, Hq)))
    layout = fa.BlockSparseLayout(mask, causal=True, device=dev)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.fwd_bsparse(qd, kd, vd, layout, True, scale)
    dq, dk, dv, _ = fa.bwd_bsparse(qd, kd, vd, o, dod, lse, layout, True, scale)
    torch.cuda.synchronize()
    Q, K, V, dO = (f64(t) for t in (q, k, v, do))
    bm = oracle.BlockMask(mask, BS)
    O, L = oracle.forward(Q, K, V, True, scale, window=bm)
    rq, rk, rv, _ = oracle.backward(Q, K, V, dO, True, scale, window=bm)
    check(f64(o), f64(lse), [f64(x) for x in (dq, dk, dv)], O, L, [rq, rk, rv], f"dilated d={d}")


@pytest.mark.parametrize("causal", [False, True])
def test_bsparse_full_mask_is_dense(fa, dev, causal):
    """Every block on: the same tiles in the same order as the dense kernels, bit for bit."""
    B, Hq, Hkv, N, d = 1, 4, 2, 1100, 128
    q, k, v, do = (I.random_tensor(91, (B, H, N, d), "bf16", tensor_id=t).to(dev)
                   for t, H in enumerate((Hq, Hkv, Hkv, Hq)))
    nb = (N + BS - 1) // BS
    layout = fa.BlockSparseLayout(np.ones((nb, nb), bool), causal=causal, device=dev)
    o, lse = fa.fwd_bsparse(q, k, v, layout, causal, 0.1)
    oc, lc = fa.fwd(q, k, v, causal, 0.1)
    g = fa.bwd_bsparse(q, k, v, o, do, lse, layout, causal, 0.1)[:3]
    gc = fa.bwd(q, k, v, oc, do, lc, causal, 0.1)[:3]
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(lse, lc)
    for a, b in zip(g, gc):
        assert torch.equal(a, b)


def test_bsparse_empty_mask(fa, dev):
    """No block on: O = 0, LSE = -inf, every gradient 0."""
    B, Hq, Hkv, N, d = 1, 2, 2, 600, 64
    q, k, v, do = (I.random_tensor(92, (B, H, N, d), "bf16", tensor_id=t).to(dev)
                   for t, H in enumerate((Hq, Hkv, Hkv, Hq)))
    layout = fa.BlockSparseLayout(np.zeros((3, 3), bool), device=dev)
    assert layout.nnz == 0
    o, lse = fa.fwd_bsparse(q, k, v, layout, False, 0.1)
    dq, dk, dv, _ = fa.bwd_bsparse(q, k, v, o, do, lse, layout, False, 0.1)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    for g in (dq, dk, dv):
        assert torch.all(g == 0)


@pytest.mark.timeout(600)
def test_bsparse_workload_sampled(fa, dev):
    """The 16K-token block-sparse workload bench.py times: sampled rows of four heads and the key columns of two
    K/V heads against the oracle; a second forward is bitwise the first."""
    w, pat = I.BSPARSE_WORKLOADS["bsparse_bf16_n16384"]
    nb = (w.N + BS - 1) // BS
    mask = I.block_pattern(nb, **pat)
    q, k, v, do = (I.full_tensor(w, t) for t in range(4))
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    layout = fa.BlockSparseLayout(mask, device=dev)
    o, lse = fa.fwd_bsparse(qd, kd, vd, layout, False, w.scale)
    dq, dk, dv, _ = fa.bwd_bsparse(qd, kd, vd, o, dod, lse, layout, False, w.scale)
    o2, lse2 = fa.fwd_bsparse(qd, kd, vd, layout, False, w.scale)
    torch.cuda.synchronize()
    print("gpu done", flush=True)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    bm = oracle.BlockMask(mask, BS)
    G = w.Hq // w.Hkv
    rows = I.sample_rows(w.N)
    got = {n: [] for n in ("O", "L", "dQ", "dK", "dV")}
    ref = {n: [] for n in got}
    for h in (0, G - 1, G, w.Hq - 1):
        g = h // G
        dQr, Or, Lr, _ = oracle.head_rows_backward_dq(f64(q[0, h]), f64(k[0, g]), f64(v[0, g]), f64(do[0, h]),
                                                      rows, False, w.scale, window=bm)
        got["O"].append(f64(o[0, h, rows])); ref["O"].append(Or)
        got["L"].append(f64(lse[0, h, rows])); ref["L"].append(Lr)
        got["dQ"].append(f64(dq[0, h, rows])); ref["dQ"].append(dQr)
    for g in (0, w.Hkv - 1):
        hs = range(g * G, (g + 1) * G)
        stats = [oracle.head_full_stats(f64(q[0, h]), f64(k[0, g]), f64(v[0, g]), f64(do[0, h]), False, w.scale,
                                        window=bm) for h in hs]
        dKc, dVc = oracle.head_cols_backward_dkdv([f64(q[0, h]) for h in hs], f64(k[0, g]), f64(v[0, g]),
                                                 [f64(do[0, h]) for h in hs], stats, rows, False, w.scale, window=bm)
        got["dK"].append(f64(dk[0, g, rows])); ref["dK"].append(dKc)
        got["dV"].append(f64(dv[0, g, rows])); ref["dV"].append(dVc)
    c = lambda d_: {n: np.concatenate(x) for n, x in d_.items()}
    G_, R_ = c(got), c(ref)
    check(G_["O"], G_["L"], [G_["dQ"], G_["dK"], G_["dV"]], R_["O"], R_["L"], [R_["dQ"], R_["dK"], R_["dV"]],
          "N16384 block-sparse")


SPLIT = [
    # B, Hq, Hkv, N, d, causal, split, global rows/cols
    (1, 4, 2, 2560, 128, False, 2, 1),
    (1, 2, 2, 2000, 64, False, 3, 2),
    (2, 2, 1, 1800, 128, True, 2, 1),
    (1, 3, 3, 1537, 64, True, 2, 2),
    (1, 4, 1, 3000, 128, False, 5, 1),
]


def global_mask(nb, n_global, seed):
    m = I.block_pattern(nb, band=1, n_global=n_global, n_random=1, seed=seed)
    if nb >= 6:
        m[nb - 2, :] = False     # a block row that sees no key (not a global one)
    return m


@pytest.mark.parametrize("shape", SPLIT, ids=lambda s: "B{}H{}x{}N{}d{}c{}s{}g{}".format(*s))
def test_bsparse_split_small(fa, dev, shape):
    """Masks with global block rows and columns run through the work split (rows and columns longer than
    `split` blocks cut into items whose partials are merged) against the oracle."""
    B, Hq, Hkv, N, d, causal, split, ng = shape
    nb = (N + BS - 1) // BS
    mask = global_mask(nb, ng, 40 + N)
    scale = 1.0 / np.sqrt(d)
    q, k, v, do = (I.random_tensor(4100 + N, (B, H, N, d), "bf16", tensor_id=t) for t, H in enumerate((Hq, Hkv, Hkv, Hq)))
    print(f"case {shape}", flush=True)
    layout = fa.BlockSparseLayout(mask, causal=causal, device=dev, split=split)
    assert layout.n_row_slots > 0 and layout.n_col_slots > 0
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.fwd_bsparse(qd, kd, vd, layout, causal, scale)
    dq, dk, dv, _ = fa.bwd_bsparse(qd, kd, vd, o, dod, lse, layout, causal, scale)
    torch.cuda.synchronize()
    Q, K, V, dO = (f64(t) for t in (q, k, v, do))
    bm = oracle.BlockMask(mask, BS)
    O, L = oracle.forward(Q, K, V, causal, scale, window=bm)
    rq, rk, rv, _ = oracle.backward(Q, K, V, dO, causal, scale, window=bm)
    check(f64(o), f64(lse), [f64(x) for x in (dq, dk, dv)], O, L, [rq, rk, rv], f"split {shape}")


def test_bsparse_split_matches_plain(fa, dev):
    """The same mask with and without the work split: the same tiles in another grouping, so the outputs agree
    to float32 summation order (compared at a quarter of the bf16 tolerances); the split forward is
    bitwise reproducible."""
    B, Hq, Hkv, N, d = 1, 8, 2, 4096, 128
    mask = global_mask(16, 1, 77)
    q, k, v, do = (I.random_tensor(4200, (B, H, N, d), "bf16", tensor_id=t).to(dev) for t, H in enumerate((Hq, Hkv, Hkv, Hq)))
    plain = fa.BlockSparseLayout(mask, device=dev, split=16)
    cut = fa.BlockSparseLayout(mask, device=dev, split=3)
    assert plain.n_row_slots == plain.n_col_slots == 0 and cut.n_row_slots > 0
    o1, l1 = fa.fwd_bsparse(q, k, v, plain, False, 0.09)
    o2, l2 = fa.fwd_bsparse(q, k, v, cut, False, 0.09)
    o3, l3 = fa.fwd_bsparse(q, k, v, cut, False, 0.09)
    g1 = fa.bwd_bsparse(q, k, v, o1, do, l1, plain, False, 0.09)[:3]
    g2 = fa.bwd_bsparse(q, k, v, o1, do, l1, cut, False, 0.09)[:3]
    torch.cuda.synchronize()
    assert torch.equal(o2, o3) and torch.equal(l2, l3)
    empty = torch.isneginf(l1)                                 # the block row that sees no key
    assert torch.equal(empty, torch.isneginf(l2)) and bool(empty.any())
    eo = float((o1.float() - o2.float()).abs().max())
    el = float((l1[~empty] - l2[~empty]).abs().max())
    errs = [rel_l2(f64(a), f64(b)) for a, b in zip(g2, g1)]
    print(f"split vs plain: O {eo:.3e}  LSE {el:.3e}  dQ/dK/dV rel-L2 {errs}", flush=True)
    assert eo <= O_TOL / 4 and el <= LSE_TOL / 4 and max(errs) <= REL_TOL / 4


@pytest.mark.timeout(600)
def test_bsparse_global_workload_sampled(fa, dev):
    """The 16K-token mask with one global block row and column (the split bench leg): sampled rows of four
    heads, among them the global row block, and key columns of two K/V heads, among them the global key
    block, against the oracle."""
    w, pat = I.BSPARSE_WORKLOADS["bsparse_global_bf16_n16384"]
    nb = (w.N + BS - 1) // BS
    mask = I.block_pattern(nb, **pat)
    q, k, v, do = (I.full_tensor(w, t) for t in range(4))
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    layout = fa.BlockSparseLayout(mask, device=dev)
    assert layout.n_row_slots > 0 and layout.n_col_slots > 0
    o, lse = fa.fwd_bsparse(qd, kd, vd, layout, False, w.scale)
    dq, dk, dv, _ = fa.bwd_bsparse(qd, kd, vd, o, dod, lse, layout, False, w.scale)
    torch.cuda.synchronize()
    print("gpu done", flush=True)
    bm = oracle.BlockMask(mask, BS)
    G = w.Hq // w.Hkv
    rows = np.unique(np.concatenate([I.sample_rows(w.N), np.arange(0, 256, 37), [255]]))
    got = {n: [] for n in ("O", "L", "dQ", "dK", "dV")}
    ref = {n: [] for n in got}
    for h in (0, G - 1, G, w.Hq - 1):
        g = h // G
        dQr, Or, Lr, _ = oracle.head_rows_backward_dq(f64(q[0, h]), f64(k[0, g]), f64(v[0, g]), f64(do[0, h]),
                                                      rows, False, w.scale, window=bm)
        got["O"].append(f64(o[0, h, rows])); ref["O"].append(Or)
        got["L"].append(f64(lse[0, h, rows])); ref["L"].append(Lr)
        got["dQ"].append(f64(dq[0, h, rows])); ref["dQ"].append(dQr)
    for g in (0, w.Hkv - 1):
        hs = range(g * G, (g + 1) * G)
        stats = [oracle.head_full_stats(f64(q[0, h]), f64(k[0, g]), f64(v[0, g]), f64(do[0, h]), False, w.scale,
                                        window=bm) for h in hs]
        dKc, dVc = oracle.head_cols_backward_dkdv([f64(q[0, h]) for h in hs], f64(k[0, g]), f64(v[0, g]),
                                                 [f64(do[0, h]) for h in hs], stats, rows, False, w.scale, window=bm)
        got["dK"].append(f64(dk[0, g, rows])); ref["dK"].append(dKc)
        got["dV"].append(f64(dv[0, g, rows])); ref["dV"].append(dVc)
        print(f"cols of kv head {g} done", flush=True)
    c = lambda d_: {n: np.concatenate(x) for n, x in d_.items()}
    G_, R_ = c(got), c(ref)
    check(G_["O"], G_["L"], [G_["dQ"], G_["dK"], G_["dV"]], R_["O"], R_["L"], [R_["dQ"], R_["dK"], R_["dV"]],
          "N16384 global row and column, split")


@pytest.mark.parametrize("d", [64, 128])
def test_bsparse_causal_raw_layout_above_diagonal(fa, dev, d):
    """A layout that is not trimmed to the lower triangle, run with causal = 1: blocks above the diagonal are
    listed (their keys are all masked), and row block 1 lists only such blocks, so its rows see no key
    (O = 0, LSE = -inf, no gradient).  Compared with the oracle's block mask with the causal mask."""
    B, Hq, Hkv, N = 1, 4, 2, 1100
    nb = (N + BS - 1) // BS
    mask = np.zeros((nb, nb), bool)
    for r, cols in {0: (0, 3), 1: (2, 4), 2: (0, 2, 3), 3: (1, 4), 4: (0, 1, 2, 3, 4)}.items():
        mask[r, list(cols)] = True
    scale = 1.0 / np.sqrt(d)
    q, k, v, do = (I.random_tensor(97 + d, (B, H, N, d), "bf16", tensor_id=t) for t, H in enumerate((Hq, Hkv, Hkv, Hq)))
    layout = fa.BlockSparseLayout(mask, causal=False, device=dev)      # not trimmed: upper blocks stay listed
    assert layout.nnz == int(mask.sum())
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.fwd_bsparse(qd, kd, vd, layout, True, scale)
    dq, dk, dv, _ = fa.bwd_bsparse(qd, kd, vd, o, dod, lse, layout, True, scale)
    torch.cuda.synchronize()
    Q, K, V, dO = (f64(t) for t in (q, k, v, do))
    bm = oracle.BlockMask(mask, BS)
    O, L = oracle.forward(Q, K, V, True, scale, window=bm)
    rq, rk, rv, _ = oracle.backward(Q, K, V, dO, True, scale, window=bm)
    assert np.all(np.isneginf(L[:, :, BS:2 * BS]))                      # row block 1 sees nothing
    check(f64(o), f64(lse), [f64(x) for x in (dq, dk, dv)], O, L, [rq, rk, rv], f"raw causal layout d={d}")
