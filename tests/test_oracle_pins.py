"""Pins of the CPU float64 oracle against what the pages and the mathematics fix.

Each test names the fact it checks.  None re-types the oracle's formula: the
checks are closed forms, invariants, central finite differences, torch's own
CPU float64 scaled_dot_product_attention (a separate library routine), and the
pages' printed memory arithmetic (tests/golden/memory_arithmetic.txt).
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, shape, sigma=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * sigma


# ---------------------------------------------------------------- V1: softmax rows

@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    q, k = rnd(1, (37, 16)), rnd(2, (37, 16))
    _, P, _, _ = oracle.probabilities(q, k, 0.25, causal)
    assert np.all(P >= 0)
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-12
    if causal:
        assert np.all(np.triu(P, 1) == 0.0)


# ---------------------------------------------------------------- V2: single key

@pytest.mark.parametrize("causal", [False, True])
def test_single_key_returns_v(causal):
    q, k, v = rnd(3, (1, 1, 1, 8)), rnd(4, (1, 1, 1, 8)), rnd(5, (1, 1, 1, 8))
    O, L = oracle.forward(q, k, v, causal, 0.7)
    assert np.array_equal(O, v)
    assert abs(L[0, 0, 0] - 0.7 * float(q[0, 0, 0] @ k[0, 0, 0])) <= 1e-14


# ---------------------------------------------------------------- V3: identical keys

@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_v(causal):
    N, d, scale = 50, 8, 0.3
    q = rnd(6, (1, 1, N, d))
    krow = rnd(7, (d,))
    k = np.broadcast_to(krow, (1, 1, N, d)).copy()
    v = rnd(8, (1, 1, N, d))
    O, L = oracle.forward(q, k, v, causal, scale)
    qk = scale * (q[0, 0] @ krow)
    if causal:
        counts = np.arange(1, N + 1)
        expect_o = np.cumsum(v[0, 0], axis=0) / counts[:, None]
        expect_l = qk + np.log(counts)
    else:
        expect_o = np.broadcast_to(v[0, 0].mean(axis=0), (N, d))
        expect_l = qk + np.log(N)
    assert np.max(np.abs(O[0, 0] - expect_o)) <= 1e-12
    assert np.max(np.abs(L[0, 0] - expect_l)) <= 1e-12


# ---------------------------------------------------------------- V4: causal row 0

def test_causal_row_zero_returns_v0():
    q, k, v = rnd(9, (2, 3, 20, 8)), rnd(10, (2, 3, 20, 8)), rnd(11, (2, 3, 20, 8))
    O, L = oracle.forward(q, k, v, True, 0.5)
    assert np.array_equal(O[:, :, 0], v[:, :, 0])
    expect = 0.5 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
    assert np.max(np.abs(L[:, :, 0] - expect)) <= 1e-14


# ---------------------------------------------------------------- V5: online == two-pass

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_online_softmax_matches_two_pass(causal, seed):
    N = 41
    q, k, v = rnd(20 + seed, (1, 2, N, 8), 3.0), rnd(30 + seed, (1, 2, N, 8), 3.0), rnd(40 + seed, (1, 2, N, 8))
    rng = np.random.default_rng(seed)
    sizes, left = [], N
    while left:
        s = int(rng.integers(1, left + 1))
        sizes.append(s)
        left -= s
    O1, L1 = oracle.forward(q, k, v, causal, 0.4)
    for blocks in (sizes, [1] * N, [N]):
        O2, L2 = oracle.forward_online(q, k, v, causal, 0.4, blocks)
        assert np.max(np.abs(O2 - O1)) <= 1e-12 * max(1.0, np.max(np.abs(O1)))
        assert np.max(np.abs(L2 - L1) / np.maximum(1.0, np.abs(L1))) <= 1e-12


# ---------------------------------------------------------------- V6: finite differences

@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_central_differences(causal):
    B, Hq, Hkv, N, d, scale = 1, 4, 2, 7, 4, 0.6
    q, k, v = rnd(50, (B, Hq, N, d)), rnd(51, (B, Hkv, N, d)), rnd(52, (B, Hkv, N, d))
    do = rnd(53, (B, Hq, N, d))

    def loss(q_, k_, v_):
        O, _ = oracle.forward(q_, k_, v_, causal, scale)
        return float(np.sum(do * O))

    dq, dk, dv, _ = oracle.backward(q, k, v, do, causal, scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        rel = np.linalg.norm(num - g) / np.linalg.norm(g)
        assert rel <= 1e-6, (name, rel)


# ---------------------------------------------------------------- V7: D identity

def test_delta_identity():
    q, k, v, do = rnd(60, (1, 2, 33, 8)), rnd(61, (1, 2, 33, 8)), rnd(62, (1, 2, 33, 8)), rnd(63, (1, 2, 33, 8))
    _, _, _, D = oracle.backward(q, k, v, do, True, 0.3)
    for h in range(2):
        _, P, _, _ = oracle.probabilities(q[0, h], k[0, h], 0.3, True)
        dP = do[0, h] @ v[0, h].T
        assert np.max(np.abs(D[0, h] - (P * dP).sum(axis=1))) <= 1e-12


# ---------------------------------------------------------------- V8: torch CPU SDPA

def _torch_reference(q, k, v, do, causal, scale):
    F = torch.nn.functional
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale,
                                       enable_gqa=tq.shape[1] != tk.shape[1])
    o.backward(torch.tensor(do, dtype=torch.float64))
    G = tq.shape[1] // tk.shape[1]
    kr = tk.detach().repeat_interleave(G, dim=1)
    s = scale * (tq.detach() @ kr.transpose(-1, -2))
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return (o.detach().numpy(), lse.numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy())


@pytest.mark.parametrize("shape,causal", [
    ((1, 2, 2, 256, 64), False),     # the tiny fp32 workload's shape
    ((2, 4, 2, 19, 8), True),
    ((1, 6, 3, 33, 16), False),
    ((1, 8, 1, 12, 4), True),
])
def test_matches_torch_cpu_float64_sdpa(shape, causal):
    B, Hq, Hkv, N, d = shape
    scale = 1.0 / np.sqrt(d)
    q, k, v, do = (rnd(70 + i, (B, H, N, d)) for i, H in enumerate((Hq, Hkv, Hkv, Hq)))
    O, L = oracle.forward(q, k, v, causal, scale)
    dq, dk, dv, _ = oracle.backward(q, k, v, do, causal, scale)
    to, tl, tdq, tdk, tdv = _torch_reference(q, k, v, do, causal, scale)
    for a, b in ((O, to), (L, tl), (dq, tdq), (dk, tdk), (dv, tdv)):
        assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(b)))


# ---------------------------------------------------------------- V9: shift invariance

def test_key_shift_invariance_large_offset():
    N, d, scale = 24, 8, 0.5
    q, k, v = rnd(80, (1, 1, N, d)), rnd(81, (1, 1, N, d)), rnd(82, (1, 1, N, d))
    w = rnd(83, (d,)) * 50.0
    O1, L1 = oracle.forward(q, k, v, False, scale)
    O2, L2 = oracle.forward(q, k + w, v, False, scale)
    assert np.max(np.abs(O2 - O1)) <= 1e-9
    shift = scale * (q[0, 0] @ w)
    assert np.max(np.abs(L2[0, 0] - (L1[0, 0] + shift))) <= 1e-9 * np.max(np.abs(shift))


# ---------------------------------------------------------------- V10: permutations

def test_permutation_equivariance():
    N, d, scale = 30, 8, 0.35
    q, k, v = rnd(90, (1, 1, N, d)), rnd(91, (1, 1, N, d)), rnd(92, (1, 1, N, d))
    pk = np.random.default_rng(93).permutation(N)
    pq = np.random.default_rng(94).permutation(N)
    O1, L1 = oracle.forward(q, k, v, False, scale)
    O2, L2 = oracle.forward(q, k[:, :, pk], v[:, :, pk], False, scale)
    assert np.max(np.abs(O2 - O1)) <= 1e-13 and np.max(np.abs(L2 - L1)) <= 1e-13
    O3, L3 = oracle.forward(q[:, :, pq], k, v, False, scale)
    assert np.max(np.abs(O3 - O1[:, :, pq])) <= 1e-13 and np.max(np.abs(L3 - L1[:, :, pq])) <= 1e-13


# ---------------------------------------------------------------- V11: grouped heads

@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_repeated_mha(causal):
    B, Hq, Hkv, N, d, scale = 2, 6, 2, 15, 8, 0.3
    G = Hq // Hkv
    q, k, v, do = rnd(100, (B, Hq, N, d)), rnd(101, (B, Hkv, N, d)), rnd(102, (B, Hkv, N, d)), rnd(103, (B, Hq, N, d))
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    O1, L1 = oracle.forward(q, k, v, causal, scale)
    O2, L2 = oracle.forward(q, kr, vr, causal, scale)
    assert np.max(np.abs(O1 - O2)) <= 1e-14 and np.max(np.abs(L1 - L2)) <= 1e-14
    dq1, dk1, dv1, _ = oracle.backward(q, k, v, do, causal, scale)
    dq2, dk2, dv2, _ = oracle.backward(q, kr, vr, do, causal, scale)
    assert np.max(np.abs(dq1 - dq2)) <= 1e-13
    assert np.max(np.abs(dk1 - dk2.reshape(B, Hkv, G, N, d).sum(axis=2))) <= 1e-12
    assert np.max(np.abs(dv1 - dv2.reshape(B, Hkv, G, N, d).sum(axis=2))) <= 1e-12


# ---------------------------------------------------------------- sampled forms == full forms

@pytest.mark.parametrize("causal", [False, True])
def test_sampled_rows_and_columns_match_full(causal):
    B, Hq, Hkv, N, d, scale = 1, 4, 2, 300, 16, 0.25
    G = Hq // Hkv
    q, k, v, do = rnd(110, (B, Hq, N, d)), rnd(111, (B, Hkv, N, d)), rnd(112, (B, Hkv, N, d)), rnd(113, (B, Hq, N, d))
    O, L = oracle.forward(q, k, v, causal, scale)
    dq, dk, dv, D = oracle.backward(q, k, v, do, causal, scale)
    rows = np.array([0, 1, 5, 128, 255, 256, 299])
    for h in range(Hq):
        g = h // G
        Or, Lr = oracle.head_rows_forward(q[0, h], k[0, g], v[0, g], rows, causal, scale)
        assert np.max(np.abs(Or - O[0, h, rows])) <= 1e-13
        assert np.max(np.abs(Lr - L[0, h, rows])) <= 1e-13
        dQr, _, _, Dr = oracle.head_rows_backward_dq(q[0, h], k[0, g], v[0, g], do[0, h], rows, causal, scale)
        assert np.max(np.abs(dQr - dq[0, h, rows])) <= 1e-12
        assert np.max(np.abs(Dr - D[0, h, rows])) <= 1e-12
    for g in range(Hkv):
        hs = range(g * G, (g + 1) * G)
        stats = [oracle.head_full_stats(q[0, h], k[0, g], v[0, g], do[0, h], causal, scale) for h in hs]
        dKc, dVc = oracle.head_cols_backward_dkdv([q[0, h] for h in hs], k[0, g], v[0, g],
                                                  [do[0, h] for h in hs], stats, rows, causal, scale)
        assert np.max(np.abs(dKc - dk[0, g, rows])) <= 1e-12
        assert np.max(np.abs(dVc - dv[0, g, rows])) <= 1e-12


# ---------------------------------------------------------------- V12: printed memory arithmetic

def test_pages_memory_arithmetic():
    lines = [ln.split("--")[0].split() for ln in open(os.path.join(GOLDEN, "memory_arithmetic.txt"))
             if ln.strip() and not ln.startswith("#")]
    assert len(lines) == 3
    for f in lines:
        if f[0] == "ratio":
            n1, n2, ratio = int(f[1]), int(f[2]), int(f[3])
            assert oracle.attention_matrix_bytes(n1, 2) == ratio * oracle.attention_matrix_bytes(n2, 2)
        else:
            n, e, rel, val = int(f[0]), int(f[1]), f[2], int(f[3])
            got = oracle.attention_matrix_bytes(n, e)
            assert (got == val) if rel == "==" else (got >= val)


# ---------------------------------------------------------------- fp8 (OCP E4M3)

def test_e4m3_decode_matches_format_definition_and_torch():
    codes = np.arange(256, dtype=np.uint8)
    d = oracle.e4m3_decode(codes)
    # format facts: largest finite 448, smallest subnormal 2^-9, smallest normal 2^-6, NaN codes
    assert np.nanmax(d) == 448.0 and d[0x7E] == 448.0
    assert d[0x01] == 2.0 ** -9 and d[0x08] == 2.0 ** -6 and d[0x38] == 1.0
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF]) and np.sum(np.isnan(d)) == 2
    t = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    ok = ~np.isnan(d)
    assert np.array_equal(d[ok], t[ok])


def test_e4m3_encode_round_trip_ties_and_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    assert np.array_equal(oracle.e4m3_encode_rne_sat(vals), codes)
    # ties go to the even mantissa: 1 + 1/16 lies halfway between 1 and 1.125
    assert oracle.e4m3_encode_rne_sat(np.array([1.0625, 1.1875]))[0] == 0x38
    assert oracle.e4m3_encode_rne_sat(np.array([1.1875]))[0] == 0x3A
    # half the smallest subnormal rounds to (signed) zero; beyond 448 saturates
    assert list(oracle.e4m3_encode_rne_sat(np.array([2.0 ** -10, -2.0 ** -10]))) == [0x00, 0x80]
    assert list(oracle.e4m3_encode_rne_sat(np.array([460.0, 1e9, -1e9]))) == [0x7E, 0x7E, 0xFE]
    x = np.random.default_rng(5).standard_normal(200000).astype(np.float32) * 60
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode_rne_sat(x), ref)


def test_quantize_per_tensor_scale_and_range():
    x = (np.random.default_rng(6).standard_normal(4096) * 3).astype(np.float32)
    codes, s = oracle.quantize_per_tensor(x)
    assert s.dtype == np.float32 and s == np.float32(np.max(np.abs(x))) / np.float32(448.0)
    back = oracle.e4m3_decode(codes) * np.float64(s)
    # E4M3 keeps 3 mantissa bits: normal values carry relative error at most 2^-4
    big = np.abs(x) > 2.0 ** -6 * s
    assert np.max(np.abs(back[big] - x[big]) / np.abs(x[big])) <= 2.0 ** -4 + 1e-7
    assert np.max(np.abs(oracle.e4m3_decode(codes))) == 448.0
    z, sz = oracle.quantize_per_tensor(np.zeros(8, np.float32))
    assert sz == np.float32(2.0 ** -120) / np.float32(448.0) and not z.any()


# ---------------------------------------------------------------- decode against a KV cache

DECODE_SHAPES = [  # B, Hq, Hkv, Nq, Nk, d
    (1, 8, 1, 1, 40, 8),
    (2, 4, 2, 3, 17, 4),
    (1, 6, 3, 5, 5, 16),
    (1, 2, 2, 7, 30, 8),
]


@pytest.mark.parametrize("shape", DECODE_SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_decode_matches_torch_cpu_float64_sdpa(shape, causal):
    """New rows at the end of the sequence: torch SDPA with an explicit bottom-right mask, and torch.logsumexp."""
    B, Hq, Hkv, Nq, Nk, d = shape
    scale = 1.0 / np.sqrt(d)
    q, k, v = rnd(90, (B, Hq, Nq, d)), rnd(91, (B, Hkv, Nk, d)), rnd(92, (B, Hkv, Nk, d))
    O, L = oracle.decode_forward(q, k, v, causal, scale)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64) for x in (q, k, v))
    mask = None
    if causal:
        mask = torch.arange(Nk)[None, :] <= torch.arange(Nk - Nq, Nk)[:, None]
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale,
                                                          enable_gqa=Hq != Hkv)
    s = scale * (tq @ tk.repeat_interleave(Hq // Hkv, dim=1).transpose(-1, -2))
    if causal:
        s = s.masked_fill(~mask, float("-inf"))
    tl = torch.logsumexp(s, dim=-1)
    assert np.max(np.abs(O - to.numpy())) <= 1e-12
    assert np.max(np.abs(L - tl.numpy())) <= 1e-12 * max(1.0, float(tl.abs().max()))


@pytest.mark.parametrize("causal", [False, True])
def test_decode_equals_last_rows_of_full_attention(causal):
    """Decoding the last Nq rows against the whole sequence's cache gives those rows of full attention."""
    B, Hq, Hkv, N, d, Nq = 1, 4, 2, 23, 8, 6
    q, k, v = rnd(95, (B, Hq, N, d)), rnd(96, (B, Hkv, N, d)), rnd(97, (B, Hkv, N, d))
    O, L = oracle.forward(q, k, v, causal, 0.4)
    Od, Ld = oracle.decode_forward(q[:, :, N - Nq:], k, v, causal, 0.4)
    assert np.max(np.abs(Od - O[:, :, N - Nq:])) <= 1e-12
    assert np.max(np.abs(Ld - L[:, :, N - Nq:])) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_decode_identical_keys_and_single_key(causal):
    """Identical cache keys: O_i = mean of the visible V rows, LSE_i = scale q_i.k + ln(count); one key returns V."""
    Hq, Nq, Nk, d, scale = 3, 4, 11, 5, 0.7
    q, v = rnd(98, (1, Hq, Nq, d)), rnd(99, (1, 1, Nk, d))
    krow = rnd(100, (d,))
    k = np.broadcast_to(krow, (1, 1, Nk, d)).copy()
    O, L = oracle.decode_forward(q, k, v, causal, scale)
    for i in range(Nq):
        cnt = Nk - Nq + i + 1 if causal else Nk
        assert np.max(np.abs(O[0, :, i] - v[0, 0, :cnt].mean(axis=0))) <= 1e-12
        assert np.max(np.abs(L[0, :, i] - (scale * q[0, :, i] @ krow + np.log(cnt)))) <= 1e-12
    O1, L1 = oracle.decode_forward(q[:, :, :1], k[:, :, :1], v[:, :, :1], causal, scale)
    assert np.max(np.abs(O1[0, :, 0] - v[0, 0, 0])) <= 1e-15
    assert np.max(np.abs(L1[0, :, 0] - scale * q[0, :, 0] @ krow)) <= 1e-12


# ---------------------------------------------------------------- sliding window (local attention)

@pytest.mark.parametrize("window", [1, 3, 7, 19, 100])
def test_local_matches_torch_cpu_float64_sdpa_with_band_mask(window):
    """Causal sliding window: torch SDPA + autograd with an explicit band mask (i - W < j <= i)."""
    B, Hq, Hkv, N, d = 1, 4, 2, 19, 8
    scale = 1.0 / np.sqrt(d)
    q, k, v, do = (rnd(110 + i, (B, H, N, d)) for i, H in enumerate((Hq, Hkv, Hkv, Hq)))
    O, L = oracle.forward(q, k, v, True, scale, window=window)
    dq, dk, dv, _ = oracle.backward(q, k, v, do, True, scale, window=window)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    i, j = torch.arange(N)[:, None], torch.arange(N)[None, :]
    band = (j <= i) & (j > i - window)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=band, scale=scale, enable_gqa=True)
    o.backward(torch.tensor(do, dtype=torch.float64))
    s = scale * (tq.detach() @ tk.detach().repeat_interleave(Hq // Hkv, dim=1).transpose(-1, -2))
    tl = torch.logsumexp(s.masked_fill(~band, float("-inf")), dim=-1)
    for a, b in ((O, o.detach()), (L, tl), (dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(a - b.numpy())) <= 1e-12 * max(1.0, float(b.abs().max()))


def test_local_window_limits():
    """W >= N is plain causal attention; W = 1 lets each row see itself only (O_i = V_i, LSE_i = scale q_i.k_i)."""
    B, Hq, Hkv, N, d, scale = 1, 2, 1, 13, 6, 0.4
    q, k, v, do = (rnd(120 + i, (B, H, N, d)) for i, H in enumerate((Hq, Hkv, Hkv, Hq)))
    for W in (N, N + 5):
        Ow, Lw = oracle.forward(q, k, v, True, scale, window=W)
        Oc, Lc = oracle.forward(q, k, v, True, scale)
        assert np.max(np.abs(Ow - Oc)) <= 1e-15 and np.max(np.abs(Lw - Lc)) <= 1e-15
    O1, L1 = oracle.forward(q, k, v, True, scale, window=1)
    for h in range(Hq):
        assert np.max(np.abs(O1[0, h] - v[0, 0])) <= 1e-15
        assert np.max(np.abs(L1[0, h] - scale * (q[0, h] * k[0, 0]).sum(axis=1))) <= 1e-12
    dq1, dk1, dv1, _ = oracle.backward(q, k, v, do, True, scale, window=1)
    # one visible key: the softmax is constant 1, so dQ = dK = 0 and dV_j = sum over heads of dO_j
    assert np.max(np.abs(dq1)) <= 1e-15 and np.max(np.abs(dk1)) <= 1e-15
    assert np.max(np.abs(dv1[0, 0] - do[0].sum(axis=0))) <= 1e-12


def test_local_backward_matches_central_differences():
    B, Hq, Hkv, N, d, scale, W = 1, 2, 1, 9, 4, 0.6, 4
    q, k, v, do = (rnd(130 + i, (B, H, N, d)) for i, H in enumerate((Hq, Hkv, Hkv, Hq)))
    dq, dk, dv, _ = oracle.backward(q, k, v, do, True, scale, window=W)
    loss = lambda q_, k_, v_: float((oracle.forward(q_, k_, v_, True, scale, window=W)[0] * do).sum())
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.linalg.norm(num - g) <= 1e-6 * np.linalg.norm(g)


def test_local_sampled_rows_and_columns_match_full():
    B, Hq, Hkv, N, d, scale, W = 1, 2, 1, 40, 8, 0.3, 11
    q, k, v, do = (rnd(140 + i, (B, H, N, d)) for i, H in enumerate((Hq, Hkv, Hkv, Hq)))
    dq, dk, dv, _ = oracle.backward(q, k, v, do, True, scale, window=W)
    O, L = oracle.forward(q, k, v, True, scale, window=W)
    rows = np.array([0, 5, 10, 11, 39])
    dQr, Or, Lr, _ = oracle.head_rows_backward_dq(q[0, 1], k[0, 0], v[0, 0], do[0, 1], rows, True, scale, window=W)
    assert np.max(np.abs(dQr - dq[0, 1, rows])) <= 1e-12 and np.max(np.abs(Or - O[0, 1, rows])) <= 1e-12
    stats = [oracle.head_full_stats(q[0, h], k[0, 0], v[0, 0], do[0, h], True, scale, window=W) for h in range(2)]
    dKc, dVc = oracle.head_cols_backward_dkdv([q[0, 0], q[0, 1]], k[0, 0], v[0, 0], [do[0, 0], do[0, 1]], stats,
                                             rows, True, scale, window=W)
    assert np.max(np.abs(dKc - dk[0, 0, rows])) <= 1e-12 and np.max(np.abs(dVc - dv[0, 0, rows])) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_decode_paged_equals_contiguous_decode(causal):
    """A shuffled block pool read through its table gives the contiguous decode of each sequence's keys."""
    B, Hq, Hkv, Nq, d, bs = 3, 4, 2, 3, 8, 4
    lens = [9, 4, 12]
    maxb = 3
    rng = np.random.default_rng(150)
    q = rnd(151, (B, Hq, Nq, d))
    kfull, vfull = rnd(152, (B, Hkv, maxb * bs, d)), rnd(153, (B, Hkv, maxb * bs, d))
    perm = rng.permutation(B * maxb)                    # block (b, i) is stored at pool slot perm[b*maxb + i]
    kc, vc = np.zeros((B * maxb, Hkv, bs, d)), np.zeros((B * maxb, Hkv, bs, d))
    table = np.zeros((B, maxb), dtype=np.int64)
    for b in range(B):
        for i in range(maxb):
            slot = perm[b * maxb + i]
            table[b, i] = slot
            kc[slot] = kfull[b, :, i * bs:(i + 1) * bs]
            vc[slot] = vfull[b, :, i * bs:(i + 1) * bs]
    O, L = oracle.decode_paged_forward(q, kc, vc, table, lens, causal, 0.35)
    for b in range(B):
        n = lens[b]
        Ob, Lb = oracle.decode_forward(q[b:b + 1], kfull[b:b + 1, :, :n], vfull[b:b + 1, :, :n], causal, 0.35)
        assert np.max(np.abs(O[b] - Ob[0])) <= 1e-12 and np.max(np.abs(L[b] - Lb[0])) <= 1e-12


def test_decode_paged_rows_without_keys():
    """An empty sequence, and causal rows before a short sequence's first key: O = 0, LSE = -inf."""
    q = rnd(160, (2, 2, 3, 4))
    kc, vc = rnd(161, (2, 1, 4, 4)), rnd(162, (2, 1, 4, 4))
    table = np.array([[0], [1]])
    O, L = oracle.decode_paged_forward(q, kc, vc, table, [0, 2], True, 0.5)
    assert np.all(O[0] == 0) and np.all(L[0] == -np.inf)
    assert np.all(O[1, :, 0] == 0) and np.all(L[1, :, 0] == -np.inf)      # row 0 of 3 would sit at position -1
    Ob, Lb = oracle.decode_forward(q[1:2, :, 1:], kc[1:2, :, :2], vc[1:2, :, :2], True, 0.5)
    assert np.max(np.abs(O[1, :, 1:] - Ob[0])) <= 1e-12 and np.max(np.abs(L[1, :, 1:] - Lb[0])) <= 1e-12


@pytest.mark.parametrize("window,sink", [(3, 1), (5, 4), (1, 7), (8, 19)])
def test_local_with_global_tokens_matches_torch_sdpa(window, sink):
    """Window plus S leading global tokens: torch SDPA + autograd with the explicit mask (j <= i and (i - W < j or j < S))."""
    B, Hq, Hkv, N, d = 1, 2, 1, 17, 8
    scale = 1.0 / np.sqrt(d)
    q, k, v, do = (rnd(170 + i, (B, H, N, d)) for i, H in enumerate((Hq, Hkv, Hkv, Hq)))
    O, L = oracle.forward(q, k, v, True, scale, window=(window, sink))
    dq, dk, dv, _ = oracle.backward(q, k, v, do, True, scale, window=(window, sink))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    i, j = torch.arange(N)[:, None], torch.arange(N)[None, :]
    mask = (j <= i) & ((j > i - window) | (j < sink))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale, enable_gqa=True)
    o.backward(torch.tensor(do, dtype=torch.float64))
    s = scale * (tq.detach() @ tk.detach().repeat_interleave(Hq // Hkv, dim=1).transpose(-1, -2))
    tl = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
    for a, b in ((O, o.detach()), (L, tl), (dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(a - b.numpy())) <= 1e-12 * max(1.0, float(b.abs().max()))
    # S = 0 is the plain window; S >= N sees every earlier key (causal)
    O0, _ = oracle.forward(q, k, v, True, scale, window=(window, 0))
    Ow, _ = oracle.forward(q, k, v, True, scale, window=window)
    Oc, _ = oracle.forward(q, k, v, True, scale)
    On, _ = oracle.forward(q, k, v, True, scale, window=(window, N))
    assert np.max(np.abs(O0 - Ow)) <= 1e-15 and np.max(np.abs(On - Oc)) <= 1e-15


# ---------------------------------------------------------------- block-sparse masks

@pytest.mark.parametrize("causal", [False, True])
def test_block_mask_matches_torch_sdpa(causal):
    """Key j visible to query i iff mask[i // bs, j // bs] (and j <= i when causal): torch SDPA + autograd."""
    B, Hq, Hkv, N, d, bs = 1, 4, 2, 21, 8, 4
    scale = 1.0 / np.sqrt(d)
    nb = (N + bs - 1) // bs
    mask = np.random.default_rng(180).random((nb, nb)) < 0.5
    np.fill_diagonal(mask, True)                      # every row sees at least its own block
    bm = oracle.BlockMask(mask, bs)
    q, k, v, do = (rnd(181 + i, (B, H, N, d)) for i, H in enumerate((Hq, Hkv, Hkv, Hq)))
    O, L = oracle.forward(q, k, v, causal, scale, window=bm)
    dq, dk, dv, _ = oracle.backward(q, k, v, do, causal, scale, window=bm)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    i, j = torch.arange(N)[:, None], torch.arange(N)[None, :]
    m = torch.tensor(mask)[i // bs, j // bs]
    if causal:
        m &= j <= i
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale, enable_gqa=True)
    o.backward(torch.tensor(do, dtype=torch.float64))
    s = scale * (tq.detach() @ tk.detach().repeat_interleave(Hq // Hkv, dim=1).transpose(-1, -2))
    tl = torch.logsumexp(s.masked_fill(~m, float("-inf")), dim=-1)
    for a, b in ((O, o.detach()), (L, tl), (dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(a - b.numpy())) <= 1e-12 * max(1.0, float(b.abs().max()))
    # all blocks on: plain attention
    On, Ln = oracle.forward(q, k, v, causal, scale, window=oracle.BlockMask(np.ones((nb, nb), bool), bs))
    Op, Lp = oracle.forward(q, k, v, causal, scale)
    assert np.max(np.abs(On - Op)) <= 1e-15 and np.max(np.abs(Ln - Lp)) <= 1e-15


def test_block_mask_rows_without_keys():
    """A query block with no visible block: O = 0, LSE = -inf, dQ = 0, and its dO reaches no dK or dV."""
    B, H, N, d, bs = 1, 1, 12, 4, 4
    mask = np.ones((3, 3), bool)
    mask[1, :] = False                                  # rows 4..7 see nothing
    bm = oracle.BlockMask(mask, bs)
    q, k, v, do = (rnd(190 + i, (B, H, N, d)) for i in range(4))
    O, L = oracle.forward(q, k, v, False, 0.5, window=bm)
    dq, dk, dv, _ = oracle.backward(q, k, v, do, False, 0.5, window=bm)
    assert np.all(O[0, 0, 4:8] == 0) and np.all(np.isneginf(L[0, 0, 4:8]))
    assert np.all(dq[0, 0, 4:8] == 0)
    do2 = do.copy()
    do2[0, 0, 4:8] += 5.0                               # the masked rows' output gradient changes nothing
    dq2, dk2, dv2, _ = oracle.backward(q, k, v, do2, False, 0.5, window=bm)
    assert np.max(np.abs(dk2 - dk)) <= 1e-12 and np.max(np.abs(dv2 - dv)) <= 1e-12
    rows = np.array([0, 5, 11])
    stats = [oracle.head_full_stats(q[0, 0], k[0, 0], v[0, 0], do[0, 0], False, 0.5, window=bm)]
    dKc, dVc = oracle.head_cols_backward_dkdv([q[0, 0]], k[0, 0], v[0, 0], [do[0, 0]], stats, rows, False, 0.5,
                                             window=bm)
    assert np.max(np.abs(dKc - dk[0, 0, rows])) <= 1e-12 and np.max(np.abs(dVc - dv[0, 0, rows])) <= 1e-12
