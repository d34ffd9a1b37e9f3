"""Pins of the oracle's attention dropout (oracle/dropout.py), CPU only.

- Philox4x32-10 against the generator's published known-answer vectors
  (Random123 distribution, "kat_vectors": counters and keys all zero, all
  ones, and the digits of pi).
- p = 0 reduces to the oracle's plain forward and backward.
- The drop rate of a large mask sits within 5 sigma of p' = floor(256 p) / 256,
  masks differ across heads, batch entries and seeds, each element's decision
  is one byte of the call of its 4 x 4 block, and the sixteen elements of a
  block are the sixteen bytes of one call (each threshold t = 0..255 drops
  exactly the bytes below it).
- The backward through a fixed mask matches central finite differences of
  the loss sum(dO * O) in float64.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

KAT = [  # counter (4 words), key (2 words), output (4 words)
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_philox_known_answers(ctr, key, out):
    got = oracle.philox4x32_10(ctr, key)
    assert [int(x) for x in got] == list(out)


def test_philox_vectorised_matches_scalar():
    rng = np.random.default_rng(3)
    ctr = rng.integers(0, 2 ** 32, size=(4, 7), dtype=np.uint64)
    key = rng.integers(0, 2 ** 32, size=(2,), dtype=np.uint64)
    vec = oracle.philox4x32_10(list(ctr), list(key))
    for i in range(7):
        one = oracle.philox4x32_10([int(c) for c in ctr[:, i]], [int(x) for x in key])
        assert [int(w[i]) for w in vec] == [int(x) for x in one]


def test_keep_mask_layout():
    """Element (i, j) is byte 4 (i mod 4) + (j mod 4) of Philox((j div 4, i div 4, b Hq + h, 0), seed halves),
    byte 4 w + e being bits 8 e .. 8 e + 7 of word w (scalar calls, element by element)."""
    seed, b, h, Hq = (7 << 32) | 12345, 1, 2, 4
    Z = oracle.keep_mask(b, h, Hq, np.arange(9), 10, 0.5, seed)
    thr = oracle.drop_threshold(0.5)
    for i in range(9):
        for j in range(10):
            w = oracle.philox4x32_10((j // 4, i // 4, b * Hq + h, 0), (12345, 7))[i % 4]
            assert Z[i, j] == (((int(w) >> (8 * (j % 4))) & 0xFF) >= thr)


def test_block_is_one_call():
    """The 16 decisions of a 4 x 4 block at thresholds t = 1..255 recover the call's 16 bytes: byte = the
    largest t that still keeps the element (the mask is monotone in t and each byte is used once)."""
    seed, b, h, Hq = 2 ** 40 + 3, 0, 3, 5
    rows, n_keys = np.arange(8, 12), 12                                  # block row 2
    masks = [oracle.keep_mask(b, h, Hq, rows, n_keys, t / 256.0, seed) for t in range(256)]
    for tprev, t in zip(range(255), range(1, 256)):
        assert not np.any(masks[t] & ~masks[tprev])                       # monotone
    byte = np.sum(masks, axis=0) - 1                                      # kept for t = 0..byte
    for jb in range(3):
        words = oracle.philox4x32_10((jb, 2, b * Hq + h, 0), (seed & 0xFFFFFFFF, seed >> 32))
        got = byte[:, 4 * jb:4 * jb + 4]                                  # [query offset, key offset]
        raw = bytes(np.array([int(w) for w in words], dtype="<u4").tobytes())
        assert [[raw[4 * r + e] for e in range(4)] for r in range(4)] == got.tolist()


def test_threshold_grid():
    assert oracle.drop_threshold(0.25) == 64 and oracle.drop_probability(0.25) == 0.25
    assert oracle.drop_threshold(0.3) == 76 and oracle.drop_probability(0.3) == 76 / 256
    assert oracle.drop_threshold(1 / 512) == 0 and oracle.drop_threshold(255.9 / 256) == 255
    assert np.all(oracle.keep_mask(0, 0, 2, np.arange(40), 40, 0.003, 5))        # p < 1/256: nothing dropped
    with pytest.raises(ValueError):
        oracle.drop_threshold(-0.01)


def test_drop_rate_and_independence():
    p = 0.3
    pp = oracle.drop_probability(p)
    Z = oracle.keep_mask(0, 0, 8, np.arange(512), 512, p, 99)
    n = Z.size
    rate = 1.0 - Z.mean()
    assert abs(rate - pp) < 5 * np.sqrt(pp * (1 - pp) / n)
    others = [oracle.keep_mask(0, 1, 8, np.arange(512), 512, p, 99),
              oracle.keep_mask(1, 0, 8, np.arange(512), 512, p, 99),
              oracle.keep_mask(0, 0, 8, np.arange(512), 512, p, 100)]
    for Y in others:
        agree = np.mean(Y == Z)
        expect = pp * pp + (1 - pp) * (1 - pp)             # two independent masks agree this often
        assert abs(agree - expect) < 5 * np.sqrt(expect * (1 - expect) / n)
    assert np.all(oracle.keep_mask(0, 0, 8, np.arange(64), 64, 0.0, 5))
    with pytest.raises(ValueError):
        oracle.drop_threshold(1.0)


@pytest.mark.parametrize("causal", [False, True])
def test_p_zero_is_plain_attention(causal):
    rng = np.random.default_rng(11)
    q, do = rng.standard_normal((2, 1, 4, 9, 8))
    k, v = rng.standard_normal((2, 1, 2, 9, 8))
    O, L = oracle.forward_dropout(q, k, v, causal, 0.3, 0.0, 1)
    O0, L0 = oracle.forward(q, k, v, causal, 0.3)
    assert np.allclose(O, O0, rtol=0, atol=1e-14) and np.allclose(L, L0, rtol=0, atol=1e-14)
    g = oracle.backward_dropout(q, k, v, do, causal, 0.3, 0.0, 1)
    g0 = oracle.backward(q, k, v, do, causal, 0.3)
    for a, b in zip(g[:3], g0[:3]):
        assert np.allclose(a, b, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_backward_finite_differences(causal):
    """Gradients of sum(dO * O) through a fixed mask (p = 0.4) against central differences."""
    rng = np.random.default_rng(21)
    B, Hq, Hkv, N, d, scale, p, seed = 1, 2, 1, 6, 3, 0.7, 0.4, 42
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    do = rng.standard_normal((B, Hq, N, d))
    dq, dk, dv, O = oracle.backward_dropout(q, k, v, do, causal, scale, p, seed)
    O_f, _ = oracle.forward_dropout(q, k, v, causal, scale, p, seed)
    assert np.allclose(O, O_f, rtol=0, atol=1e-14)
    Z = oracle.keep_mask(0, 0, Hq, np.arange(N), N, p, seed)
    assert 0 < Z.sum() < Z.size                        # the mask does drop something here

    def loss(q_, k_, v_):
        return float(np.sum(do * oracle.forward_dropout(q_, k_, v_, causal, scale, p, seed)[0]))

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v, name: xp}
            args_m = {"q": q, "k": k, "v": v, name: xm}
            num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        assert np.allclose(g, num, rtol=1e-6, atol=1e-7), name


def test_dropout_is_unbiased():
    """The mean of O over many seeds approaches the undropped O (1/(1 - p) rescale)."""
    rng = np.random.default_rng(8)
    q, k, v = rng.standard_normal((3, 1, 1, 4, 4))
    O0, _ = oracle.forward(q, k, v, False, 0.5)
    p = 0.5
    acc = np.zeros_like(O0)
    n = 4000
    for s in range(n):
        acc += oracle.forward_dropout(q, k, v, False, 0.5, p, s)[0]
    # each output is a sum of 4 terms P_ij Z_ij V_jc / (1 - p): std <= max|V| sqrt(p / (1 - p)) / sqrt(n)
    bound = 5 * np.max(np.abs(v)) * np.sqrt(p / (1 - p)) / np.sqrt(n)
    assert np.max(np.abs(acc / n - O0)) < bound
