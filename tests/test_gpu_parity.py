"""GPU parity: the HIP path (through the C ABI) against the CPU float64 oracle.

Tolerances (written here, per the workload definitions):
  fp32      : max |err| <= 1e-5 on O and LSE, <= 1e-4 on dQ, dK, dV
  bf16      : max |err| <= 2e-2 on O, <= 1e-2 on LSE, relative L2 <= 2e-2 on dQ, dK, dV
  fp8 (E4M3): relative L2 <= 6e-2 on O (oracle on the unquantised bf16 inputs)
Relative L2 is ||x - y|| / ||y|| over every compared element of one tensor
(y = oracle).  Small shapes are compared element by element in full; the full
workloads are compared on sampled (batch, head, row) slices and sampled key
columns, computed by the oracle one by one from full rows of P.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_50_amd import inputs as I

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(o=1e-5, lse=1e-5, grad_abs=1e-4), "bf16": dict(o=2e-2, lse=1e-2, grad_rel=2e-2)}


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


def check(dtype, o, lse, O, L, grads=None, ref_grads=None, tag=""):
    tol = TOL[dtype]
    eo, el = float(np.max(np.abs(o - O))), float(np.max(np.abs(lse - L)))
    print(f"[{tag}] O max|err| {eo:.3e}  LSE max|err| {el:.3e}", flush=True)
    assert eo <= tol["o"], (tag, "O", eo)
    assert el <= tol["lse"], (tag, "LSE", el)
    if grads is None:
        return
    for name, g, r in zip(("dQ", "dK", "dV"), grads, ref_grads):
        if dtype == "f32":
            e = float(np.max(np.abs(g - r)))
            print(f"[{tag}] {name} max|err| {e:.3e}", flush=True)
            assert e <= tol["grad_abs"], (tag, name, e)
        elif not np.any(r):
            # an exactly zero gradient (one key: the softmax over a single key
            # does not depend on it, so dK = 0) has no relative error; the
            # absolute bound of the float32 path applies instead
            e = float(np.max(np.abs(g)))
            print(f"[{tag}] {name} max|err| {e:.3e} (zero reference)", flush=True)
            assert e <= TOL["f32"]["grad_abs"], (tag, name, e)
        else:
            e = rel_l2(g, r)
            print(f"[{tag}] {name} rel-L2 {e:.3e}", flush=True)
            assert e <= tol["grad_rel"], (tag, name, e)


def run(fa, dev, q, k, v, do, causal, scale):
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal, scale)
    dq, dk, dv, _ = fa.bwd(qd, kd, vd, o, dod, lse, causal, scale)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


SMALL = [
    # B, Hq, Hkv, N, d, causal, dtype
    (1, 1, 1, 1, 64, False, "bf16"),
    (1, 1, 1, 1, 128, True, "bf16"),
    (1, 2, 1, 5, 64, True, "bf16"),
    (1, 2, 2, 63, 128, False, "bf16"),
    (2, 2, 2, 64, 64, True, "bf16"),
    (1, 3, 3, 65, 128, True, "bf16"),
    (1, 2, 2, 127, 64, False, "bf16"),
    (1, 4, 2, 129, 128, True, "bf16"),
    (2, 4, 1, 200, 64, True, "bf16"),
    (1, 8, 2, 257, 128, False, "bf16"),
    (1, 2, 2, 385, 128, True, "bf16"),
    (1, 1, 1, 1, 64, True, "f32"),
    (1, 2, 1, 37, 64, True, "f32"),
    (1, 2, 2, 129, 128, False, "f32"),
    (2, 4, 2, 200, 128, True, "f32"),
    (1, 2, 2, 300, 64, True, "f32"),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B{}H{}x{}N{}d{}{}{}".format(*s[:5], "c" if s[5] else "", s[6]))
def test_small_shapes_full(fa, dev, shape):
    B, Hq, Hkv, N, d, causal, dt = shape
    scale = 1.0 / np.sqrt(d)
    seed = 1000 + N + d + Hq
    q = I.random_tensor(seed, (B, Hq, N, d), dt, tensor_id=0)
    k = I.random_tensor(seed, (B, Hkv, N, d), dt, tensor_id=1)
    v = I.random_tensor(seed, (B, Hkv, N, d), dt, tensor_id=2)
    do = I.random_tensor(seed, (B, Hq, N, d), dt, tensor_id=3)
    print(f"case {shape}", flush=True)
    o, lse, dq, dk, dv = run(fa, dev, q, k, v, do, causal, scale)
    Q, K, V, dO = (f64(t) for t in (q, k, v, do))
    O, L = oracle.forward(Q, K, V, causal, scale)
    dQ, dK, dV, _ = oracle.backward(Q, K, V, dO, causal, scale)
    check(dt, f64(o), f64(lse), O, L, [f64(x) for x in (dq, dk, dv)], [dQ, dK, dV], tag=str(shape))


def _random_shapes(n, seed=20261203):
    """n shapes drawn from a fixed seed: batch 1..3, query heads 1..8 in groups
    of 1, 2, 4 or 8 per K/V head, sequence length 1..700 (tiles and query
    blocks of every raggedness), both head sizes, causal or not, bf16 or fp32."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        G = int(rng.choice([1, 2, 4, 8]))
        Hkv = int(rng.integers(1, 3)) if G < 8 else 1
        out.append((int(rng.integers(1, 4)), G * Hkv, Hkv, int(rng.integers(1, 701)), int(rng.choice([64, 128])),
                    bool(rng.integers(0, 2)), "f32" if rng.random() < 0.25 else "bf16"))
    return out


@pytest.mark.parametrize("shape", _random_shapes(20),
                         ids=lambda s: "B{}H{}x{}N{}d{}{}{}".format(*s[:5], "c" if s[5] else "", s[6]))
def test_random_shapes_full(fa, dev, shape):
    """Forward and backward on seeded random shapes, every element against the oracle."""
    test_small_shapes_full(fa, dev, shape)


@pytest.mark.parametrize("causal", [True, False])
def test_many_items_full(fa, dev, causal):
    """More work items than resident workgroups (B=4, Hq=32, Hkv=8, N=520, d=128:
    384 query blocks and 96 key blocks of 256 rows, ragged last blocks), so the
    persistent schedule runs several rounds per workgroup; every element checked."""
    test_small_shapes_full(fa, dev, (4, 32, 8, 520, 128, causal, "bf16"))


def test_tiny_f32_workload(fa, dev):
    w = I.WORKLOADS["tiny_f32"]
    q, k, v, do = (I.full_tensor(w, t) for t in range(4))
    o, lse, dq, dk, dv = run(fa, dev, q, k, v, do, w.causal, w.scale)
    Q, K, V, dO = (f64(t) for t in (q, k, v, do))
    O, L = oracle.forward(Q, K, V, w.causal, w.scale)
    dQ, dK, dV, _ = oracle.backward(Q, K, V, dO, w.causal, w.scale)
    check("f32", f64(o), f64(lse), O, L, [f64(x) for x in (dq, dk, dv)], [dQ, dK, dV], tag="tiny_f32")


def sampled_check(fa, dev, w, kv_heads_for_cols=None, fp8=False):
    """Run the whole workload on the GPU, compare sampled slices with the oracle."""
    q, k, v, do = (I.full_tensor(w, t) for t in range(4))
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    print(f"workload {w.name}: inputs on device", flush=True)
    o, lse = fa.fwd(qd, kd, vd, w.causal, w.scale)
    dq, dk, dv, _ = fa.bwd(qd, kd, vd, o, dod, lse, w.causal, w.scale)
    torch.cuda.synchronize()
    print("gpu done", flush=True)
    G = w.Hq // w.Hkv
    rows = I.sample_rows(w.N)
    heads = I.sample_heads(w)
    got = {n: [] for n in ("O", "L", "dQ", "dK", "dV")}
    ref = {n: [] for n in ("O", "L", "dQ", "dK", "dV")}
    for (b, h) in heads:
        g = h // G
        Qh, Kg, Vg, dOh = (f64(t[b, hh]) for t, hh in ((q, h), (k, g), (v, g), (do, h)))
        dQr, Or, Lr, _ = oracle.head_rows_backward_dq(Qh, Kg, Vg, dOh, rows, w.causal, w.scale)
        got["O"].append(f64(o[b, h, rows])); ref["O"].append(Or)
        got["L"].append(f64(lse[b, h, rows])); ref["L"].append(Lr)
        got["dQ"].append(f64(dq[b, h, rows])); ref["dQ"].append(dQr)
    cols_heads = kv_heads_for_cols if kv_heads_for_cols is not None else sorted({(b, h // G) for b, h in heads})
    for (b, g) in cols_heads:
        hs = list(range(g * G, (g + 1) * G))
        Kg, Vg = f64(k[b, g]), f64(v[b, g])
        qs = [f64(q[b, h]) for h in hs]
        dos = [f64(do[b, h]) for h in hs]
        stats = [oracle.head_full_stats(qq, Kg, Vg, dd, w.causal, w.scale) for qq, dd in zip(qs, dos)]
        dKc, dVc = oracle.head_cols_backward_dkdv(qs, Kg, Vg, dos, stats, rows, w.causal, w.scale)
        got["dK"].append(f64(dk[b, g, rows])); ref["dK"].append(dKc)
        got["dV"].append(f64(dv[b, g, rows])); ref["dV"].append(dVc)
        print(f"cols of kv head {(b, g)} done", flush=True)
    cat = lambda d: {n: np.concatenate(x) for n, x in d.items()}
    G_, R_ = cat(got), cat(ref)
    check("bf16", G_["O"], G_["L"], R_["O"], R_["L"], [G_["dQ"], G_["dK"], G_["dV"]],
          [R_["dQ"], R_["dK"], R_["dV"]], tag=w.name)
    del qd, kd, vd, dod, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


@pytest.mark.timeout(300)
def test_mha_bf16_n1024_workload(fa, dev):
    sampled_check(fa, dev, I.WORKLOADS["mha_bf16_n1024"])


@pytest.mark.timeout(300)
def test_causal_bf16_n4096_workload(fa, dev):
    sampled_check(fa, dev, I.WORKLOADS["causal_bf16_n4096"])


@pytest.mark.timeout(900)
def test_gqa_bf16_n16384_workload(fa, dev):
    # key columns of the K/V heads of the sampled query heads: 0 and 1 hold the
    # group-straddling query heads G - 1 and G, 7 the last one
    sampled_check(fa, dev, I.WORKLOADS["gqa_bf16_n16384"], kv_heads_for_cols=[(0, 0), (0, 1), (0, 7)])


@pytest.mark.timeout(900)
def test_long_bf16_n65536_workload(fa, dev):
    sampled_check(fa, dev, I.WORKLOADS["long_bf16_n65536"], kv_heads_for_cols=[(0, 0), (0, 7)])


# ---------------------------------------------------------------- fp8

@pytest.mark.parametrize("n", [0, 1, 1000, 4097, (1 << 20) + 3])
def test_quantize_fp8_bit_exact(fa, dev, n):
    x = (torch.randn(n, generator=torch.Generator().manual_seed(n)) * 3.0).to(torch.bfloat16)
    codes, ds = fa.quantize_fp8(x.to(dev))
    torch.cuda.synchronize()
    ref_codes, ref_s = oracle.quantize_per_tensor(x.float().numpy())
    assert ds.cpu().numpy()[0] == ref_s
    assert np.array_equal(codes.cpu().numpy(), ref_codes)


def fp8_forward_check(fa, dev, q, k, v, causal, scale, rows_by_head, tag):
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    q8, sq = fa.quantize_fp8(qd)
    k8, sk = fa.quantize_fp8(kd)
    v8, sv = fa.quantize_fp8(vd)
    descale = torch.cat([sq, sk, sv])
    o, lse = fa.fwd(q8, k8, v8, causal, scale, descale=descale)
    torch.cuda.synchronize()
    G = q.shape[1] // k.shape[1]
    got, ref = [], []
    for (b, h), rows in rows_by_head:
        Or, _ = oracle.head_rows_forward(f64(q[b, h]), f64(k[b, h // G]), f64(v[b, h // G]), rows, causal, scale)
        got.append(f64(o[b, h, rows]))
        ref.append(Or)
    e = rel_l2(np.concatenate(got), np.concatenate(ref))
    print(f"[{tag}] fp8 O rel-L2 {e:.3e}", flush=True)
    assert e <= 6e-2, (tag, e)


@pytest.mark.parametrize("N,d,causal", [(200, 64, True), (257, 128, False), (1024, 128, True), (1000, 128, False),
                                           (777, 128, True), (1000, 64, False), (333, 64, True), (50, 64, False)])
def test_fp8_forward_small(fa, dev, N, d, causal):
    B, Hq, Hkv = 1, 4, 2
    q = I.random_tensor(7, (B, Hq, N, d), "bf16", tensor_id=0)
    k = I.random_tensor(7, (B, Hkv, N, d), "bf16", tensor_id=1)
    v = I.random_tensor(7, (B, Hkv, N, d), "bf16", tensor_id=2)
    heads = [((0, h), np.arange(N)) for h in range(Hq)]
    fp8_forward_check(fa, dev, q, k, v, causal, 1 / np.sqrt(d), heads, f"fp8 N{N} d{d}")


@pytest.mark.timeout(300)
def test_fp8_forward_gqa_n16384_workload(fa, dev):
    w = I.WORKLOADS["gqa_bf16_n16384"]
    q, k, v = (I.full_tensor(w, t) for t in range(3))
    rows = I.sample_rows(w.N)
    fp8_forward_check(fa, dev, q, k, v, w.causal, w.scale, [(bh, rows) for bh in I.sample_heads(w)], w.name)


@pytest.mark.timeout(300)
def test_fp8_forward_mha_n1024_workload(fa, dev):
    """The d = 64 fp8 forward at the 1024-token workload's shape: every row of the sampled heads."""
    w = I.WORKLOADS["mha_bf16_n1024"]
    q, k, v = (I.full_tensor(w, t) for t in range(3))
    rows = np.arange(w.N)
    fp8_forward_check(fa, dev, q, k, v, w.causal, w.scale, [(bh, rows) for bh in I.sample_heads(w)], w.name)


# ---------------------------------------------------------------- properties at full size

def test_identical_keys_closed_form_full_size(fa, dev):
    """Every key equal: causal O_i = mean(V[0..i]) and LSE_i = scale q_i.k + ln(i+1), checked on all rows."""
    B, H, N, d = 1, 2, 4096, 128
    scale = 1 / np.sqrt(d)
    q = I.random_tensor(3, (B, H, N, d), "bf16", tensor_id=0)
    krow = I.random_tensor(3, (1, 1, 1, d), "bf16", tensor_id=1)
    k = krow.expand(B, H, N, d).contiguous()
    v = I.random_tensor(3, (B, H, N, d), "bf16", tensor_id=2)
    o, lse = fa.fwd(q.to(dev), k.to(dev), v.to(dev), True, scale)
    torch.cuda.synchronize()
    V = f64(v)
    counts = np.arange(1, N + 1)[None, None, :, None]
    O = np.cumsum(V, axis=2) / counts
    L = scale * np.einsum("bhnd,d->bhn", f64(q), f64(krow)[0, 0, 0]) + np.log(np.arange(1, N + 1))
    check("bf16", f64(o), f64(lse), O, L, tag="identical keys")


def test_deterministic_bitwise(fa, dev):
    B, Hq, Hkv, N, d = 2, 4, 2, 1000, 128
    q = I.random_tensor(5, (B, Hq, N, d), "bf16", tensor_id=0).to(dev)
    k = I.random_tensor(5, (B, Hkv, N, d), "bf16", tensor_id=1).to(dev)
    v = I.random_tensor(5, (B, Hkv, N, d), "bf16", tensor_id=2).to(dev)
    do = I.random_tensor(5, (B, Hq, N, d), "bf16", tensor_id=3).to(dev)
    outs = []
    for _ in range(2):
        o, lse = fa.fwd(q, k, v, True, 0.1)
        dq, dk, dv, _ = fa.bwd(q, k, v, o, do, lse, True, 0.1)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (o, lse, dq, dk, dv)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
