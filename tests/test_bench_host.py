"""Host-side checks of bench.py: the one-GPU refusal, the flop and byte
models it reports against, the traffic lookup's staleness rule, and the
untimed settle loop (with a stand-in for torch's events).  No GPU is used."""
import hashlib
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from exact_io_aware_50_amd import inputs as I  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_credited_flops_of_the_headline_workload():
    w = I.WORKLOADS["causal_bf16_n4096"]
    fwd, bwd = bench.credited(w)
    assert fwd == 4 * 4 * 32 * 4096 * 4096 * 128 / 2
    assert bwd == 2.5 * fwd
    kf = bench.kernel_flops(w)
    assert kf["fwd"] == fwd and kf["bwd_dkdv"] == 2 * fwd and kf["bwd_dq"] == 1.5 * fwd


def test_local_pairs_brute_force():
    for N, W in [(1, 1), (10, 3), (64, 64), (100, 7), (5, 9)]:
        brute = sum(1 for i in range(N) for j in range(N) if j <= i and i - W < j)
        assert bench.local_pairs(N, W) == brute


def test_block_pairs_brute_force():
    rng = np.random.default_rng(0)
    N, bs = 700, 256
    nb = (N + bs - 1) // bs
    mask = rng.random((nb, nb)) < 0.5
    brute = sum(1 for i in range(N) for j in range(N) if mask[i // bs, j // bs])
    assert bench.block_pairs(mask, N, bs) == brute


def test_decode_bytes():
    dw = I.DECODE_WORKLOADS["decode_gqa_bf16_n16384"]
    kv = 2 * dw.B * dw.Hkv * dw.Nk * dw.d * 2
    assert bench.decode_bytes(dw) == kv + 2 * dw.B * dw.Hq * dw.Nq * dw.d * 2 + 4 * dw.B * dw.Hq * dw.Nq


def test_stored_traffic_is_dropped_when_the_source_changes(tmp_path, monkeypatch):
    csrc = tmp_path / "exact_io_aware_50_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "a.hip").write_bytes(b"kernel a")
    (csrc / "b.hpp").write_bytes(b"header b")
    digest = hashlib.sha256(b"kernel a" + b"header b").hexdigest()
    rec = tmp_path / "traffic.txt"
    rec.write_text("# comment\n"
                   f"fwd wl bytes_per_launch=123 read=100 write=23 source=a.hip+b.hpp sha256={digest}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.stored_traffic("fwd", "wl") == 123.0
    assert bench.stored_traffic("fwd", "other") is None
    (csrc / "b.hpp").write_bytes(b"header b, edited")
    assert bench.stored_traffic("fwd", "wl") is None


class _Event:
    log = []

    def record(self, stream):
        _Event.log.append(("record", stream))

    def synchronize(self):
        _Event.log.append(("sync",))


def _fake_torch():
    return types.SimpleNamespace(cuda=types.SimpleNamespace(Event=_Event))


@pytest.mark.parametrize("ms", [0.0, -5.0])
def test_settle_off(ms):
    calls = []
    bench.settle(_fake_torch(), "s", lambda: calls.append(1), ms)
    assert calls == []


def test_settle_runs_for_its_time_and_keeps_one_batch_queued():
    _Event.log = []
    calls = []
    bench.settle(_fake_torch(), "s", lambda: calls.append(1), 20.0, batch=3)
    records = [e for e in _Event.log if e[0] == "record"]
    syncs = [e for e in _Event.log if e[0] == "sync"]
    assert len(calls) == 3 * len(records) and len(records) >= 1
    assert all(e[1] == "s" for e in records)
    # every batch but the newest is waited for: the last one is still queued on return
    assert len(syncs) == len(records) - 1
