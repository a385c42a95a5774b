"""CPU checks of the benchmark's own accounting: the algorithmic bytes and FLOPs it divides by, the
settle phase's stopping rule, and that the committed counter records belong to the kernel sources in
the tree (a record taken on other sources would put stale figures into the JSON line)."""
import glob
import json
import os
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mlra_workloads import WORKLOADS  # noqa: E402


def _fake_inputs(w, lengths):
    """The attributes algorithmic_bytes reads, without allocating the caches."""
    tokens = sum(lengths)
    return types.SimpleNamespace(w=w, seqlens=list(lengths), block_table=None,
                                 cache_bytes=lambda: tokens * w.token_elems * w.elem_bytes)


def test_algorithmic_bytes_of_the_headline():
    # 1,048,576 cached tokens of 512 + 64 bf16 elements; queries 32 x 32 x 576 bf16; 32 int32 lengths;
    # W_UV 4 x 32 x 128 x 128 fp32 and the fp32 output 32 x 32 x 128 on top for the whole step.
    w = WORKLOADS[2]
    b = bench.algorithmic_bytes(_fake_inputs(w, [32768] * 32))
    assert b["cache"] == 1_048_576 * 1152
    assert b["attention"] == 1_209_139_328
    assert b["step"] == 1_218_052_224


def test_flops_per_head_and_token():
    # QK over 512 latent + 64 RoPE channels (the RoPE dot counted once) and PV over 512 latent channels.
    assert bench.flop_per_head_token(WORKLOADS[2]) == 2 * (512 + 64) + 2 * 512
    assert bench.flop_per_head_token(WORKLOADS[4]) == 2 * (512 + 64) + 2 * 512
    assert bench.flop_per_head_token(WORKLOADS[7]) == 2 * (128 + 64) + 2 * 128


class _Clock:
    """A stand-in for the benchmark's perf_counter that advances only when a fake step runs."""

    def __init__(self):
        self.t = 0.0

    def __call__(self):
        return self.t


def _fake_device(monkeypatch):
    import torch
    clock = _Clock()
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    monkeypatch.setattr(bench.time, "perf_counter", clock)
    return clock


def test_settle_stops_once_three_windows_agree(monkeypatch):
    clock = _fake_device(monkeypatch)
    calls = [0]

    def step():  # 300 us for the first 60 calls, then 200 us
        calls[0] += 1
        clock.t += 300e-6 if calls[0] <= 60 else 200e-6

    # Windows of 20 steps end at 6, 12, 18 ms (slow), then 22, 26, 30 ms (steady). The three slow windows
    # agree before min_ms, so only the steady ones can end it, at 30 ms.
    r = bench.settle(step, min_ms=29, max_ms=1000, window=20)
    assert r["agreed"] and r["windows"] == 6
    assert r["settle_ms"] == pytest.approx(30.0)
    assert r["first_window_us"] == pytest.approx(300.0) and r["last_windows_us"] == [200.0, 200.0, 200.0]


def test_settle_gives_up_at_its_cap(monkeypatch):
    clock = _fake_device(monkeypatch)
    calls = [0]

    def step():  # alternates between 100 us and 800 us windows: no three ever agree within 1.5 %
        calls[0] += 1
        clock.t += 100e-6 if ((calls[0] - 1) // 20) % 2 else 800e-6

    r = bench.settle(step, min_ms=5, max_ms=60, window=20)
    assert not r["agreed"]
    assert 60 <= r["settle_ms"] < 60 + 16  # stops at the first window that ends past the cap


def _records(prefix):
    return sorted(glob.glob(os.path.join(ROOT, "profiles", f"{prefix}_decode_*.json")))


@pytest.mark.parametrize("kind", ["traffic", "mfma"])
def test_counter_records_belong_to_the_current_kernel_sources(kind):
    paths = _records(kind)
    assert paths, f"no {kind} records under profiles/"
    want = bench.kernel_source_hash()
    lookup = bench.traffic_record if kind == "traffic" else bench.mfma_record
    for p in paths:
        rec = json.load(open(p))
        name = os.path.basename(p)[len(kind) + len("_decode_"):-len(".json")]
        assert rec["kernel_source_sha256"] == want, f"{p} was taken on other kernel sources"
        assert lookup(name) is not None, name
