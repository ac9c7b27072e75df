"""Host-side checks of the benchmark's arithmetic (no GPU): the pages'
attention-latency-overhead measure and the two-GPU projection model, on
hand-worked inputs, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_overhead_reduction_hand_worked():
    # t_exact 100, t_approx 10, hit 7/8: 100 / (8.75 + 12.5) = 80/17
    assert bench.overhead_reduction(100.0, 10.0, 0.875) == pytest.approx(
        80.0 / 17.0, rel=1e-12)
    # every layer commits: the full ratio; none commits: no reduction
    assert bench.overhead_reduction(100.0, 10.0, 1.0) == pytest.approx(10.0)
    assert bench.overhead_reduction(100.0, 10.0, 0.0) == pytest.approx(1.0)
    # the approximation as slow as exact attention: no reduction at any hit
    for h in (0.0, 0.3, 1.0):
        assert bench.overhead_reduction(50.0, 50.0, h) == pytest.approx(1.0)


def test_overhead_reduction_monotone_in_hit_rate():
    vals = [bench.overhead_reduction(96.0, 10.0, h / 10) for h in range(11)]
    assert all(a < b for a, b in zip(vals, vals[1:]))


def test_project_layer_hand_worked():
    """approx 10, exact to verified output 100, exact-only 98, post 80, hit
    1/2, link 5 (p2p) and 10 (all-reduce):
      one GPU  98 + 80 = 178
      commit   max(10 + 80, 100 + 5) = 105
      discard  100 + 5 + 80 = 185
      ALSpec   (105 + 185) / 2 = 145
      TP2      178 / 2 + 2 * 10 = 109"""
    u = bench.project_layer(10.0, 100.0, 98.0, 80.0, 0.5, 5.0, 10.0)
    assert u == {"one_gpu": 178.0, "alspec_2gpu_commit": 105.0,
                 "alspec_2gpu_discard": 185.0, "alspec_2gpu": 145.0,
                 "tp_2gpu": 109.0}
    # a commit bounded by the speculative side: max picks approx + post
    u2 = bench.project_layer(30.0, 60.0, 58.0, 80.0, 1.0, 2.0, 2.0)
    assert u2["alspec_2gpu"] == u2["alspec_2gpu_commit"] == 110.0


def test_projection_sweeps_the_link():
    seq = {"approx_latency_us_mean": 12.0, "exact_latency_us_mean": 100.0}
    pr = bench.projection(seq, 98.0, 81.0, 0.67)
    assert [e["link_us"] for e in pr["link_sweep"]] == list(bench.LINK_US)
    prev = None
    for e in pr["link_sweep"]:
        L = e["link_us"]
        u = bench.project_layer(12.0, 100.0, 98.0, 81.0, 0.67, L, L)
        assert e["us_per_layer"] == u
        assert e["speedup_vs_one_gpu"]["alspec_2gpu"] == pytest.approx(
            u["one_gpu"] / u["alspec_2gpu"])
        # slower links never help either placement
        if prev is not None:
            assert e["us_per_layer"]["alspec_2gpu"] >= prev["alspec_2gpu"]
            assert e["us_per_layer"]["tp_2gpu"] >= prev["tp_2gpu"]
        prev = e["us_per_layer"]
    assert "not a measurement" in pr["note"]


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_post_probe_at_size_products(monkeypatch):
    """The probe is asked for each post-attention product's weight bytes
    (Llama-3-8B layer, bf16) and its four launch times add up to the layer
    ceiling, set against the measured layer time."""
    from synth import device as sdev
    asked = []

    def fake(sizes):
        asked.extend(sizes)
        # 5000 GB/s at every size: t = bytes / 5e9 us
        return {n: {"us": n / 5e3 / 1e3, "GBps": 5000.0, "blocks": 512,
                    "loads_in_flight": 2, "nontemporal": True}
                for n in sizes}
    monkeypatch.setattr(sdev, "probe_read_sizes", fake)
    res = bench.post_probe_at_size({"us_per_layer": 100.0})
    want = {"o_proj": 4096 * 4096 * 2, "gate_up": 2 * 14336 * 4096 * 2,
            "down": 4096 * 14336 * 2, "next_qkv": 6144 * 4096 * 2}
    assert sorted(asked) == sorted(want.values())
    for k, nb in want.items():
        assert res[k]["bytes"] == nb
        assert res[k]["us"] == pytest.approx(nb / 5e6)
    total = sum(want.values()) / 5e6
    assert res["layer_probe_us"] == pytest.approx(total)
    assert res["layer_frac_of_probe"] == pytest.approx(total / 100.0)
