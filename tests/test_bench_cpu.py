"""Host-side logic of bench.py (no GPU): the algorithmic FLOP and byte counts
its rooflines divide by, the gate on the committed HBM counters, and the
refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def brute_pairs(Nq, Nk, causal):
    """Visible (query, key) pairs by enumeration, bottom-right causal alignment."""
    return sum(1 for i in range(Nq) for j in range(Nk) if not causal or j <= i + (Nk - Nq))


@pytest.mark.parametrize("Nq,Nk", [(1, 1), (5, 5), (7, 3), (3, 7), (64, 200), (200, 64), (1, 50), (50, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_flops_counts_visible_pairs(Nq, Nk, causal):
    d, B, H = 128, 2, 3
    assert bench.prefill_flops(B, H, Nq, Nk, d, causal) == 4.0 * d * B * H * brute_pairs(Nq, Nk, causal)


def test_long_context_flop_figure():
    # B=1, H=32, N=8192, d=128 causal: 4*d*H*N(N+1)/2
    assert bench.prefill_flops(1, 32, 8192, 8192, 128, True) == 549822922752.0


def test_decode_bytes_figure():
    # K and V of B=64, Hkv=8, Nk=32768, d=128 bf16 once, plus Q and O (bf16) and the fp32 LSE
    assert bench.decode_bytes(64, 32, 8, 32768, 128) == 2 * 64 * 8 * 32768 * 128 * 2 + 64 * 32 * 128 * 2 * 2 + 64 * 32 * 4
    assert bench.decode_bytes(64, 32, 8, 32768, 128) == 8590991360


def test_traffic_only_for_matching_sources(monkeypatch):
    with open(bench.PROFILE_COUNTERS) as f:
        rec = json.load(f)
    name, entry = next(iter(rec["kernels"].items()))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: rec["kernel_source_hash"])
    assert bench.load_traffic(name) == entry["hbm_bytes_per_launch"] > 0
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.load_traffic(name) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_padded_causal_flops_counts_visible_pairs():
    # row i of sequence b sees keys j <= i with j < L_b (Nq = Nk = N)
    N, d, H = 37, 64, 3
    lens = [0, 1, 20, 36, 37, 50]
    brute = sum(1 for L in lens for i in range(N) for j in range(N) if j <= i and j < min(L, N))
    assert bench.padded_causal_flops(H, N, lens, d) == 4.0 * d * H * brute
    assert bench.padded_causal_flops(32, 4096, [4096] * 4, 128) == bench.prefill_flops(4, 32, 4096, 4096, 128, True)


def test_stats_of_launch_times():
    st = bench.stats_ms([5.0, 1.0, 3.0, 2.0, 4.0, 10.0, 6.0, 7.0, 8.0, 9.0])
    assert st["min_ms"] == 1.0 and st["median_ms"] == 5.5 and st["mean_ms"] == 5.5 and st["p90_ms"] == 9.0
    assert bench.stats_ms([2.0])["p90_ms"] == 2.0
