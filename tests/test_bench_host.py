"""Host-side checks of bench.py that need no GPU: the one-GPU rule and the
bookkeeping that ties the roofline's traffic figure to the decode sources."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for a refused run


def test_traffic_comes_from_a_profile_of_the_current_sources():
    """Every decode workload's committed counter summary carries the hash of
    the decode sources it was taken with; the bench reports its traffic only
    while that hash matches the sources."""
    h = bench.decode_source_hash()
    for wl in ("llama3_8b_gqa_bf16", "llama13b_mha_f16", "long_context_bf16",
               "shared_prefix_bf16"):
        t = bench.measured_traffic(wl)
        with open(os.path.join(bench.PROFILES, f"decode_{wl}_traffic.md")) as f:
            text = f.read()
        assert (f"decode_source_sha256: {h}" in text) == (t is not None), wl


def test_traffic_is_dropped_once_the_sources_change(monkeypatch):
    monkeypatch.setattr(bench, "decode_source_hash", lambda: "0" * 16)
    assert bench.measured_traffic("llama3_8b_gqa_bf16") is None
