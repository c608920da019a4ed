"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the counted FLOPs against a
brute-force pair count, and the rule that stored counters are reported only for the
kernel sources they were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.parametrize("seqlens,w0", [((1,), 1), ((7,), 3), ((5, 12, 1), 4), ((30,), 100),
                                        ((16, 16), 16)])
def test_prefill_flops_match_pair_count(seqlens, w0):
    Hq, D = 3, 8
    causal = window = 0
    for L in seqlens:
        for i in range(L):
            for j in range(i + 1):
                causal += 1
                window += (i - j) < w0
    F, Fc = bench.prefill_flops(seqlens, w0, Hq, D)
    assert Fc == 4 * D * Hq * causal
    assert F == 4 * D * Hq * causal + 2 * D * Hq * window


def _fake_tree(tmp_path, kind_sources):
    for rel, text in kind_sources.items():
        p = tmp_path / rel
        p.parent.mkdir(parents=True, exist_ok=True)
        p.write_text(text)
    (tmp_path / "profiles").mkdir(exist_ok=True)


def test_stored_counters_follow_the_kernel_source(tmp_path, monkeypatch):
    srcs = {rel: f"// {rel}\n" for rel in bench.KERNEL_SOURCES["prefill"]}
    _fake_tree(tmp_path, srcs)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.source_hash("prefill")
    traffic = {"copy": {"bytes_read": 1024, "bytes_written": 1024, "FETCH_SIZE_KiB": 0.5,
                        "WRITE_SIZE_KiB": 1.0},
               "prefill": {"source_sha256": h, "FETCH_SIZE_KiB": 10.0, "WRITE_SIZE_KiB": 3.0}}
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(traffic))
    counters = {"source_sha256": h, "derived": {"executed_flops": 5.0, "mfma_busy_frac": 0.5,
                                                 "coexec_frac": 0.2}}
    (tmp_path / "profiles" / "prefill_counters.json").write_text(json.dumps(counters))
    # read factor 1024 / 512 = 2, write factor 1: 10 KiB * 2 + 3 KiB
    assert bench.hbm_traffic("prefill") == pytest.approx((10.0 * 2 + 3.0) * 1024)
    assert bench.mfma_counters("prefill")["executed_flops"] == 5.0
    # any change to a kernel source voids both
    first = bench.KERNEL_SOURCES["prefill"][0]
    (tmp_path / first).write_text("// changed\n")
    assert bench.hbm_traffic("prefill") is None
    assert bench.mfma_counters("prefill") is None


def test_missing_counter_files_give_none(tmp_path, monkeypatch):
    _fake_tree(tmp_path, {rel: "x" for rel in bench.KERNEL_SOURCES["prefill"]})
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.hbm_traffic("prefill") is None
    assert bench.mfma_counters("prefill") is None
