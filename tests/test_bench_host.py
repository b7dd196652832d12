"""Host-side pieces of bench.py, checked without a GPU.

The algorithmic byte counts that the roofline fractions divide by, against the page's
figures (tests/golden/page_figures.json: the bf16 table of V = 262,144 rows of d = 2,816)
and plain arithmetic; the roofline arithmetic; the traffic lookup refusing a profile
taken on other kernel sources; the source hash covering every file the timed kernels
are built from; and the refusal of more than one GPU.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from diffusion_self_conditioning_amd import workloads as wl  # noqa: E402

GOLDEN = os.path.join(ROOT, "tests", "golden", "page_figures.json")


def test_byte_counts_of_the_whole_vocabulary_step():
    w = wl.get("full")
    page = json.load(open(GOLDEN))
    table = 262144 * 2816 * 2
    assert page["embedding_bytes_bf16"]["value"] == table
    assert page["canvas_len"]["value"] == w.rows and page["vocab"]["value"] == w.k
    assert page["hidden"]["value"] == w.d
    logits = 256 * 262144 * 4
    staged = 256 * 262144 * 2
    out = 256 * 2816 * 4
    assert bench.contraction_bytes(w, fused=False) == table + staged == 1_610_612_736
    assert bench.contraction_bytes(w, fused=True) == table + logits
    # the e4m3 table: one byte per code
    assert bench.contraction_bytes(w, False, 1) == table // 2 + staged
    assert bench.step_bytes_logits_once(w) == logits + table + out + 16 * 256 == 1_747_718_144
    assert bench.step_bytes_two_pass(w) == (logits + 16 * 256) + (table + logits + out) \
        == 2_016_153_600


def test_byte_counts_of_the_rank_slice():
    w = wl.get("rank")
    K = 131072 - 65536
    assert w.k == K
    assert bench.contraction_bytes(w, fused=False) == 2 * K * 2816 + 2 * 256 * K
    assert bench.step_bytes_two_pass(w) == 707_530_752


def test_roofline_arithmetic():
    # 1.6 GB in 200 us is 8 TB/s: the HBM peak
    r = bench.roofline(flops=10**9, nbytes=1_600_000_000, us=200.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(8000.0) and r["frac"] == pytest.approx(1.0)
    # 2.5 PFLOP in 1 s is the bf16 peak; few bytes make it MFMA-bound
    r = bench.roofline(flops=2_500 * 10**12, nbytes=10**6, us=1e6)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["frac"] == pytest.approx(1.0)


def test_traffic_lookup_requires_the_current_kernel_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_soft_embed_pp_kernel_full.json").write_text(json.dumps(
        {"kernel_hash": "0" * 16, "bytes_per_launch": 123}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_hash", lambda: "f" * 16)
    val, why = bench.measured_traffic("soft_embed_pp_kernel", "full")
    assert val is None and "not these" in why
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    val, why = bench.measured_traffic("soft_embed_pp_kernel", "full")
    assert val == 123
    val, why = bench.measured_traffic("soft_embed_pp_kernel", "rank")
    assert val is None and "no counter summary" in why


def test_kernel_hash_covers_every_source_of_the_timed_kernels():
    csrc = os.path.join(ROOT, "diffusion_self_conditioning_amd", "csrc")
    # kernels no timed step launches: the sampler, the e4m3 quantiser, the partial sum
    # across ranks, the no-allocation entry point's array and the MFMA-rate probe
    outside = {"accept.hip", "quant.hip", "reduce.hip", "scratch.hip", "probe.hip"}
    sources = {f for f in os.listdir(csrc) if f.endswith((".hip", ".h", ".cpp"))}
    assert sources - outside == set(bench.KERNEL_SOURCES)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
