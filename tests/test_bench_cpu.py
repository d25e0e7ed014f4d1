"""Host logic of bench.py (no GPU): the one-GPU refusal, the algorithmic byte
and flop counts the roofline divides by, the G-sweep fit, and the committed
profile summaries it reads only while they match the library sources."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


@pytest.mark.parametrize("B,H,G,d,N,itemsize,want", [
    # tiny float32 decode, H=8, d=64, N=128 at G=2 / 8 / 1: K/V + q/out + lengths
    (1, 8, 2, 64, 128, 4, 131_072 + 4_096 + 4),
    (1, 8, 8, 64, 128, 4, 524_288 + 4_096 + 4),
    (1, 8, 1, 64, 128, 4, 65_536 + 4_096 + 4),
    # Llama-7B-sized layer, B=16, H=32, d=128, N=1024, bf16, G = 32 / 8 / 4 / 1
    (16, 32, 32, 128, 1024, 2, 268_435_456 + 262_144 + 64),
    (16, 32, 8, 128, 1024, 2, 67_108_864 + 262_144 + 64),
    (16, 32, 4, 128, 1024, 2, 33_554_432 + 262_144 + 64),
    (16, 32, 1, 128, 1024, 2, 8_388_608 + 262_144 + 64),
    # T5-XXL-sized cross-attention, B=32, H=64, G=8, d=64, N=2048
    (32, 64, 8, 64, 2048, 2, 134_217_728 + 524_288 + 128),
])
def test_decode_bytes(B, H, G, d, N, itemsize, want):
    assert bench.decode_bytes(B, H, G, d, B * N, itemsize) == want


def test_decode_flops_do_not_depend_on_G():
    # 4 B H N d for every G (the arithmetic is unchanged; only K/V bytes shrink)
    assert bench.decode_flops(32, 16 * 1024, 128) == 268_435_456
    assert bench.decode_flops(8, 128, 64) == 262_144


def test_prefill_flops():
    # 2 B H d T (T + 1): the unmasked pairs j <= i, two products, a MAC as 2 flops
    assert bench.prefill_flops(2, 4096, 32, 128) == 274_945_015_808
    assert bench.prefill_flops(1, 1, 1, 1) == 4          # one pair: 2 d flops in each product


def test_split_partials_are_overhead_only_with_splits():
    assert bench.split_partial_bytes(16, 32, 128, 1) == 0
    assert bench.split_partial_bytes(16, 32, 128, 2) == 2 * 16 * 32 * 2 * 130 * 4


def test_g_sweep_fit_recovers_a_line():
    fixed_s, bw = 8.3e-6, 7.7e12
    pts = [{"G": g, "bytes_per_call": b, "ms_per_call": (fixed_s + b / bw) * 1e3}
           for g, b in ((32, 268_697_664), (8, 67_371_072), (4, 33_816_640), (1, 8_650_816))]
    fit = bench.g_sweep_fit(pts)
    assert fit["fixed_us"] == pytest.approx(8.3, abs=0.01)
    assert fit["marginal_GBps"] == pytest.approx(7700.0, rel=1e-3)


def test_committed_profiles_are_read_only_while_they_match(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
    good = tmp_path / "good.md"
    good.write_text('x\n```json\n{"kernel_source_sha256_16": "%s", "kernel_mean_us": {"a": 1.5}}\n```\n' % h)
    stale = tmp_path / "stale.md"
    stale.write_text('```json\n{"kernel_source_sha256_16": "0000000000000000", "kernel_mean_us": {"a": 1.5}}\n```\n')
    assert bench._stored_json(str(good))["kernel_mean_us"] == {"a": 1.5}
    assert bench._stored_json(str(stale)) is None
    assert bench._stored_json(str(tmp_path / "missing.md")) is None
    monkeypatch.setattr(bench, "TRACE_FILE", str(stale))
    assert bench.stored_kernel_means() == {}
