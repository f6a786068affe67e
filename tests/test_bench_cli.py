"""bench.py's contract pieces that need no GPU: the one-GPU guard, the
roofline's byte and flop accounting, and the rule that the counter-based
traffic is reported only for the kernel source it was measured on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_decode_algorithmic_bytes():
    # per pool: 128 bf16 key channels + 1 valid byte read, 4 score bytes written (a pool's
    # start is first_valid + p * kpool: one value per sequence, not a per-pool read)
    assert bench.score_bytes_per_pool() == 256 + 1 + 4
    Q, P, H, D = 4, 65536, 32, 128
    total = bench.score_bytes_per_pool() * Q * P + Q * H * D * 2 + Q * H * 4 + 2 * D * 4
    assert total == 68453888                          # 68.45 MB per launch


def test_prefill_candidate_pairs_closed_form():
    # the prefill rows sit at positions 126976..131071 of a sequence with no
    # padding and kpool 4: pool p (tokens 4p..4p+3) is a candidate of the row
    # at position pos iff 4p + 3 <= pos, i.e. floor((pos + 1) / 4) pools
    pairs = sum((pos + 1) // 4 for pos in range(131072 - 4096, 131072))
    assert pairs == 132119552
    assert 2 * 32 * 128 * pairs == 1082323369984


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    measured = bench.measured_traffic()
    text = open(bench.TRAFFIC_FILE).read()
    if measured is not None:
        assert measured > 0
    # the same summary with another source hash is ignored
    stale = tmp_path / "traffic.txt"
    stale.write_text("\n".join(
        ("source_sha256: " + "0" * 64) if line.startswith("source_sha256:") else line
        for line in text.splitlines()))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic() is None


def test_step_algorithmic_bytes():
    # the long-context decode step: 4 rows x 65536 pools, K 512, W 2048, 64 x 512 latent
    import bench
    score = bench.score_bytes_per_pool() * 4 * 65536 + 4 * 32 * 128 * 2 + 4 * 32 * 4 + 2 * 128 * 4
    total = bench.step_algorithmic_bytes(4, 65536, 512, 2048, 64, 512, score)
    gathered = 4 * 2048 * 1024                       # each listed latent row once
    assert total == score + 4 * 65536 * 4 + 4 * 512 * 4 + 4 * 2048 * 4 + gathered + 2 * 4 * 64 * 512 * 2 \
        + 4 * 64 * 4 + 4 * 2048 * 4
    assert 78e6 < total < 80e6                       # ~78.5 MB: 9.8 us at 8 TB/s
