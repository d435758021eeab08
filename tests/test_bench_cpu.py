"""CPU checks of the benchmark's bookkeeping: algorithmic byte counts, the
hash gate on recorded HBM traffic, and the one-GPU contract."""
import os
import subprocess
import sys

import numpy as np

import bench
import decode_inputs as di

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_bytes_of_the_batch16_workload():
    # 16640 context tokens x 8 KV heads x 64 dims x 4 bytes for each of K and
    # V, q and out rows (16 x 32 x 64 x 4 each), the table entries the
    # contexts use (ceil(ctx / 16) each, 4 bytes) and the 16 lengths.
    cfg = di.CONFIGS["llama1b_b16"]
    lay = di.make_layout(cfg)
    ctx = lay.context_lens.astype(np.int64)
    kv = int(ctx.sum()) * 8 * 64 * 4 * 2
    qo = 2 * 16 * 32 * 64 * 4
    tables = int(((ctx + 15) // 16).sum()) * 4
    assert bench.decode_bytes(cfg, ctx) == kv + qo + tables + 4 * 16 == 68_423_836
    # the fused step also reads each sequence's new K and V rows and writes
    # them to the pool: the per-launch figure the counter summaries use
    assert (lay.slot_mapping >= 0).sum() == 16
    assert 68_423_836 + 4 * 16 * 8 * 64 * 4 == 68_554_908


def test_write_and_rope_bytes():
    cfg = di.CONFIGS["llama1b_b16"]
    row = 8 * 64 * 4
    assert bench.write_bytes(cfg, 16, 16) == 4 * 16 * row + 4 * 16
    assert bench.write_bytes(cfg, 16, 3) == 2 * 16 * row + 2 * 3 * row + 4 * 16
    qrow = 32 * 64 * 4
    assert bench.rope_write_bytes(cfg, 4, 2) == 4 * (2 * qrow + 2 * row + 8) + 2 * 2 * row


def test_recorded_traffic_is_used_only_for_the_current_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    for rel in bench.KERNEL_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, rel), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    sha = bench.kernel_source_sha256()
    f = prof / "paged_decode_w_pmc.md"
    f.write_text(f"hbm_bytes_per_launch: 1234\nkernel_source_sha256: {sha}\n")
    assert bench.measured_traffic("w") == 1234.0
    f.write_text("hbm_bytes_per_launch: 1234\nkernel_source_sha256: " + "0" * 64 + "\n")
    assert bench.measured_traffic("w") is None
    assert bench.measured_traffic("absent") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
