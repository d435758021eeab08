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
    f = prof / "summary_pmc.md"
    f.write_text(f"<!-- w hbm_bytes_per_launch: 1234 -->\n<!-- v hbm_bytes_per_launch: 99 -->\n"
                 f"kernel_source_sha256: {sha}\n")
    assert bench.measured_traffic("w", str(f)) == 1234.0
    assert bench.measured_traffic("v", str(f)) == 99.0
    assert bench.measured_traffic("absent", str(f)) is None
    f.write_text("<!-- w hbm_bytes_per_launch: 1234 -->\nkernel_source_sha256: " + "0" * 64 + "\n")
    assert bench.measured_traffic("w", str(f)) is None
    assert bench.measured_traffic("w", str(prof / "missing.md")) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_planned_waves_matches_the_workspace_size():
    # the summariser's copy of the automatic wave rule must agree with the
    # library: the decode workspace holds two records per wavefront
    import paged_attention_decode_photon_amd as pa
    import bench
    for name, cfg in di.CONFIGS.items():
        lay = di.make_layout(cfg)
        desc = pa.DecodeDesc(len(lay.context_lens), cfg.num_q_heads, lay.max_blocks_per_seq,
                             lay.max_context_len, 0,
                             pa.KvDesc(lay.num_blocks, cfg.num_kv_heads, cfg.block_size,
                                       cfg.head_dim, {"f32": pa.F32, "f16": pa.F16,
                                                      "bf16": pa.BF16}[cfg.dtype]), 0)
        ws = pa.workspace_bytes(desc)
        if ws == 0:
            continue
        counters = (len(lay.context_lens) * cfg.num_kv_heads * 8 + 255) // 256 * 256
        rec = ((2 * cfg.group + cfg.group * cfg.head_dim + 3) & ~3) * 4
        assert (ws - counters) == bench.planned_waves(desc) * 2 * rec, name


def test_decode_kernel_names_parse_in_both_forms():
    import bench
    assert bench.decode_kernel_sig("_ZN6photon12_GLOBAL__N_119paged_decode_kernelIDF16bDF16bLi64ELi4EEEvNS0_10KernelArgsE") \
        == ("__bf16", "__bf16", 64, 4)
    assert bench.decode_kernel_sig("_ZN6photon12_GLOBAL__N_119paged_decode_kernelIDF16_fLi128ELi2EEEvNS0_10KernelArgsE") \
        == ("_Float16", "float", 128, 2)
    assert bench.decode_kernel_sig("void photon::(anonymous namespace)::paged_decode_kernel<float, float, 64, 4>(photon::(anonymous namespace)::KernelArgs)") \
        == ("float", "float", 64, 4)
    assert bench.decode_kernel_sig("paged_mq_kernel<float, float, 64, 4>") is None


def test_kernel_names_in_summaries():
    import bench
    assert bench.short_kernel_name("void photon::rope_kv_cache_write_kernel<float, 64, false>(x)") \
        == "rope_kv_cache_write_kernel<float, 64, false>"
    assert bench.short_kernel_name("photon::kv_cache_write_kernel(x)") == "kv_cache_write_kernel"
    assert bench.short_kernel_name("_ZN6photon12_GLOBAL__N_113gather_kernelILi256EEEvNS0_10GatherArgsE") \
        == "gather_kernel<256>"


def test_probe_kernels_in_summaries():
    import bench
    assert bench.short_kernel_name(
        "_ZN6photon12_GLOBAL__N_120gather_staged_kernelILi256ELi2EEEvNS0_10GatherArgsEi") \
        == "gather_staged_kernel<256, 2>"
    assert bench.short_kernel_name(
        "void photon::(anonymous namespace)::gather_staged_kernel<128, 8>(x, int)") \
        == "gather_staged_kernel<128, 8>"
    assert bench.short_kernel_name(
        "_ZN6photon12_GLOBAL__N_119gather_queue_kernelILi512EEEvNS0_10GatherArgsEPyii") \
        == "gather_queue_kernel<512>"
    groups = {("gather_kernel<256>", 65536): [15.4, 15.6], ("gather_staged_kernel<256, 4>", 65536): [15.1],
              ("gather_queue_kernel<256>", 65536): [27.0], ("stream_read_kernel", 262144): [13.0],
              ("paged_mq_kernel<float, float, 64, 4>", 256): [25.0]}
    rows = {(d, s): (m, c) for d, s, m, c in bench.probe_rows(groups)}
    assert rows == {("gather, register sets", "1024 waves"): (15.5, True),
                    ("gather, LDS ring", "256 workgroups x 4 tiles"): (15.1, True),
                    ("gather, queue-driven", "1024 waves, 900/1000 static, 4-tile pieces"): (27.0, False),
                    ("stream read", "4096 waves"): (13.0, False)}
