"""C-ABI checks that need no GPU: exported symbols and argument validation.

Every call here fails validation (or has nothing to launch), which the
library guarantees happens before its first HIP call.
"""
import ctypes
import os
import re
import subprocess

import pytest

import paged_attention_decode_photon_amd as pa

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADER = os.path.join(INCLUDE, "photon_decode.h")
HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))
FAKE = 0x10000  # aligned, never dereferenced: each call below fails validation first


def declared_functions():
    names = []
    for h in HEADERS:
        names += re.findall(r"PHOTON_API\s+[\w\s\*]+?\b(photon_\w+)\s*\(", open(h).read())
    return names


def test_header_declares_the_entry_points():
    names = set(declared_functions())
    assert {"photon_kv_cache_write", "photon_paged_attn_decode", "photon_rope_kv_cache_write",
            "photon_paged_attn_workspace_bytes", "photon_status_str", "photon_sched_create",
            "photon_sched_schedule", "photon_sched_update"} <= names


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports_every_declared_symbol(name):
    assert hasattr(pa.lib, name)


def test_abi_version_matches_header():
    m = re.search(r"#define PHOTON_ABI_VERSION (\d+)", open(HEADER).read())
    assert pa.lib.photon_abi_version() == int(m.group(1))


def test_status_names():
    for code, name in [(0, "PHOTON_OK"), (1, "PHOTON_ERR_INVALID_ARG"),
                       (2, "PHOTON_ERR_UNSUPPORTED"), (3, "PHOTON_ERR_WORKSPACE"),
                       (4, "PHOTON_ERR_HIP")]:
        assert pa.lib.photon_status_str(code).decode() == name


def kv(nb=64, hkv=8, bs=16, d=64, dtype=pa.F32):
    return pa.KvDesc(nb, hkv, bs, d, dtype)


def dd(b=16, hq=32, mb=128, maxctx=2048, part=0, flags=0, **kw):
    return pa.DecodeDesc(b, hq, mb, maxctx, part, kv(**kw), flags)


def test_binding_structs_match_the_header(tmp_path):
    # Compile the header with the host C compiler and compare the layout of
    # both descriptors with the ctypes mirrors the binding passes.
    prog = tmp_path / "layout.c"
    prog.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "photon_decode.h"\n'
        "int main(void) {\n"
        '  printf("%zu %zu %zu %zu %zu %d %d %zu %zu\\n", sizeof(photon_kv_desc),\n'
        "         sizeof(photon_decode_desc), offsetof(photon_decode_desc, kv),\n"
        "         offsetof(photon_decode_desc, flags), offsetof(photon_kv_desc, dtype), PHOTON_BF16,\n"
        "         PHOTON_DECODE_OUT_F32, sizeof(photon_rope_desc),\n"
        "         offsetof(photon_rope_desc, adjacent_pairs));\n"
        "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), "-o", str(exe),
                           str(prog)])
    got = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    assert got == [ctypes.sizeof(pa.KvDesc), ctypes.sizeof(pa.DecodeDesc),
                   pa.DecodeDesc.kv.offset, pa.DecodeDesc.flags.offset, pa.KvDesc.dtype.offset,
                   pa.BF16, pa.DECODE_OUT_F32, ctypes.sizeof(pa.RopeDesc),
                   pa.RopeDesc.adjacent_pairs.offset]


def write(desc, n=4, k=FAKE, v=FAKE, slots=FAKE, kc=FAKE, vc=FAKE):
    return pa.lib.photon_kv_cache_write(k, v, slots, n, kc, vc,
                                        ctypes.byref(desc) if desc is not None else None, None)


def detail():
    return pa.lib.photon_last_error_detail().decode()


@pytest.mark.parametrize("desc,code", [
    (None, pa.ERR_INVALID_ARG),
    (kv(nb=0), pa.ERR_INVALID_ARG),
    (kv(hkv=-1), pa.ERR_INVALID_ARG),
    (kv(dtype=7), pa.ERR_INVALID_ARG),
    (kv(bs=8), pa.ERR_UNSUPPORTED),
    (kv(d=96), pa.ERR_UNSUPPORTED),
    (kv(nb=1 << 28, bs=16), pa.ERR_INVALID_ARG),  # slots overflow int32
])
def test_cache_write_rejects_bad_descriptor(desc, code):
    assert write(desc) == code
    assert detail()


def test_cache_write_rejects_bad_pointers():
    assert write(kv(), k=None) == pa.ERR_INVALID_ARG
    assert write(kv(), slots=None) == pa.ERR_INVALID_ARG
    assert write(kv(), kc=FAKE + 8) == pa.ERR_INVALID_ARG   # pool not 16-byte aligned
    assert write(kv(), slots=FAKE + 2) == pa.ERR_INVALID_ARG
    assert write(kv(), n=-1) == pa.ERR_INVALID_ARG


def test_cache_write_with_no_tokens_launches_nothing():
    assert write(kv(), n=0, k=None, v=None, slots=None, kc=None, vc=None) == pa.OK


def test_partition_quantum_and_auto_size():
    # fp32 / d64 / group 4: two 16-token blocks per unit of work
    assert pa.lib.photon_paged_attn_partition_quantum(ctypes.byref(dd())) == 32
    # group 8 with fp32 rows: one block per unit keeps the partial scores in registers
    assert pa.lib.photon_paged_attn_partition_quantum(ctypes.byref(dd(hq=64))) == 16
    # fp16 / d128 / group 2
    assert pa.lib.photon_paged_attn_partition_quantum(
        ctypes.byref(dd(hq=16, d=128, dtype=pa.F16))) == 32
    # bf16 rows are as wide as fp16 rows, with or without fp32 output
    for flags in (0, pa.DECODE_OUT_F32):
        assert pa.lib.photon_paged_attn_partition_quantum(
            ctypes.byref(dd(dtype=pa.BF16, flags=flags))) == 32
    # auto: 16 seqs x 8 KV heads x 64 units = 8192 units over 1024 waves
    assert pa.lib.photon_paged_attn_partition_tokens(ctypes.byref(dd())) == 8 * 32
    # 3 units per wave -> 2731 waves, rounded up to whole workgroups
    assert pa.lib.photon_paged_attn_partition_tokens(ctypes.byref(dd(part=96))) == 96
    # a small batch gets one wave per unit
    assert pa.lib.photon_paged_attn_partition_tokens(ctypes.byref(dd(b=1, maxctx=512))) == 32


def test_workspace_size_formula():
    # 3 seqs x 2 KV heads x ceil(640/32) = 120 units; 2 units per wave -> 60 waves
    d = dd(b=3, hq=8, mb=40, maxctx=640, part=64, hkv=2)
    counters = (3 * 2 * 8 + 255) // 256 * 256  # one 64-bit word per (sequence, KV head)
    record = (2 * 4 + 4 * 64) * 4
    assert pa.workspace_bytes(d) == counters + 60 * 2 * record
    assert pa.workspace_bytes(dd(b=0)) == 0
    # contexts of at most one quantum are never split: no workspace at all
    assert pa.workspace_bytes(dd(maxctx=32)) == 0
    assert pa.workspace_bytes(dd(maxctx=33)) > 0


@pytest.mark.parametrize("desc,code", [
    (dd(hq=30), pa.ERR_INVALID_ARG),            # Hq not a multiple of Hkv
    (dd(hq=128), pa.ERR_UNSUPPORTED),           # group 16
    (dd(hq=24), pa.ERR_UNSUPPORTED),            # group 3
    (dd(maxctx=128 * 16 + 1), pa.ERR_INVALID_ARG),
    (dd(maxctx=-1), pa.ERR_INVALID_ARG),
    (dd(part=48), pa.ERR_INVALID_ARG),          # not a multiple of the quantum
    (dd(part=-32), pa.ERR_INVALID_ARG),
    (dd(b=-1), pa.ERR_INVALID_ARG),
    (dd(b=2049), pa.ERR_UNSUPPORTED),
    # 2048 x 8 KV heads x 150,000 units of 32 tokens: past 32-bit unit indexing
    (dd(b=2048, mb=300_000, maxctx=300_000 * 16), pa.ERR_UNSUPPORTED),
    (dd(bs=32), pa.ERR_UNSUPPORTED),
    (dd(flags=2), pa.ERR_INVALID_ARG),          # unknown flag bit
    (dd(flags=-1), pa.ERR_INVALID_ARG),
    (dd(dtype=3), pa.ERR_INVALID_ARG),
])
def test_decode_rejects_bad_descriptor(desc, code):
    n = ctypes.c_size_t(0)
    assert pa.lib.photon_paged_attn_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)) == code
    assert _decode(desc) == code
    assert detail()


def _decode(desc, q=FAKE, kc=FAKE, vc=FAKE, tables=FAKE, lens=FAKE, scale=0.125, out=FAKE,
            ws=FAKE, ws_bytes=1 << 30):
    return pa.lib.photon_paged_attn_decode(q, kc, vc, tables, lens, scale,
                                           ctypes.byref(desc) if desc is not None else None,
                                           out, ws, ws_bytes, None)


def test_decode_rejects_bad_pointers_scale_and_workspace():
    d = dd(part=256)
    need = pa.workspace_bytes(d)
    assert need > 0
    assert _decode(None) == pa.ERR_INVALID_ARG
    assert _decode(d, q=None) == pa.ERR_INVALID_ARG
    assert _decode(d, out=FAKE + 4) == pa.ERR_INVALID_ARG
    assert _decode(d, tables=FAKE + 1) == pa.ERR_INVALID_ARG
    assert _decode(d, scale=float("nan")) == pa.ERR_INVALID_ARG
    assert _decode(d, scale=float("inf")) == pa.ERR_INVALID_ARG
    assert _decode(d, ws_bytes=need - 1) == pa.ERR_WORKSPACE
    assert _decode(d, ws=None, ws_bytes=need) == pa.ERR_INVALID_ARG
    assert _decode(d, ws=FAKE + 8, ws_bytes=need) == pa.ERR_INVALID_ARG


def test_decode_with_no_sequences_launches_nothing():
    assert _decode(dd(b=0), q=None, kc=None, vc=None, tables=None, lens=None, out=None,
                   ws=None, ws_bytes=0) == pa.OK


def _rope(kvd=None, rope=None, n=4, hq=32, q=FAKE, q_out=FAKE + 0x100000, k=FAKE, v=FAKE,
          pos=FAKE, slots=FAKE, kc=FAKE, vc=FAKE):
    kvd = kv() if kvd is None else kvd
    rope = pa.RopeDesc(1e4, 0, 0) if rope is None else rope
    return pa.lib.photon_rope_kv_cache_write(q, q_out, k, v, pos, slots, n, hq, kc, vc,
                                             ctypes.byref(kvd),
                                             ctypes.byref(rope) if rope is not False else None,
                                             None)


@pytest.mark.parametrize("kw,code", [
    (dict(rope=False), pa.ERR_INVALID_ARG),
    (dict(rope=pa.RopeDesc(0.0, 0, 0)), pa.ERR_INVALID_ARG),
    (dict(rope=pa.RopeDesc(-1e4, 0, 0)), pa.ERR_INVALID_ARG),
    (dict(rope=pa.RopeDesc(float("nan"), 0, 0)), pa.ERR_INVALID_ARG),
    (dict(rope=pa.RopeDesc(float("inf"), 0, 0)), pa.ERR_INVALID_ARG),
    (dict(rope=pa.RopeDesc(1e4, 2, 0)), pa.ERR_INVALID_ARG),
    (dict(rope=pa.RopeDesc(1e4, 0, 1)), pa.ERR_INVALID_ARG),
    (dict(kvd=kv(d=96)), pa.ERR_UNSUPPORTED),
    (dict(kvd=kv(dtype=5)), pa.ERR_INVALID_ARG),
    (dict(hq=0), pa.ERR_INVALID_ARG),
    (dict(n=-1), pa.ERR_INVALID_ARG),
    (dict(q=None), pa.ERR_INVALID_ARG),
    (dict(pos=None), pa.ERR_INVALID_ARG),
    (dict(q_out=FAKE + 8), pa.ERR_INVALID_ARG),      # misaligned
    (dict(pos=FAKE + 2), pa.ERR_INVALID_ARG),
    (dict(q_out=FAKE + 16), pa.ERR_INVALID_ARG),     # overlaps q without being q
])
def test_rope_cache_write_rejects_bad_arguments(kw, code):
    assert _rope(**kw) == code
    assert detail()


def test_rope_cache_write_with_no_tokens_launches_nothing():
    assert _rope(n=0, q=None, q_out=None, k=None, v=None, pos=None, slots=None, kc=None,
                 vc=None) == pa.OK


def test_scheduler_structs_match_the_header(tmp_path):
    from paged_attention_decode_photon_amd import sched
    prog = tmp_path / "sched_layout.c"
    prog.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "photon_sched.h"\n'
        "int main(void) {\n"
        '  printf("%zu %zu %zu %zu %zu %zu\\n", sizeof(photon_sched_config), sizeof(photon_sched_batch),\n'
        "         offsetof(photon_sched_batch, request_ids), offsetof(photon_sched_batch, preempted_ids),\n"
        "         sizeof(photon_sched_request_info), offsetof(photon_sched_request_info, num_preemptions));\n"
        "  return 0;\n}\n")
    exe = tmp_path / "sched_layout"
    subprocess.check_call(["gcc", "-std=c11", "-I", INCLUDE, "-o", str(exe), str(prog)])
    got = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    assert got == [ctypes.sizeof(sched.SchedConfig), ctypes.sizeof(sched.SchedBatch),
                   sched.SchedBatch.request_ids.offset, sched.SchedBatch.preempted_ids.offset,
                   ctypes.sizeof(sched.SchedRequestInfo), sched.SchedRequestInfo.num_preemptions.offset]


def _mq(desc, q=FAKE, kc=FAKE, vc=FAKE, tables=FAKE, lens=FAKE, qs=FAKE, scale=0.125, out=FAKE,
        ws=FAKE, ws_bytes=1 << 30):
    return pa.lib.photon_paged_attn_multi_query(q, kc, vc, tables, lens, qs, scale,
                                                ctypes.byref(desc) if desc is not None else None,
                                                out, ws, ws_bytes, None)


def mqd(b=4, t=16, hq=32, mb=8, mq=4, maxctx=100, split=0, flags=0, **kw):
    return pa.MultiQueryDesc(b, t, hq, mb, mq, maxctx, split, flags, kv(**kw))


def test_multi_query_split_and_workspace_formula():
    # 4 seqs x 8 KV heads x ceil(4*4/16)=1 tile = 32 tiles; 2000 tokens = 125 blocks
    d = mqd(mb=128, maxctx=2000)
    n = ctypes.c_size_t(0)
    assert pa.lib.photon_paged_attn_multi_query_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == 0
    # automatic: 1024 / 32 = 32 splits wanted -> 4 blocks each, raised to the
    # fp32 per-tile minimum of 16 blocks -> ceil(125/16) = 8 splits
    counters = (32 * 8 + 255) // 256 * 256  # one 64-bit word per tile
    rec = 16 * (64 + 2) * 4
    assert n.value == counters + 32 * 8 * rec
    # 16-bit storage: the 32-block minimum -> ceil(125/32) = 4 splits
    d16 = mqd(mb=128, maxctx=2000, dtype=pa.F16)
    assert pa.lib.photon_paged_attn_multi_query_workspace_bytes(ctypes.byref(d16), ctypes.byref(n)) == 0
    assert n.value == counters + 32 * 4 * rec
    # fp32 with a query run of four tiles (the wide kernel): 32-block minimum
    dw = mqd(b=1, t=16, mq=16, mb=128, maxctx=2000)
    assert pa.lib.photon_paged_attn_multi_query_workspace_bytes(ctypes.byref(dw), ctypes.byref(n)) == 0
    assert n.value == (8 * 8 + 255) // 256 * 256 + 8 * 4 * 4 * rec
    d = mqd(mb=128, maxctx=2000)
    # explicit 512-token splits: 4 splits of 32 blocks
    d = mqd(mb=128, maxctx=2000, split=512)
    assert pa.lib.photon_paged_attn_multi_query_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value == counters + 32 * 4 * rec
    # one split covers everything: no workspace
    d = mqd(mb=128, maxctx=2000, split=2048)
    assert pa.lib.photon_paged_attn_multi_query_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value == 0


@pytest.mark.parametrize("desc,code", [
    (mqd(hq=30), pa.ERR_INVALID_ARG),
    (mqd(hq=128), pa.ERR_UNSUPPORTED),
    (mqd(b=-1), pa.ERR_INVALID_ARG),
    (mqd(t=-1), pa.ERR_INVALID_ARG),
    (mqd(mq=-1), pa.ERR_INVALID_ARG),
    (mqd(mq=17), pa.ERR_INVALID_ARG),           # longer than all the rows
    (mqd(mb=0), pa.ERR_INVALID_ARG),
    (mqd(flags=4), pa.ERR_INVALID_ARG),
    (mqd(b=9000), pa.ERR_UNSUPPORTED),          # grid y limit with 8 KV heads
    (mqd(d=80), pa.ERR_UNSUPPORTED),
    (mqd(dtype=9), pa.ERR_INVALID_ARG),
    (mqd(maxctx=8 * 16 + 1), pa.ERR_INVALID_ARG),   # past the tables
    (mqd(maxctx=-1), pa.ERR_INVALID_ARG),
    (mqd(split=100), pa.ERR_INVALID_ARG),           # not a multiple of 64
    (mqd(split=-64), pa.ERR_INVALID_ARG),
])
def test_multi_query_rejects_bad_descriptor(desc, code):
    assert _mq(desc) == code
    assert detail()


def test_multi_query_rejects_bad_pointers_and_scale():
    assert _mq(None) == pa.ERR_INVALID_ARG
    assert _mq(mqd(), qs=None) == pa.ERR_INVALID_ARG
    assert _mq(mqd(), out=FAKE + 8) == pa.ERR_INVALID_ARG
    assert _mq(mqd(), qs=FAKE + 2) == pa.ERR_INVALID_ARG
    assert _mq(mqd(), scale=float("nan")) == pa.ERR_INVALID_ARG
    d = mqd(mb=128, maxctx=2000)
    n = ctypes.c_size_t(0)
    pa.lib.photon_paged_attn_multi_query_workspace_bytes(ctypes.byref(d), ctypes.byref(n))
    assert _mq(d, ws_bytes=n.value - 1) == pa.ERR_WORKSPACE
    assert _mq(d, ws=None, ws_bytes=n.value) == pa.ERR_INVALID_ARG


def test_multi_query_with_nothing_to_do_launches_nothing():
    assert _mq(mqd(b=0, t=0, mq=0), q=None, kc=None, vc=None, tables=None, lens=None, qs=None,
               out=None) == pa.OK
    assert _mq(mqd(t=0, mq=0), q=None, out=None) == pa.OK


def test_decode_step_rejects_missing_new_rows():
    d = dd(part=256)
    need = pa.workspace_bytes(d)
    call = lambda kn, vn: pa.lib.photon_paged_attn_decode_step(FAKE, kn, vn, FAKE, FAKE, FAKE, FAKE,
                                                               0.125, ctypes.byref(d), FAKE, FAKE,
                                                               need, None)
    assert call(None, FAKE) == pa.ERR_INVALID_ARG
    assert call(FAKE, FAKE + 4) == pa.ERR_INVALID_ARG
    assert pa.lib.photon_paged_attn_decode_step(None, None, None, None, None, None, None, 0.125,
                                                ctypes.byref(dd(b=0)), None, None, 0, None) == pa.OK


def _binding_calls(torch, idx_dtype):
    """One call of each binding on host tensors, with index tensors of idx_dtype."""
    f32 = torch.float32
    kc = torch.zeros((4, 2, 16, 64), dtype=f32)
    vc = torch.zeros_like(kc)
    q = torch.zeros((1, 4, 64), dtype=f32)
    k = torch.zeros((1, 2, 64), dtype=f32)
    idx1 = torch.zeros(1, dtype=idx_dtype)
    tables = torch.zeros((1, 4), dtype=idx_dtype)
    qs = torch.tensor([0, 1], dtype=idx_dtype)
    return {
        "kv_cache_write": lambda: pa.kv_cache_write(k, k, idx1, kc, vc),
        "rope_kv_cache_write": lambda: pa.rope_kv_cache_write(q, k, k, idx1, idx1, kc, vc, 1e4),
        "paged_attn_decode": lambda: pa.paged_attn_decode(q, kc, vc, tables, idx1, 0.125,
                                                          max_context_len=1),
        "paged_attn_decode_step": lambda: pa.paged_attn_decode_step(q, k, k, kc, vc, tables, idx1,
                                                                    0.125, max_context_len=1),
        "paged_attn_multi_query": lambda: pa.paged_attn_multi_query(
            q, kc, vc, tables, idx1, qs, 0.125, max_query_len=1, max_context_len=1),
    }


@pytest.mark.parametrize("entry", ["kv_cache_write", "rope_kv_cache_write", "paged_attn_decode",
                                   "paged_attn_decode_step", "paged_attn_multi_query"])
def test_binding_refuses_int64_indices(entry):
    # torch's default integer type is int64; the kernels read int32, so an
    # int64 slot mapping or table would be misread.  The binding refuses it.
    torch = pytest.importorskip("torch")
    with pytest.raises(pa.PhotonError, match="int32"):
        _binding_calls(torch, torch.int64)[entry]()


@pytest.mark.parametrize("entry", ["kv_cache_write", "rope_kv_cache_write", "paged_attn_decode",
                                   "paged_attn_decode_step", "paged_attn_multi_query"])
def test_binding_refuses_host_tensors(entry):
    # a host pointer handed to a kernel would be dereferenced on the GPU
    torch = pytest.importorskip("torch")
    with pytest.raises(pa.PhotonError, match="GPU"):
        _binding_calls(torch, torch.int32)[entry]()


def test_noalloc_decode_checks_before_any_hip_call():
    m = re.search(r"#define PHOTON_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert pa.NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))

    def call(desc, q=FAKE, out=FAKE):
        return pa.lib.photon_paged_attn_decode_noalloc(q, FAKE, FAKE, FAKE, FAKE, 0.125,
                                                       ctypes.byref(desc), out, None)

    # one wave per quantum over 2048 x 8 x 64 units: 2 GB of workspace
    big = dd(b=2048, mb=128, maxctx=2048, part=32)
    assert pa.workspace_bytes(big) > pa.NOALLOC_SCRATCH_BYTES
    assert call(big) == pa.ERR_WORKSPACE
    assert "scratch" in detail()
    assert call(dd(), q=None) == pa.ERR_INVALID_ARG
    assert call(dd(), out=FAKE + 4) == pa.ERR_INVALID_ARG
    assert call(dd(b=0)) == pa.OK  # nothing to launch


def test_probes_validate_before_any_hip_call():
    lib = pa.lib

    def stream(buf=FAKE, nbytes=1 << 20, waves=64, sink=FAKE):
        return lib.photon_probe_stream_read(buf, nbytes, waves, sink, None)

    assert stream(waves=0) == pa.ERR_INVALID_ARG
    assert stream(waves=6) == pa.ERR_INVALID_ARG          # not whole workgroups
    assert stream(waves=(1 << 20) + 4) == pa.ERR_INVALID_ARG
    assert stream(sink=None) == pa.ERR_INVALID_ARG
    assert stream(buf=None) == pa.ERR_INVALID_ARG
    assert stream(buf=FAKE + 8) == pa.ERR_INVALID_ARG
    assert stream(nbytes=0) == pa.ERR_INVALID_ARG
    assert stream(nbytes=24) == pa.ERR_INVALID_ARG
    assert stream(nbytes=1 << 40, waves=4) == pa.ERR_UNSUPPORTED

    def gather(desc, kc=FAKE, waves=64):
        return lib.photon_probe_gather(kc, FAKE, FAKE, FAKE, ctypes.byref(desc), waves, FAKE, None)

    assert gather(dd(b=65)) == pa.ERR_UNSUPPORTED        # prefix sums of at most 64 sequences
    assert gather(dd(bs=32)) == pa.ERR_UNSUPPORTED
    assert gather(dd(dtype=7)) == pa.ERR_INVALID_ARG
    assert gather(dd(maxctx=128 * 16 + 1)) == pa.ERR_INVALID_ARG
    assert gather(dd(), kc=None) == pa.ERR_INVALID_ARG
    assert gather(dd(), waves=3) == pa.ERR_INVALID_ARG

    def staged(desc, wgs=256, ring=2, kc=FAKE, sink=FAKE):
        return lib.photon_probe_gather_staged(kc, FAKE, FAKE, FAKE, ctypes.byref(desc), wgs, ring,
                                              sink, None)

    assert staged(dd(), wgs=0) == pa.ERR_INVALID_ARG
    assert staged(dd(), wgs=(1 << 18) + 1) == pa.ERR_INVALID_ARG
    assert staged(dd(), ring=3) == pa.ERR_UNSUPPORTED
    assert staged(dd(), ring=8) == pa.ERR_UNSUPPORTED    # 256-byte rows: 4 tiles fill 128 KiB
    assert staged(dd(d=128), ring=4) == pa.ERR_UNSUPPORTED
    assert staged(dd(b=65)) == pa.ERR_UNSUPPORTED
    assert staged(dd(), kc=None) == pa.ERR_INVALID_ARG
    assert staged(dd(), sink=None) == pa.ERR_INVALID_ARG

    def queue(desc, waves=64, permille=500, piece=4, q=FAKE):
        return lib.photon_probe_gather_queue(FAKE, FAKE, FAKE, FAKE, ctypes.byref(desc), waves,
                                             permille, piece, q, FAKE, None)

    assert queue(dd(), waves=6) == pa.ERR_INVALID_ARG
    assert queue(dd(), permille=-1) == pa.ERR_INVALID_ARG
    assert queue(dd(), permille=1001) == pa.ERR_INVALID_ARG
    assert queue(dd(), piece=0) == pa.ERR_INVALID_ARG
    assert queue(dd(), piece=65) == pa.ERR_INVALID_ARG
    assert queue(dd(), q=None) == pa.ERR_INVALID_ARG
    assert queue(dd(), q=FAKE + 4) == pa.ERR_INVALID_ARG
    assert queue(dd(b=65)) == pa.ERR_UNSUPPORTED
