"""The bandwidth probes read exactly the bytes they claim to read: the XOR of
their per-wavefront checksums equals the XOR of every 32-bit word of the
buffer (streaming read) or of every valid K and V row of the decode call
(the three gathers), computed here with numpy."""
import numpy as np
import pytest
import torch

import decode_inputs as di

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import paged_attention_decode_photon_amd as mod
    return mod


def xor_all(words: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(words.ravel().view(np.uint32))) if words.size else 0


def sink_xor(sink) -> int:
    return xor_all(sink.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("nbytes,waves", [(16, 4), (1 << 20, 8), ((1 << 20) + 48, 1024),
                                          (68_157_440, 4096), (3 * 4096 + 16, 8192)])
def test_stream_read_checksum(pa, nbytes, waves):
    rng = np.random.default_rng(nbytes % 1000)
    host = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    sink = pa.probe_stream_read(buf, waves)
    torch.cuda.synchronize()
    got, want = sink_xor(sink), xor_all(host)
    assert got == want, f"{nbytes} bytes, {waves} waves: {got:#x} != {want:#x}"


def valid_rows_xor(kc: np.ndarray, vc: np.ndarray, tables, ctx) -> int:
    acc = 0
    for b, c in enumerate(ctx):
        for n in range(-(-int(c) // 16)):
            rows = min(16, int(c) - 16 * n)
            blk = tables[b, n]
            acc ^= xor_all(np.ascontiguousarray(kc[blk, :, :rows]).view(np.uint32))
            acc ^= xor_all(np.ascontiguousarray(vc[blk, :, :rows]).view(np.uint32))
    return acc


@pytest.mark.parametrize("name", ["tiny", "llama1b_b1", "llama1b_b16", "cb_b64", "llama1b_b16_bf16"])
@pytest.mark.parametrize("waves", [4, 1024, 8192])
def test_gather_checksum(pa, name, waves):
    cfg = di.CONFIGS[name]
    lay = di.make_layout(cfg)
    t = di.make_layer(cfg, lay)
    # poison every row no sequence may read: the checksum would change if
    # the probe read one
    kc = di.poison_unused(cfg, lay, t.k_cache)
    vc = di.poison_unused(cfg, lay, t.v_cache)
    sink = pa.probe_gather(di.to_torch(kc).to("cuda:0"), di.to_torch(vc).to("cuda:0"),
                           di.to_torch(lay.block_tables).to("cuda:0"),
                           di.to_torch(lay.context_lens).to("cuda:0"), lay.max_context_len, waves)
    torch.cuda.synchronize()
    got = sink_xor(sink)
    want = valid_rows_xor(di.storage_bits(kc), di.storage_bits(vc), lay.block_tables,
                          lay.context_lens)
    assert got == want, f"{name}, {waves} waves: {got:#x} != {want:#x}"


def test_gather_head_dim_128(pa):
    # 512-byte rows (fp32, head_dim 128) and 256-byte rows (fp16, head_dim 128)
    rng = np.random.default_rng(5)
    for dtype in (np.float32, np.float16):
        ctx = np.array([0, 1, 17, 300, 33], np.int32)
        need = (ctx + 15) // 16
        nb = int(need.sum()) + 2
        perm = rng.permutation(nb).astype(np.int32)
        tables = np.full((5, int(need.max())), -1, np.int32)
        p = 0
        for i, n in enumerate(need):
            tables[i, :n] = perm[p:p + n]
            p += n
        kc = rng.standard_normal((nb, 3, 16, 128)).astype(dtype)
        vc = rng.standard_normal((nb, 3, 16, 128)).astype(dtype)
        sink = pa.probe_gather(torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(),
                               torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda(),
                               300, 64)
        torch.cuda.synchronize()
        bits = np.uint32 if dtype == np.float32 else np.uint16
        got = sink_xor(sink)
        want = valid_rows_xor(kc.view(bits), vc.view(bits), tables, ctx)
        assert got == want, f"{np.dtype(dtype)}: {got:#x} != {want:#x}"


def gather_case(name):
    cfg = di.CONFIGS[name]
    lay = di.make_layout(cfg)
    t = di.make_layer(cfg, lay)
    kc = di.poison_unused(cfg, lay, t.k_cache)
    vc = di.poison_unused(cfg, lay, t.v_cache)
    dev = [di.to_torch(x).to("cuda:0") for x in (kc, vc, lay.block_tables, lay.context_lens)]
    want = valid_rows_xor(di.storage_bits(kc), di.storage_bits(vc), lay.block_tables,
                          lay.context_lens)
    return dev, lay.max_context_len, want


@pytest.mark.parametrize("name", ["tiny", "llama1b_b1", "llama1b_b16", "cb_b64", "llama1b_b16_bf16"])
def test_staged_gather_checksum(pa, name):
    (kc, vc, tables, lens), max_ctx, want = gather_case(name)
    rings = (2, 4, 8) if di.CONFIGS[name].elem_bytes == 2 else (2, 4)
    for wgs in (1, 7, 256, 1024):
        for ring in rings:
            sink = pa.probe_gather_staged(kc, vc, tables, lens, max_ctx, wgs, ring)
            torch.cuda.synchronize()
            got = sink_xor(sink)
            assert got == want, f"{name}, {wgs} workgroups, ring {ring}: {got:#x} != {want:#x}"


@pytest.mark.parametrize("name", ["tiny", "llama1b_b1", "llama1b_b16", "cb_b64", "llama1b_b16_bf16"])
def test_queue_gather_checksum(pa, name):
    (kc, vc, tables, lens), max_ctx, want = gather_case(name)
    queue = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    for waves in (4, 1024):
        for permille, piece in ((0, 1), (500, 4), (900, 16), (1000, 8), (0, 64)):
            for rep in range(2):  # the second call relies on the first leaving zero behind
                sink = pa.probe_gather_queue(kc, vc, tables, lens, max_ctx, waves, permille, piece,
                                             queue)
                torch.cuda.synchronize()
                got = sink_xor(sink)
                assert got == want, \
                    f"{name}, {waves} waves, {permille} static, pieces of {piece}, call {rep}: " \
                    f"{got:#x} != {want:#x}"
                assert int(queue.item()) == 0


def test_staged_and_queue_gathers_head_dim_128(pa):
    rng = np.random.default_rng(6)
    ctx = np.array([0, 1, 17, 300, 33], np.int32)
    need = (ctx + 15) // 16
    nb = int(need.sum()) + 2
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((5, int(need.max())), -1, np.int32)
    p = 0
    for i, n in enumerate(need):
        tables[i, :n] = perm[p:p + n]
        p += n
    for dtype, ring in ((np.float32, 2), (np.float16, 4)):
        kc = rng.standard_normal((nb, 3, 16, 128)).astype(dtype)
        vc = rng.standard_normal((nb, 3, 16, 128)).astype(dtype)
        bits = np.uint32 if dtype == np.float32 else np.uint16
        want = valid_rows_xor(kc.view(bits), vc.view(bits), tables, ctx)
        args = (torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(),
                torch.from_numpy(tables).cuda(), torch.from_numpy(ctx).cuda(), 300)
        got = sink_xor(pa.probe_gather_staged(*args, 3, ring))
        assert got == want, f"{np.dtype(dtype)} staged: {got:#x} != {want:#x}"
        queue = torch.zeros(1, dtype=torch.int64, device="cuda:0")
        got = sink_xor(pa.probe_gather_queue(*args, 64, 250, 2, queue))
        assert got == want, f"{np.dtype(dtype)} queue: {got:#x} != {want:#x}"
        assert int(queue.item()) == 0
