"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Tolerances (on every output element, fp32 accumulation throughout): max-abs
1e-4 for fp32 output (fp32 storage, or 16-bit storage with the fp32-output
flag: the inputs are exact in both); 2e-3 for fp16 output (half an fp16 ulp
of |o| < 4, plus the accumulation); for bfloat16 output 1e-4 + 2^-8 |ref|,
since rounding to nearest in bfloat16 (8 significant bits) moves a value by
at most 2^-8 of itself.  Cache writes must be bit-exact over the whole pool.  The oracle runs first on every input set,
so its precondition checks (slot and block-id ranges, context bounds) guard
each launch.
"""
import numpy as np
import pytest
import torch

import decode_inputs as di
import oracle

pytestmark = pytest.mark.gpu

TOL = {np.dtype(np.float32): 1e-4, np.dtype(np.float16): 2e-3}
DTYPES = [np.float32, np.float16, di.BF16]


def tolerance(out_dtype, ref):
    if np.dtype(out_dtype) == di.BF16:
        return 1e-4 + 2.0 ** -8 * np.abs(ref)
    return TOL[np.dtype(out_dtype)]


@pytest.fixture(scope="module")
def pa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import paged_attention_decode_photon_amd as mod
    return mod


def dev(a):
    return di.to_torch(a).to("cuda:0")


def host(t):
    return di.from_torch(t)


def gpu_decode(pa, q, kc, vc, tables, ctx, scale, max_ctx=None, part=0, out_dtype=None):
    out = pa.paged_attn_decode(dev(q), dev(kc), dev(vc), dev(tables), dev(ctx), scale,
                               max_context_len=int(ctx.max()) if max_ctx is None else max_ctx,
                               partition_tokens=part, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return host(out)


def assert_close(got, ref, dtype, what=""):
    g = di.as_float64(got)
    err = np.abs(g - ref)
    worst = float(np.nanmax(err)) if err.size else 0.0
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    assert (err <= tolerance(dtype, ref)).all(), f"{what}: max-abs error {worst:.3e}"
    return worst


def random_case(rng, dtype, b, hq, hkv, d, ctx_list=None, max_ctx=64, spare=3):
    ctx = np.array(ctx_list, np.int32) if ctx_list is not None else \
        rng.integers(0, max_ctx + 1, b).astype(np.int32)
    b = len(ctx)
    need = (ctx.astype(np.int64) + 15) // 16
    nb = int(need.sum()) + spare
    mb = max(int(need.max()), 1)
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((b, mb), -1, np.int32)
    p = 0
    for i, n in enumerate(need):
        tables[i, :n] = perm[p:p + n]
        p += n
    q = di.cast(rng.standard_normal((b, hq, d)), dtype)
    kc = di.cast(rng.standard_normal((nb, hkv, 16, d)), dtype)
    vc = di.cast(rng.standard_normal((nb, hkv, 16, d)), dtype)
    return q, kc, vc, tables, ctx


# ----------------------------------------------------------------- cache write

@pytest.mark.parametrize("dtype,hkv,d", [(np.float32, 8, 64), (np.float16, 8, 64),
                                         (np.float16, 8, 128), (np.float32, 2, 128),
                                         (di.BF16, 8, 64), (di.BF16, 8, 128)])
def test_cache_write_bit_exact(pa, dtype, hkv, d):
    rng = np.random.default_rng(20)
    nb, t = 300, 77
    kc = di.cast(rng.standard_normal((nb, hkv, 16, d)), dtype)
    vc = di.cast(rng.standard_normal((nb, hkv, 16, d)), dtype)
    k = di.cast(rng.standard_normal((t, hkv, d)), dtype)
    v = di.cast(rng.standard_normal((t, hkv, d)), dtype)
    if np.dtype(dtype).itemsize == 2:  # NaN payloads, infinities and subnormals must survive
        k.view(np.uint16)[0, 0, :8] = [0x7E01, 0xFC00, 0x0001, 0x8001, 0x7C00, 0x7D55, 0xFFFF, 0x03FF]
    slots = di.random_injective_slots(nb, 16, t, rng, pad_fraction=0.15)
    ek, ev = oracle.kv_cache_write(k, v, slots, kc, vc)
    gk, gv = dev(kc), dev(vc)
    pa.kv_cache_write(dev(k), dev(v), dev(slots), gk, gv)
    torch.cuda.synchronize()
    assert host(gk).tobytes() == ek.tobytes()
    assert host(gv).tobytes() == ev.tobytes()


def test_cache_write_all_padding_is_noop(pa):
    rng = np.random.default_rng(21)
    kc = rng.standard_normal((4, 2, 16, 64)).astype(np.float32)
    gk, gv = dev(kc), dev(kc)
    k = dev(np.ones((5, 2, 64), np.float32))
    pa.kv_cache_write(k, k, dev(np.full(5, -1, np.int32)), gk, gv)
    torch.cuda.synchronize()
    assert host(gk).tobytes() == kc.tobytes() and host(gv).tobytes() == kc.tobytes()


# ------------------------------------------------------------ decode vs oracle

@pytest.mark.parametrize("name,layer", [("tiny", 0), ("llama1b_b1", 0), ("llama1b_b16", 0),
                                        ("llama1b_b16", 11), ("cb_b64", 0),
                                        ("llama1b_b16_bf16", 0), ("llama1b_b16_bf16", 15)])
def test_decode_matches_oracle_on_workloads(pa, name, layer):
    cfg = di.CONFIGS[name]
    lay = di.make_layout(cfg)
    t = di.make_layer(cfg, lay, layer)
    ref = oracle.paged_attn_decode(t.q, t.k_cache, t.v_cache, lay.block_tables,
                                   lay.context_lens, cfg.scale)
    got = gpu_decode(pa, t.q, t.k_cache, t.v_cache, lay.block_tables, lay.context_lens, cfg.scale)
    err = assert_close(got, ref, cfg.np_dtype, name)
    print(f"{name} layer {layer}: max-abs {err:.3e}")


def test_decode_qwen3_long_full(pa):
    # The full-size Qwen3-shaped workload (8 x 32768 tokens, fp16, d128) in
    # the launch configuration the benchmark uses (automatic partitioning,
    # max_context_len = the longest context); every output element of all
    # eight sequences is compared with the oracle (all host threads, a few
    # seconds).
    cfg = di.CONFIGS["qwen3_long"]
    lay = di.make_layout(cfg)
    t = di.make_layer(cfg, lay)
    got = gpu_decode(pa, t.q, t.k_cache, t.v_cache, lay.block_tables, lay.context_lens, cfg.scale)
    ref = oracle.paged_attn_decode(t.q, t.k_cache, t.v_cache, lay.block_tables, lay.context_lens,
                                   cfg.scale, num_threads=0)
    assert got.shape == ref.shape == (8, 16, 128)
    for b in range(8):
        err = assert_close(got[b:b + 1], ref[b:b + 1], cfg.np_dtype, f"qwen3_long seq {b}")
        print(f"qwen3_long seq {b}: max-abs {err:.3e}")


@pytest.mark.parametrize("name", ["tiny", "cb_b64", "llama1b_b16_bf16"])
def test_decode_step_writes_then_attends(pa, name):
    # The step writes each sequence's new K/V at logical position ctx-1 and
    # then attends over all ctx tokens, the new one included.
    cfg = di.CONFIGS[name]
    lay = di.make_layout(cfg)
    t = di.make_layer(cfg, lay)
    ek, ev = oracle.kv_cache_write(t.k_new, t.v_new, lay.slot_mapping, t.k_cache, t.v_cache)
    ref = oracle.paged_attn_decode(t.q, ek, ev, lay.block_tables, lay.context_lens, cfg.scale)
    gk, gv = dev(t.k_cache), dev(t.v_cache)
    pa.kv_cache_write(dev(t.k_new), dev(t.v_new), dev(lay.slot_mapping), gk, gv)
    out = pa.paged_attn_decode(dev(t.q), gk, gv, dev(lay.block_tables), dev(lay.context_lens),
                               cfg.scale, max_context_len=lay.max_context_len)
    torch.cuda.synchronize()
    assert host(gk).tobytes() == ek.tobytes() and host(gv).tobytes() == ev.tobytes()
    assert_close(host(out), ref, cfg.np_dtype, name)


@pytest.mark.parametrize("name", ["tiny", "cb_b64", "llama1b_b16_bf16"])
def test_unread_slots_never_reach_the_output(pa, name):
    cfg = di.CONFIGS[name]
    lay = di.make_layout(cfg, num_blocks=None)
    t = di.make_layer(cfg, lay)
    args = (lay.block_tables, lay.context_lens, cfg.scale)
    clean = gpu_decode(pa, t.q, t.k_cache, t.v_cache, *args)
    kp = di.poison_unused(cfg, lay, t.k_cache)
    vp = di.poison_unused(cfg, lay, t.v_cache)
    poisoned = gpu_decode(pa, t.q, kp, vp, *args)
    assert np.isfinite(di.as_float64(poisoned)).all()
    assert poisoned.tobytes() == clean.tobytes()


def test_block_permutation_and_repeat_are_bit_identical(pa):
    rng = np.random.default_rng(22)
    q, kc, vc, tables, ctx = random_case(rng, np.float32, 12, 32, 8, 64, max_ctx=700, spare=20)
    base = gpu_decode(pa, q, kc, vc, tables, ctx, 0.125, part=128)
    again = gpu_decode(pa, q, kc, vc, tables, ctx, 0.125, part=128)
    assert base.tobytes() == again.tobytes()
    pi = rng.permutation(kc.shape[0])
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[pi], vc2[pi] = kc, vc
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1).astype(np.int32)
    perm = gpu_decode(pa, q, kc2, vc2, t2, ctx, 0.125, part=128)
    assert perm.tobytes() == base.tobytes()


@pytest.mark.parametrize("dtype,hq,hkv,d", [(np.float32, 32, 8, 64), (np.float16, 32, 8, 64),
                                            (np.float16, 16, 8, 128), (di.BF16, 32, 8, 64)])
def test_partition_sizes_agree_with_oracle(pa, dtype, hq, hkv, d):
    rng = np.random.default_rng(23)
    q, kc, vc, tables, ctx = random_case(rng, dtype, 6, hq, hkv, d,
                                         ctx_list=[1, 17, 255, 256, 257, 1100])
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.11)
    desc = pa.decode_desc(dev(q), dev(kc), dev(tables), int(ctx.max()))
    qu = pa.partition_quantum(desc)
    for part in sorted({qu, 2 * qu, 4 * qu, 128, 256, 512, 2048}):
        if part % qu:
            continue
        got = gpu_decode(pa, q, kc, vc, tables, ctx, 0.11, part=part)
        assert_close(got, ref, dtype, f"partition {part}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_every_built_shape(pa, dtype, d, group):
    rng = np.random.default_rng(1000 + group * 10 + d + DTYPES.index(dtype))
    hkv = 2
    ctx = [0, 1, 15, 16, 17, 31, 33, 64, 100, 333]
    q, kc, vc, tables, ctx = random_case(rng, dtype, len(ctx), hkv * group, hkv, d, ctx_list=ctx)
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, float(np.float32(d ** -0.5)))
    for part in (0, 64):
        got = gpu_decode(pa, q, kc, vc, tables, ctx, float(np.float32(d ** -0.5)), part=part)
        assert_close(got, ref, dtype, f"G{group} d{d} part {part}")
        assert (di.as_float64(got[0]) == 0).all()  # empty context -> zero row


@pytest.mark.parametrize("dtype", [np.float16, di.BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_fp32_output_for_16bit_storage(pa, dtype, d, group):
    # The fp32-output kernels skip the final rounding: fp32 tolerance applies.
    rng = np.random.default_rng(2000 + group * 10 + d + DTYPES.index(dtype))
    hkv = 2
    ctx = [0, 1, 16, 17, 63, 200, 333, 1000]
    q, kc, vc, tables, ctx = random_case(rng, dtype, len(ctx), hkv * group, hkv, d, ctx_list=ctx)
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, float(np.float32(d ** -0.5)))
    for part in (0, 64):
        got = gpu_decode(pa, q, kc, vc, tables, ctx, float(np.float32(d ** -0.5)), part=part,
                         out_dtype=torch.float32)
        assert got.dtype == np.float32
        assert_close(got, ref, np.float32, f"fp32 out G{group} d{d} part {part}")
        assert (got[0] == 0).all()


def test_context_edges_around_partition_boundaries(pa):
    rng = np.random.default_rng(24)
    ctx = [0, 1, 2, 15, 16, 17, 127, 128, 129, 255, 256, 257, 511, 512, 513, 1000]
    q, kc, vc, tables, ctx = random_case(rng, np.float32, 0, 32, 8, 64, ctx_list=ctx)
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.125)
    for part in (0, 128, 256, 512):
        got = gpu_decode(pa, q, kc, vc, tables, ctx, 0.125, part=part)
        assert_close(got, ref, np.float32, f"partition {part}")


def test_max_context_len_may_exceed_every_context(pa):
    rng = np.random.default_rng(25)
    q, kc, vc, tables, ctx = random_case(rng, np.float32, 5, 8, 2, 64, max_ctx=90)
    tables = np.concatenate([tables, np.full((5, 20), -1, np.int32)], axis=1)
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.125)
    got = gpu_decode(pa, q, kc, vc, tables, ctx, 0.125, max_ctx=tables.shape[1] * 16)
    assert_close(got, ref, np.float32, "loose max_context_len")


@pytest.mark.parametrize("scale", [-0.3, 4.0, 40.0])
def test_large_and_negative_scores(pa, scale):
    # scale 40 puts scores in the hundreds: exp only stays finite after the
    # running maximum is subtracted.
    rng = np.random.default_rng(26)
    q, kc, vc, tables, ctx = random_case(rng, np.float32, 4, 8, 2, 64, ctx_list=[5, 70, 300, 31])
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, scale)
    for part in (0, 64):
        got = gpu_decode(pa, q, kc, vc, tables, ctx, scale, part=part)
        assert_close(got, ref, np.float32, f"scale {scale}")


def test_workspace_reused_across_calls_stays_zeroed(pa):
    # Arrival counters live at the start of the workspace; every call that
    # finishes leaves them at zero, and one workspace serves calls of any shape.
    rng = np.random.default_rng(27)
    q, kc, vc, tables, ctx = random_case(rng, np.float32, 9, 32, 8, 64, max_ctx=900)
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.125)
    args = [dev(q), dev(kc), dev(vc), dev(tables), dev(ctx)]
    sizes = {}
    for part in (32, 64, 128, 256):
        desc = pa.decode_desc(args[0], args[1], args[3], int(ctx.max()), part)
        sizes[part] = pa.workspace_bytes(desc)
    ws = pa.new_workspace(max(sizes.values()), "cuda:0")
    ws.zero_()
    for rep in range(2):
        for part in (32, 64, 128, 256):
            out = pa.paged_attn_decode(*args, 0.125, max_context_len=int(ctx.max()), workspace=ws,
                                       partition_tokens=part)
            torch.cuda.synchronize()
            assert_close(host(out), ref, np.float32, f"partition {part} rep {rep}")
            counters = host(ws[: 9 * 8 * 8].view(torch.int64))
            assert (counters == 0).all(), f"counters left at {counters[counters != 0]}"


def _stale_patterns(n_words, rng):
    """Counter contents a workspace may hold before a call: random words,
    all ones, small counts with a zero tag, counts tagged with another call's
    number (what a call that stopped early would leave), and a mix."""
    tagged = (np.uint64(0x5A5A5A5A) << np.uint64(32)) | rng.integers(1, 40, n_words, dtype=np.uint64)
    return {
        "random": rng.integers(0, 2**64 - 1, n_words, dtype=np.uint64, endpoint=True),
        "all_ones": np.full(n_words, np.uint64(2**64 - 1)),
        "small_counts": rng.integers(1, 40, n_words, dtype=np.uint64),
        "other_call": tagged,
        "mixed": np.where(rng.random(n_words) < 0.5, tagged, np.uint64(0)),
    }


@pytest.mark.parametrize("fused", [False, True])
def test_workspace_contents_before_a_call_do_not_matter(pa, fused):
    # Fill the whole workspace (counters and records) with arbitrary values
    # before each call: the result must still match the oracle, and the call
    # must leave every counter it used at zero.
    rng = np.random.default_rng(28)
    cfg = di.CONFIGS["cb_b64"]
    lay = di.make_layout(cfg)
    t = di.make_layer(cfg, lay)
    if fused:
        ek, ev = oracle.kv_cache_write(t.k_new, t.v_new, lay.slot_mapping, t.k_cache, t.v_cache)
        ref = oracle.paged_attn_decode(t.q, ek, ev, lay.block_tables, lay.context_lens, cfg.scale)
    else:
        ref = oracle.paged_attn_decode(t.q, t.k_cache, t.v_cache, lay.block_tables,
                                       lay.context_lens, cfg.scale)
    q, tables, lens = dev(t.q), dev(lay.block_tables), dev(lay.context_lens)
    kc0, vc0 = dev(t.k_cache), dev(t.v_cache)
    for part in (0, 64):
        desc = pa.decode_desc(q, kc0, tables, lay.max_context_len, part)
        nbytes = pa.workspace_bytes(desc)
        ws = pa.new_workspace(nbytes, "cuda:0")
        n_words = 64 * 8  # one counter per (sequence, KV head)
        for name, words in _stale_patterns(n_words, rng).items():
            junk = rng.integers(0, 256, ws.numel(), dtype=np.uint8)
            junk[: n_words * 8] = words.view(np.uint8)
            ws.copy_(torch.from_numpy(junk))
            before = words.view(np.int64)
            kc, vc = kc0.clone(), vc0.clone()
            if fused:
                out = pa.paged_attn_decode_step(q, dev(t.k_new), dev(t.v_new), kc, vc, tables, lens,
                                                cfg.scale, max_context_len=lay.max_context_len,
                                                workspace=ws, partition_tokens=part)
            else:
                out = pa.paged_attn_decode(q, kc, vc, tables, lens, cfg.scale,
                                           max_context_len=lay.max_context_len, workspace=ws,
                                           partition_tokens=part)
            torch.cuda.synchronize()
            assert_close(host(out), ref, cfg.np_dtype, f"{name}, partition {part}")
            # counters of split segments are released to zero; the others
            # are never touched
            counters = host(ws[: n_words * 8].view(torch.int64))
            assert ((counters == 0) | (counters == before)).all(), name
            assert (counters == 0).sum() >= 64, name


def test_no_workspace_when_no_context_can_split(pa):
    # max_context_len within one partition quantum: no segment is ever split,
    # so the workspace query returns 0 and the call takes no workspace.
    rng = np.random.default_rng(29)
    q, kc, vc, tables, ctx = random_case(rng, np.float32, 40, 32, 8, 64, max_ctx=32)
    desc = pa.decode_desc(dev(q), dev(kc), dev(tables), 32)
    assert pa.partition_quantum(desc) == 32
    assert pa.workspace_bytes(desc) == 0
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.125)
    got = gpu_decode(pa, q, kc, vc, tables, ctx, 0.125, max_ctx=32)
    assert_close(got, ref, np.float32, "no workspace")


def test_hip_graph_replays_match_eager(pa):
    # Write + decode captured in a HIP graph and replayed several times, with
    # eager work in between; every replay must equal the eager result.
    cfg = di.CONFIGS["cb_b64"]
    lay = di.make_layout(cfg)
    t = di.make_layer(cfg, lay)
    q, kn, vn = dev(t.q), dev(t.k_new), dev(t.v_new)
    tables, lens, slots = dev(lay.block_tables), dev(lay.context_lens), dev(lay.slot_mapping)
    kc0, vc0 = dev(t.k_cache), dev(t.v_cache)
    desc = pa.decode_desc(q, kc0, tables, lay.max_context_len)
    ws = pa.new_workspace(pa.workspace_bytes(desc), "cuda:0")
    kc, vc = kc0.clone(), vc0.clone()
    eager = torch.empty_like(q)
    pa.kv_cache_write(kn, vn, slots, kc, vc)
    pa.paged_attn_decode(q, kc, vc, tables, lens, cfg.scale, max_context_len=lay.max_context_len,
                         out=eager, workspace=ws)
    torch.cuda.synchronize()
    kc, vc = kc0.clone(), vc0.clone()
    out = torch.zeros_like(q)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pa.kv_cache_write(kn, vn, slots, kc, vc)
        pa.paged_attn_decode(q, kc, vc, tables, lens, cfg.scale,
                             max_context_len=lay.max_context_len, out=out, workspace=ws)
    for rep in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert host(out).tobytes() == host(eager).tobytes(), f"replay {rep} differs"
        # eager work between replays, on the same workspace
        other = pa.paged_attn_decode(q, kc, vc, tables, lens, cfg.scale,
                                     max_context_len=lay.max_context_len, workspace=ws)
        torch.cuda.synchronize()
        assert host(other).tobytes() == host(eager).tobytes()


# --------------------------------------------------------- fused decode step

def derived_slots(tables, ctx, bs=16):
    """Slot of position ctx-1 of each sequence (-1 for an empty context)."""
    out = np.full(len(ctx), -1, np.int32)
    for b, c in enumerate(ctx):
        if c > 0:
            out[b] = tables[b, (c - 1) // bs] * bs + (c - 1) % bs
    return out


@pytest.mark.parametrize("name", ["tiny", "llama1b_b1", "llama1b_b16", "cb_b64", "llama1b_b16_bf16"])
def test_fused_step_equals_write_then_decode(pa, name):
    cfg = di.CONFIGS[name]
    lay = di.make_layout(cfg)
    t = di.make_layer(cfg, lay, 1)
    slots = derived_slots(lay.block_tables, lay.context_lens)
    assert (slots == lay.slot_mapping).all()
    ek, ev = oracle.kv_cache_write(t.k_new, t.v_new, slots, t.k_cache, t.v_cache)
    ref = oracle.paged_attn_decode(t.q, ek, ev, lay.block_tables, lay.context_lens, cfg.scale)
    q, kn, vn = dev(t.q), dev(t.k_new), dev(t.v_new)
    tables, lens = dev(lay.block_tables), dev(lay.context_lens)
    # fused
    gk, gv = dev(t.k_cache), dev(t.v_cache)
    fused = pa.paged_attn_decode_step(q, kn, vn, gk, gv, tables, lens, cfg.scale,
                                      max_context_len=lay.max_context_len)
    # unfused: the cache-write kernel, then the decode kernel
    uk, uv = dev(t.k_cache), dev(t.v_cache)
    pa.kv_cache_write(kn, vn, dev(slots), uk, uv)
    unfused = pa.paged_attn_decode(q, uk, uv, tables, lens, cfg.scale,
                                   max_context_len=lay.max_context_len)
    torch.cuda.synchronize()
    assert host(gk).tobytes() == ek.tobytes() and host(gv).tobytes() == ev.tobytes()
    assert host(fused).tobytes() == host(unfused).tobytes()
    assert_close(host(fused), ref, cfg.np_dtype, name)


@pytest.mark.parametrize("part", [0, 32, 64, 128, 512])
def test_fused_step_ragged_batch_and_partitions(pa, part):
    # empty contexts, contexts ending on a block boundary, and partition
    # sizes that put a segment's last chunk in the middle of a wave's slice
    rng = np.random.default_rng(31)
    ctx = [0, 1, 16, 17, 31, 32, 33, 300, 0, 1000, 64, 2]
    q, kc, vc, tables, ctx = random_case(rng, np.float32, 0, 32, 8, 64, ctx_list=ctx, spare=5)
    kn = rng.standard_normal((len(ctx), 8, 64)).astype(np.float32)
    vn = rng.standard_normal((len(ctx), 8, 64)).astype(np.float32)
    slots = derived_slots(tables, ctx)
    ek, ev = oracle.kv_cache_write(kn, vn, slots, kc, vc)
    ref = oracle.paged_attn_decode(q, ek, ev, tables, ctx, 0.125)
    gk, gv = dev(kc), dev(vc)
    out = pa.paged_attn_decode_step(dev(q), dev(kn), dev(vn), gk, gv, dev(tables), dev(ctx), 0.125,
                                    max_context_len=int(ctx.max()), partition_tokens=part)
    torch.cuda.synchronize()
    assert host(gk).tobytes() == ek.tobytes() and host(gv).tobytes() == ev.tobytes()
    got = host(out)
    assert_close(got, ref, np.float32, f"partition {part}")
    assert (got[0] == 0).all() and (got[8] == 0).all()


@pytest.mark.parametrize("dtype", [np.float32, di.BF16])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_fused_step_every_group(pa, dtype, group, d):
    # up to four query heads per KV head a wave keeps two chunks in flight,
    # with eight one; pieces of one, two and many chunks append the new row
    rng = np.random.default_rng(32 + group + d)
    ctx = [1, 17, 40, 65, 700, 2, 129, 31, 0, 300]
    hkv = 2
    q, kc, vc, tables, ctx = random_case(rng, dtype, 0, hkv * group, hkv, d, ctx_list=ctx, spare=4)
    kn = di.cast(rng.standard_normal((len(ctx), hkv, d)), dtype)
    vn = di.cast(rng.standard_normal((len(ctx), hkv, d)), dtype)
    slots = derived_slots(tables, ctx)
    ek, ev = oracle.kv_cache_write(kn, vn, slots, kc, vc)
    ref = oracle.paged_attn_decode(q, ek, ev, tables, ctx, 0.09)
    gk, gv = dev(kc), dev(vc)
    for part in (0, 64):
        gk.copy_(dev(kc))
        gv.copy_(dev(vc))
        out = pa.paged_attn_decode_step(dev(q), dev(kn), dev(vn), gk, gv, dev(tables), dev(ctx), 0.09,
                                        max_context_len=int(ctx.max()), partition_tokens=part)
        torch.cuda.synchronize()
        assert host(gk).tobytes() == ek.tobytes() and host(gv).tobytes() == ev.tobytes()
        assert_close(host(out), ref, dtype, f"G{group} d{d} partition {part}")


def test_fused_step_graph_replays_match_eager(pa):
    cfg = di.CONFIGS["cb_b64"]
    lay = di.make_layout(cfg)
    t = di.make_layer(cfg, lay)
    q, kn, vn = dev(t.q), dev(t.k_new), dev(t.v_new)
    tables, lens = dev(lay.block_tables), dev(lay.context_lens)
    desc = pa.decode_desc(q, dev(t.k_cache), tables, lay.max_context_len)
    ws = pa.new_workspace(pa.workspace_bytes(desc), "cuda:0")
    kc, vc = dev(t.k_cache), dev(t.v_cache)
    eager = pa.paged_attn_decode_step(q, kn, vn, kc, vc, tables, lens, cfg.scale,
                                      max_context_len=lay.max_context_len, workspace=ws)
    torch.cuda.synchronize()
    out = torch.zeros_like(q)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pa.paged_attn_decode_step(q, kn, vn, kc, vc, tables, lens, cfg.scale,
                                  max_context_len=lay.max_context_len, out=out, workspace=ws)
    for rep in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert host(out).tobytes() == host(eager).tobytes(), f"replay {rep} differs"


# ---------------------------------------------------------------- limits

def test_decode_at_the_largest_batch(pa):
    # 2048 sequences (the most a call takes), ragged short contexts with
    # empty ones mixed in, through the fused step and the plain decode
    rng = np.random.default_rng(40)
    ctx = rng.integers(0, 80, 2048).astype(np.int32)
    ctx[::97] = 0
    q, kc, vc, tables, ctx = random_case(rng, np.float16, 0, 16, 8, 64, ctx_list=ctx)
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.125)
    got = gpu_decode(pa, q, kc, vc, tables, ctx, 0.125)
    assert_close(got, ref, np.float16, "B=2048")
    assert (di.as_float64(got[ctx == 0]) == 0).all()


def test_context_filling_the_whole_table(pa):
    # every sequence uses every entry of its table row, the last block full
    rng = np.random.default_rng(41)
    ctx = [16 * 40] * 3 + [16 * 40 - 1]
    q, kc, vc, tables, ctx = random_case(rng, np.float32, 0, 32, 8, 64, ctx_list=ctx)
    assert tables.shape[1] * 16 == int(ctx.max())
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.125)
    for part in (0, 32, 640):
        got = gpu_decode(pa, q, kc, vc, tables, ctx, 0.125, max_ctx=tables.shape[1] * 16, part=part)
        assert_close(got, ref, np.float32, f"full tables, partition {part}")


def test_cache_write_many_tokens(pa):
    # 65536 tokens into a pool of 8192 blocks: bit-exact over the whole pool
    rng = np.random.default_rng(42)
    nb, hkv, d, t = 8192, 8, 64, 65536
    kc = rng.standard_normal((nb, hkv, 16, d)).astype(np.float16)
    vc = rng.standard_normal((nb, hkv, 16, d)).astype(np.float16)
    k = rng.standard_normal((t, hkv, d)).astype(np.float16)
    v = rng.standard_normal((t, hkv, d)).astype(np.float16)
    slots = di.random_injective_slots(nb, 16, t, rng, pad_fraction=0.1)
    ek, ev = oracle.kv_cache_write(k, v, slots, kc, vc)
    gk, gv = dev(kc), dev(vc)
    pa.kv_cache_write(dev(k), dev(v), dev(slots), gk, gv)
    torch.cuda.synchronize()
    assert host(gk).tobytes() == ek.tobytes() and host(gv).tobytes() == ev.tobytes()


def contexts_with_chunks(rng, b, target, ct=32, most=5):
    # b contexts (some empty) whose ceil(ctx / ct) sum to exactly `target`
    chunks = rng.integers(0, most + 1, b)
    while chunks.sum() != target:
        i = int(rng.integers(0, b))
        if chunks.sum() < target and chunks[i] < most:
            chunks[i] += 1
        elif chunks.sum() > target and chunks[i] > 0:
            chunks[i] -= 1
    low = np.maximum((chunks - 1) * ct + 1, 0)
    ctx = np.where(chunks > 0, rng.integers(low, chunks * ct + 1), 0)
    assert int(((ctx + ct - 1) // ct).sum()) == target
    return ctx.astype(np.int32)


@pytest.mark.parametrize("b", [64, 65])
@pytest.mark.parametrize("target", [47, 48, 49, 80, 81, 160])
@pytest.mark.parametrize("part", [0, 64])
def test_split_regimes_around_the_boundary_charge(pa, b, target, part):
    # 32 query / 8 KV heads, D 64: 32-token units, 8 units per 32-token
    # stretch of a sequence.  48 stretches (384 units, three per slice at
    # the 128-wave floor) is where the split starts charging a segment
    # change, 80 (640 units) where slices reach five units; 64 sequences
    # keep the prefix sums in registers, 65 use the workgroup's LDS.  Empty
    # contexts are mixed in.
    rng = np.random.default_rng(1000 + 10 * b + target + part)
    ctx = contexts_with_chunks(rng, b, target)
    q, kc, vc, tables, ctx = random_case(rng, np.float32, 0, 32, 8, 64, ctx_list=ctx)
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.125)
    got = gpu_decode(pa, q, kc, vc, tables, ctx, 0.125, part=part)
    assert_close(got, ref, np.float32, f"B={b} chunks={target} part={part}")
    assert (di.as_float64(got[ctx == 0]) == 0).all()


@pytest.mark.parametrize("b", [64, 65])
def test_split_regimes_bf16_fused_step(pa, b):
    # the same boundary for bf16 storage through the fused append + decode
    rng = np.random.default_rng(2000 + b)
    ctx = contexts_with_chunks(rng, b, 49)
    ctx = np.maximum(ctx, 1).astype(np.int32)
    q, kc, vc, tables, ctx = random_case(rng, di.BF16, 0, 32, 8, 64, ctx_list=ctx)
    k_new = di.cast(rng.standard_normal((b, 8, 64)), di.BF16)
    v_new = di.cast(rng.standard_normal((b, 8, 64)), di.BF16)
    slots = derived_slots(tables, ctx)
    kw, vw = oracle.kv_cache_write(k_new, v_new, slots, kc, vc)
    ref = oracle.paged_attn_decode(q, kw, vw, tables, ctx, 0.125)
    kcd, vcd = dev(kc), dev(vc)
    out = pa.paged_attn_decode_step(dev(q), dev(k_new), dev(v_new), kcd, vcd, dev(tables),
                                    dev(ctx), 0.125, max_context_len=int(ctx.max()))
    torch.cuda.synchronize()
    assert_close(host(out), ref, di.BF16, f"fused B={b}")
    assert host(kcd).tobytes() == kw.tobytes() and host(vcd).tobytes() == vw.tobytes()


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("part", [32, 64, 96, 128, 160])
def test_pieces_of_one_to_five_chunks(pa, dtype, part):
    # Slices of part/32 chunks over contexts of 1-192 tokens give pieces of
    # one to five 32-token chunks, ragged at both ends: the decode loop's
    # one-chunk path, and its exits after an even and after an odd number of
    # chunks (the next chunk's loads are issued before the current one is
    # used, alternating two register sets).  Plain call and fused step.
    rng = np.random.default_rng(3000 + part)
    ctx = rng.integers(1, 6 * 32 + 1, 24).astype(np.int32)
    q, kc, vc, tables, ctx = random_case(rng, dtype, 0, 32, 8, 64, ctx_list=ctx)
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.125)
    assert_close(gpu_decode(pa, q, kc, vc, tables, ctx, 0.125, part=part), ref, dtype,
                 f"part={part}")
    k_new = di.cast(rng.standard_normal((len(ctx), 8, 64)), dtype)
    v_new = di.cast(rng.standard_normal((len(ctx), 8, 64)), dtype)
    kw, vw = oracle.kv_cache_write(k_new, v_new, derived_slots(tables, ctx), kc, vc)
    ref = oracle.paged_attn_decode(q, kw, vw, tables, ctx, 0.125)
    kcd, vcd = dev(kc), dev(vc)
    out = pa.paged_attn_decode_step(dev(q), dev(k_new), dev(v_new), kcd, vcd, dev(tables),
                                    dev(ctx), 0.125, max_context_len=int(ctx.max()),
                                    partition_tokens=part)
    torch.cuda.synchronize()
    assert_close(host(out), ref, dtype, f"fused part={part}")
    assert host(kcd).tobytes() == kw.tobytes() and host(vcd).tobytes() == vw.tobytes()


@pytest.mark.parametrize("dtype", [np.float32, di.BF16])
@pytest.mark.parametrize("n", [2048, 4103, 8192])
def test_one_long_sequence(pa, dtype, n):
    # Batch 1 with 32 query / 8 KV heads: 512-2048 units over 128 or more
    # waves, so each of the eight segments is cut into 16 or more slices
    # (several merge passes) and, from 384 units on, segment changes are
    # charged.  Plain call and fused step.
    rng = np.random.default_rng(4000 + n)
    q, kc, vc, tables, ctx = random_case(rng, dtype, 0, 32, 8, 64, ctx_list=[n])
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.125)
    assert_close(gpu_decode(pa, q, kc, vc, tables, ctx, 0.125), ref, dtype, f"n={n}")
    k_new = di.cast(rng.standard_normal((1, 8, 64)), dtype)
    v_new = di.cast(rng.standard_normal((1, 8, 64)), dtype)
    kw, vw = oracle.kv_cache_write(k_new, v_new, derived_slots(tables, ctx), kc, vc)
    ref = oracle.paged_attn_decode(q, kw, vw, tables, ctx, 0.125)
    kcd, vcd = dev(kc), dev(vc)
    out = pa.paged_attn_decode_step(dev(q), dev(k_new), dev(v_new), kcd, vcd, dev(tables),
                                    dev(ctx), 0.125, max_context_len=n)
    torch.cuda.synchronize()
    assert_close(host(out), ref, dtype, f"fused n={n}")
    assert host(kcd).tobytes() == kw.tobytes() and host(vcd).tobytes() == vw.tobytes()
