"""GPU parity of multi-query paged attention (causal tail) against the fp64 oracle.

Tolerances as for the decode step: max-abs 1e-4 for fp32 output (fp32
storage, or 16-bit storage with fp32 output: products are exact on the
matrix cores and the softmax weights travel as a 16-bit value plus its
rounding residual), 2e-3 for fp16 output, 1e-4 + 2^-8 |ref| for bfloat16
output.  Every output row is compared with the multi-query oracle, the
512-row chunked prefill included; sampled rows of it are also compared with
the decode oracle over the row's prefix (a row at position p equals the
decode step over the first p + 1 tokens, a pinned property of the oracle).
"""
import numpy as np
import pytest
import torch

import decode_inputs as di
import oracle
from tests.test_oracle_multi_query import ragged_case

pytestmark = pytest.mark.gpu

DTYPES = [np.float32, np.float16, di.BF16]


@pytest.fixture(scope="module")
def pa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import paged_attention_decode_photon_amd as mod
    return mod


def dev(a):
    return di.to_torch(a).to("cuda:0")


def tolerance(out_dtype, ref):
    if np.dtype(out_dtype) == di.BF16:
        return 1e-4 + 2.0 ** -8 * np.abs(ref)
    return {np.dtype(np.float32): 1e-4, np.dtype(np.float16): 2e-3}[np.dtype(out_dtype)]


def assert_close(got, ref, out_dtype, what):
    g = di.as_float64(got)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    assert (err <= tolerance(out_dtype, ref)).all(), f"{what}: max-abs error {err.max():.3e}"
    return float(err.max()) if err.size else 0.0


def gpu_mq(pa, q, kc, vc, tables, ctx, qs, scale, out_dtype=None, split=0):
    out = pa.paged_attn_multi_query(dev(q), dev(kc), dev(vc), dev(tables), dev(ctx), dev(qs), scale,
                                    max_query_len=int(np.diff(qs).max()),
                                    max_context_len=int(ctx.max()), out_dtype=out_dtype,
                                    split_tokens=split)
    torch.cuda.synchronize()
    return di.from_torch(out)


QLENS = [0, 1, 3, 5, 8, 16, 2, 37]
EXTRA = [0, 0, 40, 1, 300, 17, 700, 0]   # cached tokens before the new ones


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_every_built_shape(pa, dtype, d, group):
    rng = np.random.default_rng(600 + group * 10 + d + DTYPES.index(dtype))
    hkv = 2
    ctx = [q + e for q, e in zip(QLENS, EXTRA)]
    ctx[0] = 5   # a sequence with no new tokens still has a cache
    q, kc, vc, tables, ctx, qs = ragged_case(rng, dtype, QLENS, ctx, hkv * group, hkv, d, 16)
    scale = float(np.float32(d ** -0.5))
    ref = oracle.paged_attn_multi_query(q, kc, vc, tables, ctx, qs, scale)
    got = gpu_mq(pa, q, kc, vc, tables, ctx, qs, scale)
    assert_close(got, ref, dtype, f"G{group} d{d}")
    if dtype != np.float32:
        got32 = gpu_mq(pa, q, kc, vc, tables, ctx, qs, scale, out_dtype=torch.float32)
        assert got32.dtype == np.float32
        assert_close(got32, ref, np.float32, f"G{group} d{d} fp32 out")


def test_one_new_token_matches_the_decode_kernel_within_tolerance(pa):
    cfg = di.CONFIGS["llama1b_b16"]
    lay = di.make_layout(cfg)
    t = di.make_layer(cfg, lay, 3)
    qs = np.arange(len(lay.context_lens) + 1, dtype=np.int32)
    ref = oracle.paged_attn_decode(t.q, t.k_cache, t.v_cache, lay.block_tables, lay.context_lens,
                                   cfg.scale)
    got = gpu_mq(pa, t.q, t.k_cache, t.v_cache, lay.block_tables, lay.context_lens, qs, cfg.scale)
    assert_close(got, ref, np.float32, "q_len 1")


@pytest.mark.parametrize("dtype", [np.float32, di.BF16])
def test_speculative_verify_shape(pa, dtype):
    # batch 16, four tokens per sequence (a draft of three plus the last
    # accepted one), Llama-3.2-1B heads, contexts of the batch-16 workload
    cfg = di.CONFIGS["llama1b_b16"]
    rng = np.random.default_rng(610)
    lay = di.make_layout(cfg)
    n = 4
    q = di.cast(rng.standard_normal((16 * n, 32, 64)), dtype)
    kc = di.cast(rng.standard_normal((lay.num_blocks, 8, 16, 64)), dtype)
    vc = di.cast(rng.standard_normal((lay.num_blocks, 8, 16, 64)), dtype)
    qs = np.arange(0, 16 * n + 1, n, dtype=np.int32)
    ref = oracle.paged_attn_multi_query(q, kc, vc, lay.block_tables, lay.context_lens, qs, cfg.scale)
    got = gpu_mq(pa, q, kc, vc, lay.block_tables, lay.context_lens, qs, cfg.scale)
    assert_close(got, ref, dtype, "speculative verify")


def test_chunked_prefill_every_row(pa):
    # four sequences, each computing a 512-token chunk of a longer prompt
    # (1836 query rows); every row is compared with the multi-query oracle,
    # and sampled rows also with the decode oracle over the row's prefix
    rng = np.random.default_rng(611)
    qlens, ctx = [512, 512, 300, 512], [2048, 512, 1500, 4000]
    q, kc, vc, tables, ctx, qs = ragged_case(rng, np.float16, qlens, ctx, 32, 8, 64, 16)
    got = gpu_mq(pa, q, kc, vc, tables, ctx, qs, 0.125)
    ref = oracle.paged_attn_multi_query(q, kc, vc, tables, ctx, qs, 0.125)
    assert_close(got, ref, np.float16, "chunked prefill, all rows")
    for b in range(4):
        for j in (0, 1, 255, qlens[b] - 1):
            row = qs[b] + j
            p = ctx[b] - qlens[b] + j
            ref = oracle.paged_attn_decode(q[row:row + 1], kc, vc, tables[b:b + 1],
                                           np.array([p + 1], np.int32), 0.125)
            assert_close(got[row:row + 1], ref, np.float16, f"seq {b} row {j}")


def test_unread_slots_and_future_keys_never_reach_a_row(pa):
    rng = np.random.default_rng(612)
    q, kc, vc, tables, ctx, qs = ragged_case(rng, np.float32, [6, 3], [50, 9], 8, 2, 64, 16, spare=4)
    base = gpu_mq(pa, q, kc, vc, tables, ctx, qs, 0.125)
    kp, vp = kc.copy(), vc.copy()
    used = np.zeros(kc.shape[0], bool)
    for b, c in enumerate(ctx):
        nblk = -(-int(c) // 16)
        used[tables[b, :nblk]] = True
        if c % 16:
            kp[tables[b, nblk - 1], :, c % 16:] = np.nan
            vp[tables[b, nblk - 1], :, c % 16:] = np.nan
    kp[~used] = np.nan
    vp[~used] = np.nan
    assert (gpu_mq(pa, q, kp, vp, tables, ctx, qs, 0.125) == base).all()
    # a key and value at position 46 are seen by rows at 46..49 only
    blk, off = tables[0, 46 // 16], 46 % 16
    kp[blk, :, off] = 30.0
    vp[blk, :, off] = -5.0
    got = gpu_mq(pa, q, kp, vp, tables, ctx, qs, 0.125)
    assert (got[:2] == base[:2]).all() and (got[6:] == base[6:]).all()
    assert not np.allclose(got[2:6], base[2:6])


def test_repeat_is_bit_identical(pa):
    rng = np.random.default_rng(613)
    q, kc, vc, tables, ctx, qs = ragged_case(rng, di.BF16, [9, 33, 1], [400, 33, 2000], 16, 8, 128, 16)
    a = gpu_mq(pa, q, kc, vc, tables, ctx, qs, 0.09)
    b = gpu_mq(pa, q, kc, vc, tables, ctx, qs, 0.09)
    assert a.tobytes() == b.tobytes()


@pytest.mark.parametrize("dtype", [np.float32, di.BF16])
@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.7])
@pytest.mark.parametrize("longest", [2, 40])
def test_any_finite_scale(pa, dtype, scale, longest):
    # positive scales fold into the exponent, others are applied first; a
    # zero scale averages the visible rows.  A longest query run of 2 tokens
    # (8 rows) runs the per-tile kernel, one of 40 (160 rows) the wide one.
    rng = np.random.default_rng(630)
    qlens, ctx = [3 if longest > 3 else 1, longest, 1], [300, 900, 17]
    q, kc, vc, tables, ctx, qs = ragged_case(rng, dtype, qlens, ctx, 8, 2, 64, 16)
    ref = oracle.paged_attn_multi_query(q, kc, vc, tables, ctx, qs, scale)
    got = gpu_mq(pa, q, kc, vc, tables, ctx, qs, scale)
    assert_close(got, ref, dtype, f"scale {scale}")


@pytest.mark.parametrize("split", [0, 64, 128, 512, 4096])
def test_kv_split_sizes_agree_with_oracle(pa, split):
    # long contexts with short and long query runs: many tiles span several
    # splits, some rows see none of a split's keys
    rng = np.random.default_rng(620)
    qlens, ctx = [1, 4, 20, 64, 3], [3000, 1500, 700, 2100, 64]
    q, kc, vc, tables, ctx, qs = ragged_case(rng, np.float32, qlens, ctx, 8, 2, 64, 16)
    ref = oracle.paged_attn_multi_query(q, kc, vc, tables, ctx, qs, 0.125)
    got = gpu_mq(pa, q, kc, vc, tables, ctx, qs, 0.125, split=split)
    assert_close(got, ref, np.float32, f"split {split}")


def test_split_workspace_reused_stays_zeroed(pa):
    rng = np.random.default_rng(621)
    q, kc, vc, tables, ctx, qs = ragged_case(rng, np.float16, [4, 4, 9], [900, 2000, 40], 16, 4, 128, 16)
    ref = oracle.paged_attn_multi_query(q, kc, vc, tables, ctx, qs, 0.09)
    args = [dev(q), dev(kc), dev(vc), dev(tables), dev(ctx), dev(qs)]
    sizes = {}
    for split in (64, 256, 0):
        d = pa.multi_query_desc(args[0], args[1], args[3], 3, 9, int(ctx.max()), split)
        sizes[split] = pa.multi_query_workspace_bytes(d)
    assert all(v > 0 for v in sizes.values())
    ws = pa.new_workspace(max(sizes.values()), "cuda:0")
    ws.zero_()
    tiles = 3 * 4 * ((9 * 4 + 15) // 16)
    for rep in range(3):
        for split in (64, 256, 0):
            before = np.zeros(tiles, np.int64)
            if rep == 2:  # arbitrary contents before the call (counters and records)
                junk = rng.integers(0, 256, ws.numel(), dtype=np.uint8)
                ws.copy_(torch.from_numpy(junk))
                before = junk[: tiles * 8].view(np.int64)
            out = pa.paged_attn_multi_query(*args, 0.09, max_query_len=9, max_context_len=int(ctx.max()),
                                            workspace=ws, split_tokens=split)
            torch.cuda.synchronize()
            assert_close(di.from_torch(out), ref, np.float16, f"split {split} rep {rep}")
            # counters of split tiles are released to zero; the others are
            # never touched
            counters = ws[: tiles * 8].view(torch.int64).cpu().numpy()
            assert ((counters == 0) | (counters == before)).all()
            assert (counters == 0).any()
