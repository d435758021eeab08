"""Pins for the oracle's multi-query paged attention with a causal tail.

Checked against things the oracle does not use: torch's float64
scaled_dot_product_attention with an explicit causal mask on the gathered
K/V, the single-query decode oracle (pinned separately) when every sequence
has one new token, closed forms (a row that sees one token returns that
token's V row), and causality (keys past a row's position cannot change it).
"""
import math

import numpy as np
import pytest
import torch

import decode_inputs as di
import oracle


def ragged_case(rng, dtype, qlens, ctxs, hq, hkv, d, bs, spare=2):
    qlens = np.array(qlens, np.int64)
    ctx = np.array(ctxs, np.int32)
    b = len(ctx)
    need = (ctx.astype(np.int64) + bs - 1) // bs
    nb = int(need.sum()) + spare
    mb = max(int(need.max()), 1)
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((b, mb), -1, np.int32)
    p = 0
    for i, n in enumerate(need):
        tables[i, :n] = perm[p:p + n]
        p += n
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = di.cast(rng.standard_normal((int(qs[-1]), hq, d)), dtype)
    kc = di.cast(rng.standard_normal((nb, hkv, bs, d)), dtype)
    vc = di.cast(rng.standard_normal((nb, hkv, bs, d)), dtype)
    return q, kc, vc, tables, ctx, qs


def dense_causal_sdpa(q, kc, vc, tables, ctx, qs, scale):
    t_all, hq, d = q.shape
    hkv, bs = kc.shape[1], kc.shape[2]
    grp = hq // hkv
    out = np.zeros((t_all, hq, d))
    for b in range(len(ctx)):
        n, c = int(qs[b + 1] - qs[b]), int(ctx[b])
        if n == 0:
            continue
        t = np.arange(c)
        k = di.as_float64(kc[tables[b, t // bs], :, t % bs, :])   # [c, Hkv, d]
        v = di.as_float64(vc[tables[b, t // bs], :, t % bs, :])
        kt = torch.from_numpy(np.ascontiguousarray(np.repeat(k.transpose(1, 0, 2), grp, axis=0)))
        vt = torch.from_numpy(np.ascontiguousarray(np.repeat(v.transpose(1, 0, 2), grp, axis=0)))
        qt = torch.from_numpy(np.ascontiguousarray(di.as_float64(q[qs[b]:qs[b + 1]]).transpose(1, 0, 2)))
        pos = c - n + np.arange(n)
        mask = torch.from_numpy(t[None, :] <= pos[:, None])            # [n, c], True = attend
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
        out[qs[b]:qs[b + 1]] = o.numpy().transpose(1, 0, 2)
    return out


@pytest.mark.parametrize("dtype", [np.float32, np.float16, di.BF16])
@pytest.mark.parametrize("seed", range(4))
def test_matches_torch_sdpa_with_causal_mask(dtype, seed):
    rng = np.random.default_rng(500 + seed)
    hkv = int(rng.choice([1, 2]))
    grp = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([8, 64]))
    bs = int(rng.choice([1, 4, 16]))
    b = int(rng.integers(1, 5))
    qlens = rng.integers(0, 9, b)
    ctxs = qlens + rng.integers(0, 40, b)
    ctxs[0] = max(ctxs[0], 1)
    qlens[0] = max(qlens[0], 1)
    q, kc, vc, tables, ctx, qs = ragged_case(rng, dtype, qlens, ctxs, hkv * grp, hkv, d, bs)
    scale = float(np.float32(1 / math.sqrt(d)))
    got = oracle.paged_attn_multi_query(q, kc, vc, tables, ctx, qs, scale)
    ref = dense_causal_sdpa(q, kc, vc, tables, ctx, qs, scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_one_new_token_per_sequence_is_the_decode_step():
    rng = np.random.default_rng(510)
    q, kc, vc, tables, ctx, qs = ragged_case(rng, np.float32, [1] * 6, [1, 5, 16, 17, 40, 100],
                                             8, 2, 64, 16)
    got = oracle.paged_attn_multi_query(q, kc, vc, tables, ctx, qs, 0.125)
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.125)
    assert np.array_equal(got, ref)


def test_whole_prompt_rows_are_prefix_decodes():
    # A prompt computed at once: row j sees exactly positions 0..j, so it
    # equals a decode step over a context of j + 1 tokens; row 0 returns V[0].
    rng = np.random.default_rng(511)
    n = 37
    q, kc, vc, tables, ctx, qs = ragged_case(rng, np.float16, [n], [n], 4, 1, 64, 16)
    got = oracle.paged_attn_multi_query(q, kc, vc, tables, ctx, qs, 0.2)
    v0 = di.as_float64(vc[tables[0, 0], 0, 0])
    assert np.array_equal(got[0], np.broadcast_to(v0, (4, 64)))
    for j in (1, 15, 16, 36):
        ref = oracle.paged_attn_decode(q[j:j + 1], kc, vc, tables, np.array([j + 1], np.int32), 0.2)
        assert np.array_equal(got[j], ref[0])


def test_keys_past_a_rows_position_cannot_change_it():
    rng = np.random.default_rng(512)
    q, kc, vc, tables, ctx, qs = ragged_case(rng, np.float32, [5], [30], 4, 2, 64, 4)
    base = oracle.paged_attn_multi_query(q, kc, vc, tables, ctx, qs, 0.3)
    # rows sit at positions 25..29; overwrite position 27 in K and V
    blk, off = tables[0, 27 // 4], 27 % 4
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[blk, :, off] = 50.0
    vc2[blk, :, off] = -7.0
    got = oracle.paged_attn_multi_query(q, kc2, vc2, tables, ctx, qs, 0.3)
    assert np.array_equal(got[:2], base[:2])          # positions 25, 26 do not see 27
    assert not np.allclose(got[2:], base[2:])          # 27, 28, 29 do


def test_multi_query_preconditions():
    kc = np.zeros((4, 1, 4, 8), np.float32)
    q = np.zeros((3, 2, 8), np.float32)
    tables = np.array([[0, 1, 2]], np.int32)
    for ctx, qs, code in [([2], [0, 3], oracle.ERR_CTX),        # fewer cached tokens than rows
                          ([13], [0, 3], oracle.ERR_CTX),       # past the table
                          ([5], [1, 3], oracle.ERR_ARG)]:       # must start at 0
        with pytest.raises(oracle.OracleError) as e:
            oracle.paged_attn_multi_query(q[:qs[1] - qs[0]] if qs[0] else q, kc, kc, tables,
                                          np.array(ctx, np.int32), np.array(qs, np.int32), 1.0)
        assert e.value.code == code
