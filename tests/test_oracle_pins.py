"""Pins for the CPU oracle: checks against facts that do not come from the oracle itself.

Each test pins the oracle to something fixed by the mathematics or by a
library routine that the oracle does not use: hand-worked golden cases,
dense attention via torch's scaled_dot_product_attention, closed forms,
invariances, and exhaustive decoding of binary16 and bfloat16 (against
numpy's and torch's own conversions).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import decode_inputs as di
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    if isinstance(x, str):
        neg = x.startswith("-")
        s = x.lstrip("-")
        if s.startswith("ln"):
            v = math.log(float(s[2:]))
        else:
            v = float(Fraction(s))
        return -v if neg else v
    return float(x)


def _arr(nested):
    return np.vectorize(_num, otypes=[np.float64])(np.array(nested, dtype=object))


# ---------------------------------------------------------------- golden cases

def test_golden_two_blocks_gqa():
    g = json.load(open(os.path.join(GOLDEN, "attn_two_blocks_gqa.json")))
    nb, hkv, bs, d = g["num_blocks"], g["num_kv_heads"], g["block_size"], g["head_dim"]
    table = np.array(g["block_tables"], dtype=np.int32)
    ctx = np.array(g["context_lens"], dtype=np.int32)
    kc = np.full((nb, hkv, bs, d), g["unread_fill"], dtype=np.float32)
    vc = kc.copy()
    lk, lv = _arr(g["logical_k"]), _arr(g["logical_v_head0"])
    for t in range(int(ctx[0])):
        blk, off = table[0, t // bs], t % bs
        kc[blk, :, off, :] = lk[t]
        vc[blk, 0, off, :] = lv[t]
        vc[blk, 1, off, :] = -lv[t]
    q = _arr(g["q"]).astype(np.float32)
    out = oracle.paged_attn_decode(q, kc, vc, table, ctx, g["scale"])
    np.testing.assert_allclose(out, _arr(g["expected_out"]), rtol=0, atol=g["tolerance"])


def test_golden_cache_write():
    g = json.load(open(os.path.join(GOLDEN, "cache_write_tiny.json")))
    shape = (g["num_blocks"], g["num_kv_heads"], g["block_size"], g["head_dim"])
    kc = np.full(shape, g["fill"], dtype=np.float32)
    vc = kc.copy()
    k = np.array(g["k"], dtype=np.float32)
    nk, nv = oracle.kv_cache_write(k, -k, np.array(g["slot_mapping"], np.int32), kc, vc)
    np.testing.assert_array_equal(nk.ravel(), np.array(g["expected_k_cache"], np.float32))
    np.testing.assert_array_equal(nv.ravel(), np.array(g["expected_v_cache"], np.float32))
    assert (kc == g["fill"]).all(), "oracle must not modify its inputs"


# ------------------------------------------------------ dense library cross-check

def _dense_sdpa(q, kc, vc, tables, ctx, scale):
    """Gather each sequence's logical K/V and run torch SDPA in float64 on the CPU."""
    b, hq, d = q.shape
    hkv, bs = kc.shape[1], kc.shape[2]
    grp = hq // hkv
    out = np.zeros((b, hq, d))
    for i in range(b):
        c = int(ctx[i])
        if c == 0:
            continue
        t = np.arange(c)
        k = di.as_float64(kc[tables[i, t // bs], :, t % bs, :])  # [c, Hkv, d]
        v = di.as_float64(vc[tables[i, t // bs], :, t % bs, :])
        kt = torch.from_numpy(np.ascontiguousarray(np.repeat(k.transpose(1, 0, 2), grp, axis=0)))
        vt = torch.from_numpy(np.ascontiguousarray(np.repeat(v.transpose(1, 0, 2), grp, axis=0)))
        qt = torch.from_numpy(di.as_float64(q[i])[:, None, :])
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=float(scale))
        out[i] = o[:, 0, :].numpy()
    return out


def _random_case(rng, dtype, b, hq, hkv, d, bs, max_ctx, spare=2):
    ctx = rng.integers(0, max_ctx + 1, b).astype(np.int32)
    ctx[0] = max_ctx
    need = (ctx + bs - 1) // bs
    nb = int(need.sum()) + spare
    mb = int(need.max())
    perm = rng.permutation(nb).astype(np.int32)
    tables = np.full((b, mb), -1, np.int32)
    p = 0
    for i, n in enumerate(need):
        tables[i, :n] = perm[p:p + n]
        p += n
    q = di.cast(rng.standard_normal((b, hq, d)), dtype)
    kc = di.cast(rng.standard_normal((nb, hkv, bs, d)), dtype)
    vc = di.cast(rng.standard_normal((nb, hkv, bs, d)), dtype)
    return q, kc, vc, tables, ctx


@pytest.mark.parametrize("dtype", [np.float32, np.float16, di.BF16])
@pytest.mark.parametrize("seed", range(6))
def test_matches_torch_sdpa_float64(dtype, seed):
    rng = np.random.default_rng(100 + seed)
    hkv = int(rng.choice([1, 2, 4]))
    grp = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([4, 8, 64]))
    bs = int(rng.choice([1, 4, 16]))
    q, kc, vc, tables, ctx = _random_case(rng, dtype, int(rng.integers(1, 5)), hkv * grp, hkv,
                                          d, bs, int(rng.integers(1, 65)))
    scale = float(np.float32(1 / math.sqrt(d)))
    got = oracle.paged_attn_decode(q, kc, vc, tables, ctx, scale)
    ref = _dense_sdpa(q, kc, vc, tables, ctx, scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_tiny_config_matches_sdpa():
    cfg = di.CONFIGS["tiny"]
    lay = di.make_layout(cfg)
    t = di.make_layer(cfg, lay)
    got = oracle.paged_attn_decode(t.q, t.k_cache, t.v_cache, lay.block_tables,
                                   lay.context_lens, cfg.scale)
    ref = _dense_sdpa(t.q, t.k_cache, t.v_cache, lay.block_tables, lay.context_lens, cfg.scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# -------------------------------------------------------------- closed forms

def _single_seq(rng, dtype, ctx, hq=4, hkv=2, d=16, bs=4):
    q, kc, vc, tables, _ = _random_case(rng, dtype, 1, hq, hkv, d, bs, ctx, spare=1)
    return q, kc, vc, tables, np.array([ctx], np.int32)


@pytest.mark.parametrize("dtype", [np.float32, np.float16, di.BF16])
def test_one_token_returns_its_value_row(dtype):
    rng = np.random.default_rng(7)
    q, kc, vc, tables, ctx = _single_seq(rng, dtype, 1)
    out = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.3)
    v0 = di.as_float64(vc[tables[0, 0], :, 0, :])  # [Hkv, d]
    np.testing.assert_array_equal(out[0], np.repeat(v0, 2, axis=0))


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(8)
    q, kc, vc, tables, ctx = _single_seq(rng, np.float32, 23)
    q[:] = 0
    out = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.25)
    t = np.arange(23)
    v = vc[tables[0, t // 4], :, t % 4, :].astype(np.float64)  # [23, Hkv, d]
    np.testing.assert_allclose(out[0], np.repeat(v.mean(axis=0), 2, axis=0), rtol=0, atol=1e-12)


def test_constant_values_pass_through():
    rng = np.random.default_rng(9)
    q, kc, vc, tables, ctx = _single_seq(rng, np.float32, 19)
    c = rng.standard_normal(16).astype(np.float32)
    vc[:] = c
    out = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 1.0)
    np.testing.assert_allclose(out[0], np.broadcast_to(c, (4, 16)), rtol=0, atol=1e-12)


@pytest.mark.parametrize("lam", [30.0, 1000.0])
def test_dominant_key_selects_its_value(lam):
    # One key parallel to the query with a huge score: the softmax puts all
    # weight on it.  At lam=1000 the scores exceed exp's range, so a missing
    # maximum subtraction would give inf/NaN.
    rng = np.random.default_rng(10)
    q, kc, vc, tables, ctx = _single_seq(rng, np.float32, 21, hq=1, hkv=1)
    q[0, 0] /= np.linalg.norm(q[0, 0])
    star = 13
    blk, off = tables[0, star // 4], star % 4
    kc[blk, 0, off] = lam * q[0, 0]
    out = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 1.0)
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out[0, 0], vc[blk, 0, off].astype(np.float64), rtol=0, atol=1e-6)


def test_empty_context_gives_zero_row():
    rng = np.random.default_rng(11)
    q, kc, vc, tables, _ = _random_case(rng, np.float32, 3, 4, 2, 8, 4, 9)
    ctx = np.array([9, 0, 5], np.int32)
    out = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.5)
    assert (out[1] == 0).all()
    ref = _dense_sdpa(q, kc, vc, tables, ctx, 0.5)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariances

@pytest.mark.parametrize("dtype", [np.float32, np.float16, di.BF16])
def test_physical_block_permutation_is_bit_identical(dtype):
    rng = np.random.default_rng(12)
    q, kc, vc, tables, ctx = _random_case(rng, dtype, 4, 8, 2, 16, 4, 45, spare=5)
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.25)
    pi = rng.permutation(kc.shape[0])
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[pi], vc2[pi] = kc, vc
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1).astype(np.int32)
    got = oracle.paged_attn_decode(q, kc2, vc2, t2, ctx, 0.25)
    assert np.array_equal(got, ref)


def test_gqa_equals_mha_with_repeated_kv_heads():
    rng = np.random.default_rng(13)
    grp = 4
    q, kc, vc, tables, ctx = _random_case(rng, np.float32, 3, 2 * grp, 2, 16, 4, 30)
    ref = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.25)
    kr = np.ascontiguousarray(np.repeat(kc, grp, axis=1))
    vr = np.ascontiguousarray(np.repeat(vc, grp, axis=1))
    got = oracle.paged_attn_decode(q, kr, vr, tables, ctx, 0.25)
    assert np.array_equal(got, ref)


def test_softmax_rows_sum_to_one_and_vanish_past_context():
    rng = np.random.default_rng(14)
    q, kc, vc, tables, ctx = _random_case(rng, np.float32, 5, 8, 4, 32, 16, 70)
    _, p = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 0.2, return_probs=True)
    for i, c in enumerate(ctx):
        if c == 0:
            assert (p[i] == 0).all()
            continue
        np.testing.assert_allclose(p[i, :, :c].sum(axis=1), 1.0, rtol=0, atol=1e-12)
        assert (p[i, :, c:] == 0).all()
        assert (p[i, :, :c] > 0).all()


def test_unread_slots_never_reach_the_output():
    # NaN in every slot past a context and in every block no table uses.
    cfg = di.CONFIGS["tiny"]
    lay = di.make_layout(cfg)
    t = di.make_layer(cfg, lay)
    ref = oracle.paged_attn_decode(t.q, t.k_cache, t.v_cache, lay.block_tables,
                                   lay.context_lens, cfg.scale)
    kp = di.poison_unused(cfg, lay, t.k_cache)
    vp = di.poison_unused(cfg, lay, t.v_cache)
    assert np.isnan(kp).sum() > 0
    assert np.isnan(di.as_float64(kp)).sum() == np.isnan(kp).sum()
    got = oracle.paged_attn_decode(t.q, kp, vp, lay.block_tables, lay.context_lens, cfg.scale)
    assert np.array_equal(got, ref)


# -------------------------------------------------------------- binary16

def test_half_decoder_matches_numpy_on_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    # The pool path widens through the decoder: route every pattern through
    # a one-token attention (ctx 1 -> out equals the V row exactly).
    d = 64
    vals = bits.view(np.float16).reshape(-1, d)  # 1024 rows of 64
    n = vals.shape[0]
    vc = np.ascontiguousarray(vals.reshape(n, 1, 1, d))
    kc = np.zeros_like(vc)
    q = np.zeros((n, 1, d), np.float16)
    tables = np.arange(n, dtype=np.int32).reshape(n, 1)
    ctx = np.ones(n, np.int32)
    out = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 1.0)
    got = out.reshape(-1)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # and the scalar entry point on a spread of patterns
    for b in [0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x7C00, 0xFC00, 0xC000]:
        assert oracle.half_to_double(b) == float(np.uint16(b).view(np.float16))


# ------------------------------------------------------------- bfloat16

def test_bfloat16_decoder_matches_torch_on_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    d = 64
    vals = bits.view(di.BF16).reshape(-1, d)
    n = vals.shape[0]
    vc = np.ascontiguousarray(vals.reshape(n, 1, 1, d))
    kc = np.zeros(vc.shape, np.uint16).view(di.BF16)
    q = np.zeros((n, 1, d), np.uint16).view(di.BF16)
    tables = np.arange(n, dtype=np.int32).reshape(n, 1)
    ctx = np.ones(n, np.int32)
    got = oracle.paged_attn_decode(q, kc, vc, tables, ctx, 1.0).reshape(-1)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # the scalar entry point: zero, subnormals, one, the largest finite, infinities
    for b, v in [(0x0000, 0.0), (0x0001, 2.0 ** -133), (0x007F, 127 * 2.0 ** -133),
                 (0x0080, 2.0 ** -126), (0x3F80, 1.0), (0xBFC0, -1.5),
                 (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127), (0x7F80, math.inf), (0xFF80, -math.inf)]:
        assert oracle.bfloat16_to_double(b) == v
    assert math.isnan(oracle.bfloat16_to_double(0x7FC0))


def test_bfloat16_rounding_of_inputs_matches_torch():
    # The input generator rounds float32 draws to bfloat16 itself; torch's
    # float32 -> bfloat16 conversion (round to nearest even) must agree.
    x = np.random.default_rng(16).standard_normal(1 << 16).astype(np.float32)
    x[:6] = [1.00390625, 1.01171875, -1.00390625, 3.0e38, 1e-39, 0.0]  # ties and edges
    got = di.to_storage(x, di.BF16).view(np.uint16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------- cache write

@pytest.mark.parametrize("dtype", [np.float32, np.float16, di.BF16])
def test_cache_write_brute_force(dtype):
    rng = np.random.default_rng(15)
    nb, hkv, bs, d, t = 12, 3, 16, 64, 40
    kc = di.cast(rng.standard_normal((nb, hkv, bs, d)), dtype)
    vc = di.cast(rng.standard_normal((nb, hkv, bs, d)), dtype)
    k = di.cast(rng.standard_normal((t, hkv, d)), dtype)
    v = di.cast(rng.standard_normal((t, hkv, d)), dtype)
    slots = di.random_injective_slots(nb, bs, t, rng, pad_fraction=0.2)
    assert (slots == -1).any()
    nk, nv = oracle.kv_cache_write(k, v, slots, kc, vc)
    ek, ev = kc.copy(), vc.copy()
    touched = np.zeros((nb, bs), bool)
    for i in range(t):
        s = int(slots[i])
        if s < 0:
            continue
        for h in range(hkv):
            ek[s // bs, h, s % bs] = k[i, h]
            ev[s // bs, h, s % bs] = v[i, h]
        touched[s // bs, s % bs] = True
    assert nk.tobytes() == ek.tobytes() and nv.tobytes() == ev.tobytes()
    untouched = ~touched
    assert nk.transpose(0, 2, 1, 3)[untouched].tobytes() == \
        kc.transpose(0, 2, 1, 3)[untouched].tobytes()


def test_cache_write_copies_raw_bits():
    # NaN payloads and subnormals survive: the write copies bytes.
    bits = np.array([0x7E01, 0xFC00, 0x0001, 0x8001, 0x7C00, 0x3555, 0x7D55, 0xFFFF], np.uint16)
    k = np.tile(bits, 8).view(np.float16).reshape(1, 1, 64)
    kc = np.zeros((2, 1, 16, 64), np.float16)
    nk, nv = oracle.kv_cache_write(k, k, np.array([17], np.int32), kc, kc)
    assert nk[1, 0, 1].view(np.uint16).tobytes() == k[0, 0].view(np.uint16).tobytes()


def test_cache_write_padding_only_is_noop():
    kc = np.arange(2 * 1 * 4 * 8, dtype=np.float32).reshape(2, 1, 4, 8)
    k = np.ones((3, 1, 8), np.float32)
    nk, nv = oracle.kv_cache_write(k, k, np.full(3, -1, np.int32), kc, kc)
    assert nk.tobytes() == kc.tobytes() and nv.tobytes() == kc.tobytes()


# ------------------------------------------------------ precondition errors

def _expect(code, fn, *a, **kw):
    with pytest.raises(oracle.OracleError) as e:
        fn(*a, **kw)
    assert e.value.code == code


def test_precondition_errors():
    kc = np.zeros((4, 2, 4, 8), np.float32)
    k = np.zeros((2, 2, 8), np.float32)
    _expect(oracle.ERR_SLOT_DUP, oracle.kv_cache_write, k, k, np.array([5, 5], np.int32), kc, kc)
    _expect(oracle.ERR_SLOT_RANGE, oracle.kv_cache_write, k, k, np.array([16, 0], np.int32), kc, kc)
    _expect(oracle.ERR_SLOT_RANGE, oracle.kv_cache_write, k, k, np.array([-2, 0], np.int32), kc, kc)
    q = np.zeros((1, 4, 8), np.float32)
    _expect(oracle.ERR_BLOCK_RANGE, oracle.paged_attn_decode, q, kc, kc,
            np.array([[0, 4]], np.int32), np.array([5], np.int32), 1.0)
    _expect(oracle.ERR_BLOCK_RANGE, oracle.paged_attn_decode, q, kc, kc,
            np.array([[-1, 0]], np.int32), np.array([2], np.int32), 1.0)
    _expect(oracle.ERR_CTX, oracle.paged_attn_decode, q, kc, kc,
            np.array([[0, 1]], np.int32), np.array([9], np.int32), 1.0)
    _expect(oracle.ERR_CTX, oracle.paged_attn_decode, q, kc, kc,
            np.array([[0, 1]], np.int32), np.array([-1], np.int32), 1.0)
    q3 = np.zeros((1, 3, 8), np.float32)
    _expect(oracle.ERR_HEADS, oracle.paged_attn_decode, q3, kc, kc,
            np.array([[0, 1]], np.int32), np.array([5], np.int32), 1.0)
    # table entries past ceil(ctx/bs) are never looked at
    out = oracle.paged_attn_decode(q, kc, kc, np.array([[0, 99]], np.int32),
                                   np.array([4], np.int32), 1.0)
    assert (out == 0).all()
