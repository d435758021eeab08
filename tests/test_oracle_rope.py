"""Pins for the oracle's rotary position embedding.

The pages name batched RoPE among the fused operations and give no formula;
the oracle implements the textbook rotation.  It is pinned here to things
the oracle does not use: transformers' own GPT-J (adjacent pairs) and Llama
(rotate-half) routines with frequencies from transformers' sinusoid table,
complex multiplication by exp(i * angle), and the identities of a rotation
(position 0 is the identity, norms are kept, scores depend only on the
position difference).
"""
import numpy as np
import pytest
import torch

import decode_inputs as di
import oracle


def _gptj_sin_cos(positions, d):
    from transformers.models.gptj.modeling_gptj import create_sinusoidal_positions
    table = create_sinusoidal_positions(int(max(positions)) + 1, d).double()  # [P, D]: sin | cos
    sel = table[torch.as_tensor(positions, dtype=torch.long)]
    return sel[:, : d // 2], sel[:, d // 2:]


@pytest.mark.parametrize("dtype", [np.float32, np.float16, di.BF16])
def test_adjacent_pairs_match_transformers_gptj(dtype):
    from transformers.models.gptj.modeling_gptj import apply_rotary_pos_emb
    rng = np.random.default_rng(300)
    pos = np.array([0, 1, 2, 7, 31, 63, 40], np.int32)
    x = di.cast(rng.standard_normal((len(pos), 3, 64)), dtype)
    got = oracle.rope(x, pos, 10000.0, interleaved=True)
    sin, cos = _gptj_sin_cos(pos, 64)
    ref = apply_rotary_pos_emb(torch.from_numpy(oracle.widen(x))[None], sin[None], cos[None])[0]
    # transformers forms the angles in float32: about 1e-7 relative at angles <= 63
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-4)


@pytest.mark.parametrize("d", [64, 128])
def test_rotate_half_matches_transformers_llama(d):
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    rng = np.random.default_rng(301 + d)
    pos = np.array([0, 5, 17, 63, 100, 3], np.int32)
    q = rng.standard_normal((len(pos), 4, d)).astype(np.float32)
    k = rng.standard_normal((len(pos), 2, d)).astype(np.float32)
    sin, cos = _gptj_sin_cos(pos, d)
    cos2, sin2 = torch.cat([cos, cos], -1)[None], torch.cat([sin, sin], -1)[None]  # [1, T, D]
    rq, rk = apply_rotary_pos_emb(torch.from_numpy(q.astype(np.float64))[None],
                                  torch.from_numpy(k.astype(np.float64))[None], cos2, sin2,
                                  unsqueeze_dim=2)
    np.testing.assert_allclose(oracle.rope(q, pos, 10000.0), rq[0].numpy(), rtol=0, atol=1e-4)
    np.testing.assert_allclose(oracle.rope(k, pos, 10000.0), rk[0].numpy(), rtol=0, atol=1e-4)


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("base", [10000.0, 500000.0, 1e6])
def test_complex_multiplication_form(interleaved, base):
    # Pair j as the complex number a + ib, multiplied by exp(i * pos * base^(-2j/D)).
    rng = np.random.default_rng(302)
    d = 64
    pos = np.array([0, 1, 1000, 32767, 131071], np.int32)
    x = rng.standard_normal((len(pos), 2, d)).astype(np.float32)
    got = oracle.rope(x, pos, base, interleaved)
    j = np.arange(d // 2)
    ia, ib = (2 * j, 2 * j + 1) if interleaved else (j, j + d // 2)
    z = x[..., ia].astype(np.float64) + 1j * x[..., ib].astype(np.float64)
    theta = np.power(base, -2.0 * j / d)
    zr = z * np.exp(1j * pos[:, None, None] * theta)
    np.testing.assert_allclose(got[..., ia], zr.real, rtol=0, atol=1e-9)
    np.testing.assert_allclose(got[..., ib], zr.imag, rtol=0, atol=1e-9)


def test_two_dimensional_closed_form():
    # D = 2: one pair, frequency base^0 = 1, so the angle is the position itself.
    pos = np.array([0, 1, 2, 100, 12345], np.int32)
    x = np.array([[[0.75, -1.5]]] * len(pos), np.float32)
    got = oracle.rope(x, pos, 777.0)
    c, s = np.cos(pos.astype(np.float64)), np.sin(pos.astype(np.float64))
    np.testing.assert_allclose(got[:, 0, 0], 0.75 * c + 1.5 * s, rtol=0, atol=1e-14)
    np.testing.assert_allclose(got[:, 0, 1], 0.75 * s - 1.5 * c, rtol=0, atol=1e-14)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotation_identities(interleaved):
    rng = np.random.default_rng(303)
    d = 128
    x = rng.standard_normal((4, 3, d)).astype(np.float32)
    x64 = x.astype(np.float64)
    # position 0 is the identity, exactly
    assert np.array_equal(oracle.rope(x, np.zeros(4, np.int32), 1e4, interleaved), x64)
    # every pair keeps its length
    j = np.arange(d // 2)
    ia, ib = (2 * j, 2 * j + 1) if interleaved else (j, j + d // 2)
    r = oracle.rope(x, np.array([3, 999, 4096, 77777], np.int32), 1e4, interleaved)
    np.testing.assert_allclose(r[..., ia] ** 2 + r[..., ib] ** 2, x64[..., ia] ** 2 + x64[..., ib] ** 2,
                               rtol=1e-13, atol=0)
    # <R(m) q, R(n) k> depends only on m - n
    q, k = x[:1, :1], x[1:2, :1]
    for m, n, shift in [(10, 3, 1000), (5000, 4990, 12345), (0, 700, 65000)]:
        a = oracle.rope(q, np.array([m], np.int32), 1e4, interleaved).ravel() @ \
            oracle.rope(k, np.array([n], np.int32), 1e4, interleaved).ravel()
        b = oracle.rope(q, np.array([m + shift], np.int32), 1e4, interleaved).ravel() @ \
            oracle.rope(k, np.array([n + shift], np.int32), 1e4, interleaved).ravel()
        assert abs(a - b) <= 1e-10 * max(1.0, abs(a))


def test_widen_matches_library_conversions():
    bits = np.arange(65536, dtype=np.uint16)
    h = oracle.widen(bits.view(np.float16))
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(h), np.isnan(ref)) and np.array_equal(h[~np.isnan(ref)], ref[~np.isnan(ref)])
    b = oracle.widen(bits.view(di.BF16))
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(np.isnan(b), np.isnan(ref)) and np.array_equal(b[~np.isnan(ref)], ref[~np.isnan(ref)])


@pytest.mark.parametrize("dtype", [np.float32, np.float16, di.BF16])
def test_rope_then_cache_write(dtype):
    rng = np.random.default_rng(304)
    nb, hkv, hq, d, t = 10, 2, 8, 64, 12
    kc = di.cast(rng.standard_normal((nb, hkv, 16, d)), dtype)
    vc = di.cast(rng.standard_normal((nb, hkv, 16, d)), dtype)
    q = di.cast(rng.standard_normal((t, hq, d)), dtype)
    k = di.cast(rng.standard_normal((t, hkv, d)), dtype)
    v = di.cast(rng.standard_normal((t, hkv, d)), dtype)
    pos = rng.integers(0, 5000, t).astype(np.int32)
    slots = di.random_injective_slots(nb, 16, t, rng, pad_fraction=0.25)
    qo, kn, vn = oracle.rope_kv_cache_write(q, k, v, pos, slots, kc, vc, 1e4)
    assert np.array_equal(qo, oracle.rope(q, pos, 1e4))
    kr = oracle.rope(k, pos, 1e4)
    written = np.zeros((nb, 16), bool)
    for i, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(kn[s // 16, :, s % 16], kr[i])
            assert vn[s // 16, :, s % 16].tobytes() == v[i].tobytes()
            written[s // 16, s % 16] = True
    base = oracle.widen(kc)
    assert np.array_equal(kn.transpose(0, 2, 1, 3)[~written], base.transpose(0, 2, 1, 3)[~written])
    assert vn.transpose(0, 2, 1, 3)[~written].tobytes() == vc.transpose(0, 2, 1, 3)[~written].tobytes()


def test_rope_rejects_bad_arguments():
    x = np.zeros((2, 1, 8), np.float32)
    for kw in [dict(positions=np.array([0, -1], np.int32), base=1e4),
               dict(positions=np.array([0, 1], np.int32), base=0.0),
               dict(positions=np.array([0, 1], np.int32), base=-5.0)]:
        with pytest.raises(oracle.OracleError):
            oracle.rope(x, **kw)
    with pytest.raises(oracle.OracleError):
        oracle.rope(np.zeros((2, 1, 7), np.float32), np.array([0, 1], np.int32), 1e4)
