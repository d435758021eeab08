"""GPU parity of the fused rotary embedding + cache write against the fp64 oracle.

Tolerances (element-wise): 1e-5 for fp32 storage (an fp32 rotation of
values below 8 in magnitude, with sines and cosines rounded once to fp32);
for 16-bit storage 1e-5 plus the final rounding's bound, 2^-11 |ref| for
fp16 (11 significant bits) and 2^-8 |ref| for bfloat16 (8 significant bits).
The v rows, and every pool row not written, must be bit-exact.
"""
import numpy as np
import pytest
import torch

import decode_inputs as di
import oracle

pytestmark = pytest.mark.gpu

DTYPES = [np.float32, np.float16, di.BF16]


@pytest.fixture(scope="module")
def pa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import paged_attention_decode_photon_amd as mod
    return mod


def dev(a):
    return di.to_torch(a).to("cuda:0")


def host(t):
    return di.from_torch(t)


def tolerance(dtype, ref):
    rel = {np.dtype(np.float32): 0.0, np.dtype(np.float16): 2.0 ** -11, di.BF16: 2.0 ** -8}
    return 1e-5 + rel[np.dtype(dtype)] * np.abs(ref)


def assert_close(got, ref, dtype, what):
    g = di.as_float64(got)
    assert np.isfinite(g).all(), f"{what}: non-finite"
    err = np.abs(g - ref)
    assert (err <= tolerance(dtype, ref)).all(), f"{what}: max error {err.max():.3e}"


def case(rng, dtype, t, hq, hkv, d, nb=40, pad=0.2):
    q = di.cast(rng.standard_normal((t, hq, d)), dtype)
    k = di.cast(rng.standard_normal((t, hkv, d)), dtype)
    v = di.cast(rng.standard_normal((t, hkv, d)), dtype)
    kc = di.cast(rng.standard_normal((nb, hkv, 16, d)), dtype)
    vc = di.cast(rng.standard_normal((nb, hkv, 16, d)), dtype)
    pos = rng.integers(0, 131072, t).astype(np.int32)
    pos[:3] = [0, 1, 131071]
    slots = di.random_injective_slots(nb, 16, t, rng, pad_fraction=pad)
    return q, k, v, kc, vc, pos, slots


def check_pools(gk, gv, kc, vc, slots, ref_k, ref_v, dtype, what):
    written = np.zeros(kc.shape[0] * 16, bool)
    written[slots[slots >= 0]] = True
    written = written.reshape(-1, 16)
    got_k = host(gk)
    # written K rows are rotated values; every other row keeps its bits
    assert_close(got_k.transpose(0, 2, 1, 3)[written], ref_k.transpose(0, 2, 1, 3)[written], dtype,
                 f"{what} k rows")
    assert got_k.transpose(0, 2, 1, 3)[~written].tobytes() == \
        kc.transpose(0, 2, 1, 3)[~written].tobytes()
    assert host(gv).tobytes() == ref_v.tobytes(), f"{what}: v pool differs"


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("adjacent", [False, True])
def test_rope_cache_write_matches_oracle(pa, dtype, d, adjacent):
    rng = np.random.default_rng(400 + d + DTYPES.index(dtype) * 7 + adjacent)
    q, k, v, kc, vc, pos, slots = case(rng, dtype, 77, 8, 2, d)
    base = 500000.0
    ref_q, ref_k, ref_v = oracle.rope_kv_cache_write(q, k, v, pos, slots, kc, vc, base, adjacent)
    gk, gv = dev(kc), dev(vc)
    qo = pa.rope_kv_cache_write(dev(q), dev(k), dev(v), dev(pos), dev(slots), gk, gv, base,
                                adjacent_pairs=adjacent)
    torch.cuda.synchronize()
    assert_close(host(qo), ref_q, dtype, "q_out")
    check_pools(gk, gv, kc, vc, slots, ref_k, ref_v, dtype, "pools")


def test_rope_in_place_and_padding_only(pa):
    rng = np.random.default_rng(410)
    q, k, v, kc, vc, pos, _ = case(rng, np.float32, 20, 32, 8, 64)
    slots = np.full(20, -1, np.int32)
    ref_q = oracle.rope(q, pos, 1e4)
    gq, gk, gv = dev(q), dev(kc), dev(vc)
    out = pa.rope_kv_cache_write(gq, dev(k), dev(v), dev(pos), dev(slots), gk, gv, 1e4, q_out=gq)
    torch.cuda.synchronize()
    assert out.data_ptr() == gq.data_ptr()
    assert_close(host(gq), ref_q, np.float32, "in-place q")
    assert host(gk).tobytes() == kc.tobytes() and host(gv).tobytes() == vc.tobytes()


def test_position_zero_is_identity_bit_exact(pa):
    # cos 0 = 1 and sin 0 = 0 exactly, so the rotation at position 0 keeps every bit.
    rng = np.random.default_rng(411)
    q, k, v, kc, vc, _, slots = case(rng, np.float16, 9, 4, 2, 128, pad=0.0)
    pos = np.zeros(9, np.int32)
    gk, gv = dev(kc), dev(vc)
    qo = pa.rope_kv_cache_write(dev(q), dev(k), dev(v), dev(pos), dev(slots), gk, gv, 1e6)
    torch.cuda.synchronize()
    assert host(qo).tobytes() == q.tobytes()
    got = host(gk)
    for i, s in enumerate(slots):
        assert got[s // 16, :, s % 16].tobytes() == k[i].tobytes()


@pytest.mark.parametrize("name", ["llama1b_b16", "cb_b64"])
def test_decode_step_with_rope(pa, name):
    # One decode step: rotate q and k at position ctx-1, write k and v, then
    # attend with the rotated q.  The oracle composes the same three steps,
    # rounding its rotated q and k once to the storage type.
    cfg = di.CONFIGS[name]
    lay = di.make_layout(cfg)
    t = di.make_layer(cfg, lay)
    dt = cfg.np_dtype
    ref_q, ref_k64, ref_v = oracle.rope_kv_cache_write(t.q, t.k_new, t.v_new, lay.positions,
                                                       lay.slot_mapping, t.k_cache, t.v_cache,
                                                       cfg.rope_base)
    ref = oracle.paged_attn_decode(di.cast(ref_q, dt), di.cast(ref_k64, dt), ref_v, lay.block_tables,
                                   lay.context_lens, cfg.scale)
    gk, gv = dev(t.k_cache), dev(t.v_cache)
    qr = pa.rope_kv_cache_write(dev(t.q), dev(t.k_new), dev(t.v_new), dev(lay.positions),
                                dev(lay.slot_mapping), gk, gv, cfg.rope_base)
    out = pa.paged_attn_decode(qr, gk, gv, dev(lay.block_tables), dev(lay.context_lens), cfg.scale,
                               max_context_len=lay.max_context_len)
    torch.cuda.synchronize()
    tol = 1e-4 if dt == np.float32 else 2e-3
    err = np.abs(di.as_float64(host(out)) - ref).max()
    assert err <= tol, f"{name}: max-abs error {err:.3e}"
