"""The decode entry point that allocates nothing
(photon_paged_attn_decode_noalloc), against the regular decode entry point.

Both run the same kernels; the no-alloc call uses the library's static
per-GPU scratch array as its workspace.  Two calls in a row on one GPU, the
second with a smaller input (so it reuses the array with stale contents
from the first): each must equal photon_paged_attn_decode bit for bit and
the oracle within the decode tolerance.
"""
import numpy as np
import pytest
import torch

import decode_inputs as di
import oracle

pytestmark = pytest.mark.gpu

TOL = {np.dtype(np.float32): 1e-4, np.dtype(np.float16): 2e-3}


@pytest.fixture(scope="module")
def pa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import paged_attention_decode_photon_amd as mod
    return mod


def test_noalloc_decode_equals_decode_on_two_calls(pa):
    dev = torch.device("cuda:0")
    for name in ("cb_b64", "llama1b_b1"):  # 64 ragged f16 sequences, then one fp32 sequence
        cfg = di.CONFIGS[name]
        lay = di.make_layout(cfg)
        t = di.make_layer(cfg, lay)
        print(f"no-alloc decode: {name}", flush=True)
        q, kc, vc = (di.to_torch(a).to(dev) for a in (t.q, t.k_cache, t.v_cache))
        tables, lens = di.to_torch(lay.block_tables).to(dev), di.to_torch(lay.context_lens).to(dev)
        desc = pa.decode_desc(q, kc, tables, lay.max_context_len)
        assert 0 < pa.workspace_bytes(desc) <= pa.NOALLOC_SCRATCH_BYTES
        want = pa.paged_attn_decode(q, kc, vc, tables, lens, cfg.scale,
                                    max_context_len=lay.max_context_len)
        got = torch.full_like(q, float("nan"))
        pa.paged_attn_decode_noalloc(q, kc, vc, tables, lens, cfg.scale, lay.max_context_len, got)
        torch.cuda.synchronize()
        assert di.from_torch(got).tobytes() == di.from_torch(want).tobytes(), name
        ref = oracle.paged_attn_decode(t.q, t.k_cache, t.v_cache, lay.block_tables,
                                       lay.context_lens, cfg.scale)
        err = np.abs(di.as_float64(di.from_torch(got)) - ref)
        assert (err <= TOL[np.dtype(cfg.np_dtype)]).all(), f"{name}: max-abs {err.max():.3e}"
