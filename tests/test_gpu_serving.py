"""Continuous batching end to end: scheduler -> fused rotary write -> attention.

The native scheduler turns a seeded request trace into steps; every step's
new tokens get synthetic q/k/v, are rotated and written to the pools by
photon_rope_kv_cache_write, and attend through photon_paged_attn_multi_query
(prefill chunks and decode tokens in one call).  The CPU side replays the
same steps with the reference scheduler and the fp64 oracles (rotary write,
then multi-query attention over its own copy of the pools).  Outputs must
agree within the fp32 tolerance at every step, with preemption and
re-admission in the trace.
"""
import numpy as np
import pytest
import torch

import decode_inputs as di
import oracle
from oracle.scheduler import OracleScheduler

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import paged_attention_decode_photon_amd as mod
    return mod


def test_scheduler_driven_steps_match_the_oracles(pa):
    from paged_attention_decode_photon_amd.sched import Scheduler
    tc = di.TRACES["tight"]
    trace = di.make_request_trace(tc)
    hq, hkv, d, base, scale = 8, 2, 64, 5e5, 0.125
    nb, bs = tc.num_blocks, tc.block_size
    rng = np.random.default_rng(700)
    kc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    gk, gv = torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda()
    nat, ref = Scheduler(**tc.sched_config()), OracleScheduler(**tc.sched_config())
    i, done, step, checked, preempted = 0, 0, 0, 0, 0
    while done < len(trace):
        while i < len(trace) and trace[i][0] <= step:
            nat.add_request(*trace[i][1:])
            ref.add_request(*trace[i][1:])
            i += 1
        out = nat.schedule()
        rout = ref.schedule()
        assert out["slot_mapping"].tolist() == rout["slot_mapping"]
        preempted += len(out["preempted"])
        t = len(out["slot_mapping"])
        if t:
            q = rng.standard_normal((t, hq, d)).astype(np.float32)
            k = rng.standard_normal((t, hkv, d)).astype(np.float32)
            v = rng.standard_normal((t, hkv, d)).astype(np.float32)
            # CPU: rotate, write, attend
            rq, k64, vc = oracle.rope_kv_cache_write(q, k, v, out["positions"], out["slot_mapping"],
                                                     kc, vc, base)
            kc = k64.astype(np.float32)
            expect = oracle.paged_attn_multi_query(rq.astype(np.float32), kc, vc, out["block_tables"],
                                                   out["context_lens"], out["query_start"], scale)
            # GPU: the same, through the C ABI
            dq = pa.rope_kv_cache_write(torch.from_numpy(q).cuda(), torch.from_numpy(k).cuda(),
                                        torch.from_numpy(v).cuda(),
                                        torch.from_numpy(out["positions"]).cuda(),
                                        torch.from_numpy(out["slot_mapping"]).cuda(), gk, gv, base)
            got = pa.paged_attn_multi_query(dq, gk, gv, torch.from_numpy(out["block_tables"]).cuda(),
                                            torch.from_numpy(out["context_lens"]).cuda(),
                                            torch.from_numpy(out["query_start"]).cuda(), scale,
                                            max_query_len=int(np.diff(out["query_start"]).max()),
                                            max_context_len=int(out["context_lens"].max()))
            torch.cuda.synchronize()
            err = np.abs(got.cpu().numpy().astype(np.float64) - expect).max()
            assert err <= 1e-4, f"step {step}: max-abs error {err:.3e}"
            checked += 1
        fin = nat.update().tolist()
        assert fin == ref.update()
        done += len(fin)
        step += 1
    assert checked > 20 and preempted > 0
