"""The decode step captured in a HIP graph: replays with fresh inputs give exactly what the same
calls give when launched one by one, and the library allocates nothing during capture."""
import numpy as np
import pytest
import torch

import paged_kv_cache_324_amd as pa
from workloads import make_batch, rope_tables

from _gpu import log, upload

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("mode", ["rope_then_decode", "step", "step_rope"])
@pytest.mark.parametrize("partition", [0, 128])
def test_graph_replays_match_eager(partition, mode):
    b = make_batch(B=12, Hq=16, Hkv=4, D=128, BS=16, dtype="bf16", scale=128 ** -0.5, seed=4242,
                   lens_range=(40, 700))
    d = upload(b)
    dt = d.q.dtype
    rng = np.random.default_rng(7)
    cos, sin = rope_tables(int(b.max_context_len) + 1, b.D)
    cos_d, sin_d = torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda()
    pos = torch.from_numpy((b.context_lens.astype(np.int64) - 1)).cuda()
    # static buffers the graph reads and writes
    q = d.q.clone()
    key, value = d.key_new.clone(), d.value_new.clone()
    out = torch.empty_like(q)
    ws = pa.decode_workspace(b.B, b.Hq, b.D, b.max_context_len, partition, "cuda")
    order = torch.from_numpy(pa.pa_decode_order(b.context_lens)).cuda()
    kc, vc = d.k_cache, d.v_cache

    def step(q_, k_, v_, kc_, vc_, out_, ws_):
        if mode == "step":
            # one launch: store this step's K/V rows and attend
            pa.pa_decode_step(out_, q_, k_, v_, d.slot_mapping, kc_, vc_, d.block_tables,
                              d.context_lens, b.scale, b.max_context_len, partition, workspace=ws_,
                              seq_order=order)
        elif mode == "step_rope":
            # one launch: rotate q and the new key, store this step's K/V rows and attend
            pa.pa_decode_step_rope(out_, q_, k_, v_, d.slot_mapping, pos, cos_d, sin_d, kc_, vc_,
                                   d.block_tables, d.context_lens, b.scale, b.max_context_len,
                                   partition, workspace=ws_, seq_order=order)
        else:
            # rotary embedding of q (in place) and K on its way into the cache, then decode
            pa.pa_rope_reshape_and_cache(q_, k_, v_, kc_, vc_, pos, cos_d, sin_d, d.slot_mapping)
            pa.pa_decode(out_, q_, kc_, vc_, d.block_tables, d.context_lens, b.scale,
                         b.max_context_len, partition, workspace=ws_, seq_order=order)

    # warm up on a side stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(q.clone(), key, value, kc.clone(), vc.clone(), torch.empty_like(out), ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(q, key, value, kc, vc, out, ws)
    torch.cuda.synchronize()

    for r in range(4):
        # fresh inputs for this replay (eager copies between replays)
        q.copy_(torch.from_numpy(rng.standard_normal(q.shape).astype(np.float32)).to(dt))
        key.copy_(torch.from_numpy(rng.standard_normal(key.shape).astype(np.float32)).to(dt))
        value.copy_(torch.from_numpy(rng.standard_normal(value.shape).astype(np.float32)).to(dt))
        q_e, kc_e, vc_e = q.clone(), kc.clone(), vc.clone()
        out_e = torch.empty_like(out)
        ws_e = pa.decode_workspace(b.B, b.Hq, b.D, b.max_context_len, partition, "cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        step(q_e, key, value, kc_e, vc_e, out_e, ws_e)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), _bits(out_e)), f"replay {r}: output differs"
        assert np.array_equal(_bits(q), _bits(q_e)), f"replay {r}: rotated q differs"
        assert torch.equal(kc.view(torch.int16), kc_e.view(torch.int16)), f"replay {r}: K cache"
        assert torch.equal(vc.view(torch.int16), vc_e.view(torch.int16)), f"replay {r}: V cache"
        assert torch.isfinite(out.float()).all()
    log(f"graph partition={partition} {mode}: 4 replays bit-identical to eager")
