"""GPU parity of the fused rotary embedding + cache write (pa_rope_reshape_and_cache) against
the oracle, bit for bit, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from oracle import rope
from paged_kv_cache_324_amd import PAError, pa_rope_reshape_and_cache
from workloads import make_config, rope_tables, to_u16

from _gpu import bits_to_device, log

pytestmark = pytest.mark.gpu

SENTINEL = 0x1234


def _rows(rng, shape, dt):
    return to_u16(rng.standard_normal(shape).astype(np.float32), dt)


def _tdt(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float16


def _u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_both(q, k, v, pos, slots, cos, sin, NB, BS, dt, with_q=True):
    """Device and oracle results: (q_dev, kc_dev, vc_dev), (q_ref, kc_ref, vc_ref)."""
    T, Hkv, D = k.shape
    tdt = _tdt(dt)
    kc = torch.full((NB, BS, Hkv, D), SENTINEL, dtype=torch.int16, device="cuda").view(tdt)
    vc = torch.full((NB, BS, Hkv, D), SENTINEL, dtype=torch.int16, device="cuda").view(tdt)
    qd = bits_to_device(q, tdt) if with_q else None
    pa_rope_reshape_and_cache(qd, bits_to_device(k, tdt), bits_to_device(v, tdt), kc, vc,
                              torch.from_numpy(np.asarray(pos, np.int64)).cuda(),
                              torch.from_numpy(cos).cuda(), torch.from_numpy(sin).cuda(),
                              torch.from_numpy(np.asarray(slots, np.int64)).cuda())
    torch.cuda.synchronize()
    hk = np.full((NB, BS, Hkv, D), SENTINEL, np.uint16)
    hv = hk.copy()
    qr = rope.rope_reshape_and_cache(q if with_q else None, k, v, hk, hv, pos, cos, sin, slots, dt)
    return (None if qd is None else _u16(qd), _u16(kc), _u16(vc)), (qr, hk, hv)


SWEEP = [(dt, D, BS, wq) for dt in ("bf16", "f16") for D in (64, 128) for BS in (16, 256)
         for wq in (True, False)]


@pytest.mark.parametrize("dt,D,BS,with_q", SWEEP)
def test_bit_exact_against_oracle(dt, D, BS, with_q):
    rng = np.random.default_rng(9900 + SWEEP.index((dt, D, BS, with_q)))
    T, Hq, Hkv, NB, P = 301, 12, 3, 40, 4096
    q, k, v = _rows(rng, (T, Hq, D), dt), _rows(rng, (T, Hkv, D), dt), _rows(rng, (T, Hkv, D), dt)
    cos, sin = rope_tables(P, D)
    pos = rng.integers(0, P, T)
    pos[[3, 50]] = [P, -7]                                    # outside the table
    slots = rng.permutation(NB * BS)[:T].astype(np.int64)     # distinct slots
    slots[[4, 60]] = [-1, NB * BS + 3]                         # padding, outside the pool
    got, ref = run_both(q, k, v, pos, slots, cos, sin, NB, BS, dt, with_q)
    if with_q:
        assert np.array_equal(got[0], ref[0])
    assert np.array_equal(got[1], ref[1])
    assert np.array_equal(got[2], ref[2])


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f16", 64)])
def test_long_chunk_odd_count_with_skipped_rows(dt, D):
    """A chunk of 2048+ tokens, where workgroups take two tokens each: an odd count leaves the
    last workgroup one token short, and rows to skip fall on both tokens of a pair."""
    rng = np.random.default_rng(9950 + D)
    T, Hq, Hkv, NB, BS, P = 2051, 8, 2, 160, 16, 8192
    q, k, v = _rows(rng, (T, Hq, D), dt), _rows(rng, (T, Hkv, D), dt), _rows(rng, (T, Hkv, D), dt)
    cos, sin = rope_tables(P, D)
    pos = rng.integers(0, P, T)
    pos[[0, 7, 1000, 1001, T - 1]] = [P, -1, -7, P + 5, P]        # outside the table
    slots = rng.permutation(NB * BS)[:T].astype(np.int64)
    slots[[1, 6, 1001, 2048, T - 2]] = [-1, NB * BS, -1, NB * BS + 9, -1]
    got, ref = run_both(q, k, v, pos, slots, cos, sin, NB, BS, dt)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)


def test_quarter_turns_and_special_values():
    """Exact angles give exact results; infinities and NaNs travel as the arithmetic says."""
    dt, D, T, Hkv, NB, BS = "bf16", 128, 8, 2, 4, 16
    c = np.array([1, 0, -1, 0], np.float32)
    s = np.array([0, 1, 0, -1], np.float32)
    cos, sin = np.repeat(c[:, None], D // 2, 1), np.repeat(s[:, None], D // 2, 1)
    rng = np.random.default_rng(1)
    k = _rows(rng, (T, Hkv, D), dt)
    k[0, 0, 0] = 0x7F80                                       # +inf in the first half
    k[1, 1, D - 1] = 0x7FC0                                   # NaN in the second half
    q = _rows(rng, (T, 4, D), dt)
    got, ref = run_both(q, k, k.copy(), np.arange(T) % 4, np.arange(T), cos, sin, NB, BS, dt)
    # inf * 0 is a NaN whose sign bit differs between hosts; any NaN matches any NaN
    for g, r in zip(got, ref):
        gf, rf = oracle.decode_u16(g, dt), oracle.decode_u16(r, dt)
        assert np.array_equal(gf, rf, equal_nan=True)
        both = ~np.isnan(rf)
        assert np.array_equal(g[both], r[both])
    assert np.isinf(oracle.decode_u16(got[1], dt)[0, 0, 0, 0])   # token 0, slot 0, theta 0


def test_empty_and_rejected_calls():
    dt, D = "f16", 64
    tdt = _tdt(dt)
    kc = torch.zeros((2, 16, 1, D), dtype=tdt, device="cuda")
    cos = torch.ones((4, D // 2), dtype=torch.float32, device="cuda")
    e = torch.empty((0, 1, D), dtype=tdt, device="cuda")
    i = torch.empty((0,), dtype=torch.int64, device="cuda")
    pa_rope_reshape_and_cache(None, e, e, kc, kc.clone(), i, cos, cos, i)    # no-op
    k = torch.zeros((1, 1, D), dtype=tdt, device="cuda")
    one = torch.zeros((1,), dtype=torch.int64, device="cuda")
    with pytest.raises(PAError):     # head_dim 96 is not supported
        pa_rope_reshape_and_cache(None, torch.zeros((1, 1, 96), dtype=tdt, device="cuda"),
                                  torch.zeros((1, 1, 96), dtype=tdt, device="cuda"),
                                  torch.zeros((2, 16, 1, 96), dtype=tdt, device="cuda"),
                                  torch.zeros((2, 16, 1, 96), dtype=tdt, device="cuda"), one,
                                  torch.ones((4, 48), dtype=torch.float32, device="cuda"),
                                  torch.ones((4, 48), dtype=torch.float32, device="cuda"), one)
    torch.cuda.synchronize()
    assert torch.all(kc == 0) and torch.all(k == 0)


@pytest.mark.parametrize("name", ["qwen3_0p6b_decode", "llama2_70b_decode_bs16", "chunked_prefill"])
def test_full_size_step(name):
    """The workload's step at its real shape: its new tokens (one per sequence for decode, the
    whole chunk for prefill) at their positions, scattered into the real-size pool."""
    b = make_config(name)
    rng = np.random.default_rng(77)
    T = len(b.slot_mapping)
    q = b.q if b.q.shape[0] == T else _rows(rng, (T, b.Hq, b.D), b.dtype)
    pos = np.concatenate([np.arange(int(L) - int(n), int(L))
                          for L, n in zip(b.context_lens, b.n_new)]).astype(np.int64)
    assert pos.shape == (T,)
    cos, sin = rope_tables(int(pos.max()) + 1, b.D)
    log(f"rope {name}: T={T} Hq={b.Hq} Hkv={b.Hkv} pool {b.NB}x{b.BS}")
    tdt = _tdt(b.dtype)
    shape = (b.NB, b.BS, b.Hkv, b.D)
    kc = torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda").view(tdt)
    vc = torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda").view(tdt)
    qd = bits_to_device(q, tdt)
    slot_d = torch.from_numpy(b.slot_mapping).cuda()
    pa_rope_reshape_and_cache(qd, bits_to_device(b.key_new, tdt), bits_to_device(b.value_new, tdt),
                              kc, vc, torch.from_numpy(pos).cuda(), torch.from_numpy(cos).cuda(),
                              torch.from_numpy(sin).cuda(), slot_d)
    torch.cuda.synchronize()
    assert np.array_equal(_u16(qd), rope.rotate(q, pos, cos, sin, b.dtype))
    k_rows = kc.view(torch.int16).view(-1, b.Hkv, b.D)[slot_d]
    v_rows = vc.view(torch.int16).view(-1, b.Hkv, b.D)[slot_d]
    assert np.array_equal(k_rows.cpu().numpy().view(np.uint16),
                          rope.rotate(b.key_new, pos, cos, sin, b.dtype))
    assert np.array_equal(v_rows.cpu().numpy().view(np.uint16), b.value_new)
    changed = int((kc.view(torch.int16) != SENTINEL).any(-1).any(-1).sum())
    assert changed == T   # nothing outside the step's slots was written
