"""Pins for the CPU oracle (no GPU).

Each pin ties the oracle to something other than itself: the worked example
printed on the page "Nano-vLLM-Ascend" (section 2.1), torch's float64
``scaled_dot_product_attention`` (a library routine) on dense layouts, a
pure-Python brute force, closed forms and invariants.  The mutation tests at the
end plant plausible mistakes in the oracle and check that some pin catches them.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import brute_force
from oracle import paged_attention as PA
from workloads import POISON_U16, make_batch, to_u16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_count_example.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            k, v = (s.strip() for s in line.split("=", 1))
            vals[k] = float(v)
    return vals


# ---------------------------------------------------------------- block arithmetic
def test_worked_example_block_count():
    g = _golden()
    BS, L = int(g["block_size"]), int(g["L"])
    assert oracle.blocks_needed(L, BS) == int(g["blocks"])
    assert oracle.slots_allocated(L, BS) == int(g["slots"])
    assert round(100 * oracle.waste_fraction(L, BS), 1) == g["waste_percent_1dp"]
    assert math.floor(100 * oracle.prealloc_waste(L, int(g["prealloc_capacity"]))) == \
        int(g["prealloc_waste_percent_int"])


def test_block_count_edges():
    for BS in (16, 32, 256):
        assert oracle.blocks_needed(0, BS) == 0
        assert oracle.blocks_needed(1, BS) == 1
        assert oracle.blocks_needed(BS, BS) == 1
        assert oracle.blocks_needed(BS + 1, BS) == 2
        for L in range(1, 3 * BS):
            n = oracle.blocks_needed(L, BS)
            assert (n - 1) * BS < L <= n * BS


def test_utilisation_above_93_percent_on_qwen3_shaped_lengths():
    g = _golden()
    rng = np.random.default_rng(7)
    lens = rng.integers(200, 2048, size=128, endpoint=True)
    assert 100 * oracle.pool_utilisation(lens, 16) > g["utilisation_percent_min"]


# ---------------------------------------------------------------- helpers
def _after_new_tokens(b):
    kc, vc = b.k_blocks.copy(), b.v_blocks.copy()
    oracle.reshape_and_cache(b.key_new, b.value_new, kc, vc, b.slot_mapping_compact)
    return kc, vc


def _dense_case(seed, L, Hq, Hkv, D, BS, dtype):
    """Identity block table: logical block j is physical block j."""
    rng = np.random.default_rng(seed)
    n = -(-L // BS)
    kc = to_u16(rng.standard_normal((n, BS, Hkv, D)).astype(np.float32), dtype)
    vc = to_u16(rng.standard_normal((n, BS, Hkv, D)).astype(np.float32), dtype)
    q = to_u16(rng.standard_normal((1, Hq, D)).astype(np.float32), dtype)
    table = np.arange(n, dtype=np.int32)[None]
    return q, kc, vc, table


def _sdpa_decode_err(seed=0, L=37, Hq=8, Hkv=2, D=16, BS=16, dtype="bf16"):
    q, kc, vc, table = _dense_case(seed, L, Hq, Hkv, D, BS, dtype)
    scale = 1.0 / math.sqrt(D)
    out = oracle.paged_decode(q, kc, vc, table, np.array([L]), scale, dtype)
    K = oracle.decode_u16(kc, dtype).reshape(-1, Hkv, D)[:L]
    V = oracle.decode_u16(vc, dtype).reshape(-1, Hkv, D)[:L]
    qt = torch.from_numpy(oracle.decode_u16(q, dtype))[:, :, None, :]       # [1,Hq,1,D]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]  # [1,Hkv,L,D]
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    ref = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)[:, :, 0]
    return float(np.max(np.abs(out - ref.numpy())))


def _sdpa_causal_err(seed=1, L=29, Hq=4, Hkv=2, D=8, BS=4, dtype="bf16"):
    """c = 0: the chunk is the whole sequence, so attention is plain causal."""
    rng = np.random.default_rng(seed)
    _, kc, vc, table = _dense_case(seed, L, Hq, Hkv, D, BS, dtype)
    q = to_u16(rng.standard_normal((L, Hq, D)).astype(np.float32), dtype)
    scale = 1.0 / math.sqrt(D)
    out = oracle.paged_prefill(q, kc, vc, table, np.array([L]), np.array([0, L]), scale, dtype)
    K = oracle.decode_u16(kc, dtype).reshape(-1, Hkv, D)[:L]
    V = oracle.decode_u16(vc, dtype).reshape(-1, Hkv, D)[:L]
    qt = torch.from_numpy(np.ascontiguousarray(oracle.decode_u16(q, dtype).transpose(1, 0, 2)))[None]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2)))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2)))[None]
    ref = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, is_causal=True, enable_gqa=True)
    return float(np.max(np.abs(out - ref[0].numpy().transpose(1, 0, 2))))


def _brute_decode_err(seed, dtype="bf16", B=3, Hq=4, Hkv=2, D=8, BS=4):
    b = make_batch(B=B, Hq=Hq, Hkv=Hkv, D=D, BS=BS, dtype=dtype, scale=0.37, seed=seed,
                   lens_range=(1, 40))
    kc, vc = _after_new_tokens(b)
    out = oracle.paged_decode(b.q, kc, vc, b.block_tables_compact, b.context_lens, b.scale, dtype)
    ref = np.array(brute_force.decode(b.q, kc, vc, b.block_tables_compact, b.context_lens,
                                      b.scale, dtype))
    return float(np.max(np.abs(out - ref)))


def _chunk_vs_decode_err(seed=3):
    """Row t of a chunk equals a decode of the same query with L = c + t + 1."""
    b = make_batch(B=2, Hq=4, Hkv=2, D=8, BS=4, dtype="bf16", scale=0.3, seed=seed,
                   n_new=6, ctx_range=(0, 13))
    kc, vc = _after_new_tokens(b)
    out = oracle.paged_prefill(b.q, kc, vc, b.block_tables_compact, b.context_lens,
                               b.query_start_loc, b.scale, "bf16")
    err = 0.0
    for i in range(b.B):
        s0, n = int(b.query_start_loc[i]), int(b.n_new[i])
        c = int(b.context_lens[i]) - n
        for t in range(n):
            d = oracle.paged_decode(b.q[s0 + t][None], kc, vc, b.block_tables_compact[i:i + 1],
                                    np.array([c + t + 1]), b.scale, "bf16")
            err = max(err, float(np.max(np.abs(d[0] - out[s0 + t]))))
    return err


# ---------------------------------------------------------------- decode pins
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_equals_torch_sdpa_dense(G):
    assert _sdpa_decode_err(seed=G, Hq=2 * G, Hkv=2) < 1e-12


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_equals_brute_force(seed, dtype):
    assert _brute_decode_err(seed, dtype) < 1e-12


def test_decode_equals_brute_force_bs16_g1():
    assert _brute_decode_err(11, "f16", B=2, Hq=2, Hkv=2, D=4, BS=16) < 1e-12


def test_decode_single_token_is_v0_exactly():
    b = make_batch(B=3, Hq=4, Hkv=2, D=8, BS=4, dtype="bf16", scale=0.5, seed=5, lens=[1, 1, 1])
    kc, vc = _after_new_tokens(b)
    out = oracle.paged_decode(b.q, kc, vc, b.block_tables_compact, b.context_lens, b.scale, "bf16")
    for i in range(3):
        for h in range(4):
            v0 = oracle.decode_u16(b.value_new[i, h // 2], "bf16")
            assert np.array_equal(out[i, h], v0)


def test_decode_zero_query_is_mean_of_values():
    b = make_batch(B=2, Hq=2, Hkv=1, D=8, BS=4, dtype="bf16", scale=1.0, seed=6, lens=[13, 30])
    kc, vc = _after_new_tokens(b)
    q0 = np.zeros_like(b.q)
    out = oracle.paged_decode(q0, kc, vc, b.block_tables_compact, b.context_lens, 1.0, "bf16")
    for i in range(2):
        L = int(b.context_lens[i])
        V = oracle.decode_u16(np.concatenate([vc[c] for c in b.block_tables_compact[i, :-(-L // 4)]]),
                              "bf16")[:L, 0]
        np.testing.assert_allclose(out[i, 0], V.mean(axis=0), rtol=0, atol=1e-12)


def test_decode_constant_values():
    b = make_batch(B=2, Hq=4, Hkv=2, D=8, BS=4, dtype="f16", scale=0.4, seed=8, lens_range=(1, 30))
    kc, vc = _after_new_tokens(b)
    vc[:] = to_u16(np.full(vc.shape, 1.5, np.float32), "f16")
    out = oracle.paged_decode(b.q, kc, vc, b.block_tables_compact, b.context_lens, b.scale, "f16")
    np.testing.assert_allclose(out, 1.5, rtol=0, atol=1e-12)


def test_softmax_rows_sum_to_one_and_onehot_values_give_probs():
    D = 16
    b = make_batch(B=3, Hq=2, Hkv=2, D=D, BS=4, dtype="bf16", scale=0.6, seed=9, lens_range=(1, D))
    kc, vc = _after_new_tokens(b)
    out, probs = oracle.paged_decode(b.q, kc, vc, b.block_tables_compact, b.context_lens, b.scale,
                                     "bf16", return_probs=True)
    for p in probs:
        np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    # V_j = e_j: output row is the probability row
    one = to_u16(np.ones(1, np.float32), "bf16")[0]
    for i in range(b.B):
        L = int(b.context_lens[i])
        for j in range(L):
            blk, off = b.block_tables_compact[i, j // 4], j % 4
            vc[blk, off] = 0
            vc[blk, off, :, j] = one
    out = oracle.paged_decode(b.q, kc, vc, b.block_tables_compact, b.context_lens, b.scale, "bf16")
    for i in range(b.B):
        L = int(b.context_lens[i])
        np.testing.assert_allclose(out[i, :, :L], probs[i], atol=1e-15)
        assert np.all(out[i, :, L:] == 0)


def test_needle_selects_one_value_row():
    """q = e0, scale 1, K_j[0] = -100 except the target (+100): the output is V_target."""
    b = make_batch(B=2, Hq=2, Hkv=1, D=8, BS=4, dtype="bf16", scale=1.0, seed=10, lens=[23, 9])
    kc, vc = _after_new_tokens(b)
    q = np.zeros_like(b.q)
    q[:, :, 0] = to_u16(np.ones(1, np.float32), "bf16")[0]
    for i, target in ((0, 17), (1, 0)):
        L = int(b.context_lens[i])
        for j in range(L):
            blk, off = b.block_tables_compact[i, j // 4], j % 4
            kc[blk, off, :, :] = 0
            kc[blk, off, :, 0] = to_u16(np.array([100.0 if j == target else -100.0], np.float32),
                                        "bf16")[0]
        out = oracle.paged_decode(q[i:i + 1], kc, vc, b.block_tables_compact[i:i + 1],
                                  b.context_lens[i:i + 1], 1.0, "bf16")
        blk, off = b.block_tables_compact[i, target // 4], target % 4
        np.testing.assert_allclose(out[0, 0], oracle.decode_u16(vc[blk, off, 0], "bf16"),
                                   rtol=0, atol=1e-80)


def test_decode_block_permutation_invariance():
    b = make_batch(B=4, Hq=4, Hkv=2, D=8, BS=4, dtype="bf16", scale=0.3, seed=12,
                   lens_range=(1, 50))
    kc, vc = _after_new_tokens(b)
    out = oracle.paged_decode(b.q, kc, vc, b.block_tables_compact, b.context_lens, b.scale, "bf16")
    rng = np.random.default_rng(0)
    perm = rng.permutation(len(kc))
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    bt2 = np.where(b.block_tables_compact >= 0, perm[np.maximum(b.block_tables_compact, 0)], -1)
    out2 = oracle.paged_decode(b.q, kc2, vc2, bt2, b.context_lens, b.scale, "bf16")
    assert np.array_equal(out, out2)


def test_decode_zero_length_gives_zero_row():
    b = make_batch(B=2, Hq=2, Hkv=2, D=8, BS=4, dtype="bf16", scale=0.3, seed=13, lens=[5, 7])
    kc, vc = _after_new_tokens(b)
    lens = b.context_lens.copy()
    lens[1] = 0
    out = oracle.paged_decode(b.q, kc, vc, b.block_tables_compact, lens, b.scale, "bf16")
    assert np.all(out[1] == 0) and np.all(np.isfinite(out))


def test_decode_one_matches_batch():
    b = make_batch(B=3, Hq=8, Hkv=2, D=16, BS=16, dtype="bf16", scale=0.25, seed=14,
                   lens_range=(1, 70))
    kc, vc = _after_new_tokens(b)
    out = oracle.paged_decode(b.q, kc, vc, b.block_tables_compact, b.context_lens, b.scale, "bf16")
    for i in range(3):
        for h in (0, 3, 7):
            one = oracle.paged_decode_one(i, h, b.q, kc, vc, b.block_tables_compact,
                                          b.context_lens, b.scale, "bf16")
            np.testing.assert_allclose(one, out[i, h], rtol=0, atol=1e-13)


def test_decode_ignores_poisoned_tail_slots():
    """Tail slots of each last block hold NaN: they never reach the output."""
    b = make_batch(B=4, Hq=2, Hkv=1, D=8, BS=16, dtype="f16", scale=0.3, seed=15,
                   lens_range=(1, 60))
    kc, vc = _after_new_tokens(b)
    out = oracle.paged_decode(b.q, kc, vc, b.block_tables_compact, b.context_lens, b.scale, "f16")
    assert np.all(np.isfinite(out))
    assert np.any(kc == POISON_U16)  # poison really present


# ---------------------------------------------------------------- prefill pins
def test_prefill_without_cache_equals_causal_sdpa():
    assert _sdpa_causal_err() < 1e-12


def test_prefill_rows_equal_successive_decodes():
    assert _chunk_vs_decode_err() < 1e-12


def test_prefill_equals_brute_force():
    b = make_batch(B=2, Hq=4, Hkv=2, D=4, BS=4, dtype="bf16", scale=0.45, seed=16,
                   n_new=5, ctx_range=(0, 11))
    kc, vc = _after_new_tokens(b)
    out = oracle.paged_prefill(b.q, kc, vc, b.block_tables_compact, b.context_lens,
                               b.query_start_loc, b.scale, "bf16")
    ref = np.array(brute_force.prefill(b.q, kc, vc, b.block_tables_compact, b.context_lens,
                                       b.query_start_loc, b.scale, "bf16"))
    assert np.max(np.abs(out - ref)) < 1e-12


def test_prefill_chunk_split_invariance():
    """One chunk of 8 new tokens == two chunks of 4 over the same cache."""
    b = make_batch(B=1, Hq=4, Hkv=2, D=8, BS=4, dtype="bf16", scale=0.3, seed=17,
                   n_new=8, ctx_range=(3, 9))
    kc, vc = _after_new_tokens(b)
    L = int(b.context_lens[0])
    whole = oracle.paged_prefill(b.q, kc, vc, b.block_tables_compact, b.context_lens,
                                 b.query_start_loc, b.scale, "bf16")
    first = oracle.paged_prefill(b.q[:4], kc, vc, b.block_tables_compact, np.array([L - 4]),
                                 np.array([0, 4]), b.scale, "bf16")
    second = oracle.paged_prefill(b.q[4:], kc, vc, b.block_tables_compact, np.array([L]),
                                  np.array([0, 4]), b.scale, "bf16")
    np.testing.assert_allclose(np.concatenate([first, second]), whole, rtol=0, atol=1e-13)


def test_prefill_row_subset():
    b = make_batch(B=2, Hq=2, Hkv=1, D=8, BS=4, dtype="bf16", scale=0.3, seed=18,
                   n_new=6, ctx_range=(0, 9))
    kc, vc = _after_new_tokens(b)
    args = (b.q, kc, vc, b.block_tables_compact, b.context_lens, b.query_start_loc, b.scale, "bf16")
    full = oracle.paged_prefill(*args)
    rows = [0, 5, 7, 11]
    part = oracle.paged_prefill(*args, rows=rows)
    np.testing.assert_allclose(part[rows], full[rows], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- reshape_and_cache pins
def test_reshape_round_trip_through_block_tables():
    b = make_batch(B=5, Hq=4, Hkv=2, D=8, BS=4, dtype="bf16", scale=0.3, seed=19,
                   n_new=3, ctx_range=(0, 20))
    kc, vc = _after_new_tokens(b)
    for i in range(b.B):
        L, n = int(b.context_lens[i]), int(b.n_new[i])
        for t in range(n):
            pos = L - n + t
            blk, off = b.block_tables_compact[i, pos // 4], pos % 4
            row = int(b.query_start_loc[i]) + t
            assert np.array_equal(kc[blk, off], b.key_new[row])
            assert np.array_equal(vc[blk, off], b.value_new[row])


def test_reshape_skips_padding_and_leaves_other_slots():
    b = make_batch(B=4, Hq=2, Hkv=2, D=8, BS=4, dtype="f16", scale=0.3, seed=20,
                   lens_range=(2, 30))
    slots = b.slot_mapping_compact.copy()
    slots[1] = -1
    kc, vc = b.k_blocks.copy(), b.v_blocks.copy()
    oracle.reshape_and_cache(b.key_new, b.value_new, kc, vc, slots)
    written = np.zeros(kc.shape[:2], dtype=bool)
    for s in slots[slots >= 0]:
        written[s // 4, s % 4] = True
    assert np.array_equal(kc[~written], b.k_blocks[~written])
    assert np.array_equal(vc[~written], b.v_blocks[~written])
    s1 = b.slot_mapping_compact[1]
    assert np.all(kc[s1 // 4, s1 % 4] == POISON_U16)


# ---------------------------------------------------------------- planted mistakes
def test_mutation_gqa_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(PA, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)
    assert _sdpa_decode_err(seed=2, Hq=8, Hkv=2) > 1e-3


def test_mutation_causal_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(PA, "visible_keys", lambda c, t: c + t)
    with np.errstate(invalid="ignore"):
        err1 = _sdpa_causal_err()
        err2 = _chunk_vs_decode_err()
    assert not (err1 < 1e-6) and not (err2 < 1e-6)


def test_mutation_slot_split_is_caught(monkeypatch):
    monkeypatch.setattr(PA, "slot_position", lambda slot, BS: (slot % BS, slot // BS))
    with pytest.raises((AssertionError, IndexError)):
        test_reshape_round_trip_through_block_tables()


def test_mutation_dropped_scale_is_caught(monkeypatch):
    real = PA.attend
    monkeypatch.setattr(PA, "attend", lambda q, K, V, scale, mask=None: real(q, K, V, 1.0, mask))
    assert _sdpa_decode_err(seed=4) > 1e-3


def test_mutation_block_table_offset_is_caught(monkeypatch):
    real = PA.gather_sequence

    def shifted(cache, row, L, dtype, out_dtype=np.float64):
        return real(cache, np.roll(np.asarray(row)[:-(-L // cache.shape[1])], 1), L, dtype, out_dtype)

    monkeypatch.setattr(PA, "gather_sequence", shifted)
    with np.errstate(invalid="ignore"):
        err = _brute_decode_err(21)
    assert not (err < 1e-6)  # NaN (a poisoned slot read) also counts as caught
