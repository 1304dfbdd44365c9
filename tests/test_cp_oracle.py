"""Pins of the context-parallel oracle (``oracle/context_parallel.py``), on the CPU."""
import numpy as np
import pytest

import oracle
from oracle import context_parallel as cp
from workloads import make_batch

from _shards import split_context


def _batch(seed, **kw):
    args = dict(B=5, Hq=8, Hkv=2, D=64, BS=16, dtype="bf16", scale=0.125, seed=seed,
                lens_range=(1, 400))
    args.update(kw)
    return make_batch(**args)


def _caches(b):
    kc, vc = b.k_blocks.copy(), b.v_blocks.copy()
    oracle.reshape_and_cache(b.key_new, b.value_new, kc, vc, b.slot_mapping_compact)
    return kc, vc


@pytest.mark.parametrize("n,mode", [(1, "contiguous"), (2, "contiguous"), (4, "round_robin"),
                                    (7, "contiguous"), (3, "round_robin")])
def test_merged_shards_equal_full_attention(n, mode):
    b = _batch(100 + n)
    kc, vc = _caches(b)
    parts = [cp.shard_partial(b.q, kc, vc, tc, lens, b.scale, b.dtype)
             for tc, _, lens in split_context(b, n, mode)]
    got = cp.merge_partials(*[np.stack(x) for x in zip(*parts)])
    ref = oracle.paged_decode(b.q, kc, vc, b.block_tables_compact, b.context_lens, b.scale, b.dtype)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_single_shard_is_identity_and_empty_shards_drop_out():
    b = _batch(200, B=4, lens=[5, 0, 40, 16])
    kc, vc = _caches(b)
    o, m, l = cp.shard_partial(b.q, kc, vc, b.block_tables_compact, b.context_lens, b.scale, b.dtype)
    assert np.array_equal(cp.merge_partials(o[None], m[None], l[None]), np.where(l[..., None] > 0, o, 0))
    empty = (np.full_like(o, 123.0), np.full_like(m, 50.0), np.zeros_like(l))   # l = 0: ignored
    got = cp.merge_partials(np.stack([o, empty[0]]), np.stack([m, empty[1]]), np.stack([l, empty[2]]))
    np.testing.assert_allclose(got, np.where(l[..., None] > 0, o, 0), rtol=0, atol=1e-14)
    assert np.all(got[1] == 0)                                   # the empty sequence


def test_m_l_scaling_freedom():
    b = _batch(300)
    kc, vc = _caches(b)
    parts = [cp.shard_partial(b.q, kc, vc, tc, lens, b.scale, b.dtype)
             for tc, _, lens in split_context(b, 3, "round_robin")]
    os, ms, ls = [np.stack(x) for x in zip(*parts)]
    c = np.random.default_rng(1).uniform(-20, 20, ms.shape)
    np.testing.assert_allclose(cp.merge_partials(os, ms + c, ls * np.exp2(-c)),
                               cp.merge_partials(os, ms, ls), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("mutation", ["natural_exp", "no_l_weight", "mean_of_shards"])
def test_pins_catch_planted_mistakes(mutation, monkeypatch):
    real = cp.merge_partials

    def wrong(os, ms, ls):
        os, ms, ls = np.asarray(os, float), np.asarray(ms, float), np.asarray(ls, float)
        M = ms.max(axis=0)
        if mutation == "natural_exp":
            w = ls * np.exp(ms - M)
        elif mutation == "no_l_weight":
            w = np.exp2(ms - M)
        else:
            w = np.ones_like(ls)
        return np.einsum("nbh,nbhd->bhd", w, os) / w.sum(axis=0)[..., None]
    monkeypatch.setattr(cp, "merge_partials", wrong)
    with pytest.raises(AssertionError):
        test_merged_shards_equal_full_attention(4, "round_robin")
    monkeypatch.setattr(cp, "merge_partials", real)
