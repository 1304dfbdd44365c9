"""The seeded input generators: reproducibility and the structure each workload promises."""
import numpy as np

from workloads import CONFIGS, POISON_U16, make_batch, make_config, to_u16


def test_same_seed_same_batch():
    a = make_batch(B=6, Hq=4, Hkv=2, D=8, BS=16, dtype="bf16", scale=0.1, seed=1, lens_range=(1, 90))
    b = make_batch(B=6, Hq=4, Hkv=2, D=8, BS=16, dtype="bf16", scale=0.1, seed=1, lens_range=(1, 90))
    c = make_batch(B=6, Hq=4, Hkv=2, D=8, BS=16, dtype="bf16", scale=0.1, seed=2, lens_range=(1, 90))
    for f in ("context_lens", "block_tables", "q", "k_blocks", "v_blocks", "key_new", "slot_mapping"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    assert not np.array_equal(a.q, c.q)


def test_tiny_config_uses_distinct_blocks_of_its_pool():
    b = make_config("tiny_decode")
    assert b.NB == 128 and b.B == 4 and b.D == 64 and b.dtype == "f16"
    used = b.block_tables[b.block_tables >= 0]
    assert len(np.unique(used)) == len(used)
    assert used.min() >= 0 and used.max() < 128
    assert np.all((b.context_lens >= 1) & (b.context_lens <= 256))


def test_slot_mapping_agrees_with_block_tables():
    b = make_batch(B=5, Hq=4, Hkv=2, D=8, BS=16, dtype="bf16", scale=0.1, seed=3,
                   n_new=20, ctx_range=(0, 50))
    for i in range(b.B):
        L, n = int(b.context_lens[i]), int(b.n_new[i])
        for t in range(n):
            pos, row = L - n + t, int(b.query_start_loc[i]) + t
            assert b.slot_mapping[row] // 16 == b.block_tables[i, pos // 16]
            assert b.slot_mapping[row] % 16 == pos % 16
            cblk = b.slot_mapping_compact[row] // 16
            assert b.phys_ids[cblk] == b.block_tables[i, pos // 16]
    # compact and physical tables describe the same blocks
    m = b.block_tables >= 0
    assert np.array_equal(b.phys_ids[b.block_tables_compact[m]], b.block_tables[m])
    assert np.all(b.block_tables_compact[~m] == -1)


def test_poison_marks_new_and_tail_slots_only():
    b = make_batch(B=4, Hq=2, Hkv=2, D=8, BS=16, dtype="f16", scale=0.1, seed=4,
                   n_new=3, ctx_range=(0, 40))
    for i in range(b.B):
        L, n = int(b.context_lens[i]), int(b.n_new[i])
        for pos in range(-(-L // 16) * 16):
            blk, off = b.block_tables_compact[i, pos // 16], pos % 16
            poisoned = np.all(b.k_blocks[blk, off] == POISON_U16)
            assert poisoned == (pos >= L - n)


def test_prefix_sharing_structure():
    b = make_batch(B=6, Hq=4, Hkv=2, D=8, BS=16, dtype="bf16", scale=0.1, seed=5,
                   lens_range=(300, 700), share=0.10)
    total = 0
    for k in range(0, 6, 2):
        n0 = -(-int(b.context_lens[k]) // 16)
        n1 = -(-int(b.context_lens[k + 1]) // 16)
        s = int(np.floor(0.10 * min(n0, n1)))
        total += s
        assert np.array_equal(b.block_tables[k + 1, :s], b.block_tables[k, :s])
        assert s < n1 - 1 and s < n0 - 1        # never the last block
        own = set(b.block_tables[k + 1, s:n1]) | set(b.block_tables[k, s:n0])
        assert not (own & set(b.block_tables[k, :s]))
    assert total == b.shared_pairs > 0
    used = b.block_tables[b.block_tables >= 0]
    assert len(np.unique(used)) == len(used) - total
    assert b.unique_kv_bytes() < b.kv_bytes()


def test_named_configs_match_their_recipe():
    c = CONFIGS
    assert (c["qwen3_0p6b_decode"]["B"], c["qwen3_0p6b_decode"]["Hq"], c["qwen3_0p6b_decode"]["Hkv"],
            c["qwen3_0p6b_decode"]["D"], c["qwen3_0p6b_decode"]["BS"], c["qwen3_0p6b_decode"]["NB"]) \
        == (128, 16, 8, 128, 16, 300_000)
    assert c["long_splitk_decode"]["BS"] == 256 and c["long_splitk_decode"]["partition"] == 512
    assert c["chunked_prefill"]["n_new"] == 512 and c["chunked_prefill"]["Hq"] == 32
    assert c["llama2_70b_decode_bs16"]["share"] == 0.10


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e38], np.float32)
    bits = to_u16(x, "bf16")
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert back[0] == 1.0 and back[1] == 1.0          # tie at 1 + 2^-8 rounds to even (1.0)
    assert back[2] == np.float32(1.0078125)           # above the tie rounds up
    assert back[3] == -2.5
