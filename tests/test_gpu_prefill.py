"""GPU parity of the MFMA chunked-prefill kernel against the CPU oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_324_amd import (pa_decode, pa_decode_order, pa_prefill_chunk,
                                    pa_reshape_and_cache)
from workloads import make_batch, make_config

from _gpu import (check_close, check_full, config_batch, host_caches_after_write, log,
                  to_bits, to_f64, upload)

pytestmark = pytest.mark.gpu


def _prefill(b, d, ordered=False, q=None, lens=None, qsl=None, max_q=None):
    pa_reshape_and_cache(d.key_new, d.value_new, d.k_cache, d.v_cache, d.slot_mapping)
    q = d.q if q is None else q
    out = torch.empty_like(q)
    order = torch.from_numpy(pa_decode_order(b.context_lens)).cuda() if ordered else None
    pa_prefill_chunk(out, q, d.k_cache, d.v_cache, d.block_tables,
                     d.context_lens if lens is None else lens,
                     d.query_start_loc if qsl is None else qsl,
                     b.max_query_len if max_q is None else max_q, b.scale, seq_order=order)
    torch.cuda.synchronize()
    return out


def _oracle(b, rows=None):
    kc, vc = host_caches_after_write(b)
    return oracle.paged_prefill(b.q, kc, vc, b.block_tables_compact, b.context_lens,
                                b.query_start_loc, b.scale, b.dtype, rows=rows)


def test_prefill_chunked_config_full_size():
    """Every query row of the chunked-prefill workload (8 x 512 new tokens after 0-8192
    cached ones) against the float64 oracle."""
    b = config_batch("chunked_prefill")
    log(f"prefill chunked config: B={b.B} T={b.num_tokens} ctx={(b.context_lens - b.n_new).tolist()}")
    got = to_f64(_prefill(b, upload(b), ordered=True))
    check_full(got, _oracle(b), "chunked_prefill", b.dtype)


SWEEP = [(dt, D, BS, G) for dt in ("bf16", "f16") for D in (128, 64) for BS in (16, 32, 256)
         for G in (1, 2, 4, 8)]


@pytest.mark.parametrize("dt,D,BS,G", SWEEP)
def test_prefill_shape_sweep(dt, D, BS, G):
    Hkv = 2
    b = make_batch(B=3, Hq=Hkv * G, Hkv=Hkv, D=D, BS=BS, dtype=dt, scale=D ** -0.5,
                   seed=2000 + SWEEP.index((dt, D, BS, G)), n_new=150, ctx_range=(0, 400))
    got = to_f64(_prefill(b, upload(b)))
    check_close(got, _oracle(b), f"prefill {dt} D{D} BS{BS} G{G}")


@pytest.mark.parametrize("n_new,ctx", [(1, (0, 0)), (17, (0, 0)), (64, (63, 65)), (300, (1000, 1400))])
def test_prefill_head_dim_64_chunk_lengths(n_new, ctx):
    b = make_batch(B=4, Hq=32, Hkv=8, D=64, BS=16, dtype="bf16", scale=0.125,
                   seed=3050 + n_new, n_new=n_new, ctx_range=ctx)
    got = to_f64(_prefill(b, upload(b), ordered=True))
    check_close(got, _oracle(b), f"prefill D64 n={n_new} ctx={ctx}")


def test_prefill_head_dim_64_rows_equal_decodes():
    """Row t of a head_dim-64 chunk equals a GPU decode of the same query with context c + t + 1."""
    b = make_batch(B=2, Hq=16, Hkv=4, D=64, BS=32, dtype="f16", scale=0.125, seed=3210,
                   n_new=40, ctx_range=(100, 300))
    d = upload(b)
    got = to_f64(_prefill(b, d))
    for i in range(b.B):
        s0, n = int(b.query_start_loc[i]), int(b.n_new[i])
        c = int(b.context_lens[i]) - n
        ts = [0, 1, 31, 32, 39]
        q = d.q[s0 + torch.tensor(ts, device="cuda")].contiguous()
        lens = torch.tensor([c + t + 1 for t in ts], dtype=torch.int32, device="cuda")
        tables = d.block_tables[i:i + 1].repeat(len(ts), 1).contiguous()
        out = torch.empty_like(q)
        pa_decode(out, q, d.k_cache, d.v_cache, tables, lens, b.scale, c + n, 0)
        torch.cuda.synchronize()
        check_close(got[[s0 + t for t in ts]], to_f64(out), "D64 chunk vs decodes")


@pytest.mark.parametrize("n_new,ctx", [(1, (0, 0)), (1, (700, 900)), (17, (0, 0)),
                                       (64, (63, 65)), (129, (0, 5)), (300, (1000, 1400))])
def test_prefill_chunk_lengths(n_new, ctx):
    b = make_batch(B=4, Hq=32, Hkv=8, D=128, BS=16, dtype="bf16", scale=128 ** -0.5,
                   seed=3000 + n_new, n_new=n_new, ctx_range=ctx)
    got = to_f64(_prefill(b, upload(b), ordered=True))
    check_close(got, _oracle(b), f"prefill n={n_new} ctx={ctx}")


def test_prefill_without_cache_is_causal_attention():
    b = make_batch(B=2, Hq=8, Hkv=2, D=128, BS=16, dtype="bf16", scale=128 ** -0.5, seed=3100,
                   n_new=200, ctx_range=(0, 0))
    got = to_f64(_prefill(b, upload(b)))
    check_close(got, _oracle(b), "pure causal")
    # first token of each sequence sees only itself: its value row exactly
    for i in range(b.B):
        s0 = int(b.query_start_loc[i])
        for h in range(8):
            v0 = oracle.decode_u16(b.value_new[s0, h // 4], "bf16")
            assert np.array_equal(got[s0, h], v0)


def test_prefill_rows_equal_decodes_on_gpu():
    """Row t of a chunk equals a GPU decode of the same query with context c + t + 1."""
    b = make_batch(B=2, Hq=16, Hkv=8, D=128, BS=16, dtype="bf16", scale=128 ** -0.5, seed=3200,
                   n_new=48, ctx_range=(100, 300))
    d = upload(b)
    got = to_f64(_prefill(b, d))
    for i in range(b.B):
        s0, n = int(b.query_start_loc[i]), int(b.n_new[i])
        c = int(b.context_lens[i]) - n
        ts = [0, 1, 15, 16, 47]
        q = d.q[s0 + torch.tensor(ts, device="cuda")].contiguous()
        lens = torch.tensor([c + t + 1 for t in ts], dtype=torch.int32, device="cuda")
        tables = d.block_tables[i:i + 1].repeat(len(ts), 1).contiguous()
        out = torch.empty_like(q)
        pa_decode(out, q, d.k_cache, d.v_cache, tables, lens, b.scale, c + n, 0)
        torch.cuda.synchronize()
        check_close(got[[s0 + t for t in ts]], to_f64(out), "chunk vs decodes")


def test_prefill_chunk_split_invariance():
    """A 256-token chunk equals two 128-token chunks over the same cache."""
    b = make_batch(B=2, Hq=32, Hkv=8, D=128, BS=16, dtype="bf16", scale=128 ** -0.5, seed=3300,
                   n_new=256, ctx_range=(0, 600))
    d = upload(b)
    whole = to_f64(_prefill(b, d))
    halves = np.zeros_like(whole)
    for part in range(2):
        rows = torch.cat([torch.arange(int(b.query_start_loc[i]) + 128 * part,
                                       int(b.query_start_loc[i]) + 128 * (part + 1))
                          for i in range(b.B)]).cuda()
        lens = d.context_lens - (128 if part == 0 else 0)
        qsl = torch.tensor([0, 128, 256], dtype=torch.int32, device="cuda")
        out = torch.empty((256, 32, 128), dtype=d.q.dtype, device="cuda")
        pa_prefill_chunk(out, d.q[rows].contiguous(), d.k_cache, d.v_cache, d.block_tables,
                         lens.contiguous(), qsl, 128, b.scale)
        torch.cuda.synchronize()
        halves[rows.cpu().numpy()] = to_f64(out)
    check_close(halves, whole, "two half chunks")
    assert np.max(np.abs(halves - whole)) < 2e-2


def test_prefill_seq_order_changes_no_bits():
    b = make_batch(B=5, Hq=16, Hkv=4, D=128, BS=32, dtype="bf16", scale=128 ** -0.5, seed=3400,
                   n_new=70, ctx_range=(0, 900))
    d = upload(b)
    a = to_bits(_prefill(b, d, ordered=False))
    c = to_bits(_prefill(b, d, ordered=True))
    assert np.array_equal(a, c)
