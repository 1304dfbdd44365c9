"""Plain CPU oracle for paged attention (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library:
its own 16-bit decoding, its own index arithmetic, plain NumPy in float64.

What it computes, and where the pages define it:

* Attention is ``softmax(q @ k.T / sqrt(d)) @ v`` -- page "Nano-vLLM-Ascend",
  section 2.2.1 (the "before" listing of the attention computation).  The scale
  is passed explicitly (section 4.2, problem 2 of the same page names the
  ``1/sqrt(d)`` factor as the first thing to check).
* The KV cache is cut into fixed 16-token blocks; a sequence of L tokens holds
  ``ceil(L/16)`` blocks -- same page, section 2.1 (worked example L = 1000).
* A block stores K and V as ``(block_size, num_heads, head_dim)`` and a block
  table maps a sequence's logical positions to physical blocks -- same page,
  section 2.1 (``Block`` / ``BlockTable``).
* Softmax is evaluated in at least fp32 with the row maximum subtracted -- page
  "vLLM-Ascend ...", section 3.1, problem 2 (fp16 accumulation faults cured by
  computing the softmax in float).  This oracle uses float64 throughout.

Readings where the pages are silent (each listed in the design notes):
query head h reads KV head ``h // G`` (G = Hq/Hkv, contiguous groups); a
sequence of length 0 yields a zero output row; slots < 0 are padding and are not
written; in a prefill chunk of n new tokens after c cached ones, new token t
sees keys ``0 .. c+t`` (bottom-right causal alignment).
"""
from __future__ import annotations

import math

import numpy as np


# --------------------------------------------------------------------------
# 16-bit storage decoding (exact)
# --------------------------------------------------------------------------
def decode_u16(bits: np.ndarray, dtype: str, out_dtype=np.float64) -> np.ndarray:
    """Exact value of fp16 / bf16 bit patterns."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        f32 = (bits.astype(np.uint32) << 16).view(np.float32)
    elif dtype == "f16":
        f32 = bits.view(np.float16).astype(np.float32)
    else:
        raise ValueError(dtype)
    return f32.astype(out_dtype)


# --------------------------------------------------------------------------
# Block arithmetic (page "Nano-vLLM-Ascend", section 2.1)
# --------------------------------------------------------------------------
def blocks_needed(L: int, block_size: int = 16) -> int:
    """Number of blocks a sequence of L tokens occupies: ceil(L / block_size)."""
    return -(-int(L) // int(block_size))


def slots_allocated(L: int, block_size: int = 16) -> int:
    return blocks_needed(L, block_size) * int(block_size)


def waste_fraction(L: int, block_size: int = 16) -> float:
    """Unused slots over allocated slots for one sequence."""
    s = slots_allocated(L, block_size)
    return (s - int(L)) / s if s else 0.0


def prealloc_waste(L: int, capacity: int) -> float:
    """Waste of reserving a contiguous region of ``capacity`` tokens for L tokens."""
    return (int(capacity) - int(L)) / int(capacity)


def pool_utilisation(lens, block_size: int = 16) -> float:
    """Occupied slots over allocated slots for a whole batch."""
    lens = [int(x) for x in lens]
    alloc = sum(slots_allocated(L, block_size) for L in lens)
    return sum(lens) / alloc if alloc else 1.0


def slot_position(slot: int, block_size: int) -> tuple[int, int]:
    """Physical (block, offset) of a flat cache slot index."""
    return slot // block_size, slot % block_size


def logical_to_physical(block_table_row, j: int, block_size: int) -> tuple[int, int]:
    """(physical block, offset) holding logical token j of a sequence."""
    return int(block_table_row[j // block_size]), j % block_size


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h: contiguous groups of G = Hq/Hkv query heads."""
    return h // (Hq // Hkv)


def visible_keys(c: int, t: int) -> int:
    """Keys visible to new token t of a chunk that follows c cached tokens."""
    return c + t + 1


# --------------------------------------------------------------------------
# reshape_and_cache: scatter new K/V rows into their slots (a bit copy)
# --------------------------------------------------------------------------
def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping) -> None:
    """For every token t with slot >= 0: cache[block, offset] = row t, all KV heads.

    ``k_cache``/``v_cache`` are uint16 ``[NB][BS][Hkv][D]`` arrays updated in place.
    """
    BS = k_cache.shape[1]
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        b, o = slot_position(slot, BS)
        k_cache[b, o] = key[t]
        v_cache[b, o] = value[t]


# --------------------------------------------------------------------------
# attention over a paged sequence
# --------------------------------------------------------------------------
def gather_sequence(cache, block_table_row, L: int, dtype: str, out_dtype=np.float64):
    """Logical rows 0..L-1 of one sequence, ``[L][Hkv][D]``, walked through its block table."""
    BS = cache.shape[1]
    n = blocks_needed(L, BS)
    rows = np.empty((n * BS,) + cache.shape[2:], dtype=np.uint16)
    for j in range(n):
        rows[j * BS:(j + 1) * BS] = cache[int(block_table_row[j])]
    return decode_u16(rows[:L], dtype, out_dtype)


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax with the row maximum subtracted (last axis)."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attend(qrows, K, V, scale: float, mask=None):
    """softmax(scale * q K^T) V for a stack of query rows against one KV head.

    qrows ``[n][D]``, K/V ``[L][D]``, optional boolean ``mask [n][L]`` (True = visible).
    Returns (out ``[n][D]``, probabilities ``[n][L]``).
    """
    s = scale * (qrows @ K.T)
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    p = softmax_rows(s)
    if mask is not None:
        p = np.where(mask, p, 0.0)
    return p @ V, p


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, dtype: str,
                 return_probs: bool = False, acc=np.float64):
    """Decode attention: one query row per sequence and query head.

    q ``[B][Hq][D]`` bits; caches ``[NB][BS][Hkv][D]`` bits; returns ``[B][Hq][D]``
    in ``acc`` (float64 by default).  ``return_probs`` also returns, per
    sequence, the ``[Hq][L]`` softmax rows.
    """
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    out = np.zeros((B, Hq, D), dtype=acc)
    probs = []
    for i in range(B):
        L = int(context_lens[i])
        if L <= 0:
            probs.append(np.zeros((Hq, 0), dtype=acc))
            continue
        K = gather_sequence(k_cache, block_tables[i], L, dtype, acc)
        V = gather_sequence(v_cache, block_tables[i], L, dtype, acc)
        qi = decode_u16(q[i], dtype, acc)
        p_i = np.empty((Hq, L), dtype=acc)
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            o, p = attend(qi[h:h + 1], K[:, kvh], V[:, kvh], scale)
            out[i, h] = o[0]
            p_i[h] = p[0]
        probs.append(p_i)
    return (out, probs) if return_probs else out


def paged_decode_one(i: int, h: int, q, k_cache, v_cache, block_tables, context_lens,
                     scale: float, dtype: str, acc=np.float64):
    """Decode output of a single (sequence i, query head h); ``[D]``."""
    Hq = q.shape[1]
    Hkv = k_cache.shape[2]
    L = int(context_lens[i])
    if L <= 0:
        return np.zeros(q.shape[2], dtype=acc)
    kvh = kv_head_of(h, Hq, Hkv)
    K = gather_sequence(k_cache[:, :, kvh:kvh + 1], block_tables[i], L, dtype, acc)[:, 0]
    V = gather_sequence(v_cache[:, :, kvh:kvh + 1], block_tables[i], L, dtype, acc)[:, 0]
    qh = decode_u16(q[i, h], dtype, acc)
    o, _ = attend(qh[None], K, V, scale)
    return o[0]


def paged_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start_loc,
                  scale: float, dtype: str, rows=None, acc=np.float64):
    """Chunked-prefill attention over a paged cache.

    Sequence i owns query rows ``query_start_loc[i] .. query_start_loc[i+1]-1``
    (n_i new tokens); its first ``c_i = context_lens[i] - n_i`` tokens were cached
    earlier and the new tokens' K/V are already in the cache.  New token t sees
    keys ``0 .. c_i + t``.  ``rows`` optionally restricts the computed query rows
    (others stay zero).  Returns ``[T][Hq][D]``.
    """
    T, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    B = len(context_lens)
    out = np.zeros((T, Hq, D), dtype=acc)
    wanted = None if rows is None else set(int(r) for r in rows)
    for i in range(B):
        s0, s1 = int(query_start_loc[i]), int(query_start_loc[i + 1])
        n = s1 - s0
        L = int(context_lens[i])
        if n <= 0 or L <= 0:
            continue
        c = L - n
        ts = [t for t in range(n) if wanted is None or (s0 + t) in wanted]
        if not ts:
            continue
        K = gather_sequence(k_cache, block_tables[i], L, dtype, acc)
        V = gather_sequence(v_cache, block_tables[i], L, dtype, acc)
        ts_a = np.asarray(ts)
        mask = np.arange(L)[None, :] < np.array([visible_keys(c, t) for t in ts])[:, None]
        qi = decode_u16(q[s0 + ts_a], dtype, acc)  # [len(ts)][Hq][D]
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            o, _ = attend(qi[:, h], K[:, kvh], V[:, kvh], scale, mask)
            out[s0 + ts_a, h] = o
    return out
