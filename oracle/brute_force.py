"""Pure-Python float64 brute force for tiny paged-attention inputs (TEST INFRASTRUCTURE ONLY).

No NumPy arithmetic: every score, exponential and weighted sum is an explicit
Python loop, and every key is fetched by walking the block table token by token
(page "Nano-vLLM-Ascend", section 2.1: the block table maps logical positions to
physical blocks).  Attention is ``softmax(q.k / sqrt(d)) v`` (same page, section
2.2.1) with the scale passed in.  Only for inputs of a few dozen tokens.
"""
from __future__ import annotations

import math
import struct


def _bits_to_float(bits: int, dtype: str) -> float:
    bits = int(bits) & 0xFFFF
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", bits << 16))[0]
    if dtype == "f16":
        return struct.unpack("<e", struct.pack("<H", bits))[0]
    raise ValueError(dtype)


def _attend(qv, keys, vals, scale):
    scores = [scale * math.fsum(a * b for a, b in zip(qv, k)) for k in keys]
    top = max(scores)
    w = [math.exp(s - top) for s in scores]
    z = math.fsum(w)
    D = len(vals[0])
    return [math.fsum(w[j] * vals[j][d] for j in range(len(vals))) / z for d in range(D)]


def _row(cache, table_row, j, kvh, BS, dtype):
    blk = int(table_row[j // BS])
    off = j % BS
    return [_bits_to_float(x, dtype) for x in cache[blk][off][kvh]]


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype):
    """Nested-list result ``[B][Hq][D]``; inputs may be NumPy arrays of bits."""
    B, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k_cache[0][0])
    BS = len(k_cache[0])
    G = Hq // Hkv
    out = []
    for i in range(B):
        L = int(context_lens[i])
        rows = []
        for h in range(Hq):
            if L == 0:
                rows.append([0.0] * D)
                continue
            kvh = h // G
            qv = [_bits_to_float(x, dtype) for x in q[i][h]]
            keys = [_row(k_cache, block_tables[i], j, kvh, BS, dtype) for j in range(L)]
            vals = [_row(v_cache, block_tables[i], j, kvh, BS, dtype) for j in range(L)]
            rows.append(_attend(qv, keys, vals, scale))
        out.append(rows)
    return out


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, dtype):
    """Nested-list result ``[T][Hq][D]``: new token t of sequence i sees keys 0..c_i+t."""
    T, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k_cache[0][0])
    BS = len(k_cache[0])
    G = Hq // Hkv
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(T)]
    for i in range(len(context_lens)):
        s0, s1 = int(query_start_loc[i]), int(query_start_loc[i + 1])
        L = int(context_lens[i])
        c = L - (s1 - s0)
        for t in range(s1 - s0):
            vis = c + t + 1
            for h in range(Hq):
                kvh = h // G
                qv = [_bits_to_float(x, dtype) for x in q[s0 + t][h]]
                keys = [_row(k_cache, block_tables[i], j, kvh, BS, dtype) for j in range(vis)]
                vals = [_row(v_cache, block_tables[i], j, kvh, BS, dtype) for j in range(vis)]
                out[s0 + t][h] = _attend(qv, keys, vals, scale)
    return out
