"""Context-parallel decode: shard partials and their merge (TEST INFRASTRUCTURE ONLY).

Only ``tests/`` may import this module.  It shares no code with the HIP library.

The pages scale long contexts by splitting a sequence's context across devices
(page "vllm-ascend architecture", sections 1.1 and 3.1: context parallelism for
long sequences).  Each shard attends over its own keys and produces, per
(sequence, query head), the shard's softmax-normalised output ``o`` together with
the two numbers that let shards be combined exactly: ``m`` (the shard's maximum
score, base-2 logarithm scale: ``m = max_j s_j * log2(e)`` with ``s_j = scale * q . K_j``)
and ``l = sum_j 2^(s_j log2 e - m)``.  Merging: ``M = max m``,
``w = l * 2^(m - M)``, ``out = sum w o / sum w``.  A shard holding no key of a
sequence contributes ``l = 0`` (its ``m`` and ``o`` are irrelevant).

The pair ``(m, l)`` is defined only up to ``(m + c, l * 2^-c)``; every consumer
uses ``l * 2^m``, so tests compare that product.
"""
from __future__ import annotations

import math

import numpy as np

from .paged_attention import decode_u16, gather_sequence, kv_head_of

LOG2E = 1.0 / math.log(2.0)


def shard_partial(q, k_cache, v_cache, block_tables, context_lens, scale: float, dtype: str):
    """Per (sequence, query head) partial of one shard: ``(o [B][Hq][D], m [B][Hq], l [B][Hq])``
    in float64.  The shard's keys of sequence i are its logical tokens ``0 .. L_i - 1`` walked
    through the shard's block table (a shard's table lists only the shard's blocks)."""
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    o = np.zeros((B, Hq, D))
    m = np.full((B, Hq), -np.inf)
    l = np.zeros((B, Hq))
    for i in range(B):
        L = int(context_lens[i])
        if L <= 0:
            continue
        K = gather_sequence(k_cache, block_tables[i], L, dtype)
        V = gather_sequence(v_cache, block_tables[i], L, dtype)
        qi = decode_u16(q[i], dtype)
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            s2 = scale * (K[:, kvh] @ qi[h]) * LOG2E     # scores in base-2 units
            m[i, h] = s2.max()
            p = np.exp2(s2 - m[i, h])
            l[i, h] = p.sum()
            o[i, h] = (p @ V[:, kvh]) / l[i, h]
    return o, m, l


def merge_partials(os, ms, ls):
    """Merge shard partials ``o [N][B][Hq][D]``, ``m, l [N][B][Hq]`` into ``[B][Hq][D]``;
    rows whose shards are all empty give zeros."""
    os, ms, ls = np.asarray(os, float), np.asarray(ms, float), np.asarray(ls, float)
    M = np.max(np.where(ls > 0, ms, -np.inf), axis=0)
    w = np.where(ls > 0, ls * np.exp2(np.where(ls > 0, ms, 0.0) - np.where(np.isfinite(M), M, 0.0)), 0.0)
    den = w.sum(axis=0)
    out = np.einsum("nbh,nbhd->bhd", w, os)
    return np.where(den[..., None] > 0, out / np.where(den > 0, den, 1.0)[..., None], 0.0)
