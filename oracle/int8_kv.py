"""INT8 KV cache: quantisation and attention over it (TEST INFRASTRUCTURE ONLY).

Only ``tests/`` may import this module.  It shares no code with the HIP library.

The pages list INT8 quantisation of the KV cache as the next step for
throughput (page "Nano-vLLM-Ascend", section 4.3, advanced optimisations: KV
cache compression, INT8 quantisation) and warn that the attention scores'
precision is what has to be kept (page "vLLM-Ascend ...", section 5, mixed
precision).  They fix no scheme; the reading taken here is the plainest one that
keeps each score's precision local:

* symmetric, per token and KV head: ``scale = amax / 127`` with
  ``amax = max_d |x_d|`` over the head's ``head_dim`` values, and
  ``code_d = rint(x_d / scale)`` (round half to even), codes in [-127, 127];
  an all-zero row has scale 0 and codes 0;
* everything in IEEE float32 (the inputs are 16-bit, so |x_d| and amax are
  exact in float32; the two divisions are correctly rounded), so the device
  reaches the same codes and scales bit for bit;
* the value used by attention is ``code_d * scale`` (exact in float64).

Cache layout (the library's), head-major within a block: codes
``int8 [NB][Hkv][BS][D]``; scales ``float32 [NB][Hkv][BS]``.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import attend, blocks_needed, decode_u16, kv_head_of


def quantize_rows(bits: np.ndarray, dtype: str):
    """16-bit rows ``[..., D]`` -> (codes int8 ``[..., D]``, scales float32 ``[...]``)."""
    x = decode_u16(bits, dtype, out_dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    codes = np.rint(x / safe[..., None]).astype(np.float32)
    codes = np.where(scale[..., None] > 0, codes, np.float32(0.0))
    assert np.all(np.abs(codes) <= 127)
    return codes.astype(np.int8), scale


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Codes ``[..., D]`` times their row scales ``[...]`` in float64 (exact)."""
    return codes.astype(np.float64) * scales.astype(np.float64)[..., None]


def reshape_and_cache_int8(key, value, k_codes, v_codes, k_scales, v_scales, slot_mapping,
                           dtype: str) -> None:
    """Quantise this step's rows ``[T][Hkv][D]`` (16-bit bits) into their slots, in place.

    Caches: codes ``[NB][Hkv][BS][D]`` int8, scales ``[NB][Hkv][BS]`` float32.
    Slots < 0 (padding) and slots outside the pool are skipped.
    """
    NB, BS = k_codes.shape[0], k_codes.shape[2]
    kq, ks = quantize_rows(key, dtype)
    vq, vs = quantize_rows(value, dtype)
    for t, slot in enumerate(np.asarray(slot_mapping)):
        slot = int(slot)
        if slot < 0 or slot >= NB * BS:
            continue
        b, o = slot // BS, slot % BS
        k_codes[b, :, o] = kq[t]
        v_codes[b, :, o] = vq[t]
        k_scales[b, :, o] = ks[t]
        v_scales[b, :, o] = vs[t]


def gather_int8(codes, scales, block_table_row, L: int) -> np.ndarray:
    """Dequantised logical rows 0..L-1 of one sequence, ``[L][Hkv][D]`` float64."""
    BS = codes.shape[2]
    parts = []
    for j in range(blocks_needed(L, BS)):
        b = int(block_table_row[j])
        parts.append(dequantize(codes[b], scales[b]).transpose(1, 0, 2))  # [BS][Hkv][D]
    return np.concatenate(parts)[:L]


def paged_decode_int8(q, k_codes, v_codes, k_scales, v_scales, block_tables, context_lens,
                      scale: float, dtype: str):
    """Decode attention over the dequantised cache: ``softmax(scale q K'^T) V'`` with
    ``K'`` = code x scale per token and head; q is 16-bit bits ``[B][Hq][D]``;
    a sequence of length 0 gives a zero row.  Returns ``[B][Hq][D]`` float64."""
    B, Hq, D = q.shape
    Hkv = k_codes.shape[1]
    out = np.zeros((B, Hq, D))
    for i in range(B):
        L = int(context_lens[i])
        if L <= 0:
            continue
        K = gather_int8(k_codes, k_scales, block_tables[i], L)
        V = gather_int8(v_codes, v_scales, block_tables[i], L)
        qi = decode_u16(q[i], dtype)
        for h in range(Hq):
            kvh = kv_head_of(h, Hq, Hkv)
            o, _ = attend(qi[h:h + 1], K[:, kvh], V[:, kvh], scale)
            out[i, h] = o[0]
    return out
