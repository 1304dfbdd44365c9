"""Rotary position embedding fused with the KV-cache write (TEST INFRASTRUCTURE ONLY).

Only ``tests/`` may import this module.  It shares no code with the HIP library.

The pages wrap a device rotary-multiply primitive in an autograd function whose
forward maps ``(x, cos, sin)`` to the rotated ``x`` and whose backward applies
the same primitive with ``-sin`` (page "Nano-vLLM-Ascend", section 5.1, custom
operator example).  The pages do not spell out the primitive; the reading taken
here is the one the models they serve (Llama3, Qwen3; section 3.1) use: the head
dimension is cut into halves ``x1 = x[:D/2]``, ``x2 = x[D/2:]`` and pair
``(x1_i, x2_i)`` is turned by angle ``theta_{p,i}`` of the token's position p:

    y1_i = x1_i cos_i - x2_i sin_i,     y2_i = x2_i cos_i + x1_i sin_i.

This is linear in x with transpose equal to the same map with ``-sin``, which is
exactly the backward the pages give (a rotation's transpose is its inverse).

Arithmetic (fixed here so that the device kernel can be compared bit for bit):
inputs are 16-bit (fp16/bf16) values, the table rows ``cos[p]``, ``sin[p]`` are
float32 ``[max_position][D/2]``; every product and the one sum/difference are
rounded to float32 separately (no fused multiply-add), and the result is rounded
once to the 16-bit type, nearest-even.

Fused step (the pages name removing separate passes by fusing operators, page
"vLLM-Ascend ...", section 5): for each token t with a valid position, its key
rows are rotated and written with its value rows into cache slot
``slot_mapping[t]`` exactly as ``reshape_and_cache`` does, and its query rows
(when given) are rotated in place.  A token whose position lies outside the
table is left alone entirely (query untouched, nothing written).
"""
from __future__ import annotations

import numpy as np

from .paged_attention import decode_u16, reshape_and_cache


def encode_u16(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to fp16/bf16 bit patterns, nearest-even."""
    x32 = np.asarray(x32, dtype=np.float32)
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = x32.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16          # carry rounds up, ties to even
    nan = np.isnan(x32)
    out = np.where(nan, (u >> 16) | 0x40, rounded)          # keep NaNs NaN (quiet bit)
    return out.astype(np.uint16)


def rotate_f32(x_bits, positions, cos, sin, dtype: str) -> np.ndarray:
    """Rotated rows in float32 before the final rounding: x_bits [T][H][D] 16-bit,
    positions [T] (each in range), cos/sin float32 [max_position][D/2]."""
    x = decode_u16(x_bits, dtype, out_dtype=np.float32)
    D = x.shape[-1]
    h = D // 2
    x1, x2 = x[..., :h], x[..., h:]
    pos = np.asarray(positions, dtype=np.int64)
    c = np.asarray(cos, np.float32)[pos][:, None, :]        # [T][1][D/2], one row per token
    s = np.asarray(sin, np.float32)[pos][:, None, :]
    y1 = (x1 * c) - (x2 * s)                                 # float32, each op rounded
    y2 = (x2 * c) + (x1 * s)
    return np.concatenate([y1, y2], axis=-1).astype(np.float32)


def rotate(x_bits, positions, cos, sin, dtype: str) -> np.ndarray:
    """Rotated rows as 16-bit bit patterns (see ``rotate_f32``)."""
    return encode_u16(rotate_f32(x_bits, positions, cos, sin, dtype), dtype)


def rope_reshape_and_cache(q, key, value, k_cache, v_cache, positions, cos, sin, slot_mapping,
                           dtype: str):
    """The fused step.  q [T][Hq][D] or None, key/value [T][Hkv][D] (16-bit bits);
    caches [NB][BS][Hkv][D] are updated in place; returns the rotated q (None if q is None).
    Tokens with positions outside [0, len(cos)) change nothing."""
    pos = np.asarray(positions, dtype=np.int64)
    ok = (pos >= 0) & (pos < len(cos))
    safe = np.where(ok, pos, 0)
    slots = np.asarray(slot_mapping, np.int64)
    num_slots = k_cache.shape[0] * k_cache.shape[1]
    slots = np.where(ok & (slots < num_slots), slots, -1)   # out-of-pool slots are skipped too
    k_rot = rotate(key, safe, cos, sin, dtype)
    reshape_and_cache(k_rot, value, k_cache, v_cache, slots)
    if q is None:
        return None
    q_rot = rotate(q, safe, cos, sin, dtype)
    return np.where(ok[:, None, None], q_rot, np.asarray(q, np.uint16))
