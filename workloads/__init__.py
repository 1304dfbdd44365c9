"""Seeded synthetic inputs for paged-attention workloads.

This module only *draws inputs*: sequence lengths, block tables (which physical
KV block holds each logical block of a sequence), slot mappings for the new
tokens, and N(0,1) query / key / value values rounded to the storage dtype.
It holds none of the attention arithmetic, so both the CPU oracle and the HIP
path can consume it without sharing any of the method's code.

Cache layout drawn here is the per-block layout of the page "Nano-vLLM-Ascend"
(section 2.1, the ``Block`` structure whose K and V tensors are shaped
``(block_size, num_heads, head_dim)``): a cache is ``[num_blocks][block_size]
[num_kv_heads][head_dim]``, with separate K and V caches.

Everything returned is a NumPy array; 16-bit floating values are returned as
their raw ``uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

POISON_U16 = 0xFFFF  # a NaN in both fp16 and bf16: marks slots that hold no token yet

# Named workloads.  Shapes follow the workloads the pages describe:
#   * Qwen3-0.6B batch study (page "Nano-vLLM-Ascend", section 3.2.1: batch > 128,
#     prompt and output lengths drawn from 100..1024),
#   * Llama2-70B deployment (page "vLLM-Ascend ...", section 4) with prefix-block
#     sharing for long contexts (same page, section 4),
#   * 256-token blocks (same page, section 2.2 tuning table),
#   * chunked prefill (page "vllm-ascend architecture", section 1.1 / 3.1).
# partition: tokens per split-K partition of a decode (0 = unsplit); None where
# the workload fixes none: the caller then asks the library for the device's
# choice (pa_decode_partition_hint).
CONFIGS = {
    "tiny_decode": dict(
        kind="decode", B=4, Hq=8, Hkv=8, D=64, BS=16, NB=128, lens=(1, 256),
        dtype="f16", scale=1.0 / 8.0, share=0.0, partition=0, seed=324_001),
    "qwen3_0p6b_decode": dict(
        kind="decode", B=128, Hq=16, Hkv=8, D=128, BS=16, NB=300_000, lens=(200, 2048),
        dtype="bf16", scale=1.0 / math.sqrt(128), share=0.0, partition=0, seed=324_002),
    "llama2_70b_decode_bs16": dict(
        kind="decode", B=64, Hq=64, Hkv=8, D=128, BS=16, NB=None, lens=(4096, 8192),
        dtype="bf16", scale=1.0 / math.sqrt(128), share=0.10, partition=None, seed=324_003),
    "llama2_70b_decode_bs32": dict(
        kind="decode", B=64, Hq=64, Hkv=8, D=128, BS=32, NB=None, lens=(4096, 8192),
        dtype="bf16", scale=1.0 / math.sqrt(128), share=0.10, partition=None, seed=324_003),
    "long_splitk_decode": dict(
        kind="decode", B=8, Hq=32, Hkv=8, D=128, BS=256, NB=2048, lens=(16384, 32768),
        dtype="bf16", scale=1.0 / math.sqrt(128), share=0.0, partition=512, seed=324_004),
    "chunked_prefill": dict(
        kind="prefill", B=8, Hq=32, Hkv=8, D=128, BS=16, NB=8192, ctx=(0, 8192), n_new=512,
        dtype="bf16", scale=1.0 / math.sqrt(128), share=0.0, partition=0, seed=324_005),
}


@dataclasses.dataclass
class PagedBatch:
    """One step's inputs.

    ``k_blocks``/``v_blocks`` hold only the physical blocks the batch references
    (``phys_ids[c]`` is the physical id of compact block ``c``), in the state the
    cache is in *before* the step's new tokens are written: slots of earlier
    tokens hold values, slots reserved for this step's new tokens and the unused
    tail of each sequence's last block hold ``POISON_U16``.
    """
    dtype: str                 # "bf16" or "f16"
    B: int
    Hq: int
    Hkv: int
    D: int
    BS: int
    NB: int                    # physical pool size (blocks)
    scale: float
    context_lens: np.ndarray   # int32 [B], tokens each query attends over incl. this step's new ones
    n_new: np.ndarray          # int32 [B], new tokens (== queries) per sequence this step
    query_start_loc: np.ndarray  # int32 [B+1], prefix sum of n_new
    block_tables: np.ndarray   # int32 [B][max_blocks], physical ids, -1 past the end
    block_tables_compact: np.ndarray  # same, compact ids
    phys_ids: np.ndarray       # int64 [n_used], physical id of each compact block (sorted)
    k_blocks: np.ndarray       # uint16 [n_used][BS][Hkv][D]
    v_blocks: np.ndarray       # uint16 [n_used][BS][Hkv][D]
    q: np.ndarray              # uint16 [B][Hq][D] (decode) or [T][Hq][D] (prefill)
    key_new: np.ndarray        # uint16 [T][Hkv][D]
    value_new: np.ndarray      # uint16 [T][Hkv][D]
    slot_mapping: np.ndarray   # int64 [T], physical slot = block*BS + offset
    slot_mapping_compact: np.ndarray  # int64 [T], same in compact ids
    shared_pairs: int = 0      # number of logical blocks mapped onto another sequence's block

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.B else 0

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_query_len(self) -> int:
        return int(self.n_new.max()) if self.B else 0

    def kv_bytes(self) -> int:
        """Logical K+V bytes the step attends over (every token of every sequence, once)."""
        return int(self.context_lens.astype(np.int64).sum()) * self.Hkv * self.D * 2 * 2

    def unique_kv_bytes(self) -> int:
        """K+V bytes of distinct attended tokens (shared prefix blocks counted once)."""
        seen = set()
        tokens = 0
        for i in range(self.B):
            L = int(self.context_lens[i])
            for j in range(-(-L // self.BS)):
                b = int(self.block_tables[i, j])
                if b in seen:
                    continue
                seen.add(b)
                tokens += min(self.BS, L - j * self.BS)
        return tokens * self.Hkv * self.D * 2 * 2


def to_u16(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to fp16 / bf16 (round to nearest even) and return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        if not np.all(np.isfinite(x)):
            raise ValueError("bf16 rounding here is for finite values only")
        r = (u >> 16) & 1
        r += u
        r += 0x7FFF          # cannot wrap: finite floats stay below 0xFF800000
        r >>= 16
        return r.astype(np.uint16)
    raise ValueError(dtype)


def rope_tables(max_position: int, head_dim: int, base: float = 1.0e6):
    """Rotary tables as a model supplies them: cos and sin of p * base^(-2i/head_dim) for
    positions p < max_position and pair index i < head_dim / 2, computed in float64 and
    stored as float32 [max_position][head_dim / 2].  (Qwen3 uses base 1e6.)"""
    inv_freq = base ** (-np.arange(0, head_dim, 2, dtype=np.float64) / head_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _normal_u16(rng: np.random.Generator, shape, dtype: str, chunk: int = 1 << 24) -> np.ndarray:
    """N(0,1) values rounded to ``dtype``; drawn in fixed chunks of 2**24 values."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = to_u16(rng.standard_normal(e - s, dtype=np.float32), dtype)
    return out.reshape(shape)


def make_batch(*, B: int, Hq: int, Hkv: int, D: int, BS: int, dtype: str, scale: float,
               seed: int, lens=None, lens_range=None, n_new=1, ctx_range=None,
               NB: int | None = None, share: float = 0.0, pool_slack: float = 1.25) -> PagedBatch:
    """Draw one step's inputs.

    Draw order: lengths -> block tables -> q -> K/V -> new tokens.

    * decode: ``n_new=1``; ``context_lens`` drawn uniform in ``lens_range``
      (inclusive) unless given in ``lens``.
    * chunked prefill: ``n_new=n`` new query tokens per sequence after ``c``
      cached tokens, ``c`` drawn uniform in ``ctx_range``; ``context_lens = c + n``.
    * ``share``: sequences (2k, 2k+1) share a prefix: the first
      ``floor(share * min(nblocks_2k, nblocks_2k+1))`` logical blocks of sequence
      2k+1 are the physical blocks of sequence 2k (reference count 2).  Shared
      blocks are always full blocks, never a sequence's last block.
    * ``NB``: physical pool size; default ``ceil(pool_slack * blocks needed)``.
      Physical ids are a seeded random draw without replacement from the pool.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    # 1. lengths
    if ctx_range is not None:
        c = rng.integers(ctx_range[0], ctx_range[1], size=B, endpoint=True).astype(np.int64)
        nn = np.full(B, int(n_new), dtype=np.int64)
        L = c + nn
    else:
        if lens is not None:
            L = np.asarray(lens, dtype=np.int64).reshape(B)
        else:
            L = rng.integers(lens_range[0], lens_range[1], size=B, endpoint=True).astype(np.int64)
        nn = np.minimum(np.full(B, int(n_new), dtype=np.int64), L)
    nblk = -(-L // BS)
    max_blocks = int(max(1, nblk.max())) if B else 1

    # 2. block tables
    shared = np.zeros(B, dtype=np.int64)
    if share > 0:
        for k in range(0, B - 1, 2):
            shared[k + 1] = int(math.floor(share * min(nblk[k], nblk[k + 1])))
    need = int(nblk.sum() - shared.sum())
    if NB is None:
        NB = int(math.ceil(pool_slack * max(need, 1)))
    if need > NB:
        raise ValueError(f"pool of {NB} blocks cannot hold {need} blocks")
    phys = rng.permutation(NB)[:need].astype(np.int64)
    bt = np.full((B, max_blocks), -1, dtype=np.int64)
    cur = 0
    for i in range(B):
        s = int(shared[i])
        if s:
            bt[i, :s] = bt[i - 1, :s]
        n_own = int(nblk[i]) - s
        bt[i, s:s + n_own] = phys[cur:cur + n_own]
        cur += n_own
    phys_ids = np.sort(phys)
    compact_of = {int(p): c for c, p in enumerate(phys_ids)}
    btc = np.full_like(bt, -1)
    for i in range(B):
        for j in range(int(nblk[i])):
            btc[i, j] = compact_of[int(bt[i, j])]

    qsl = np.zeros(B + 1, dtype=np.int64)
    qsl[1:] = np.cumsum(nn)
    T = int(qsl[-1])

    # 3. queries: one per sequence for decode (even an empty one), one per new token for prefill
    q = _normal_u16(rng, (T if ctx_range is not None else B, Hq, D), dtype)
    # 4. cached K/V of earlier tokens (whole blocks drawn, then unwritten slots poisoned)
    n_used = len(phys_ids)
    k_blocks = _normal_u16(rng, (n_used, BS, Hkv, D), dtype)
    v_blocks = _normal_u16(rng, (n_used, BS, Hkv, D), dtype)
    for i in range(B):
        first_new = int(L[i] - nn[i])
        for pos in range(first_new, int(nblk[i]) * BS):
            cb, off = btc[i, pos // BS], pos % BS
            k_blocks[cb, off] = POISON_U16
            v_blocks[cb, off] = POISON_U16
    # 5. this step's new tokens and their slots
    key_new = _normal_u16(rng, (T, Hkv, D), dtype)
    value_new = _normal_u16(rng, (T, Hkv, D), dtype)
    slot = np.empty(T, dtype=np.int64)
    slot_c = np.empty(T, dtype=np.int64)
    for i in range(B):
        first_new = int(L[i] - nn[i])
        for t in range(int(nn[i])):
            pos = first_new + t
            slot[qsl[i] + t] = bt[i, pos // BS] * BS + pos % BS
            slot_c[qsl[i] + t] = btc[i, pos // BS] * BS + pos % BS

    return PagedBatch(
        dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, BS=BS, NB=int(NB), scale=float(scale),
        context_lens=L.astype(np.int32), n_new=nn.astype(np.int32),
        query_start_loc=qsl.astype(np.int32),
        block_tables=bt.astype(np.int32), block_tables_compact=btc.astype(np.int32),
        phys_ids=phys_ids, k_blocks=k_blocks, v_blocks=v_blocks, q=q,
        key_new=key_new, value_new=value_new, slot_mapping=slot, slot_mapping_compact=slot_c,
        shared_pairs=int(shared.sum()))


def make_config(name: str, seed: int | None = None, **overrides) -> PagedBatch:
    """Draw the named workload (see ``CONFIGS``); ``overrides`` shrink it for tests."""
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    seed = cfg["seed"] if seed is None else seed
    common = dict(B=cfg["B"], Hq=cfg["Hq"], Hkv=cfg["Hkv"], D=cfg["D"], BS=cfg["BS"],
                  dtype=cfg["dtype"], scale=cfg["scale"], seed=seed, NB=cfg.get("NB"),
                  share=cfg.get("share", 0.0))
    if cfg["kind"] == "prefill":
        return make_batch(n_new=cfg["n_new"], ctx_range=cfg["ctx"], **common)
    return make_batch(n_new=1, lens=cfg.get("lens_list"), lens_range=cfg["lens"], **common)
