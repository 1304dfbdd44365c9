"""Helpers of the GPU parity tests: put a PagedBatch on the device, run the oracle beside it."""
from __future__ import annotations

import sys
import types

import numpy as np
import torch

import oracle
from workloads import PagedBatch

# Acceptance bar for 16-bit attention outputs against the float64 oracle.
MAX_ABS = 1.5e-2
REL_L2 = 5e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(b: PagedBatch):
    return torch.bfloat16 if b.dtype == "bf16" else torch.float16


def bits_to_device(a: np.ndarray, dt, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(dt)


def upload(b: PagedBatch, device="cuda") -> types.SimpleNamespace:
    """Device pool of b.NB blocks, NaN everywhere except the referenced blocks."""
    dt = torch_dtype(b)
    shape = (b.NB, b.BS, b.Hkv, b.D)
    kc = torch.full(shape, -1, dtype=torch.int16, device=device)   # 0xFFFF = NaN
    vc = torch.full(shape, -1, dtype=torch.int16, device=device)
    idx = torch.from_numpy(b.phys_ids).to(device)
    kc[idx] = torch.from_numpy(b.k_blocks.view(np.int16)).to(device)
    vc[idx] = torch.from_numpy(b.v_blocks.view(np.int16)).to(device)
    return types.SimpleNamespace(
        k_cache=kc.view(dt), v_cache=vc.view(dt),
        q=bits_to_device(b.q, dt, device),
        key_new=bits_to_device(b.key_new, dt, device),
        value_new=bits_to_device(b.value_new, dt, device),
        slot_mapping=torch.from_numpy(b.slot_mapping).to(device),
        block_tables=torch.from_numpy(b.block_tables).to(device),
        context_lens=torch.from_numpy(b.context_lens).to(device),
        query_start_loc=torch.from_numpy(b.query_start_loc).to(device),
        idx=idx)


def host_caches_after_write(b: PagedBatch):
    """Oracle view of the cache after this step's tokens are written (compact block ids)."""
    kc, vc = b.k_blocks.copy(), b.v_blocks.copy()
    oracle.reshape_and_cache(b.key_new, b.value_new, kc, vc, b.slot_mapping_compact)
    return kc, vc


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_close(got: np.ndarray, ref: np.ndarray, what: str = "") -> tuple[float, float]:
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / denom) if denom > 0 else float(np.linalg.norm(got - ref))
    assert max_abs <= MAX_ABS, f"{what}: max abs error {max_abs:.3e} > {MAX_ABS}"
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"
    return max_abs, rel
