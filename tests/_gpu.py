"""Helpers of the GPU parity tests: put a PagedBatch on the device, run the oracle beside it."""
from __future__ import annotations

import functools
import json
import os
import sys
import types

import numpy as np
import torch

import oracle
from workloads import PagedBatch, make_config, to_u16

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


# ------------------------------------------------------------------ full-size configs
@functools.lru_cache(maxsize=2)
def config_batch(name: str) -> PagedBatch:
    """The named workload, drawn once per process (callers must not modify it)."""
    return make_config(name)


@functools.lru_cache(maxsize=2)
def config_decode_ref(name: str) -> np.ndarray:
    """Float64 oracle output of every row of the named decode workload, after its step's
    new tokens are written."""
    b = config_batch(name)
    kc, vc = host_caches_after_write(b)
    return oracle.paged_decode(b.q, kc, vc, b.block_tables_compact, b.context_lens, b.scale,
                               b.dtype)


def parity_stats(got: np.ndarray, ref: np.ndarray, dtype: str) -> dict:
    """Error figures of a full output against the oracle: max-abs and relative L2, the
    count of reference values with |o_ref| >= 4 (where half a bf16 ulp exceeds the max-abs
    bar), and the largest error in excess of rounding o_ref itself to the 16-bit type."""
    err = np.abs(got - ref)
    rounded = oracle.decode_u16(to_u16(ref.astype(np.float32), dtype), dtype)
    excess = err - np.abs(rounded - ref)
    denom = float(np.linalg.norm(ref))
    return {"elements": int(ref.size), "max_abs": float(err.max()) if err.size else 0.0,
            "rel_l2": float(np.linalg.norm(got - ref) / denom) if denom > 0 else 0.0,
            "n_ref_abs_ge_4": int((np.abs(ref) >= 4).sum()),
            "max_excess_over_rounding": float(excess.max()) if excess.size else 0.0}


def check_full(got: np.ndarray, ref: np.ndarray, case: str, dtype: str) -> dict:
    """check_close over every output element, plus a record of the error figures: logged,
    and appended as a JSON line to $PA_PARITY_LOG when that is set."""
    check_close(got, ref, case)
    st = {"case": case, **parity_stats(got, ref, dtype)}
    log(f"  parity {json.dumps(st)}")
    path = os.environ.get("PA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(st) + "\n")
    return st
