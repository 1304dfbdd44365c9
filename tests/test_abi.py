"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects bad host arguments before making any HIP call."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_324_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

INVALID, UNSUPPORTED, WORKSPACE = pa.PAError, pa.PAError, pa.PAError
P = ctypes.c_void_p(0x1000)   # a non-null host-side stand-in; never dereferenced by a rejected call


def declared_functions():
    """Every function any header under include/ declares."""
    text = "".join(open(os.path.join(ROOT, "include", f)).read()
                   for f in sorted(os.listdir(os.path.join(ROOT, "include"))) if f.endswith(".h"))
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_0-9]+\*?\s+\*?(pa_[a-z_0-9]+)\s*\(",
                                 text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return pa.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("pa_bm_create", "pa_bm_append", "pa_bm_fork", "pa_copy_blocks",
              "pa_reshape_and_cache", "pa_decode", "pa_decode_workspace_size",
              "pa_prefill_chunk", "pa_status_string", "pa_last_error", "pa_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert lib.pa_status_string(code)
    assert lib.pa_version() >> 16 == 1


def _decode(lib, **kw):
    a = dict(out=P, q=P, k=P, v=P, bt=P, lens=P, B=2, Hq=16, Hkv=8, D=128, BS=16, NB=100,
             maxb=10, maxL=160, scale=0.1, part=0, ws=None, wsb=0, dt=pa.PA_BF16)
    a.update(kw)
    return lib.pa_decode(a["out"], a["q"], a["k"], a["v"], a["bt"], a["lens"], None, a["B"], a["Hq"],
                         a["Hkv"], a["D"], a["BS"], a["NB"], a["maxb"], a["maxL"], a["scale"],
                         a["part"], a["ws"], a["wsb"], a["dt"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(out=None), -1, "null pointer"),
    (dict(bt=None), -1, "null pointer"),
    (dict(B=-1), -1, "num_seqs"),
    (dict(Hkv=5), -1, "multiple"),
    (dict(Hq=48, Hkv=3), -2, "query heads per KV head"),
    (dict(D=96), -2, "head_dim"),
    (dict(BS=8), -2, "block_size"),
    (dict(dt=7), -2, "dtype"),
    (dict(NB=0), -1, "num_blocks"),
    (dict(maxL=161), -1, "max_context_len"),
    (dict(scale=float("inf")), -1, "scale"),
    (dict(scale=float("nan")), -1, "scale"),
    (dict(scale=0.0), -1, "scale"),
    (dict(scale=-0.088), -1, "scale"),
    (dict(scale=-0.0), -1, "scale"),
    (dict(part=24), -1, "partition_size"),
    (dict(part=-16), -1, "partition_size"),
    (dict(part=32), -3, "workspace"),
    (dict(part=32, ws=P, wsb=100), -3, "workspace"),
])
def test_decode_rejects_bad_arguments(lib, kw, code, msg):
    assert _decode(lib, **kw) == code
    assert msg in lib.pa_last_error().decode()


def test_decode_zero_sequences_is_a_noop(lib):
    assert _decode(lib, B=0, out=None, q=None) == 0


def test_workspace_size(lib):
    assert lib.pa_decode_workspace_size(128, 16, 128, 2048, 0) == 0
    assert lib.pa_decode_workspace_size(128, 16, 128, 512, 512) == 0
    n = lib.pa_decode_workspace_size(128, 16, 128, 2048, 512)
    rows = 128 * 16 * 4
    assert n >= rows * 128 * 2 + rows * 2 * 4 and n % 256 == 0


def test_partition_hint(lib):
    """Split only when the (sequence, KV head) pairs leave compute units idle (256 CUs assumed
    without a device, as on MI355X)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("hint values below assume 256 compute units and no device")
    h = lib.pa_decode_partition_hint
    assert h(128, 8, 2048, 16) == 0            # 1024 pairs: enough workgroups unsplit
    assert h(64, 8, 8192, 32) == 0             # 512 pairs: two per compute unit
    assert h(8, 8, 32768, 256) == 1024         # 64 pairs: 32 partitions of the longest context
    assert h(8, 8, 4096, 256) == 512           # the 512-token floor (32 partitions would be 128)
    assert h(8, 8, 30000, 16) == 944           # rounded up to a whole block
    assert h(1, 1, 100, 16) == 0               # shorter than the minimum partition
    assert h(4, 8, 0, 16) == 0
    assert h(0, 8, 100, 16) == -1 and h(4, 8, -1, 16) == -1
    assert h(4, 8, 100, 48) == -2


def test_reshape_rejects_bad_arguments(lib):
    f = lib.pa_reshape_and_cache
    assert f(None, P, P, P, P, 4, 8, 128, 16, 100, pa.PA_BF16, None) == -1
    assert f(P, P, P, P, P, -1, 8, 128, 16, 100, pa.PA_BF16, None) == -1
    assert f(P, P, P, P, P, 4, 8, 80, 16, 100, pa.PA_BF16, None) == -2
    assert f(P, P, P, P, P, 4, 8, 128, 48, 100, pa.PA_BF16, None) == -2
    assert f(P, P, P, P, P, 4, 8, 128, 16, 0, pa.PA_BF16, None) == -1
    assert f(None, None, None, None, None, 0, 8, 128, 16, 100, pa.PA_F16, None) == 0


def test_prefill_rejects_bad_arguments(lib):
    f = lib.pa_prefill_chunk
    args = [P, P, P, P, P, P, P, None, 2, 64, 32, 8, 128, 16, 100, 10, 32, 0.1, pa.PA_BF16, None]
    bad = list(args)
    bad[6] = None
    assert f(*bad) == -1
    bad = list(args)
    bad[10] = 6     # 32 heads over 6 KV heads
    assert f(*bad) == -1
    for sc in (float("nan"), float("-inf"), 0.0, -0.0, -0.1):
        bad = list(args)
        bad[17] = sc
        assert f(*bad) == -1
        assert "scale" in lib.pa_last_error().decode()
    bad = list(args)
    bad[16] = -1
    assert f(*bad) == -1
    bad = list(args)
    bad[12] = 96    # head_dim 96 has no prefill kernel (64 and 128 do)
    assert f(*bad) == -2


def test_python_binding_names_match_c_entry_points():
    for name in ("pa_reshape_and_cache", "pa_decode", "pa_decode_step", "pa_decode_order",
                 "pa_decode_workspace_size", "pa_prefill_chunk"):
        assert callable(getattr(pa, name))


def test_decode_step_rejects_bad_arguments(lib):
    f = lib.pa_decode_step
    base = [P, P, P, P, P, P, P, P, P, None, 2, 16, 8, 128, 16, 100, 10, 160, 0.1, 0, None, 0,
            pa.PA_BF16, None]
    bad = list(base)
    bad[4] = None                          # slot_mapping
    assert f(*bad) == -1 and "null" in lib.pa_last_error().decode()
    bad = list(base)
    bad[13] = 80                           # head_dim
    assert f(*bad) == -2
    bad = list(base)
    bad[19] = 32                           # needs a workspace
    assert f(*bad) == -3


def test_decode_step_int8_rejects_bad_arguments(lib):
    f = lib.pa_decode_step_int8
    # out, q, key, value, slot_mapping, k_codes, v_codes, k_scales, v_scales, tables, lens,
    # seq_order, B, Hq, Hkv, D, BS, NB, max_blocks, max_len, scale, partition, ws, ws_bytes,
    # dtype, stream
    base = [P, P, P, P, P, P, P, P, P, P, P, None, 2, 16, 8, 128, 16, 100, 10, 160, 0.1, 0, None,
            0, pa.PA_BF16, None]
    bad = list(base)
    bad[7] = None                          # k_scales
    assert f(*bad) == -1 and "null" in lib.pa_last_error().decode()
    bad = list(base)
    bad[4] = None                          # slot_mapping
    assert f(*bad) == -1 and "null" in lib.pa_last_error().decode()
    bad = list(base)
    bad[15] = 96                           # head_dim: INT8 decode takes 64 and 128
    assert f(*bad) == -2
    bad = list(base)
    bad[21] = 32                           # needs a workspace
    assert f(*bad) == -3
    bad = list(base)
    bad[12] = 0                            # no sequences: nothing to do
    assert f(*bad) == 0


def test_decode_order_is_longest_first_and_stable():
    import numpy as np
    lens = np.array([5, 9, 5, 0, 12, 9, 1], dtype=np.int32)
    order = pa.pa_decode_order(lens)
    assert order.tolist() == [4, 1, 5, 0, 2, 6, 3]
    rng = np.random.default_rng(3)
    lens = rng.integers(0, 3000, size=1000).astype(np.int32)
    order = pa.pa_decode_order(lens)
    assert sorted(order.tolist()) == list(range(1000))
    assert np.all(np.diff(lens[order]) <= 0)
    assert pa.pa_decode_order(np.zeros(0, np.int32)).shape == (0,)


def test_bench_refuses_several_gpus():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_new_entry_points_have_bindings():
    for name in ("pa_decode_partial", "pa_merge_partials", "pa_rope_reshape_and_cache",
                 "pa_decode_int8", "pa_reshape_and_cache_int8", "pa_copy_blocks",
                 "pa_decode_partition_hint", "pa_decode_step_int8"):
        assert callable(getattr(pa, name)), name


def test_decode_partial_rejects_bad_arguments(lib):
    f = lib.pa_decode_partial
    base = [P, P, P, P, P, P, P, None, 2, 16, 8, 128, 16, 100, 10, 160, 0.1, 0, None, 0,
            pa.PA_BF16, None]
    bad = list(base)
    bad[1] = None                          # out_ml
    assert f(*bad) == -1 and "null" in lib.pa_last_error().decode()
    bad = list(base)
    bad[1] = ctypes.c_void_p(0x1004)       # out_ml not 8-byte aligned
    assert f(*bad) == -1 and "aligned" in lib.pa_last_error().decode()
    bad = list(base)
    bad[11] = 96                           # head_dim
    assert f(*bad) == -2
    bad = list(base)
    bad[17] = 32                           # needs a workspace
    assert f(*bad) == -3
    empty = list(base)
    empty[0] = empty[1] = None
    empty[8] = 0                           # no sequences: nothing to do
    assert f(*empty) == 0


@pytest.mark.parametrize("index,value,code", [
    (4, 0, -1),                            # num_shards
    (5, -1, -1),                           # num_seqs
    (6, 0, -1),                            # num_heads
    (7, 80, -2),                           # head_dim
    (8, 5, -2),                            # dtype
    (0, None, -1),                         # out
    (3, ctypes.c_void_p(0x1004), -1),      # partial_ml alignment
    (2, ctypes.c_void_p(0x1002), -1),      # partial_o alignment
    (1, ctypes.c_void_p(0x1004), -1),      # out_ml alignment
])
def test_merge_partials_rejects_bad_arguments(lib, index, value, code):
    args = [P, None, P, P, 4, 2, 16, 128, pa.PA_BF16, None]
    args[index] = value
    assert lib.pa_merge_partials(*args) == code


def test_merge_partials_empty_batch_is_a_noop(lib):
    assert lib.pa_merge_partials(None, None, None, None, 4, 0, 16, 128, pa.PA_BF16, None) == 0


@pytest.mark.parametrize("index,value,code", [
    (10, 0, -1),                           # q given with num_heads 0
    (1, None, -1),                         # key
    (5, None, -1),                         # positions
    (12, 96, -2),                          # head_dim
    (13, 8, -2),                           # block_size
    (15, 0, -1),                           # max_position
    (6, ctypes.c_void_p(0x1004), -1),      # cos table alignment
    (9, -1, -1),                           # num_tokens
    (16, 9, -2),                           # dtype
])
def test_rope_rejects_bad_arguments(lib, index, value, code):
    args = [P, P, P, P, P, P, P, P, P, 4, 16, 8, 128, 16, 100, 4096, pa.PA_BF16, None]
    args[index] = value
    assert lib.pa_rope_reshape_and_cache(*args) == code


def test_rope_without_tokens_or_queries(lib):
    f = lib.pa_rope_reshape_and_cache
    assert f(None, None, None, None, None, None, None, None, None, 0, 0, 8, 128, 16, 100, 10,
             pa.PA_F16, None) == 0
    # no queries: num_heads is ignored, a bad key still rejected
    assert f(None, None, P, P, P, P, P, P, P, 4, 0, 8, 128, 16, 100, 10, pa.PA_F16, None) == -1


@pytest.mark.parametrize("scale", [0.0, -1.0, float("nan")])
def test_int8_decode_and_steps_reject_non_positive_scale(lib, scale):
    """A non-positive or non-finite scale is rejected by every attention entry point."""
    int8 = [P, P, P, P, P, P, P, P, None, 2, 16, 8, 128, 16, 100, 10, 160, scale, 0, None, 0,
            pa.PA_BF16, None]
    assert lib.pa_decode_int8(*int8) == -1
    assert "scale" in lib.pa_last_error().decode()
    step = [P, P, P, P, P, P, P, P, P, None, 2, 16, 8, 128, 16, 100, 10, 160, scale, 0, None, 0,
            pa.PA_BF16, None]
    assert lib.pa_decode_step(*step) == -1
    assert "scale" in lib.pa_last_error().decode()


def test_decode_merge_rejects_bad_arguments(lib):
    f = lib.pa_decode_merge
    # out, lens, seq_order, B, Hq, D, max_len, partition, ws, ws_bytes, dtype, stream
    args = [P, P, None, 4, 16, 128, 2048, 512, P, 1 << 20, pa.PA_BF16, None]
    for i, v, code in [(0, None, -1), (1, None, -1), (3, -1, -1), (4, 0, -1), (5, 96, -2),
                       (10, 9, -2), (6, -1, -1), (7, -16, -1), (8, None, -3), (9, 100, -3)]:
        bad = list(args)
        bad[i] = v
        assert f(*bad) == code, (i, v)
    # nothing to merge: no partition split, or no sequence
    assert f(None, None, None, 4, 16, 128, 2048, 0, None, 0, pa.PA_BF16, None) == 0
    assert f(None, None, None, 4, 16, 128, 512, 512, None, 0, pa.PA_BF16, None) == 0
    assert f(None, None, None, 0, 16, 128, 2048, 512, None, 0, pa.PA_BF16, None) == 0


def test_decode_partitions_validates_like_decode(lib):
    a = [P, P, P, P, P, P, None, 2, 16, 8, 128, 16, 100, 10, 160, 0.1, 32, None, 0, pa.PA_BF16, None]
    assert lib.pa_decode_partitions(*a) == -3          # split without a workspace
    a[15] = -1.0
    assert lib.pa_decode_partitions(*a) == -1


def test_decode_step_scratch_rejects_a_split_beyond_the_scratch(lib):
    """The no-allocation step refuses, before any HIP call, a split whose partials would not
    fit its 16 MiB static scratch, and validates the rest like pa_decode_step."""
    # out, q, key, value, slot, kc, vc, tables, lens, order, B, Hq, Hkv, D, BS, NB, maxb, maxL,
    # scale, partition, dtype, stream
    a = [P, P, P, P, P, P, P, P, P, None, 64, 64, 8, 128, 16, 100000, 512, 8192, 0.088, 16,
         pa.PA_BF16, None]
    assert lib.pa_decode_step_scratch(*a) == -3
    assert "static scratch" in lib.pa_last_error().decode()
    a[18] = 0.0
    assert lib.pa_decode_step_scratch(*a) == -1
    a[18], a[0] = 0.088, None
    assert lib.pa_decode_step_scratch(*a) == -1


def test_checking_library_exports_the_same_entry_points():
    chk = pa.load_library(checked=True)
    for name in declared_functions():
        assert hasattr(chk, name), name
    assert chk.pa_check_indices_enabled() == 1
    assert pa.load_library().pa_check_indices_enabled() == 0


def test_index_errors_need_the_checking_library(lib):
    import ctypes
    k, f, v = ctypes.c_uint32(7), ctypes.c_uint32(7), ctypes.c_int64(7)
    assert lib.pa_take_index_errors(None, ctypes.byref(k), ctypes.byref(f), ctypes.byref(v)) == -2
    assert "PA_CHECK_INDICES" in lib.pa_last_error().decode()
    assert (k.value, f.value, v.value) == (0, 0, 0)
    assert lib.pa_take_index_errors(None, None, None, None) == -1


def test_kernel_events_and_cache_flush_reject_bad_arguments(lib):
    assert lib.pa_set_kernel_events(P, None) == -1
    assert "stop event" in lib.pa_last_error().decode()
    assert lib.pa_set_kernel_events(None, P) == 0       # arming makes no HIP call
    assert lib.pa_set_kernel_events(P, P) == 0
    assert lib.pa_set_kernel_events(None, None) == 0
    pa.pa_set_kernel_events()
    with pytest.raises(ValueError):
        pa.pa_set_kernel_events(__import__("torch").cuda.Event(enable_timing=True), 1)
    assert lib.pa_cache_flush(None, 0, None) == 0       # nothing to read
    assert lib.pa_cache_flush(None, 16, None) == -1
    assert lib.pa_cache_flush(ctypes.c_void_p(0x1008), 16, None) == -1
    assert lib.pa_cache_flush(P, 24, None) == -1
    assert lib.pa_stream_read(None, 0, None) == 0
    assert lib.pa_stream_read(None, 16, None) == -1
    assert lib.pa_stream_read(ctypes.c_void_p(0x1008), 16, None) == -1
    assert lib.pa_stream_read(P, 24, None) == -1
