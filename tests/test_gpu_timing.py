"""The measuring aids.  pa_set_kernel_events: HIP events the library's kernels record from
their own dispatch timestamps.  A stop event armed before a call takes the end of its last
kernel, across calls; the start event lies no later than the first kernel's start; both lie
inside event records queued on the stream around the call; arming changes no output bit.
pa_cache_flush and pa_stream_read: read their buffer and write nothing."""
import numpy as np
import pytest
import torch

from paged_kv_cache_324_amd import (PAError, decode_workspace, pa_cache_flush, pa_decode,
                                    pa_decode_order, pa_set_kernel_events, pa_stream_read)
from workloads import make_batch

from _gpu import log, to_bits, upload

pytestmark = pytest.mark.gpu


def _events(n):
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:            # a torch event holds no HIP event before its first record
        e.record()
    torch.cuda.synchronize()
    return ev


def _decode_case(partition):
    b = make_batch(B=32, Hq=16, Hkv=2, D=128, BS=16, dtype="bf16", scale=128 ** -0.5, seed=71,
                   lens_range=(500, 4000))
    d = upload(b)
    ws = decode_workspace(b.B, b.Hq, b.D, b.max_context_len, partition, "cuda")
    order = torch.from_numpy(pa_decode_order(b.context_lens)).cuda()

    def call(out):
        pa_decode(out, d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, b.scale,
                  b.max_context_len, partition, workspace=ws, seq_order=order)
    return d, call


@pytest.mark.parametrize("partition", [0, 256])
def test_kernel_events_lie_inside_queued_events(partition):
    d, call = _decode_case(partition)
    ref = torch.empty_like(d.q)
    call(ref)
    out = torch.empty_like(d.q)
    ks, ke, qs, qe = _events(4)
    for i in range(4):
        qs.record()
        pa_set_kernel_events(ks, ke)
        try:
            call(out)
        finally:
            pa_set_kernel_events()
        qe.record()
        torch.cuda.synchronize()
        k_ms, q_ms = ks.elapsed_time(ke), qs.elapsed_time(qe)
        lead, tail = qs.elapsed_time(ks), ke.elapsed_time(qe)
        log(f"partition {partition} call {i}: kernels {k_ms * 1e3:.1f} us, queued events "
            f"{q_ms * 1e3:.1f} us (lead {lead * 1e3:.1f}, tail {tail * 1e3:.1f})")
        assert k_ms > 0
        assert lead >= -1e-3 and tail >= -1e-3          # 1 us of timestamp granularity
        assert k_ms <= q_ms + 1e-3
    assert np.array_equal(to_bits(out), to_bits(ref))


def test_stop_event_follows_the_last_kernel_across_calls():
    d, call = _decode_case(256)
    out = torch.empty_like(d.q)
    ks, ke = _events(2)
    single, double = [], []
    for _ in range(3):
        for calls, acc in ((1, single), (2, double)):
            pa_set_kernel_events(ks, ke)     # arming again re-arms the start event
            try:
                for _ in range(calls):
                    call(out)
            finally:
                pa_set_kernel_events()
            torch.cuda.synchronize()
            acc.append(ks.elapsed_time(ke))
    s, t = float(np.median(single)), float(np.median(double))
    log(f"one call {s * 1e3:.1f} us, two calls {t * 1e3:.1f} us")
    assert 1.6 * s < t < 2.6 * s


def test_flush_end_to_call_end_brackets_the_call():
    """Stop events at the end of a flush and of the call after it: their interval holds the
    call's kernels (no shorter than start-to-stop events of the same call) and little else.
    The flush reads 1 GiB (about 180 us), so the host has enqueued the call before it ends;
    the first round, which pays first-use costs on the host, is not checked."""
    d, call = _decode_case(0)
    out = torch.empty_like(d.q)
    buf = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")
    fe, ks, ke = _events(3)
    spans, kern = [], []
    for _ in range(7):
        pa_set_kernel_events(None, fe)
        try:
            pa_cache_flush(buf)
            pa_set_kernel_events(ks, ke)
            call(out)
        finally:
            pa_set_kernel_events()
        torch.cuda.synchronize()
        spans.append(fe.elapsed_time(ke))
        kern.append(ks.elapsed_time(ke))
    log("flush end to call end " + ", ".join(f"{x * 1e3:.1f}" for x in spans) +
        " us; call start to end " + ", ".join(f"{x * 1e3:.1f}" for x in kern) + " us")
    for s, k in zip(spans[1:], kern[1:]):
        assert s >= k - 1e-3 and s < k + 0.05


def test_cache_flush_writes_nothing():
    buf = torch.arange(1 << 22, dtype=torch.int32, device="cuda")
    before = buf.clone()
    pa_cache_flush(buf)
    with pytest.raises(PAError):
        pa_cache_flush(buf[:5])             # 20 bytes: not a multiple of 16
    torch.cuda.synchronize()
    assert torch.equal(buf, before)


def test_stream_read_writes_nothing():
    buf = torch.arange(1 << 22, dtype=torch.int32, device="cuda")
    before = buf.clone()
    pa_stream_read(buf)
    pa_stream_read(buf[4:8])                # 16 bytes at a 16-byte offset
    with pytest.raises(PAError):
        pa_stream_read(buf[:5])             # 20 bytes: not a multiple of 16
    torch.cuda.synchronize()
    assert torch.equal(buf, before)


def test_arming_a_start_event_alone_is_rejected():
    ks, = _events(1)
    with pytest.raises(PAError):
        pa_set_kernel_events(ks, None)
    pa_set_kernel_events()


def test_armed_events_stay_out_of_a_graph_capture():
    """A call captured into a HIP graph while events are armed launches normally: the
    capture succeeds, the events are not recorded by the replays, and the replays give the
    eager result."""
    d, call = _decode_case(0)
    ref = torch.empty_like(d.q)
    call(ref)
    out = torch.zeros_like(d.q)
    ks, ke = _events(2)
    torch.cuda.synchronize()
    before = ks.elapsed_time(ke)
    graph = torch.cuda.CUDAGraph()
    pa_set_kernel_events(ks, ke)
    try:
        with torch.cuda.graph(graph):
            call(out)
    finally:
        pa_set_kernel_events()
    for _ in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(out), to_bits(ref))
    assert ks.elapsed_time(ke) == before
