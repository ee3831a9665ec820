"""Streams and graphs: the library only enqueues kernels on the stream it is
given (no allocation, copy, memset or synchronisation), so the whole path runs
on any stream and can be captured in a HIP graph.

* a side stream (default priority) gives the default stream's result, bit for bit;
* a captured graph, replayed three times with other eager work and
  synchronisations between the replays, matches the eager result each time."""
import numpy as np
import pytest

from synth import WORKLOADS, make_qkv

from gpu_harness import log, to_dev

pytestmark = pytest.mark.gpu

PRECISIONS = ["bf16", "mix", "fp8"]


def _setup(precision):
    import block_sparse_video_rf_amd as rf
    w = WORKLOADS["tiny"].with_(precision=precision)
    desc = rf.Desc.from_workload(w)
    q, k, v = (to_dev(x) for x in make_qkv(w))
    return rf, w, desc, q, k, v


@pytest.mark.parametrize("precision", PRECISIONS)
def test_side_stream_matches_default_stream(precision):
    import torch
    rf, w, desc, q, k, v = _setup(precision)
    ref, _ = rf.attention(q, k, v, desc)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out, _ = rf.attention(q, k, v, desc)
    side.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("precision", PRECISIONS)
def test_graph_replays_match_eager(precision):
    import torch
    rf, w, desc, q, k, v = _setup(precision)
    bufs = rf.Buffers(desc)
    eager = torch.empty_like(q)
    rf.attention(q, k, v, desc, bufs=bufs, out=eager)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    # Warm up on a side stream, then capture the four entry points.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        rf.attention(q, k, v, desc, bufs=bufs, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        rf.attention(q, k, v, desc, bufs=bufs, out=out)
    other_bufs = rf.Buffers(desc)
    q2 = (q.float() * 0.5).to(torch.bfloat16)
    for r in range(3):
        out.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), r
        # Eager work of the program between replays (other inputs, other buffers).
        rf.attention(q2, k, v, desc, bufs=other_bufs)
        torch.cuda.synchronize()
    log(f"  graph ({precision}): 3 replays bit-equal to eager")


def test_concurrent_host_threads():
    """Two host threads drive the whole path at once, each with its own buffers
    and stream (the library keeps no mutable global state): each result equals
    the single-threaded one, bit for bit."""
    import threading
    import torch
    rf, w, desc, q, k, v = _setup("bf16")
    ref, _ = rf.attention(q, k, v, desc)
    torch.cuda.synchronize()
    results, errors = {}, []

    def work(tag):
        try:
            torch.cuda.set_device(0)
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = [rf.attention(q, k, v, desc)[0] for _ in range(4)]
            s.synchronize()
            results[tag] = outs
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    assert sorted(results) == [0, 1]
    for outs in results.values():
        for o in outs:
            assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
