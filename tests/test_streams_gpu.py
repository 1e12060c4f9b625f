"""Concurrent calls on distinct streams from several host threads.

The library keeps no state between calls and allocates no device memory, so
calls on distinct streams are independent (the header's contract).  Five
host threads, each with its own stream (default priority), repeatedly run
a different entry point -- grouped forward, chunk-direction forward,
long-filter forward, backward, long-filter backward -- while the others
run; the host calls overlap (ctypes releases the interpreter lock) and so
can the kernels.
Every result must equal the same call made alone, bit for bit.
"""
import threading

import pytest
import torch

import gated_convolution_sequence_amd as hc
from gpu_util import DEV, log
from workloads import gaussian_inputs, normal_activation

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    hc.lib()
    yield
    torch.cuda.synchronize()


def _jobs():
    def grouped():
        q, k, v, h = (t.to(DEV) for t in gaussian_inputs(2, 1500, 256, 16, 128, torch.bfloat16, seed=1))
        y = torch.empty_like(q)
        return (lambda s: hc.conv_fwd(q, k, v, h, 16, out=y, stream=s)), (y,)

    def chunk_direction():
        q, k, v, h = (t.to(DEV) for t in gaussian_inputs(1, 2000, 128, 1, 65, torch.bfloat16, seed=2))
        y = torch.empty_like(q)
        return (lambda s: hc.conv_fwd(q, k, v, h, 1, out=y, stream=s)), (y,)

    def long_filter():
        q, k, v, h = (t.to(DEV) for t in gaussian_inputs(1, 3000, 64, 2, 3000, torch.bfloat16, seed=3))
        y = torch.empty_like(q)
        ws = torch.empty(hc.long_workspace_bytes(1, 3000, 64, 2, 3000), dtype=torch.uint8, device=DEV)
        return (lambda s: hc.conv_fwd_long(q, k, v, h, 2, out=y, workspace=ws, stream=s)), (y,)

    def backward():
        q, k, v, h = (t.to(DEV) for t in gaussian_inputs(1, 1200, 128, 16, 100, torch.bfloat16, seed=4))
        dy = normal_activation((1, 1200, 128), torch.bfloat16, DEV, seed=5)
        res = {}

        def run(s):
            res["g"] = hc.conv_bwd(q, k, v, h, dy, 16, stream=s)
        return run, res

    def long_backward():
        q, k, v, h = (t.to(DEV) for t in gaussian_inputs(1, 1500, 48, 3, 1500, torch.bfloat16, seed=6))
        dy = normal_activation((1, 1500, 48), torch.bfloat16, DEV, seed=7)
        ws = torch.empty(hc.bwd_long_workspace_bytes(1, 1500, 48, 3, 1500), dtype=torch.uint8, device=DEV)
        res = {}

        def run(s):
            res["g"] = hc.conv_bwd_long(q, k, v, h, dy, 3, workspace=ws, stream=s)
        return run, res
    return [grouped(), chunk_direction(), long_filter(), backward(), long_backward()]


def _snapshot(outs):
    if isinstance(outs, dict):
        return [t.clone() for t in outs["g"]]
    return [t.clone() for t in outs]


def test_concurrent_calls_on_distinct_streams():
    jobs = _jobs()
    # alone, one after the other
    ref = []
    for fn, outs in jobs:
        fn(torch.cuda.current_stream())
        torch.cuda.synchronize()
        ref.append(_snapshot(outs))
    # together: one thread and one stream per job, many calls each
    streams = [torch.cuda.Stream() for _ in jobs]
    errors = []

    def worker(i):
        try:
            fn, _ = jobs[i]
            with torch.cuda.stream(streams[i]):
                for _ in range(12):
                    fn(streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported by the main thread
            errors.append((i, repr(e)))
    log("%d threads x 12 calls on %d streams" % (len(jobs), len(jobs)))
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (fn, outs) in enumerate(jobs):
        for a, b in zip(_snapshot(outs), ref[i]):
            assert torch.equal(a, b), "job %d differs when run concurrently" % i
