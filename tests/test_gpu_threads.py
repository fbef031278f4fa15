"""echo_allreduce_sim from two host threads at once.

The C ABI promises reentrant calls: the staged call keeps its events in a
per-thread pool and its last HIP error per thread.  Two threads, each with
its own buffers and streams, run three staged calls carrying their state at
the same time (the ctypes call releases the interpreter lock, so the host
side of the calls overlaps too); each thread's outputs and state equal the
same calls run alone, bit for bit."""
import threading

import pytest
import torch

import oracle
from _helpers import DEV, assert_bits_equal, dev_u16, host_f32, host_u16, rand_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def echo():
    from error_feedback_quant_amd import echo as e
    assert torch.cuda.is_available()
    return e


# P, n, bits, tiles, streams, alpha, beta (two-timescale fused when beta > 0)
JOBS = [
    (4, 1 << 21, 4, 4, 2, 1.0, 0.0),
    (8, 1 << 21, 8, 3, 3, 0.5, 0.25),
]


def make_job(echo, job, seed):
    P, n, bits, tiles, nstreams, alpha, beta = job
    xs = [[dev_u16(rand_bf16(n, seed + 100 * c + r)) for r in range(P)] for c in range(3)]
    return xs


def run_job(echo, job, xs):
    P, n, bits, tiles, nstreams, alpha, beta = job
    comps = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)]
    slows = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)] if beta > 0 else None
    outs = [torch.empty(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    ws = torch.empty(echo.echo_allreduce_sim_workspace_bytes(P, n, bits), dtype=torch.uint8, device=DEV)
    streams = [torch.cuda.Stream() for _ in range(nstreams)]
    results = []
    for c in range(3):
        a = echo.make_sim_args(xs[c], outs, ws, bits=bits, tiles=tiles, out_dtype=oracle.OUT_BF16, ef=True,
                               alpha=alpha, beta=beta, comps=comps, slows=slows)
        echo.echo_allreduce_sim(a, streams=streams)
        streams[0].synchronize()
        results.append([host_u16(o) for o in outs])
    state = ([host_f32(x) for x in comps], [host_f32(x) for x in slows] if slows else None)
    return results, state


def test_two_threads_call_at_once(echo):
    inputs = [make_job(echo, job, 7100 + 1000 * k) for k, job in enumerate(JOBS)]
    say("threads", "alone")
    alone = [run_job(echo, job, xs) for job, xs in zip(JOBS, inputs)]
    torch.cuda.synchronize()

    say("threads", "together")
    together = [None, None]
    errors = []
    start = threading.Barrier(len(JOBS))

    def worker(k):
        try:
            torch.cuda.set_device(0)
            start.wait(timeout=60)
            together[k] = run_job(echo, JOBS[k], inputs[k])
        except Exception as e:                      # reported by the main thread
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(JOBS))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()

    for k, job in enumerate(JOBS):
        P = job[0]
        (ra, sa), (rt, st) = alone[k], together[k]
        for c in range(3):
            for r in range(P):
                assert_bits_equal(rt[c][r], ra[c][r], f"job {k} call {c} rank {r} out")
        for r in range(P):
            assert_bits_equal(st[0][r], sa[0][r], f"job {k} comp {r}")
            if sa[1] is not None:
                assert_bits_equal(st[1][r], sa[1][r], f"job {k} slow {r}")
