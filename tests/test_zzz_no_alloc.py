"""GPU check of echo_allreduce_sim_noalloc, the allocation-free variant of
echo_allreduce_sim for callers that cannot allocate device memory: through the
C ABI, its outputs and compensation equal those of echo_allreduce_sim (bit for
bit) on two calls in a row, the second with a smaller message (the static
scratch keeps the first call's contents), with tiles; a message whose
workspace exceeds the static scratch is rejected with nothing enqueued; and
the call captured in a HIP graph (what callers that cannot allocate often
are) replays bit for bit like the eager call, also five calls to a graph."""
import numpy as np
import pytest
import torch

from _helpers import DEV, assert_bits_equal, dev_u16, host_f32, host_u16, rand_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def echo():
    from error_feedback_quant_amd import echo as e
    assert torch.cuda.is_available()
    return e


def run_pair(echo, P, n, bits, tiles, seed):
    """The same call through both entry points, each with its own state."""
    xs = [dev_u16(rand_bf16(n, seed + r)) for r in range(P)]
    got = {}
    for which in ("noalloc", "workspace"):
        comps = [torch.full((n,), 0.0, dtype=torch.float32, device=DEV) for _ in range(P)]
        outs = [torch.full((n,), 0x3F3F, dtype=torch.int16, device=DEV) for _ in range(P)]
        if which == "noalloc":
            a = echo.make_sim_args(xs, outs, None, bits=bits, tiles=tiles, out_dtype=echo.OUT_BF16, ef=True,
                                   comps=comps, workspace_bytes=0)
            for _ in range(2):                      # the compensation carries into the second call
                echo.echo_allreduce_sim_noalloc(a)
        else:
            ws = torch.empty(echo.echo_allreduce_sim_workspace_bytes(P, n, bits), dtype=torch.uint8, device=DEV)
            a = echo.make_sim_args(xs, outs, ws, bits=bits, tiles=tiles, out_dtype=echo.OUT_BF16, ef=True,
                                   comps=comps)
            streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
            for _ in range(2):
                echo.echo_allreduce_sim(a, streams=streams)
        torch.cuda.synchronize()
        got[which] = ([host_u16(o) for o in outs], [host_f32(c) for c in comps])
    for r in range(P):
        assert_bits_equal(got["noalloc"][0][r], got["workspace"][0][r], f"out rank {r}")
        assert_bits_equal(got["noalloc"][1][r], got["workspace"][1][r], f"comp rank {r}")


def test_noalloc_equals_workspace_call_twice_smaller_second(echo):
    limit = echo.echo_noalloc_scratch_bytes()
    assert limit == 64 << 20
    say("noalloc", "P=4 n=2^22+512 bits=4 tiles=3")
    n1 = (1 << 22) + 512
    assert echo.echo_allreduce_sim_workspace_bytes(4, n1, 4) <= limit
    run_pair(echo, 4, n1, 4, 3, 100)
    say("noalloc", "P=8 n=2^17 bits=8 tiles=1 (smaller, after the first)")
    run_pair(echo, 8, 1 << 17, 8, 1, 200)


def test_noalloc_rejects_a_message_beyond_the_scratch(echo):
    P, bits = 4, 4
    limit = echo.echo_noalloc_scratch_bytes()
    n = 1 << 25                                    # 85 MB of workspace at P = 4
    assert echo.echo_allreduce_sim_workspace_bytes(P, n, bits) > limit
    say("noalloc reject", P, n)
    xs = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    outs = [torch.full((n,), 0x3F3F, dtype=torch.int16, device=DEV) for _ in range(P)]
    a = echo.make_sim_args(xs, outs, None, bits=bits, tiles=1, out_dtype=echo.OUT_BF16, workspace_bytes=0)
    with pytest.raises(echo.EchoError) as ei:
        echo.echo_allreduce_sim_noalloc(a)
    assert ei.value.rc == echo.ETOOBIG
    torch.cuda.synchronize()
    for o in outs:
        assert bool((o == 0x3F3F).all())           # nothing was enqueued


@pytest.mark.parametrize("tiles", [1, 3])
def test_noalloc_call_captured_in_a_graph(echo, tiles):
    """One call captured in a graph (torch.cuda.graph, on its capture stream)
    and replayed three times, with eager work and synchronizations between the
    replays: every replay gives what the same call gives eagerly, bit for bit,
    with the compensation carried from replay to replay.  The call records one
    launch (one tile) or its stages on one stream (three tiles): no memset and
    no event.  The scratch's device address was looked up by an earlier,
    eager call."""
    P, n, bits = 4, 64 * 1024, 4
    xs = [dev_u16(rand_bf16(n, 300 + r)) for r in range(P)]

    def fresh():
        comps = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)]
        outs = [torch.full((n,), 0x3F3F, dtype=torch.int16, device=DEV) for _ in range(P)]
        a = echo.make_sim_args(xs, outs, None, bits=bits, tiles=tiles, out_dtype=echo.OUT_BF16, ef=True,
                               comps=comps, workspace_bytes=0)
        return a, comps, outs

    say("noalloc graph", "tiles", tiles, "eager")
    a_e, comps_e, outs_e = fresh()
    want = []
    for _ in range(3):
        echo.echo_allreduce_sim_noalloc(a_e)
        torch.cuda.synchronize()
        want.append(([host_u16(o) for o in outs_e], [host_f32(c) for c in comps_e]))

    say("noalloc graph", "tiles", tiles, "capture")
    a, comps, outs = fresh()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        echo.echo_allreduce_sim_noalloc(a)
    torch.cuda.synchronize()
    # capturing ran nothing
    for c in comps:
        assert bool((c == 0).all())
    for k in range(3):
        say("noalloc graph", "tiles", tiles, "replay", k)
        g.replay()
        torch.cuda.synchronize()
        got_outs, got_comps = [host_u16(o) for o in outs], [host_f32(c) for c in comps]
        for r in range(P):
            assert_bits_equal(got_outs[r], want[k][0][r], f"replay {k} out rank {r}")
            assert_bits_equal(got_comps[r], want[k][1][r], f"replay {k} comp rank {r}")
        # the program's own eager work between replays
        junk = torch.randn(1 << 20, device=DEV)
        float(junk.sum())
        torch.cuda.synchronize()
    del g


@pytest.mark.parametrize("tiles", [1, 3])
def test_noalloc_calls_captured_five_to_a_graph(echo, tiles):
    """Five consecutive calls captured in one graph (as the benchmark's
    device-time measurement captures fifty), the compensation carried from
    call to call: the first replay equals five eager calls and the second
    ten, bit for bit."""
    P, n, bits, calls = 4, 64 * 1024, 4, 5
    xs = [dev_u16(rand_bf16(n, 500 + r)) for r in range(P)]

    def fresh():
        comps = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)]
        outs = [torch.full((n,), 0x3F3F, dtype=torch.int16, device=DEV) for _ in range(P)]
        a = echo.make_sim_args(xs, outs, None, bits=bits, tiles=tiles, out_dtype=echo.OUT_BF16, ef=True,
                               comps=comps, workspace_bytes=0)
        return a, comps, outs

    say("noalloc graph x5", "tiles", tiles, "eager")
    a_e, comps_e, outs_e = fresh()
    want = {}
    for c in range(1, 2 * calls + 1):
        echo.echo_allreduce_sim_noalloc(a_e)
        torch.cuda.synchronize()
        if c % calls == 0:
            want[c] = ([host_u16(o) for o in outs_e], [host_f32(x) for x in comps_e])

    say("noalloc graph x5", "tiles", tiles, "capture")
    a, comps, outs = fresh()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            echo.echo_allreduce_sim_noalloc(a)
    torch.cuda.synchronize()
    for k in (1, 2):
        say("noalloc graph x5", "tiles", tiles, "replay", k)
        g.replay()
        torch.cuda.synchronize()
        for r in range(P):
            assert_bits_equal(host_u16(outs[r]), want[k * calls][0][r], f"replay {k} out rank {r}")
            assert_bits_equal(host_f32(comps[r]), want[k * calls][1][r], f"replay {k} comp rank {r}")
    del g
