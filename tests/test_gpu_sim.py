"""GPU parity of echo_allreduce_sim (one whole call for P simulated ranks)
against the oracle's whole call, over consecutive calls that carry the
compensation state; plus the properties the Echo paper card states for
Fig. 2: identical outputs on every rank, and results independent of how
tiles are staggered across streams (Fig. 2(b))."""
import numpy as np
import pytest
import torch

import oracle
from _helpers import (DEV, assert_bits_equal, assert_f32_parity, dev_f32, dev_u16, host_f32, host_u16,
                      rand_bf16, say)

pytestmark = pytest.mark.gpu
G = 128


@pytest.fixture(scope="module")
def echo():
    from error_feedback_quant_amd import echo as e
    assert torch.cuda.is_available()
    return e


MODES = {"off": (1.0, 0.0), "classic": (1.0, 0.0), "classic_unfused": (1.0, 0.0), "two": (0.5, 0.25),
         "two_fused": (0.5, 0.25)}


def run_gpu_calls(echo, xs_list, P, n, bits, ef_mode, odt, tiles, nstreams, quant="zero_aware", group=128):
    """Run len(xs_list) consecutive calls; returns per-call outs and the final state."""
    alpha, beta = MODES[ef_mode]
    ef = ef_mode != "off"
    comps = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)] if ef else None
    errs = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)] \
        if ef_mode in ("classic_unfused", "two") else None
    slows = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)] \
        if ef_mode in ("two", "two_fused") else None
    odtype = torch.float32 if odt == oracle.OUT_F32 else torch.int16
    ws = torch.empty(echo.echo_allreduce_sim_workspace_bytes(P, n, bits, group), dtype=torch.uint8, device=DEV)
    streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(nstreams - 1)]
    results = []
    for xs in xs_list:
        xd = [dev_u16(x) for x in xs]
        outs = [torch.full((n,), 0x3F, dtype=odtype, device=DEV) for _ in range(P)]
        a = echo.make_sim_args(xd, outs, ws, bits=bits, tiles=tiles, out_dtype=odt, ef=ef, alpha=alpha,
                               beta=beta, comps=comps, slows=slows, errs=errs, quant=quant, group=group)
        echo.echo_allreduce_sim(a, streams=streams)
        torch.cuda.synchronize()
        results.append([host_f32(o) if odt == oracle.OUT_F32 else host_u16(o) for o in outs])
    state = dict(comps=[host_f32(c) for c in comps] if comps else None,
                 slows=[host_f32(s) for s in slows] if slows else None,
                 errs=[host_f32(e) for e in errs] if errs else None)
    return results, state


def run_oracle_calls(xs_list, P, n, bits, ef_mode, odt, quant="zero_aware", group=128):
    alpha, beta = MODES[ef_mode]
    ef = ef_mode != "off"
    comps = [np.zeros(n, np.float32) for _ in range(P)] if ef else None
    # the oracle always runs the unfused update (explicit error arrays)
    errs = [np.zeros(n, np.float32) for _ in range(P)] if ef_mode in ("classic_unfused", "two", "two_fused") \
        else None
    slows = [np.zeros(n, np.float32) for _ in range(P)] if ef_mode in ("two", "two_fused") else None
    results = []
    for xs in xs_list:
        outs, _, _ = oracle.allreduce(xs, bits=bits, group=group, ef=ef, alpha=alpha, beta=beta, comps=comps,
                                      slows=slows, errs=errs, out_dtype=odt, quant=quant)
        results.append(outs)
    return results, dict(comps=comps, slows=slows, errs=errs)


CASES = [
    # P, bits, ef, out, tiles, streams
    (1, 4, "classic", oracle.OUT_F32, 1, 1),
    (2, 4, "off", oracle.OUT_BF16, 2, 4),
    (3, 8, "two", oracle.OUT_F32, 3, 3),
    (4, 4, "classic", oracle.OUT_BF16, 1, 1),
    (4, 4, "classic", oracle.OUT_BF16, 5, 4),
    (4, 4, "classic_unfused", oracle.OUT_F32, 4, 2),
    (4, 4, "two", oracle.OUT_F32, 7, 4),
    (4, 8, "classic", oracle.OUT_BF16, 3, 4),
    (4, 8, "off", oracle.OUT_F32, 1, 4),
    (8, 4, "classic", oracle.OUT_BF16, 4, 4),
    (8, 8, "two", oracle.OUT_BF16, 2, 4),
    (5, 4, "classic", oracle.OUT_F32, 3, 4),
    (4, 4, "two_fused", oracle.OUT_F32, 1, 1),
    (4, 4, "two_fused", oracle.OUT_BF16, 6, 4),
    (8, 8, "two_fused", oracle.OUT_F32, 3, 2),
    (2, 4, "two_fused", oracle.OUT_F32, 2, 3),
    (1, 8, "two_fused", oracle.OUT_F32, 1, 1),
]


@pytest.mark.parametrize("P,bits,ef_mode,odt,tiles,nstreams", CASES)
def test_sim_matches_oracle_over_calls(echo, P, bits, ef_mode, odt, tiles, nstreams):
    n = P * G * 37                      # 37 groups per segment: ragged against tiles and blocks
    calls = 3
    xs_list = [[rand_bf16(n, 1000 * c + 10 * P + r, scale=1.0 + c) for r in range(P)] for c in range(calls)]
    say("sim", P, bits, ef_mode, odt, tiles, nstreams)
    got, gstate = run_gpu_calls(echo, xs_list, P, n, bits, ef_mode, odt, tiles, nstreams)
    want, wstate = run_oracle_calls(xs_list, P, n, bits, ef_mode, odt)
    for c in range(calls):
        for r in range(P):
            if odt == oracle.OUT_F32:
                assert_f32_parity(got[c][r], want[c][r], f"call {c} rank {r} out")
            assert_bits_equal(got[c][r], want[c][r], f"call {c} rank {r} out bits")
            assert_bits_equal(got[c][r], got[c][0], f"call {c}: rank {r} differs from rank 0")
    for key in ("comps", "slows", "errs"):
        if wstate[key] is not None and gstate[key] is not None:
            for r in range(P):
                assert_f32_parity(gstate[key][r], wstate[key][r], f"{key}[{r}]")
                assert_bits_equal(gstate[key][r], wstate[key][r], f"{key}[{r}] bits")


VARIANT_CASES = [
    # P, bits, ef, out, tiles, streams, quant, group
    (4, 4, "classic", oracle.OUT_BF16, 3, 4, "naive", 128),
    (4, 4, "two_fused", oracle.OUT_F32, 1, 1, "symmetric", 128),
    (4, 4, "classic", oracle.OUT_BF16, 2, 4, "zero_aware", 256),
    (8, 8, "classic_unfused", oracle.OUT_F32, 3, 2, "naive", 256),
    (3, 4, "two", oracle.OUT_F32, 2, 3, "symmetric", 256),
    (2, 8, "off", oracle.OUT_BF16, 1, 1, "naive", 128),
    (4, 4, "classic", oracle.OUT_BF16, 3, 2, "mse", 128),
    (5, 8, "two_fused", oracle.OUT_F32, 2, 3, "mse", 256),
]


@pytest.mark.parametrize("P,bits,ef_mode,odt,tiles,nstreams,quant,group", VARIANT_CASES)
def test_sim_quantizer_variants_match_oracle(echo, P, bits, ef_mode, odt, tiles, nstreams, quant, group):
    """Table 8's ablation quantizers and group size through the whole call."""
    n = P * group * 21
    xs_list = [[rand_bf16(n, 5000 * c + 10 * P + r, scale=1.0 + c) for r in range(P)] for c in range(3)]
    say("sim variant", P, bits, ef_mode, odt, tiles, nstreams, quant, group)
    got, gstate = run_gpu_calls(echo, xs_list, P, n, bits, ef_mode, odt, tiles, nstreams, quant, group)
    want, wstate = run_oracle_calls(xs_list, P, n, bits, ef_mode, odt, quant, group)
    for c in range(3):
        for r in range(P):
            assert_bits_equal(got[c][r], want[c][r], f"call {c} rank {r} out bits")
    for key in ("comps", "slows", "errs"):
        if wstate[key] is not None and gstate[key] is not None:
            for r in range(P):
                assert_bits_equal(gstate[key][r], wstate[key][r], f"{key}[{r}] bits")


@pytest.mark.parametrize("bits", [4, 8])
def test_staged_equals_serial(echo, bits):
    """Fig. 2(b): staggering tiles across streams changes only the schedule."""
    P, n = 4, 4 * G * 64
    xs_list = [[rand_bf16(n, 77 + 10 * c + r) for r in range(P)] for c in range(2)]
    say("staged vs serial", bits)
    ref, rstate = run_gpu_calls(echo, xs_list, P, n, bits, "classic", oracle.OUT_BF16, 1, 1)
    for tiles, ns in [(2, 2), (7, 4), (64, 4), (1000, 3)]:
        say("staged", bits, tiles, ns)
        got, gstate = run_gpu_calls(echo, xs_list, P, n, bits, "classic", oracle.OUT_BF16, tiles, ns)
        for c in range(2):
            for r in range(P):
                assert_bits_equal(got[c][r], ref[c][r], f"tiles {tiles} streams {ns} call {c} rank {r}")
        for r in range(P):
            assert_bits_equal(gstate["comps"][r], rstate["comps"][r], f"comp {r}")


def test_tile_count_is_capped(echo):
    """A tile count far above the cap (4096 per segment) on a message with
    more groups per segment than that: same bits as one tile, two calls."""
    P, n = 2, 2 * G * 4200
    xs_list = [[rand_bf16(n, 500 + 10 * c + r) for r in range(P)] for c in range(2)]
    say("tile cap", n)
    ref, rstate = run_gpu_calls(echo, xs_list, P, n, 4, "classic", oracle.OUT_BF16, 1, 1)
    got, gstate = run_gpu_calls(echo, xs_list, P, n, 4, "classic", oracle.OUT_BF16, 100000, 3)
    for c in range(2):
        for r in range(P):
            assert_bits_equal(got[c][r], ref[c][r], f"capped tiles call {c} rank {r}")
    for r in range(P):
        assert_bits_equal(gstate["comps"][r], rstate["comps"][r], f"comp {r}")


def test_sim_empty_message_is_a_no_op(echo):
    say("empty")
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    a = echo.make_sim_args([torch.empty(0, dtype=torch.int16, device=DEV)] * 4,
                           [torch.empty(0, dtype=torch.float32, device=DEV)] * 4, ws)
    echo.echo_allreduce_sim(a)
    torch.cuda.synchronize()


def test_sim_rejects_small_workspace(echo):
    P, n = 4, 4 * G
    xd = [torch.zeros(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    od = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)]
    ws = torch.empty(echo.echo_allreduce_sim_workspace_bytes(P, n, 4) - 256, dtype=torch.uint8, device=DEV)
    a = echo.make_sim_args(xd, od, ws)
    with pytest.raises(echo.EchoError) as ei:
        echo.echo_allreduce_sim(a)
    assert ei.value.rc == echo.EINVAL
