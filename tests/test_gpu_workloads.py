"""The workloads at full size on the GPU.

* 1 GiB message (2^29 bf16 per rank, Laplace(0,1)), P = 4 and P = 8, in the
  launch configurations the benchmark times (bf16 output, classic feedback
  written in place; one tile per segment on one stream, and tiles staggered
  over four streams), two consecutive calls.  Full parity: every output and
  compensation element against the oracle's whole call, run in host threads
  over ranges that keep segment ownership.  Sampled parity: the oracle recomputes a set of groups from every
  segment (an exact sub-problem: quantization, sums and feedback act per
  group and per element) and must match bit for bit; properties over the
  whole message: bitwise identical outputs on every rank, and the injected
  error equals the revealed errors (fed back as -comp) up to fp32 rounding.
* Depth chains (Echo paper card Fig. 1: N injection sites add their
  all-reduce output to the hidden state): 4-bit, P = 4, 2048 x 4096, 64 sites,
  and 8-bit, P = 4, 4096 x 1024, 56 sites, with classic feedback and without
  it; the 4-bit chain also with the two-timescale compensator.  Every site's
  call is checked against the oracle's whole call over the whole message,
  bit for bit; the accumulated error must equal the outstanding error debt,
  stay bounded with feedback, and grow without it (abstract: depth does not
  raise the bound).
"""
import time

import numpy as np
import pytest
import torch

import oracle
from _helpers import (DEV, assert_bits_equal, gather_chunk, host_f32, host_u16, host_workers,
                      oracle_by_chunks, say)
from error_feedback_quant_amd import inputs

pytestmark = pytest.mark.gpu
G = 128
U24 = 2.0 ** -24


@pytest.fixture(scope="module")
def echo():
    from error_feedback_quant_amd import echo as e
    assert torch.cuda.is_available()
    return e


def sample_index(P, S, n_groups, seed):
    """Element indices (device, int64) of `n_groups` group offsets taken from
    every segment (same offsets in each segment, so ownership is kept), laid
    out as a mini message of P * n_groups * 128 elements."""
    rng = np.random.default_rng(seed)
    gps = S // G
    offs = set([0, gps - 1, gps // 2, gps // 3])
    offs |= set(rng.choice(gps, size=n_groups - len(offs), replace=False).tolist())
    offs = np.array(sorted(offs)[:n_groups], dtype=np.int64)
    seg = np.arange(P, dtype=np.int64)[:, None, None] * S
    idx = seg + offs[None, :, None] * G + np.arange(G, dtype=np.int64)[None, None, :]
    return torch.from_numpy(idx.reshape(-1)).to(DEV)


def bf16_dev_to_f64(t):
    return t.view(torch.bfloat16).to(torch.float64)


@pytest.mark.parametrize("P", [4, 8])
def test_onegb_sampled_parity_and_identities(echo, P):
    n = 1 << 29
    S = n // P
    tiles, nstreams = 8, 4
    torch.cuda.empty_cache()
    say("onegb", P, "generate")
    xs = [inputs.laplace(r, n, device=DEV) for r in range(P)]
    for x in xs:
        assert bool(torch.isfinite(x.view(torch.bfloat16)).all()), "inputs must be finite"
    comps = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)]
    outs = [torch.empty(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    ws = torch.empty(echo.echo_allreduce_sim_workspace_bytes(P, n, 4), dtype=torch.uint8, device=DEV)
    streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(nstreams - 1)]
    idx = sample_index(P, S, 48, seed=P)
    mini_n = idx.numel()
    o_comps = [np.zeros(mini_n, np.float32) for _ in range(P)]
    for call in range(2):
        if call == 1:                       # fresh partials for the second call, same shapes
            for r in range(P):
                xs[r] = inputs.laplace(r + 16, n, device=DEV)
        x_mini = [host_u16(x[idx]) for x in xs]
        c_before = [c.clone() for c in comps] if call == 1 else None
        say("onegb", P, "call", call)
        a = echo.make_sim_args(xs, outs, ws, bits=4, tiles=tiles, out_dtype=oracle.OUT_BF16, ef=True,
                               comps=comps)
        echo.echo_allreduce_sim(a, streams=streams)
        torch.cuda.synchronize()
        # sampled parity against the oracle's own call on the mini message
        o_outs, _, _ = oracle.allreduce(x_mini, bits=4, ef=True, comps=o_comps, out_dtype=oracle.OUT_BF16)
        for r in range(P):
            assert_bits_equal(host_u16(outs[r][idx]), o_outs[r], f"P={P} call {call} out[{r}] sample")
            assert_bits_equal(host_f32(comps[r][idx]), o_comps[r], f"P={P} call {call} comp[{r}] sample")
        # whole message: every rank holds the same bits
        for r in range(1, P):
            assert torch.equal(outs[r], outs[0]), f"rank {r} differs"
        # whole message: out - sum(x + c) == sum(e) = -sum(comp after), chunked in fp64
        step = 1 << 26
        for a0 in range(0, n, step):
            sl = slice(a0, a0 + step)
            out = bf16_dev_to_f64(outs[0][sl])
            u_sum = torch.zeros_like(out)
            mag = torch.zeros_like(out)
            e_sum = torch.zeros_like(out)
            for r in range(P):
                u = bf16_dev_to_f64(xs[r][sl])
                if call == 1:
                    u = u + c_before[r][sl].double()
                u_sum += u
                mag += u.abs()
                e_sum -= comps[r][sl].double()
            # the bf16 output rounding is part of what the owner's error cannot see
            resid = (out - u_sum - e_sum).abs()
            # bf16 unit roundoff is 2^-8
            bound = (P + 2) * U24 * (mag + e_sum.abs() + out.abs()) + 2.0 ** -8 * out.abs()
            assert bool((resid <= bound).all()), f"P={P} call {call} chunk {a0}: {resid.max().item()}"
            del out, u_sum, mag, e_sum
        del c_before
    del xs, comps, outs, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("P", [4, 8])
def test_onegb_full_parity(echo, P):
    """Every element of the 1 GiB message (2^29 bf16 per rank, Laplace(0,1)),
    P = 4 and P = 8, bit for bit against the oracle's whole call: all P bf16
    outputs and all P compensations.  Three calls carry the feedback: the
    first back to back (one tile per segment on one stream), the second in
    the benchmark's headline schedule (4 tiles staged on 2 streams), the
    third on 4 streams.  The oracle's call runs on the host
    as independent calls on mini messages made of the same range of every
    segment, in threads (its chunked form is pinned to one whole call on the
    CPU)."""
    n = 1 << 29
    S = n // P
    L = 1 << 18
    workers = host_workers()
    torch.cuda.empty_cache()
    comps = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)]
    outs = [torch.empty(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    ws = torch.empty(echo.echo_allreduce_sim_workspace_bytes(P, n, 4), dtype=torch.uint8, device=DEV)
    c_host = [np.zeros(n, np.float32) for _ in range(P)]      # state before the call
    for call, (tiles, nstreams) in enumerate([(1, 1), (4, 2), (4, 4)]):
        say("onegb full", P, "call", call, "generate")
        xs = [inputs.laplace(r + 16 * call, n, device=DEV) for r in range(P)]
        xh = [host_u16(x) for x in xs]
        streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(nstreams - 1)]
        say("onegb full", P, "call", call, "tiles", tiles, "streams", nstreams)
        a = echo.make_sim_args(xs, outs, ws, bits=4, tiles=tiles, out_dtype=oracle.OUT_BF16, ef=True,
                               comps=comps)
        echo.echo_allreduce_sim(a, streams=streams)
        torch.cuda.synchronize()
        out_h = [host_u16(o) for o in outs]
        c_after = [host_f32(c) for c in comps]
        del xs

        def visit(sl, o_outs, o_comps, _):
            for r in range(P):
                if gather_chunk(out_h[r], sl).tobytes() != o_outs[r].tobytes():
                    return f"P={P} call {call}: out[{r}] differs in the range at {sl[0].start} of segment 0"
                if gather_chunk(c_after[r], sl).tobytes() != o_comps[r].tobytes():
                    return f"P={P} call {call}: comp[{r}] differs in the range at {sl[0].start} of segment 0"
            return None

        say("onegb full", P, "call", call, "oracle on", workers, "threads")
        t0 = time.time()
        bad = oracle_by_chunks(xh, c_host, P, L, oracle.OUT_BF16, workers, visit)
        print(f"onegb full P={P} call {call}: oracle and compare {time.time() - t0:.1f} s", flush=True)
        assert bad is None, bad
        del xh, out_h
        c_host = c_after
    del comps, outs, ws, c_host
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["ef_off", "f32_out", "two_timescale", "bits8", "naive", "symmetric", "g256",
                                  "mse"])
def test_onegb_full_parity_modes(echo, mode):
    """The benchmark's other legs at full size (1 GiB message, P = 4):
    feedback off, fp32 output, the two-timescale compensator (alpha = 0.5,
    beta = 0.25) fused into push and reduce, 8-bit codes, and Table 8's
    naive-zero-point and symmetric-grid quantizers, groups of 256, and the
    full method with its zero point searched.  Two calls carry the state, the
    first back to back (one tile on one stream), the second in the
    benchmark's headline schedule (4 tiles staged on 2 streams); every output,
    compensation and slow-memory element matches the oracle's whole call bit
    for bit."""
    P, n = 4, 1 << 29
    L = 1 << 18
    ef = mode != "ef_off"
    two = mode == "two_timescale"
    bits = 8 if mode == "bits8" else 4
    quant = mode if mode in ("naive", "symmetric", "mse") else "zero_aware"
    group = 256 if mode == "g256" else 128
    odt = oracle.OUT_F32 if mode == "f32_out" else oracle.OUT_BF16
    alpha, beta = (0.5, 0.25) if two else (1.0, 0.0)
    workers = host_workers()
    torch.cuda.empty_cache()
    comps = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)] if ef else None
    slows = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)] if two else None
    outs = [torch.empty(n, dtype=torch.float32 if odt == oracle.OUT_F32 else torch.int16, device=DEV)
            for _ in range(P)]
    ws = torch.empty(echo.echo_allreduce_sim_workspace_bytes(P, n, bits, group), dtype=torch.uint8, device=DEV)
    c_host = [np.zeros(n, np.float32) for _ in range(P)] if ef else None
    s_host = [np.zeros(n, np.float32) for _ in range(P)] if two else None
    for call, (tiles, nstreams) in enumerate([(1, 1), (4, 2)]):
        say("onegb mode", mode, "call", call, "tiles", tiles, "streams", nstreams)
        xs = [inputs.laplace(r + 16 * call, n, device=DEV) for r in range(P)]
        xh = [host_u16(x) for x in xs]
        streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(nstreams - 1)]
        a = echo.make_sim_args(xs, outs, ws, bits=bits, group=group, tiles=tiles, out_dtype=odt, ef=ef,
                               alpha=alpha, beta=beta, comps=comps, slows=slows, quant=quant)
        echo.echo_allreduce_sim(a, streams=streams)
        torch.cuda.synchronize()
        out_h = [host_f32(o) if odt == oracle.OUT_F32 else host_u16(o) for o in outs]
        c_after = [host_f32(c) for c in comps] if ef else None
        s_after = [host_f32(m) for m in slows] if two else None
        del xs

        def visit(sl, o_outs, o_c, o_s):
            for r in range(P):
                if gather_chunk(out_h[r], sl).tobytes() != o_outs[r].tobytes():
                    return f"{mode} call {call}: out[{r}] differs in the range at {sl[0].start} of segment 0"
                if ef and gather_chunk(c_after[r], sl).tobytes() != o_c[r].tobytes():
                    return f"{mode} call {call}: comp[{r}] differs in the range at {sl[0].start} of segment 0"
                if two and gather_chunk(s_after[r], sl).tobytes() != o_s[r].tobytes():
                    return f"{mode} call {call}: slow[{r}] differs in the range at {sl[0].start} of segment 0"
            return None

        t0 = time.time()
        bad = oracle_by_chunks(xh, c_host, P, L, odt, workers, visit, bits=bits, slows=s_host, alpha=alpha,
                               beta=beta, quant=quant, group=group)
        print(f"onegb mode {mode} call {call}: oracle and compare {time.time() - t0:.1f} s", flush=True)
        assert bad is None, bad
        del xh, out_h
        c_host, s_host = c_after, s_after
    del comps, slows, outs, ws
    torch.cuda.empty_cache()


def test_message_beyond_2_31_elements(echo):
    """2^31 + 2^22 elements per rank (P = 2, about 38 GB on the device):
    every element of segment 1 lies beyond 2^31, so do its fp32 byte offsets
    beyond 2^33, its code bytes beyond 2^30 and its parameter words beyond
    2^24.  One call, classic feedback written in place, bf16 output, 4 tiles
    on 2 streams.  Sampled groups, including both ends of both segments,
    match the oracle's call on the mini message bit for bit (outputs and
    compensations), and the two ranks' outputs agree over the whole message."""
    P = 2
    n = (1 << 31) + (1 << 22)
    S = n // P
    torch.cuda.empty_cache()
    say("beyond 2^31", n, "generate")
    xs = [inputs.laplace(r + 40, n, device=DEV) for r in range(P)]
    comps = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)]
    outs = [torch.empty(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    ws = torch.empty(echo.echo_allreduce_sim_workspace_bytes(P, n, 4), dtype=torch.uint8, device=DEV)
    streams = [torch.cuda.current_stream(), torch.cuda.Stream()]
    idx = sample_index(P, S, 24, seed=31)
    x_mini = [host_u16(x[idx]) for x in xs]
    o_comps = [np.zeros(idx.numel(), np.float32) for _ in range(P)]
    say("beyond 2^31", n, "call")
    a = echo.make_sim_args(xs, outs, ws, bits=4, tiles=4, out_dtype=oracle.OUT_BF16, ef=True, comps=comps)
    echo.echo_allreduce_sim(a, streams=streams)
    torch.cuda.synchronize()
    o_outs, _, _ = oracle.allreduce(x_mini, bits=4, ef=True, comps=o_comps, out_dtype=oracle.OUT_BF16)
    for r in range(P):
        assert_bits_equal(host_u16(outs[r][idx]), o_outs[r], f"out[{r}] sample")
        assert_bits_equal(host_f32(comps[r][idx]), o_comps[r], f"comp[{r}] sample")
    assert torch.equal(outs[1], outs[0]), "the ranks differ"
    del xs, comps, outs, ws
    torch.cuda.empty_cache()


def chain_run(echo, P, n, sites, bits, gen, mode, alpha=1.0, beta=0.0):
    """Depth chain on the GPU.  Every site's call is checked bit for bit
    against the oracle's whole call over the whole message: the fp32
    outputs of all ranks, the compensations and the slow memories.  The
    oracle takes as its state before each call the GPU's state after the
    previous one, which the previous site has just matched bit for bit."""
    S = n // P
    ef = mode != "off"
    two = mode == "two_timescale"
    comps = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)] if ef else None
    slows = [torch.zeros(n, dtype=torch.float32, device=DEV) for _ in range(P)] if two else None
    outs = [torch.empty(n, dtype=torch.float32, device=DEV) for _ in range(P)]
    ws = torch.empty(echo.echo_allreduce_sim_workspace_bytes(P, n, bits), dtype=torch.uint8, device=DEV)
    streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(3)]
    c_host = [np.zeros(n, np.float32) for _ in range(P)] if ef else None
    s_host = [np.zeros(n, np.float32) for _ in range(P)] if two else None
    workers = host_workers()
    L = min(S, 1 << 16)
    h = torch.zeros(n, dtype=torch.float64, device=DEV)
    h_exact = torch.zeros(n, dtype=torch.float64, device=DEV)
    rms = lambda t: float(torch.sqrt(torch.mean(t * t)))
    E_rms, d_rms, debt_gap = [], [], []
    for k in range(sites):
        xs = [gen(r, k) for r in range(P)]
        c_sum = sum(c.double() for c in comps) if ef else 0.0
        a = echo.make_sim_args(xs, outs, ws, bits=bits, tiles=4, out_dtype=oracle.OUT_F32, ef=ef,
                               alpha=alpha, beta=beta, comps=comps, slows=slows)
        echo.echo_allreduce_sim(a, streams=streams)
        x_sum = sum(x.view(torch.bfloat16).double() for x in xs)
        out = outs[0].double()
        h += out
        h_exact += x_sum
        E = h - h_exact
        E_rms.append(rms(E))
        d_rms.append(rms(out - x_sum - c_sum))
        if ef:
            debt = -sum(c.double() for c in comps)
            if two:
                debt += sum(m.double() for m in slows)
            debt_gap.append(float((E - debt).abs().max()) / max(float(E.abs().max()), 1e-30))
        for r in range(1, P):
            assert torch.equal(outs[r], outs[0])
        # whole-message parity at this site
        xh = [host_u16(x) for x in xs]
        out_h = [host_f32(o) for o in outs]
        c_after = [host_f32(c) for c in comps] if ef else None
        s_after = [host_f32(m) for m in slows] if two else None

        def visit(sl, o_outs, o_c, o_s):
            for r in range(P):
                if gather_chunk(out_h[r], sl).tobytes() != o_outs[r].tobytes():
                    return f"out[{r}] differs in the range at {sl[0].start} of segment 0"
                if ef and gather_chunk(c_after[r], sl).tobytes() != o_c[r].tobytes():
                    return f"comp[{r}] differs in the range at {sl[0].start} of segment 0"
                if two and gather_chunk(s_after[r], sl).tobytes() != o_s[r].tobytes():
                    return f"slow[{r}] differs in the range at {sl[0].start} of segment 0"
            return None

        bad = oracle_by_chunks(xh, c_host, P, L, oracle.OUT_F32, workers, visit, bits=bits, slows=s_host,
                               alpha=alpha, beta=beta)
        assert bad is None, f"{mode} site {k}: {bad}"
        c_host, s_host = c_after, s_after
        del xs, x_sum, out, E, xh, out_h
    del comps, slows, outs, ws, h, h_exact
    torch.cuda.empty_cache()
    return np.array(E_rms), np.array(d_rms), np.array(debt_gap)


def chain_gen(which):
    if which == "chain":
        P, tokens, hidden, sites, bits = 4, 2048, 4096, 64, 4
        sigma = inputs.chain_channel_scale(hidden, device=DEV)
        gen = lambda r, k: inputs.chain(r, k, tokens, hidden, sigma_h=sigma, device=DEV)
    else:
        P, tokens, hidden, sites, bits = 4, 4096, 1024, 56, 8
        gen = lambda r, k: inputs.chain8(r, k, tokens, hidden, device=DEV)
    return P, tokens * hidden, sites, bits, gen


@pytest.mark.parametrize("which", ["chain", "chain8"])
def test_depth_chain_bounded_with_feedback(echo, which):
    P, n, sites, bits, gen = chain_gen(which)
    say(which, "with feedback")
    E_ef, d_ef, gap = chain_run(echo, P, n, sites, bits, gen, "classic")
    say(which, "without feedback")
    E_off, d_off, _ = chain_run(echo, P, n, sites, bits, gen, "off")
    print(f"{which}: max RMS E with EF {E_ef.max():.3e}, max RMS delta {d_ef.max():.3e}, "
          f"RMS E_N without EF {E_off[-1]:.3e}, ratio {E_off[-1] / E_ef[-1]:.2f}, max debt gap {gap.max():.2e}",
          flush=True)
    # accumulated error == outstanding debt (fp32 rounding aside)
    assert gap.max() < 1e-3
    # bounded with feedback, independent of depth
    assert E_ef.max() <= 1.25 * d_ef.max()
    # accumulates without feedback
    assert E_off[-1] >= 4.0 * E_ef[-1]
    assert E_off[-1] > 1.5 * E_off[sites // 4]


def test_depth_chain_two_timescale(echo):
    """The 4-bit chain (64 sites, 2048 x 4096, P = 4) with the two-timescale
    compensator (alpha = 0.5, beta = 0.25) fused into push and reduce: the
    accumulated error equals the outstanding debt sum_j (M_j - c_j) at every
    site and stays within twice the largest injected error, independent of
    depth (PhantomByte article, "The cancellation rule": each error is paid
    back in later calls)."""
    P, n, sites, bits, gen = chain_gen("chain")
    say("chain two-timescale")
    E, d, gap = chain_run(echo, P, n, sites, bits, gen, "two_timescale", alpha=0.5, beta=0.25)
    print(f"chain two-timescale: max RMS E {E.max():.3e}, max RMS delta {d.max():.3e}, "
          f"ratio {E.max() / d.max():.3f}, max debt gap {gap.max():.2e}", flush=True)
    assert gap.max() < 1e-3
    assert E.max() <= 2.0 * d.max()
    # the bound does not grow with depth: the second half is no worse than 1.1x the first
    assert E[sites // 2:].max() <= 1.1 * E[:sites // 2].max()


@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (0.5, 0.25)])
def test_compensate_full_size(echo, alpha, beta):
    """echo_compensate on 2^29 + 3 elements (the state of one rank at the
    1 GiB message, plus a ragged remainder): the grid-stride loop runs many
    rounds per thread at this size.  The new compensation and slow memory
    match the oracle's update bit for bit."""
    n = (1 << 29) + 3
    say("compensate full size", alpha, beta, n)
    g = torch.Generator(device=DEV)
    g.manual_seed(20261202 + int(alpha * 1000) + int(beta * 100))
    e_d = torch.randn(n, generator=g, device=DEV) * 0.01
    c_d = torch.full((n,), 9.0, device=DEV)
    m_d = torch.randn(n, generator=g, device=DEV) * 0.02 if beta > 0 else None
    e = host_f32(e_d)
    c = np.full(n, 9.0, np.float32)
    m = host_f32(m_d).copy() if m_d is not None else None
    echo.echo_compensate(e_d, c_d, m_d, n, alpha, beta)
    torch.cuda.synchronize()
    oracle.compensate(e, c, m, n, alpha, beta)
    assert_bits_equal(host_f32(c_d), c, "comp")
    if m is not None:
        assert_bits_equal(host_f32(m_d), m, "slow")
    del e_d, c_d, m_d
    torch.cuda.empty_cache()


def test_maximum_message_size(echo):
    """The largest message the library accepts: 2^34 elements per rank
    (P = 2, feedback off, bf16 output; about 155 GB of device memory).  Every
    offset of segment 1 lies beyond 2^33 elements.  Sampled groups at both
    ends and inside both segments match the oracle bit for bit, the two
    ranks' outputs agree over the whole message, and a message one group
    pair longer is rejected."""
    P = 2
    n = 1 << 34
    S = n // P
    torch.cuda.empty_cache()
    need = P * n * 2 * 2 + echo.echo_allreduce_sim_workspace_bytes(P, n, 4) + (4 << 30)
    free, _ = torch.cuda.mem_get_info()
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of free device memory, {free / 2**30:.0f} GiB free")
    say("maximum size", n, "generate")
    xs = [inputs.laplace(r + 60, n, device=DEV) for r in range(P)]
    outs = [torch.empty(n, dtype=torch.int16, device=DEV) for _ in range(P)]
    ws = torch.empty(echo.echo_allreduce_sim_workspace_bytes(P, n, 4), dtype=torch.uint8, device=DEV)
    idx = sample_index(P, S, 24, seed=34)
    x_mini = [host_u16(x[idx]) for x in xs]
    say("maximum size", n, "call")
    a = echo.make_sim_args(xs, outs, ws, bits=4, tiles=1, out_dtype=oracle.OUT_BF16, ef=False)
    echo.echo_allreduce_sim(a)
    torch.cuda.synchronize()
    o_outs, _, _ = oracle.allreduce(x_mini, bits=4, ef=False, out_dtype=oracle.OUT_BF16)
    for r in range(P):
        assert_bits_equal(host_u16(outs[r][idx]), o_outs[r], f"out[{r}] sample")
    assert torch.equal(outs[1], outs[0]), "the ranks differ"
    assert echo.echo_allreduce_sim_workspace_bytes(P, n + 2 * G, 4) == 0   # beyond the limit
    del xs, outs, ws
    torch.cuda.empty_cache()
