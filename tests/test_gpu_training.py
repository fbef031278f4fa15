"""The training workload on the GPU: hidden 1024, 28 layers x 2 injection
sites, P = 4, batch 32 x seq 4096 bf16 partials per rank (2^27 elements),
forward then backward (reverse site order) per step, 100 steps = 11,200
calls, with the two-timescale compensator (alpha = 0.5, beta = 0.25) fused
into the kernels; each pass keeps its own compensation and slow memory,
carried across steps (Echo paper card Fig. 1: the backward pass adds its
errors at the forward pass's sites; PhantomByte article, "The cancellation rule": each error
is paid back in later calls).

Every call is checked bit for bit against the oracle on a row slice that
keeps segment ownership (the first row of every segment: an exact
sub-problem); four calls spread over the run (the first forward and first
backward call, one in the middle, the last) are checked over the whole
message against the oracle's whole call from the GPU's state before them; the state must stay bounded over the whole message, and within
each pass the accumulated error must equal the change of the outstanding
error debt (checked over the whole message every 25 steps).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from _helpers import (DEV, assert_bits_equal, gather_chunk, host_f32, host_u16, host_workers,
                      oracle_by_chunks, say)
from error_feedback_quant_amd import inputs

pytestmark = pytest.mark.gpu

P, HIDDEN, LAYERS = 4, 1024, 28
SITES = 2 * LAYERS
N = 32 * 4096 * HIDDEN                 # per rank
STEPS = int(os.environ.get("ECHO_TRAINING_STEPS", "100"))
ALPHA, BETA = 0.5, 0.25
# (step, pass, site) of the calls checked over the whole message
FULL = {(0, "fwd", 0), (0, "bwd", SITES - 1), (STEPS // 2, "fwd", LAYERS), (STEPS - 1, "bwd", 0)}


def full_call_parity(xs, outs, c_before, s_before, comps, slows, what):
    """One call over the whole message against the oracle's whole call, run
    in host threads over ranges that keep segment ownership: bf16 outputs of
    all ranks, compensations and slow memories, bit for bit."""
    xh = [host_u16(x) for x in xs]
    out_h = [host_u16(o) for o in outs]
    c_after = [host_f32(c) for c in comps]
    s_after = [host_f32(m) for m in slows]

    def visit(sl, o_outs, o_c, o_s):
        for r in range(P):
            if gather_chunk(out_h[r], sl).tobytes() != o_outs[r].tobytes():
                return f"out[{r}] differs in the range at {sl[0].start} of segment 0"
            if gather_chunk(c_after[r], sl).tobytes() != o_c[r].tobytes():
                return f"comp[{r}] differs in the range at {sl[0].start} of segment 0"
            if gather_chunk(s_after[r], sl).tobytes() != o_s[r].tobytes():
                return f"slow[{r}] differs in the range at {sl[0].start} of segment 0"
        return None

    bad = oracle_by_chunks(xh, c_before, P, 1 << 18, oracle.OUT_BF16, host_workers(), visit, bits=4,
                           slows=s_before, alpha=ALPHA, beta=BETA)
    assert bad is None, f"{what}: {bad}"


def test_training_workload_two_timescale(tmp_path):
    from error_feedback_quant_amd import echo
    S = N // P
    idx = (torch.arange(P, device=DEV)[:, None] * S + torch.arange(HIDDEN, device=DEV)[None, :]).reshape(-1)
    m = idx.numel()
    ws = torch.empty(echo.echo_allreduce_sim_workspace_bytes(P, N, 4), dtype=torch.uint8, device=DEV)
    outs = [torch.empty(N, dtype=torch.int16, device=DEV) for _ in range(P)]
    state = {p: ([torch.zeros(N, dtype=torch.float32, device=DEV) for _ in range(P)],
                 [torch.zeros(N, dtype=torch.float32, device=DEV) for _ in range(P)]) for p in ("fwd", "bwd")}
    o_state = {p: ([np.zeros(m, np.float32) for _ in range(P)], [np.zeros(m, np.float32) for _ in range(P)],
                   [np.zeros(m, np.float32) for _ in range(P)]) for p in ("fwd", "bwd")}
    debt_rms = {"fwd": [], "bwd": []}
    calls = 0
    for step in range(STEPS):
        for p in ("fwd", "bwd"):
            comps, slows = state[p]
            oc, os_, oe = o_state[p]
            check_debt = step % 25 == 24
            if check_debt:
                debt0 = sum(s.double() - c.double() for c, s in zip(comps, slows))
                E = torch.zeros(N, dtype=torch.float64, device=DEV)
            sites = range(SITES) if p == "fwd" else range(SITES - 1, -1, -1)
            for site in sites:
                xs = [inputs.training(r, step, site + (SITES if p == "bwd" else 0), p == "bwd", N, device=DEV)
                      for r in range(P)]
                full = (step, p, site) in FULL
                if full:
                    c_before = [host_f32(c) for c in comps]
                    s_before = [host_f32(m) for m in slows]
                a = echo.make_sim_args(xs, outs, ws, bits=4, tiles=1, out_dtype=echo.OUT_BF16, ef=True,
                                       alpha=ALPHA, beta=BETA, comps=comps, slows=slows)
                echo.echo_allreduce_sim(a)
                if full:
                    say(f"step {step} {p} site {site}: whole-message parity")
                    full_call_parity(xs, outs, c_before, s_before, comps, slows, f"step {step} {p} site {site}")
                    del c_before, s_before
                x_mini = [host_u16(x[idx]) for x in xs]
                o_outs, _, _ = oracle.allreduce(x_mini, bits=4, ef=True, alpha=ALPHA, beta=BETA, comps=oc,
                                                slows=os_, errs=oe, out_dtype=oracle.OUT_BF16)
                for r in range(P):
                    assert_bits_equal(host_u16(outs[r][idx]), o_outs[r], f"step {step} {p} site {site} out[{r}]")
                if check_debt:
                    E += outs[0].view(torch.bfloat16).double() - sum(x.view(torch.bfloat16).double() for x in xs)
                calls += 1
            for r in range(P):
                assert_bits_equal(host_f32(comps[r][idx]), oc[r], f"step {step} {p} comp[{r}]")
                assert_bits_equal(host_f32(slows[r][idx]), os_[r], f"step {step} {p} slow[{r}]")
            debt = sum(s.double() - c.double() for c, s in zip(comps, slows))
            debt_rms[p].append(float(torch.sqrt(torch.mean(debt * debt))))
            if check_debt:
                # within the pass: accumulated error == debt change, up to fp32 and bf16-output rounding
                gap = (E - (debt - debt0)).abs()
                out_scale = float(torch.sqrt(torch.mean(E * E))) + 1e-30
                say(f"step {step} {p}: RMS E {out_scale:.3e}, max |E - debt change| {float(gap.max()):.3e}")
                assert float(torch.sqrt(torch.mean(gap * gap))) <= 0.25 * out_scale
                del E, debt0
            del debt
        if step % 10 == 0 or step == STEPS - 1:
            say(f"step {step}: {calls} calls, debt RMS fwd {debt_rms['fwd'][-1]:.3e} bwd {debt_rms['bwd'][-1]:.3e}")
    # the two-timescale state stays bounded: no growth after the first steps
    for p in ("fwd", "bwd"):
        d = np.array(debt_rms[p])
        ref = d[: max(2, len(d) // 10)].max()
        assert d.max() <= 1.5 * ref, (p, d.max(), ref)
    assert calls == STEPS * 2 * SITES
