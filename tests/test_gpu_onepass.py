"""GPU parity of the one-launch form of echo_allreduce_sim.

A call asked for in one tile with at most 2^20 elements per rank runs as one
launch (each block takes one 512-element chunk of one segment through every
rank's push, the owner's reduce and every rank's tail, its four wavefronts
splitting the ranks).  These cases cover it over the ranks (more than four,
where a wavefront serves two), code widths, feedback forms, quantizers,
group sizes and output types, on segments whose last chunk is partly empty
(down to one group), against the oracle's whole call over three calls that
carry the state; 16 seeded random cases (ranks, segment
length up to the limit, width, quantizer, group size, feedback form, output
type) over two calls; the largest one-launch message and the smallest
message above it against the oracle; and guard regions around every buffer
the call writes."""
import numpy as np
import pytest
import torch

import oracle
from _helpers import DEV, assert_bits_equal, assert_f32_parity, dev_u16, host_f32, host_u16, rand_bf16, say
from test_gpu_sim import MODES, run_gpu_calls, run_oracle_calls

pytestmark = pytest.mark.gpu
ONEPASS_MAX = 1 << 20


@pytest.fixture(scope="module")
def echo():
    from error_feedback_quant_amd import echo as e
    assert torch.cuda.is_available()
    return e


def check(got, gstate, want, wstate, P, odt):
    for c in range(len(got)):
        for r in range(P):
            if odt == oracle.OUT_F32:
                assert_f32_parity(got[c][r], want[c][r], f"call {c} rank {r} out")
            assert_bits_equal(got[c][r], want[c][r], f"call {c} rank {r} out bits")
    for key in ("comps", "slows", "errs"):
        if wstate[key] is not None and gstate[key] is not None:
            for r in range(P):
                assert_bits_equal(gstate[key][r], wstate[key][r], f"{key}[{r}] bits")


CASES = [
    # P, bits, ef, out, quant, group, groups per segment
    (1, 4, "classic", oracle.OUT_BF16, "zero_aware", 128, 37),
    (2, 8, "off", oracle.OUT_F32, "zero_aware", 128, 37),
    (3, 4, "two", oracle.OUT_F32, "zero_aware", 128, 37),          # last chunk: one group
    (4, 4, "classic", oracle.OUT_BF16, "zero_aware", 128, 37),
    (4, 4, "classic_unfused", oracle.OUT_F32, "naive", 128, 37),
    (4, 8, "two_fused", oracle.OUT_BF16, "symmetric", 128, 5),      # one partly empty chunk per segment
    (4, 4, "classic", oracle.OUT_F32, "mse", 128, 37),
    (4, 4, "two_fused", oracle.OUT_F32, "zero_aware", 256, 19),
    (5, 8, "classic", oracle.OUT_BF16, "naive", 256, 19),           # wavefront 0 serves ranks 0 and 4
    (8, 4, "off", oracle.OUT_BF16, "zero_aware", 128, 37),
    (8, 8, "two", oracle.OUT_F32, "mse", 256, 3),
    (8, 4, "classic_unfused", oracle.OUT_BF16, "symmetric", 256, 1),  # one group of 256 per segment
    (6, 4, "two_fused", oracle.OUT_BF16, "mse", 128, 1),
    (7, 8, "off", oracle.OUT_F32, "symmetric", 128, 64),
]


@pytest.mark.parametrize("P,bits,ef_mode,odt,quant,group,gps", CASES)
def test_one_launch_matches_oracle_over_calls(echo, P, bits, ef_mode, odt, quant, group, gps):
    n = P * group * gps
    assert n <= ONEPASS_MAX
    calls = 3
    xs_list = [[rand_bf16(n, 7000 * c + 100 * P + r + bits, scale=1.0 + c) for r in range(P)] for c in range(calls)]
    say("one launch", P, bits, ef_mode, odt, quant, group, gps)
    got, gstate = run_gpu_calls(echo, xs_list, P, n, bits, ef_mode, odt, 1, 1, quant, group)
    want, wstate = run_oracle_calls(xs_list, P, n, bits, ef_mode, odt, quant, group)
    check(got, gstate, want, wstate, P, odt)


@pytest.mark.parametrize("n", [ONEPASS_MAX, ONEPASS_MAX + 4 * 128])
def test_both_sides_of_the_one_launch_limit(echo, n):
    """The largest one-launch message and the smallest one above it (the
    per-stage launches), each against the oracle."""
    P, bits = 4, 4
    xs_list = [[rand_bf16(n, 9100 + 10 * c + r) for r in range(P)] for c in range(2)]
    say("limit", n)
    got, gstate = run_gpu_calls(echo, xs_list, P, n, bits, "classic", oracle.OUT_BF16, 1, 1)
    want, wstate = run_oracle_calls(xs_list, P, n, bits, "classic", oracle.OUT_BF16)
    check(got, gstate, want, wstate, P, oracle.OUT_BF16)


@pytest.mark.parametrize("ef_mode,odt", [("classic", oracle.OUT_BF16), ("two", oracle.OUT_F32),
                                         ("two_fused", oracle.OUT_F32)])
def test_one_launch_writes_nothing_outside_the_message(echo, ef_mode, odt):
    """Every buffer the call writes sits inside a guard region filled with a
    sentinel; after the call the guards are unchanged and the message equals
    the oracle's."""
    P, bits, group, gps = 3, 4, 128, 37
    n = P * group * gps
    pad = 4096
    alpha, beta = MODES[ef_mode]
    odtype = torch.float32 if odt == oracle.OUT_F32 else torch.int16
    sentinel_f = float(np.float32(-1234.5))

    def guarded(dtype, fill):
        t = torch.full((n + 2 * pad,), fill, dtype=dtype, device=DEV)
        return t, t[pad:pad + n]

    xs = [rand_bf16(n, 9300 + r) for r in range(P)]
    outs_full, outs = zip(*[guarded(odtype, 0x3F if odtype == torch.int16 else sentinel_f) for _ in range(P)])
    comps_full, comps = zip(*[guarded(torch.float32, 0.0) for _ in range(P)])
    for c in comps_full:
        c[:pad] = sentinel_f
        c[pad + n:] = sentinel_f
    errs_full = errs = slows_full = slows = None
    if ef_mode == "two":
        errs_full, errs = zip(*[guarded(torch.float32, sentinel_f) for _ in range(P)])
    if ef_mode in ("two", "two_fused"):
        slows_full, slows = zip(*[guarded(torch.float32, 0.0) for _ in range(P)])
        for s in slows_full:
            s[:pad] = sentinel_f
            s[pad + n:] = sentinel_f
    ws_bytes = echo.echo_allreduce_sim_workspace_bytes(P, n, bits, group)
    ws_full = torch.full((ws_bytes + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
    ws = ws_full[pad:pad + ws_bytes]
    xd = [dev_u16(x) for x in xs]
    a = echo.make_sim_args(xd, list(outs), ws, bits=bits, tiles=1, out_dtype=odt, ef=True, alpha=alpha, beta=beta,
                           comps=list(comps), slows=list(slows) if slows else None,
                           errs=list(errs) if errs else None, quant="zero_aware", group=group)
    say("guards", ef_mode, odt)
    echo.echo_allreduce_sim(a)
    torch.cuda.synchronize()

    def guards_hold(full, what):
        h = full.cpu()
        assert torch.equal(h[:pad], torch.full_like(h[:pad], h[0].item())), f"{what}: front guard written"
        assert torch.equal(h[pad + (full.numel() - 2 * pad):], torch.full_like(h[:pad], h[-1].item())), \
            f"{what}: back guard written"

    for r in range(P):
        guards_hold(outs_full[r], f"out[{r}]")
        guards_hold(comps_full[r], f"comp[{r}]")
        if errs_full:
            guards_hold(errs_full[r], f"err[{r}]")
        if slows_full:
            guards_hold(slows_full[r], f"slow[{r}]")
    wsh = ws_full.cpu()
    assert torch.all(wsh[:pad] == 0xA5) and torch.all(wsh[pad + ws_bytes:] == 0xA5), "workspace guard written"
    # the guards' fill values are what the test wrote (not only uniform)
    assert outs_full[0].cpu()[0].item() == (0x3F if odtype == torch.int16 else sentinel_f)
    assert comps_full[0].cpu()[0].item() == sentinel_f

    want, wstate = run_oracle_calls([xs], P, n, bits, ef_mode, odt)
    got = [[host_f32(o) if odt == oracle.OUT_F32 else host_u16(o) for o in outs]]
    gstate = dict(comps=[host_f32(c) for c in comps], slows=[host_f32(s) for s in slows] if slows else None,
                  errs=[host_f32(e) for e in errs] if errs else None)
    check(got, gstate, want, wstate, P, odt)


def _random_case(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.integers(1, 9))
    group = int(rng.choice([128, 256]))
    # segments from one group up to the one-launch limit
    max_gps = ONEPASS_MAX // (P * group)
    gps = int(rng.choice([1, 2, 3, int(rng.integers(4, 80)), int(rng.integers(80, max_gps + 1))]))
    bits = int(rng.choice([4, 8]))
    quant = str(rng.choice(["zero_aware", "naive", "symmetric", "mse"]))
    ef_mode = str(rng.choice(list(MODES)))
    odt = int(rng.choice([oracle.OUT_F32, oracle.OUT_BF16]))
    return P, group, gps, bits, quant, ef_mode, odt


@pytest.mark.parametrize("seed", range(16))
def test_one_launch_random_cases(echo, seed):
    P, group, gps, bits, quant, ef_mode, odt = _random_case(20261203 + seed)
    n = P * group * gps
    say("one launch random", seed, P, group, gps, bits, quant, ef_mode, odt)
    xs_list = [[rand_bf16(n, 50000 + 100 * seed + 10 * c + r, scale=0.5 + c) for r in range(P)] for c in range(2)]
    got, gstate = run_gpu_calls(echo, xs_list, P, n, bits, ef_mode, odt, 1, 1, quant, group)
    want, wstate = run_oracle_calls(xs_list, P, n, bits, ef_mode, odt, quant, group)
    check(got, gstate, want, wstate, P, odt)


def _with_zero_groups(x, group):
    """bf16 partials with every third group zero (some with -0) and every
    sixth (offset 1) one constant, the same rows on every rank."""
    b = np.frombuffer(x.tobytes(), np.uint16).copy().reshape(-1, group)
    b[0::3] = 0x0000
    b[0::9, ::2] = 0x8000                       # -0
    b[1::6] = 0x3F40                            # 0.75
    return b.reshape(-1)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("quant", ["zero_aware", "naive", "symmetric", "mse"])
def test_one_launch_groups_zero_on_every_rank(echo, quant, bits):
    """Zero (and, for the naive quantizer, constant) groups on every rank
    through the one-launch call over three calls with classic feedback: the
    pushes store scale 0 for them, the owner decodes those peers' words and
    stores its all-zero sums with scale 0, and the compensation stays zero
    there; bit for bit against the oracle."""
    P, group, gps = 4, 128, 18
    n = P * group * gps
    xs_list = [[_with_zero_groups(rand_bf16(n, 9700 + 10 * c + r + bits), group) for r in range(P)]
               for c in range(3)]
    say("one launch zero groups", quant, bits)
    got, gstate = run_gpu_calls(echo, xs_list, P, n, bits, "classic", oracle.OUT_BF16, 1, 1, quant, group)
    want, wstate = run_oracle_calls(xs_list, P, n, bits, "classic", oracle.OUT_BF16, quant, group)
    check(got, gstate, want, wstate, P, oracle.OUT_BF16)
    zero_rows = np.arange(n // group)[0::3]
    for r in range(P):
        assert np.all(wstate["comps"][r].reshape(-1, group)[zero_rows] == 0)
