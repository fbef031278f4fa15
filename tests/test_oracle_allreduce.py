"""Pins for the oracle's all-reduce call and compensator (CPU only).

Structure of the call: Echo paper card, Fig. 2(a) and appendix Fig. 4 (push of
non-owned segments as codes; the owner adds three decoded copies to its own
copy, which is never quantized, in fp32; the total is quantized a single time;
every rank decodes the same code); abstract (no element is quantized more than
twice, whatever P; the sum reveals the injected error; returning it cancels
it in later calls; with feedback the accumulated error does not grow with
depth).  The
two-timescale compensator is named in the PhantomByte article ("The
cancellation rule") without equations; the reading is an error debt (fast
fraction alpha returned at the next call, slow memory released at rate beta).
"""
import json
import os

import numpy as np
import pytest

import oracle
from error_feedback_quant_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U24 = 2.0 ** -24


def bf16_to_f64(x):
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_partials(P, n, seed, scale=1.0, decimals=None):
    rng = np.random.default_rng(seed)
    xs = []
    for _ in range(P):
        v = rng.standard_normal(n) * scale
        if decimals is not None:
            v = np.round(v, decimals)
        xs.append(oracle.f32_to_bf16_bits(v.astype(np.float32)))
    return xs


def run_steps(xs, bits, g, comps=None, tiles=None):
    """Run the call through the oracle's step functions (push per rank,
    reduce per owner, decode per rank), optionally tile by tile, with error
    outputs and no compensator update.  Returns outs, errs, codes."""
    P, n = len(xs), xs[0].size
    S = n // P
    cb = oracle.code_bytes(n, bits)
    pc = [np.zeros(cb, np.uint8) for _ in range(P)]
    pp = [np.zeros(2 * (n // g), np.uint16) for _ in range(P)]
    sc = np.zeros(cb, np.uint8)
    sp = np.zeros(2 * (n // g), np.uint16)
    errs = [np.zeros(n, np.float32) for _ in range(P)]
    outs = [np.zeros(n, np.float32) for _ in range(P)]
    bounds = tiles or [(0, S)]
    for (tb, tl) in bounds:
        for r in range(P):
            oracle.quantize_ef(xs[r], None if comps is None else comps[r], n, P, r, tb, tl, bits, g,
                               pc[r], pp[r], errs[r])
    for (tb, tl) in bounds:
        for o in range(P):
            oracle.reduce_segment(xs[o], None if comps is None else comps[o], pc, pp, P, o, n, tb, tl,
                                  bits, g, sc, sp, errs[o])
    for (tb, tl) in bounds:
        for r in range(P):
            oracle.gather_dequant(sc, sp, n, tb, tl, P, bits, g, outs[r], oracle.OUT_F32)
    return outs, errs, (pc, pp, sc, sp)


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("bits", [4, 8])
def test_identical_outputs_and_at_most_two_quantizations(P, bits):
    n = P * 128 * 3
    xs = rand_partials(P, n, 100 + P + bits)
    for odt in (oracle.OUT_F32, oracle.OUT_BF16):
        outs, qdepth, qwork = oracle.allreduce(xs, bits=bits, out_dtype=odt, want_counts=True)
        for r in range(1, P):
            assert outs[r].tobytes() == outs[0].tobytes()          # bitwise identical on every rank
        # counted along every path into every output element
        assert qdepth.max() <= 2
        assert np.all(qdepth == (2 if P > 1 else 1))
        # every rank quantizes exactly n elements per call, whatever P is
        assert np.all(qwork == n)


@pytest.mark.parametrize("P", [2, 4, 8])
@pytest.mark.parametrize("bits", [4, 8])
def test_sum_reveals_the_injected_error(P, bits):
    """out - sum_j x_j equals sum_j e_j (push errors on non-owned segments and
    the owner's requantization error), up to the fp32 rounding of the sum and
    of each error: (P + 1) * 2^-24 * (sum |t| + sum |e|)."""
    n = P * 128 * 4
    xs = rand_partials(P, n, 200 + P + bits)
    xs[0][:64] = oracle.f32_to_bf16_bits(np.full(64, 37.0, np.float32))   # one group with an outlier
    outs, errs, _ = run_steps(xs, bits, 128)
    xsum = sum(bf16_to_f64(x) for x in xs)
    esum = sum(e.astype(np.float64) for e in errs)
    tabs = sum(np.abs(bf16_to_f64(x)) + np.abs(e.astype(np.float64)) for x, e in zip(xs, errs))
    lhs = outs[0].astype(np.float64) - xsum
    assert np.all(np.abs(lhs - esum) <= (P + 1) * U24 * (tabs + np.abs(esum)) + 1e-30)
    assert np.abs(esum).max() > 0                                           # the errors are not trivially zero


def test_fig4_shaped_example():
    """The worked example's shape (appendix Fig. 4): P = 4, b = 4, each
    segment is one group of two elements, inputs with one decimal.  Checks what the figure
    states: identical values on every rank; the owner's own copy enters the sum
    unquantized (its rank records no push error there, and the error identity
    only closes if the own copy is exact); the last row (out - sum x) is the
    injected error, equal to the sum of the revealed shares."""
    spec = json.load(open(os.path.join(GOLDEN, "fig4_shape.json")))
    P, bits, g, n = spec["P"], spec["bits"], spec["group"], spec["n"]
    for seed in range(50):
        xs = rand_partials(P, n, 300 + seed, decimals=spec["input_decimals"])
        outs, errs, (pc, pp, sc, sp) = run_steps(xs, bits, g)
        for r in range(1, P):
            assert outs[r].tobytes() == outs[0].tobytes()
        S = n // P
        for o in range(P):
            seg = slice(o * S, (o + 1) * S)
            # the own segment's push codes were never written by its owner
            assert not pc[o][o * S // 2:(o + 1) * S // 2].any()
        xsum = sum(bf16_to_f64(x) for x in xs)
        esum = sum(e.astype(np.float64) for e in errs)
        tabs = sum(np.abs(bf16_to_f64(x)) + np.abs(e.astype(np.float64)) for x, e in zip(xs, errs))
        assert np.all(np.abs(outs[0] - xsum - esum) <= (P + 1) * U24 * (tabs + np.abs(esum)))


def test_single_rank_is_one_round_trip():
    """P = 1: no push, so the output is one quantize/dequantize of the input."""
    n = 128 * 16
    (x,) = rand_partials(1, n, 400)
    outs, qdepth, _ = oracle.allreduce([x], bits=4, want_counts=True)
    v = bf16_to_f64(x).astype(np.float32)
    for k in range(n // 128):
        q, sh, zh = oracle.quantize_group(v[k * 128:(k + 1) * 128], 4)
        want = np.array([oracle.dequant(int(a), sh, zh) for a in q], np.float32)
        assert np.array_equal(outs[0][k * 128:(k + 1) * 128], want)
    assert np.all(qdepth == 1)


@pytest.mark.parametrize("P", [2, 4, 8])
def test_one_contributor_on_the_grid_is_exact(P):
    """If one rank holds values already on a 4-bit grid with a power-of-two
    scale (so exactly representable in bfloat16) and every other rank holds
    zeros, the push is lossless, the fp32 sum adds only exact zeros and the
    requantization is lossless: every rank gets the input back exactly.  Pins
    the composition (which rank's codes, which segment, which group)."""
    rng = np.random.default_rng(500 + P)
    n = P * 128 * 2
    for src in range(P):
        v = np.zeros(n, np.float32)
        for grp in range(n // 128):
            s = 2.0 ** int(rng.integers(-8, 4))
            z = int(rng.integers(0, 16))
            k = rng.integers(0, 16, size=128)
            k[rng.integers(0, 64)] = 0
            k[64 + rng.integers(0, 64)] = 15
            v[grp * 128:(grp + 1) * 128] = (k - z) * s
        xs = [np.zeros(n, np.uint16) for _ in range(P)]
        xs[src] = oracle.f32_to_bf16_bits(v)
        assert np.array_equal(bf16_to_f64(xs[src]), v.astype(np.float64))
        outs, _, _ = oracle.allreduce(xs, bits=4)
        for r in range(P):
            assert np.array_equal(outs[r], v)


@pytest.mark.parametrize("bits", [4, 8])
def test_tiles_are_independent(bits):
    """Splitting each segment into tiles (multiples of g) and running the
    steps tile by tile in any order gives the same bits as whole segments."""
    P, g = 4, 128
    n = P * g * 12
    xs = rand_partials(P, n, 600 + bits)
    comps = [np.random.default_rng(7 + r).standard_normal(n).astype(np.float32) * 0.01 for r in range(P)]
    whole, ew, cw = run_steps(xs, bits, g, comps=comps)
    S = n // P
    tiles = [(0, 3 * g), (3 * g, g), (4 * g, 5 * g), (9 * g, 3 * g)]
    assert sum(t[1] for t in tiles) == S
    tiled, et, ct = run_steps(xs, bits, g, comps=comps, tiles=tiles[::-1])
    for r in range(P):
        assert whole[r].tobytes() == tiled[r].tobytes()
        assert ew[r].tobytes() == et[r].tobytes()
    for a, b in zip(cw[0] + cw[1] + [cw[2], cw[3]], ct[0] + ct[1] + [ct[2], ct[3]]):
        assert a.tobytes() == b.tobytes()


def test_fused_negated_error_equals_classic_update():
    """With alpha = 1 and beta = 0 the update c' = -(1 * e) is exactly -e, so
    writing -e straight into the compensation buffer (fused) gives the same
    bits as computing e and running the compensator."""
    P, n = 4, 4 * 128 * 8
    c1 = [np.zeros(n, np.float32) for _ in range(P)]
    c2 = [np.zeros(n, np.float32) for _ in range(P)]
    errs = [np.zeros(n, np.float32) for _ in range(P)]
    for k in range(5):
        xs = rand_partials(P, n, 700 + k)
        o1, _, _ = oracle.allreduce(xs, ef=True, comps=c1)
        o2, _, _ = oracle.allreduce(xs, ef=True, comps=c2, errs=errs)
        assert o1[0].tobytes() == o2[0].tobytes()
        for a, b in zip(c1, c2):
            assert a.tobytes() == b.tobytes()


@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (0.5, 0.25), (0.75, 0.1), (0.3, 1.0)])
def test_compensator_conserves_the_error_debt(alpha, beta):
    """Whatever is not returned now is kept: -c' + M' = e + M (the new error
    plus the old debt), up to the four fp32 roundings of the update."""
    rng = np.random.default_rng(800)
    n = 1 << 14
    e = rng.standard_normal(n).astype(np.float32)
    M = (rng.standard_normal(n) * 3).astype(np.float32)
    c = np.zeros(n, np.float32)
    if beta == 0.0:
        oracle.compensate(e, c, None, n, alpha, beta)
        assert np.array_equal(c, -e * np.float32(alpha))
        assert np.array_equal(c.view(np.uint32), (-e).view(np.uint32)) if alpha == 1.0 else True
        return
    M0 = M.copy()
    oracle.compensate(e, c, M, n, alpha, beta)
    lhs = -c.astype(np.float64) + M.astype(np.float64)
    rhs = e.astype(np.float64) + M0.astype(np.float64)
    tol = 4 * U24 * (np.abs(e) + np.abs(M0)).astype(np.float64)
    assert np.all(np.abs(lhs - rhs) <= tol)
    # the fast part returns alpha of the new error and beta of the old debt
    assert np.all(np.abs(-c - (alpha * e.astype(np.float64) + beta * M0)) <= tol)


def test_compensator_rejects_bad_constants():
    n = 128
    e = np.zeros(n, np.float32)
    c = np.zeros(n, np.float32)
    M = np.zeros(n, np.float32)
    for a, b, m in [(0.0, 0.0, None), (1.5, 0.0, None), (0.5, 0.0, None), (1.0, 0.5, None),
                    (1.0, -0.1, M), (1.0, 1.5, M), (0.5, 0.0, M)]:
        with pytest.raises(oracle.OracleError):
            oracle.compensate(e, c, m, n, a, b)


def _chain_partials(P, tokens, hidden, sites, sigma):
    def f(site):
        if site >= sites:
            return None
        return [inputs.as_numpy_u16(inputs.chain(r, site, tokens, hidden, sigma_h=sigma)) for r in range(P)]
    return f


@pytest.mark.parametrize("mode", ["off", "classic", "two_timescale"])
def test_depth_chain_closed_form(mode):
    """Over a chain of N sites (Fig. 1) the accumulated error equals the
    outstanding error debt: E_k = sum_j (M_j - c_j) after site k.  With classic
    feedback (alpha = 1) that is E_k = delta_k, the newest error alone; without
    feedback E_k is the sum of every delta.  Holds up to the uncaptured fp32
    roundings (of x + c, of the sum and of each error), k * (P + 3) * 2^-24 * |.|."""
    P, tokens, hidden, N = 4, 8, 512, 64
    n = tokens * hidden
    sigma = inputs.chain_channel_scale(hidden)
    part = _chain_partials(P, tokens, hidden, N, sigma)
    if mode == "off":
        res = oracle.depth_chain(part, P, n, ef=False)
        cum = np.cumsum(res["delta"], axis=0)
        assert np.allclose(res["E"], cum, rtol=0, atol=1e-9)
        return
    if mode == "classic":
        res = oracle.depth_chain(part, P, n, ef=True, alpha=1.0, beta=0.0, fused=True)
    else:
        res = oracle.depth_chain(part, P, n, ef=True, alpha=0.5, beta=0.25, fused=False)
    E, debt = res["E"], res["debt"]
    scale = np.abs(E).max() + np.abs(debt).max() + 1.0
    for k in range(N):
        tol = (k + 1) * (P + 3) * U24 * 64 * scale
        assert np.abs(E[k] - debt[k]).max() <= tol, (k, np.abs(E[k] - debt[k]).max(), tol)
    if mode == "classic":
        # E_k is just the error injected at the last site
        assert np.abs(E[-1] - res["delta"][-1]).max() <= N * (P + 3) * U24 * 64 * scale


def test_depth_chain_error_bounded_with_feedback_grows_without():
    """Abstract: with feedback the accumulated error stays at the size of one
    site's error however many sites there are, and without it the error piles up (about sqrt(N) for independent
    sites).  Thresholds: with classic feedback max_k RMS(E_k) <= 1.25 *
    max_k RMS(delta_k); two-timescale <= 2x; without feedback RMS(E_N) is at
    least 4x the feedback run's at N = 64."""
    P, tokens, hidden, N = 4, 8, 512, 64
    n = tokens * hidden
    sigma = inputs.chain_channel_scale(hidden)
    part = _chain_partials(P, tokens, hidden, N, sigma)
    rms = lambda a: np.sqrt(np.mean(a * a, axis=-1))
    off = oracle.depth_chain(part, P, n, ef=False)
    ef1 = oracle.depth_chain(part, P, n, ef=True, alpha=1.0, beta=0.0)
    ef2 = oracle.depth_chain(part, P, n, ef=True, alpha=0.5, beta=0.25, fused=False)
    assert rms(ef1["E"]).max() <= 1.25 * rms(ef1["delta"]).max()
    assert rms(ef2["E"]).max() <= 2.0 * rms(ef2["delta"]).max()
    assert rms(off["E"])[-1] >= 4.0 * rms(ef1["E"])[-1]
    # growth without feedback: the second half's error is larger than the first's
    assert rms(off["E"])[N - 1] > 1.5 * rms(off["E"])[N // 4]


def test_argument_checks():
    n, P = 4 * 128, 4
    x = np.zeros(n, np.uint16)
    codes = np.zeros(n, np.uint8)
    params = np.zeros(2 * n // 128, np.uint16)
    bad = [
        dict(bits=3), dict(bits=4, group=3), dict(rank=4), dict(rank=-1), dict(P=0),
        dict(tile_begin=64), dict(tile_len=129), dict(tile_begin=128, tile_len=128 * 1),
    ]
    for b in bad:
        kw = dict(n=n, P=P, rank=0, tile_begin=0, tile_len=128, bits=4, group=128)
        kw.update(b)
        if kw == dict(n=n, P=P, rank=0, tile_begin=128, tile_len=128, bits=4, group=128):
            continue   # that one is valid (tile inside the segment)
        with pytest.raises(oracle.OracleError):
            oracle.quantize_ef(x, None, kw["n"], kw["P"], kw["rank"], kw["tile_begin"], kw["tile_len"],
                               kw["bits"], kw["group"], codes, params, None)
    with pytest.raises(oracle.OracleError):   # n not a multiple of P * g
        oracle.quantize_ef(x, None, n - 128, P, 0, 0, 0, 4, 128, codes, params, None)


@pytest.mark.parametrize("P,bits,out_dtype", [(4, 4, oracle.OUT_BF16), (8, 4, oracle.OUT_BF16), (3, 8, oracle.OUT_F32)])
def test_chunked_calls_equal_one_whole_call(P, bits, out_dtype):
    """The full-size GPU parity test computes the oracle's call as
    independent calls on mini messages made of the same range of every
    segment, in host threads.  That is valid because quantization, the
    owner's sum and the feedback act per group and per element: here the
    chunked result must equal one call on the whole message, bit for bit,
    with a nonzero compensation carried in and written back."""
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    from _helpers import oracle_by_chunks, gather_chunk

    S = 128 * 24
    n = P * S
    rng = np.random.default_rng(7 + P)
    xs = [oracle.f32_to_bf16_bits(rng.laplace(size=n).astype(np.float32)) for _ in range(P)]
    comps0 = [(rng.standard_normal(n) * 0.05).astype(np.float32) for _ in range(P)]
    kept = [c.copy() for c in comps0]
    whole_c = [c.copy() for c in comps0]
    whole, _, _ = oracle.allreduce(xs, bits=bits, ef=True, comps=whole_c, out_dtype=out_dtype)

    slows0 = [(rng.standard_normal(n) * 0.02).astype(np.float32) for _ in range(P)]
    kept_s = [m.copy() for m in slows0]
    two_c = [c.copy() for c in comps0]
    two_s = [m.copy() for m in slows0]
    two, _, _ = oracle.allreduce(xs, bits=bits, ef=True, alpha=0.5, beta=0.25, comps=two_c, slows=two_s,
                                 out_dtype=out_dtype)

    def visit(sl, outs, cm, sm):
        for r in range(P):
            if gather_chunk(whole[r], sl).tobytes() != outs[r].tobytes():
                return f"out[{r}] at {sl[0].start}"
            if gather_chunk(whole_c[r], sl).tobytes() != cm[r].tobytes():
                return f"comp[{r}] at {sl[0].start}"
        return None

    def visit_two(sl, outs, cm, sm):
        for r in range(P):
            if gather_chunk(two[r], sl).tobytes() != outs[r].tobytes():
                return f"out[{r}] at {sl[0].start}"
            if gather_chunk(two_c[r], sl).tobytes() != cm[r].tobytes():
                return f"comp[{r}] at {sl[0].start}"
            if gather_chunk(two_s[r], sl).tobytes() != sm[r].tobytes():
                return f"slow[{r}] at {sl[0].start}"
        return None

    for L in (128, 384, 128 * 8):
        assert oracle_by_chunks(xs, comps0, P, L, out_dtype, 4, visit, bits=bits) is None, L
        assert oracle_by_chunks(xs, comps0, P, L, out_dtype, 4, visit_two, bits=bits, slows=slows0,
                                alpha=0.5, beta=0.25) is None, L
    # the chunked calls leave their input state untouched
    assert all(c.tobytes() == k.tobytes() for c, k in zip(comps0, kept))
    assert all(m.tobytes() == k.tobytes() for m, k in zip(slows0, kept_s))


@pytest.mark.parametrize("alpha,beta", [(0.5, 0.25), (0.75, 0.1)])
def test_two_timescale_error_bound_independent_of_depth(alpha, beta):
    """Elementwise bound for the two-timescale compensator: each rank's
    outstanding debt M - c stays within (1 + (1 - alpha) / beta) * max|e|
    (the slow memory is a geometric sum of (1 - alpha) e with ratio 1 - beta;
    the fast part returns alpha e + beta M), so the accumulated error over a
    chain, the sum of the P debts, stays within P (1 + (1 - alpha) / beta)
    max|e| at every depth, where max|e| runs over every error injected so
    far.  The e_j come from the unfused form (errors written out, then the
    compensator)."""
    P, tokens, hidden, N = 4, 8, 512, 64
    n = tokens * hidden
    sigma = inputs.chain_channel_scale(hidden)
    part = _chain_partials(P, tokens, hidden, N, sigma)
    comps = [np.zeros(n, np.float32) for _ in range(P)]
    slows = [np.zeros(n, np.float32) for _ in range(P)]
    errs = [np.zeros(n, np.float32) for _ in range(P)]
    h = np.zeros(n)
    h_exact = np.zeros(n)
    emax = 0.0
    factor = P * (1.0 + (1.0 - alpha) / beta)
    worst = 0.0
    for k in range(N):
        xs = part(k)
        outs, _, _ = oracle.allreduce(xs, bits=4, ef=True, alpha=alpha, beta=beta, comps=comps,
                                      slows=slows, errs=errs)
        emax = max(emax, max(float(np.abs(e).max()) for e in errs))
        h += outs[0].astype(np.float64)
        for x in xs:
            h_exact += bf16_to_f64(x)
        E = np.abs(h - h_exact)
        # fp32 roundings of the update and of the sums: a relative slack far above their size
        slack = (k + 1) * 64 * (P + 3) * U24 * (np.abs(h).max() + 1.0)
        assert E.max() <= factor * emax * (1 + 1e-5) + slack, (k, E.max(), factor * emax)
        worst = max(worst, E.max() / (factor * emax))
    # the bound is not vacuous: the chain uses a sizeable part of it
    assert worst > 0.05


@pytest.mark.parametrize("bits,ratio", [(4, 16 / 4.25), (8, 16 / 8.25)])
def test_wire_bytes_per_pushed_element(bits, ratio):
    """Abstract: a 4-bit payload makes the all-reduce's traffic almost four
    times smaller than a 16-bit one.  Count the bytes the push writes for one
    rank's non-owned segments (codes plus one binary16 scale and zero per
    group of 128, found by writing over two different sentinels): 4.25 bits
    per element at b = 4, so 16 / 4.25 = 3.76x fewer bytes than bf16."""
    P, g = 4, 128
    S = g * 16
    n = P * S
    xs = rand_partials(P, n, 41)
    written = []
    for fill in (0x00, 0xFF):
        codes = np.full(oracle.code_bytes(n, bits), fill, np.uint8)
        params = np.full(2 * (n // g), fill * 0x0101, np.uint16)
        oracle.quantize_ef(xs[0], None, n, P, 0, 0, S, bits, g, codes, params, None)
        written.append((codes.copy(), params.view(np.uint8).copy()))
    (c0, p0), (c1, p1) = written
    # a byte was written if it holds the same value after both sentinels
    code_bytes = int(np.count_nonzero(c0 == c1))
    param_bytes = int(np.count_nonzero(p0 == p1))
    pushed = (P - 1) * S
    assert code_bytes == pushed * bits // 8
    assert param_bytes == pushed // g * 4
    bits_per_elem = 8 * (code_bytes + param_bytes) / pushed
    assert bits_per_elem == bits + 32 / g
    assert abs(16 / bits_per_elem - ratio) < 1e-12
    if bits == 4:
        assert 3.5 < 16 / bits_per_elem < 4.0        # almost four times fewer bytes


@pytest.mark.parametrize("quant,group", [("naive", 128), ("symmetric", 128), ("zero_aware", 256), ("mse", 128),
                                         ("mse", 256)])
def test_chunked_calls_equal_one_whole_call_variants(quant, group):
    """The chunked form of the oracle's call (as the full-size GPU parity runs
    it) for Table 8's quantizers and groups of 256: equal to one whole call,
    bit for bit."""
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    from _helpers import oracle_by_chunks, gather_chunk

    P, S = 4, 256 * 12
    n = P * S
    rng = np.random.default_rng(11)
    xs = [oracle.f32_to_bf16_bits(rng.laplace(size=n).astype(np.float32)) for _ in range(P)]
    comps0 = [(rng.standard_normal(n) * 0.05).astype(np.float32) for _ in range(P)]
    whole_c = [c.copy() for c in comps0]
    whole, _, _ = oracle.allreduce(xs, bits=4, group=group, ef=True, comps=whole_c, out_dtype=oracle.OUT_BF16,
                                   quant=quant)

    def visit(sl, outs, cm, sm):
        for r in range(P):
            if gather_chunk(whole[r], sl).tobytes() != outs[r].tobytes():
                return f"out[{r}] at {sl[0].start}"
            if gather_chunk(whole_c[r], sl).tobytes() != cm[r].tobytes():
                return f"comp[{r}] at {sl[0].start}"
        return None

    for L in (256, 256 * 4):
        assert oracle_by_chunks(xs, comps0, P, L, oracle.OUT_BF16, 4, visit, quant=quant, group=group) is None
