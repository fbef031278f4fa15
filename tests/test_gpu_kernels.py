"""GPU parity of each libecho entry point against the CPU oracle.

Each test runs the same seeded inputs through the C ABI on the GPU and
through the oracle on the host, over the single-call workload's shape (P = 4,
64 x 1024 per rank) and ragged tiles that leave partial blocks, and compares:
codes and parameters byte for byte, fp32 errors/outputs within 1e-6 relative
(the bar for floating point), bf16 outputs bit for bit.  Buffers start filled
with a sentinel on both sides, so writes outside the tile are caught too.
Push codes fed to the reduce test come from the oracle, so each kernel is
checked on its own.
"""
import numpy as np
import pytest
import torch

import oracle
from _helpers import (DEV, assert_bits_equal, assert_f32_parity, dev_f32, dev_u8, dev_u16, host_f32,
                      host_u8, host_u16, params_dev, rand_bf16, say)
from error_feedback_quant_amd import inputs

pytestmark = pytest.mark.gpu

P, N = 4, 64 * 1024
S = N // P
G = 128
TILES = [(0, S), (3 * G, S - 5 * G), (S - G, G), (7 * G, 33 * G)]


@pytest.fixture(scope="module")
def echo():
    from error_feedback_quant_amd import echo as e
    assert torch.cuda.is_available()
    return e


def single_inputs():
    return [inputs.as_numpy_u16(inputs.single(r)) for r in range(P)]


def sentinel_f32(n):
    return np.full(n, np.float32(-7.5e-3), dtype=np.float32)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("mode", ["plain", "comp_err", "comp_negated_inplace", "err_only", "comp_only"])
def test_quantize_ef(echo, bits, mode):
    xs = single_inputs()
    rng = np.random.default_rng(11 + bits)
    cb = oracle.code_bytes(N, bits)
    for rank in range(P):
        for tb, tl in TILES:
            say("quantize_ef", bits, mode, rank, tb, tl)
            comp = (rng.standard_normal(N) * 0.05).astype(np.float32) if "comp" in mode else None
            want_codes = np.full(cb, 0xAB, np.uint8)
            want_params = np.full(2 * N // G, 0xCDCD, np.uint16)
            flags = 0
            if mode == "comp_negated_inplace":
                want_err = comp.copy()
                flags = oracle.ERR_NEGATED
            elif mode in ("comp_err", "err_only"):
                want_err = sentinel_f32(N)
            else:
                want_err = None
            oracle.quantize_ef(xs[rank], comp.copy() if comp is not None else None, N, P, rank, tb, tl, bits,
                               G, want_codes, want_params, want_err, flags)
            if mode == "comp_negated_inplace":
                # the oracle's err aliases its own comp copy on the GPU side too
                pass
            x_d = dev_u16(xs[rank])
            comp_d = dev_f32(comp) if comp is not None else None
            codes_d = dev_u8(np.full(cb, 0xAB, np.uint8))
            params_d = params_dev(N // G)
            if mode == "comp_negated_inplace":
                err_d = comp_d
            elif want_err is not None:
                err_d = dev_f32(sentinel_f32(N))
            else:
                err_d = None
            echo.echo_quantize_ef(x_d, comp_d, N, P, rank, tb, tl, bits, G, codes_d, params_d, err_d, flags)
            torch.cuda.synchronize()
            assert_bits_equal(host_u8(codes_d), want_codes, "codes")
            assert_bits_equal(host_u16(params_d), want_params, "params")
            if want_err is not None:
                assert_f32_parity(host_f32(err_d), want_err, "err")
                assert_bits_equal(host_f32(err_d), want_err, "err bits")


def oracle_push_all(xs, comps, bits):
    cb = oracle.code_bytes(N, bits)
    pc = [np.zeros(cb, np.uint8) for _ in range(P)]
    pp = [np.zeros(2 * N // G, np.uint16) for _ in range(P)]
    for r in range(P):
        oracle.quantize_ef(xs[r], comps[r] if comps else None, N, P, r, 0, S, bits, G, pc[r], pp[r], None)
    return pc, pp


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("with_comp", [False, True])
@pytest.mark.parametrize("Pn", [1, 2, 4, 8])
def test_reduce_segment(echo, bits, with_comp, Pn):
    n = Pn * 16 * G
    Sn = n // Pn
    xs = [rand_bf16(n, 30 + r + 10 * Pn) for r in range(Pn)]
    rng = np.random.default_rng(3 + Pn)
    comps = [(rng.standard_normal(n) * 0.05).astype(np.float32) for _ in range(Pn)] if with_comp else None
    cb = oracle.code_bytes(n, bits)
    pc = [np.zeros(cb, np.uint8) for _ in range(Pn)]
    pp = [np.zeros(2 * n // G, np.uint16) for _ in range(Pn)]
    for r in range(Pn):
        oracle.quantize_ef(xs[r], comps[r] if comps else None, n, Pn, r, 0, Sn, bits, G, pc[r], pp[r], None)
    pc_d = [dev_u8(a) for a in pc]
    pp_d = [dev_u16(a) for a in pp]
    for owner in range(Pn):
        for tb, tl in [(0, Sn), (G, Sn - 3 * G), (Sn - G, G)]:
            for negate in (0, oracle.ERR_NEGATED):
                say("reduce_segment", bits, with_comp, Pn, owner, tb, tl, negate)
                sc = np.full(cb, 0x5A, np.uint8)
                sp = np.full(2 * n // G, 0x1234, np.uint16)
                err = sentinel_f32(n)
                oracle.reduce_segment(xs[owner], comps[owner] if comps else None, pc, pp, Pn, owner, n, tb, tl,
                                      bits, G, sc, sp, err, negate)
                sc_d = dev_u8(np.full(cb, 0x5A, np.uint8))
                sp_d = params_dev(n // G, 0x1234)
                err_d = dev_f32(sentinel_f32(n))
                echo.echo_reduce_segment(dev_u16(xs[owner]), dev_f32(comps[owner]) if comps else None,
                                         [None if j == owner else pc_d[j] for j in range(Pn)],
                                         [None if j == owner else pp_d[j] for j in range(Pn)],
                                         Pn, owner, n, tb, tl, bits, G, sc_d, sp_d, err_d, negate)
                torch.cuda.synchronize()
                assert_bits_equal(host_u8(sc_d), sc, "sum codes")
                assert_bits_equal(host_u16(sp_d), sp, "sum params")
                assert_f32_parity(host_f32(err_d), err, "own err")
                assert_bits_equal(host_f32(err_d), err, "own err bits")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("odt", [oracle.OUT_F32, oracle.OUT_BF16])
def test_gather_dequant(echo, bits, odt):
    xs = single_inputs()
    pc, pp = oracle_push_all(xs, None, bits)
    cb = oracle.code_bytes(N, bits)
    sc = np.zeros(cb, np.uint8)
    sp = np.zeros(2 * N // G, np.uint16)
    for o in range(P):
        oracle.reduce_segment(xs[o], None, pc, pp, P, o, N, 0, S, bits, G, sc, sp, None)
    sc_d, sp_d = dev_u8(sc), dev_u16(sp)
    for tb, tl in TILES:
        say("gather_dequant", bits, odt, tb, tl)
        if odt == oracle.OUT_F32:
            want = sentinel_f32(N)
            out_d = dev_f32(sentinel_f32(N))
        else:
            want = np.full(N, 0xBEEF, np.uint16)
            out_d = dev_u16(np.full(N, 0xBEEF, np.uint16))
        oracle.gather_dequant(sc, sp, N, tb, tl, P, bits, G, want, odt)
        echo.echo_gather_dequant(sc_d, sp_d, N, tb, tl, P, bits, G, out_d, odt)
        torch.cuda.synchronize()
        if odt == oracle.OUT_F32:
            assert_f32_parity(host_f32(out_d), want, "out")
            assert_bits_equal(host_f32(out_d), want, "out bits")
        else:
            assert_bits_equal(host_u16(out_d), want, "bf16 out")


@pytest.mark.parametrize("alpha,beta", [(1.0, 0.0), (0.5, 0.25), (0.75, 0.1), (0.3, 1.0)])
@pytest.mark.parametrize("n", [0, 3, 4096, 4096 + 3, 1 << 20])
def test_compensate(echo, alpha, beta, n):
    say("compensate", alpha, beta, n)
    rng = np.random.default_rng(n + int(alpha * 100))
    e = (rng.standard_normal(n) * 0.01).astype(np.float32)
    M = (rng.standard_normal(n) * 0.02).astype(np.float32) if beta > 0 else None
    c = np.full(n, 9.0, np.float32)
    Mw = M.copy() if M is not None else None
    oracle.compensate(e, c, Mw, n, alpha, beta)
    e_d = dev_f32(e)
    c_d = dev_f32(np.full(n, 9.0, np.float32))
    M_d = dev_f32(M) if M is not None else None
    echo.echo_compensate(e_d, c_d, M_d, n, alpha, beta)
    torch.cuda.synchronize()
    assert_bits_equal(host_f32(c_d), c, "comp")
    if M is not None:
        assert_bits_equal(host_f32(M_d), Mw, "slow")
    # in place: comp_next aliasing err
    if n:
        e2 = dev_f32(e)
        M2 = dev_f32(M) if M is not None else None
        echo.echo_compensate(e2, e2, M2, n, alpha, beta)
        torch.cuda.synchronize()
        assert_bits_equal(host_f32(e2), c, "comp in place")


def edge_groups(bits):
    """fp32 groups (fed as comp with x = 0, so u = comp exactly) that hit the
    quantizer's special cases: an all-zero group, one-sided groups (z = 0 and
    z = Qm), binary16-subnormal and underflowing scales, an overflowing scale
    (clamped to 65504), exact ties in rint for codes and for the zero point,
    a scale that is an exact binary16 midpoint, and negative zeros."""
    Qm = (1 << bits) - 1
    rng = np.random.default_rng(5)
    gs = []
    gs.append(np.zeros(G))
    z = np.zeros(G); z[::3] = -0.0; gs.append(z)
    gs.append(np.abs(rng.standard_normal(G)))
    gs.append(-np.abs(rng.standard_normal(G)))
    gs.append(rng.standard_normal(G) * 1e-6)                 # subnormal binary16 scale
    gs.append(rng.standard_normal(G) * 1e-9)                 # scale underflows -> 2^-24
    gs.append(rng.standard_normal(G) * 1e7)                  # scale overflows -> 65504
    s = 2.0 ** -4                                            # exact scale, inv = 16
    lo, hi = -8.0 * s, (Qm - 8.0) * s                        # z = 8 exactly
    t = np.concatenate([[lo, hi], (np.arange(-8, Qm - 8) + 0.5) * s])  # every code tie
    gs.append(np.resize(t, G))
    lo = -8.5 * s; hi = lo + Qm * s                          # zero point tie at 8.5
    gs.append(np.resize(np.array([lo, hi, 0.0, 0.5 * s, -0.5 * s]), G))
    mid = 1.0 + 2.0 ** -11                                   # halfway between binary16 1 and 1+2^-10
    gs.append(np.resize(np.array([0.0, Qm * mid, 3.0, 7.25]), G))
    gs.append(np.resize(np.array([0.0, Qm * (1.0 + 3 * 2.0 ** -11)]), G))  # the other tie direction
    gs.append(np.full(G, 3.0))                               # constant nonzero group
    # exact ties with an odd integer zero point (z = 3: the zero point must be
    # added after rounding), and zero-point ties at 2.5 (-> 2) and 3.5 (-> 4)
    for z2 in (6, 5, 7):                                     # -lo/s = z2 / 2
        lo = -0.5 * z2 * s; hi = lo + Qm * s
        t = np.concatenate([[lo, hi], (np.arange(-z2, 2 * Qm - z2) * 0.5) * s])
        gs.append(np.resize(t, G))
    gs.append(np.resize(np.array([-3 * s, (Qm - 3) * s, 0.5 * s, 1.5 * s, -0.5 * s, 2.5 * s, -2.5 * s]), G))
    return [g.astype(np.float32) for g in gs]


@pytest.mark.parametrize("bits", [4, 8])
def test_quantizer_edge_groups(echo, bits):
    groups = edge_groups(bits)
    assert len(groups) % P == 0
    n = G * len(groups)              # the groups spread over the P segments
    Sn = n // P
    comp = np.concatenate(groups).astype(np.float32)
    x = np.zeros(n, np.uint16)
    for rank in range(P):
        say("edge groups", bits, rank)
        cb = oracle.code_bytes(n, bits)
        wc = np.zeros(cb, np.uint8); wp = np.zeros(2 * n // G, np.uint16); we = np.zeros(n, np.float32)
        oracle.quantize_ef(x, comp, n, P, rank, 0, Sn, bits, G, wc, wp, we)
        cd = dev_u8(np.zeros(cb, np.uint8)); pd = params_dev(n // G, 0); ed = dev_f32(np.zeros(n, np.float32))
        echo.echo_quantize_ef(dev_u16(x), dev_f32(comp), n, P, rank, 0, Sn, bits, G, cd, pd, ed, 0)
        torch.cuda.synchronize()
        assert_bits_equal(host_u8(cd), wc, "edge codes")
        assert_bits_equal(host_u16(pd), wp, "edge params")
        assert_bits_equal(host_f32(ed), we, "edge err")
    # the scale-tie groups really produced binary16 midpoints and clamps
    sc = wp[0::2]
    assert 0x7BFF in set(sc.tolist()) and 0x0001 in set(sc.tolist())


def variant_inputs(P, n, seed):
    """Partials mixing two-sided, one-sided, near-zero and exact-zero groups,
    plus a small fp32 compensation, so every quantizer meets its edge cases."""
    rng = np.random.default_rng(seed)
    xs = []
    for r in range(P):
        v = rng.standard_normal(n).astype(np.float32)
        blocks = v.reshape(-1, 128)
        blocks[1::7] = np.abs(blocks[1::7]) + 0.5          # positive, away from 0
        blocks[2::7] = -np.abs(blocks[2::7])               # non-positive
        blocks[3::7] *= 1e-3                               # near zero
        blocks[4::7, ::5] = 0.0                            # exact zeros inside a group
        blocks[5::11] = 0.0                                # all-zero rows
        xs.append(oracle.f32_to_bf16_bits(v))
    comps = [(rng.standard_normal(n) * 0.01).astype(np.float32) for _ in range(P)]
    return xs, comps


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [128, 256])
@pytest.mark.parametrize("quant", ["zero_aware", "naive", "symmetric", "mse"])
def test_quantizer_variants_each_step(echo, quant, group, bits):
    """Table 8's quantizers (full method, naive zero point, symmetric grid),
    the full method with its zero point searched, and group size 256: push,
    owner reduce and tail decode, step by step, bit for bit against the
    oracle, on whole segments and a ragged tile."""
    P = 4
    n = P * 256 * 19                      # 19 groups of 256 (38 rows) per segment
    Sn = n // P
    flag = echo.QUANTS[quant]
    xs, comps = variant_inputs(P, n, 7 + bits + group)
    cb = oracle.code_bytes(n, bits)
    ng = n // group
    for tb, tl in [(0, Sn), (group, Sn - 3 * group)]:
        say("variant push", quant, group, bits, tb, tl)
        pc_h = [np.full(cb, 0x3C, np.uint8) for _ in range(P)]
        pp_h = [np.full(2 * ng, 0x7777, np.uint16) for _ in range(P)]
        err_h = [np.full(n, np.float32(-1.5), np.float32) for _ in range(P)]
        pc_d = [dev_u8(a) for a in pc_h]
        pp_d = [dev_u16(a) for a in pp_h]
        err_d = [dev_f32(a) for a in err_h]
        for r in range(P):
            oracle.quantize_ef(xs[r], comps[r], n, P, r, tb, tl, bits, group, pc_h[r], pp_h[r], err_h[r], flag)
            echo.echo_quantize_ef(dev_u16(xs[r]), dev_f32(comps[r]), n, P, r, tb, tl, bits, group, pc_d[r],
                                  pp_d[r], err_d[r], flag)
        torch.cuda.synchronize()
        for r in range(P):
            assert_bits_equal(host_u8(pc_d[r]), pc_h[r], f"push codes {r}")
            assert_bits_equal(host_u16(pp_d[r]), pp_h[r], f"push params {r}")
            assert_bits_equal(host_f32(err_d[r]), err_h[r], f"push err {r}")
        say("variant reduce", quant, group, bits, tb, tl)
        sc_h = np.full(cb, 0x11, np.uint8)
        sp_h = np.full(2 * ng, 0x2222, np.uint16)
        sc_d, sp_d = dev_u8(sc_h), dev_u16(sp_h)
        oe_h = [np.full(n, np.float32(2.5), np.float32) for _ in range(P)]
        oe_d = [dev_f32(a) for a in oe_h]
        for o in range(P):
            oracle.reduce_segment(xs[o], comps[o], pc_h, pp_h, P, o, n, tb, tl, bits, group, sc_h, sp_h,
                                  oe_h[o], flag | oracle.ERR_NEGATED)
            echo.echo_reduce_segment(dev_u16(xs[o]), dev_f32(comps[o]), pc_d, pp_d, P, o, n, tb, tl, bits,
                                     group, sc_d, sp_d, oe_d[o], flag | echo.ERR_NEGATED)
        torch.cuda.synchronize()
        assert_bits_equal(host_u8(sc_d), sc_h, "sum codes")
        assert_bits_equal(host_u16(sp_d), sp_h, "sum params")
        for o in range(P):
            assert_bits_equal(host_f32(oe_d[o]), oe_h[o], f"owner err {o}")
        for odt in (oracle.OUT_F32, oracle.OUT_BF16):
            say("variant gather", quant, group, bits, tb, tl, odt)
            if odt == oracle.OUT_F32:
                want, out_d = sentinel_f32(n), dev_f32(sentinel_f32(n))
            else:
                want, out_d = np.full(n, 0xBEEF, np.uint16), dev_u16(np.full(n, 0xBEEF, np.uint16))
            oracle.gather_dequant(sc_h, sp_h, n, tb, tl, P, bits, group, want, odt)
            echo.echo_gather_dequant(sc_d, sp_d, n, tb, tl, P, bits, group, out_d, odt)
            torch.cuda.synchronize()
            got = host_f32(out_d) if odt == oracle.OUT_F32 else host_u16(out_d)
            assert_bits_equal(got, want, "decoded output")


@pytest.mark.parametrize("quant", ["naive", "symmetric", "mse"])
def test_quantizer_variant_edge_groups(echo, quant):
    """The edge groups of the full method's test, through each ablation."""
    flag = echo.QUANTS[quant]
    for bits in (4, 8):
        groups = edge_groups(bits)
        n = G * len(groups)
        Sn = n // P
        comp = np.concatenate(groups).astype(np.float32)
        x = np.zeros(n, np.uint16)
        for rank in range(P):
            say("variant edge groups", quant, bits, rank)
            cb = oracle.code_bytes(n, bits)
            wc = np.zeros(cb, np.uint8); wp = np.zeros(2 * n // G, np.uint16); we = np.zeros(n, np.float32)
            oracle.quantize_ef(x, comp, n, P, rank, 0, Sn, bits, G, wc, wp, we, flag)
            cd = dev_u8(np.zeros(cb, np.uint8)); pd = params_dev(n // G, 0); ed = dev_f32(np.zeros(n, np.float32))
            echo.echo_quantize_ef(dev_u16(x), dev_f32(comp), n, P, rank, 0, Sn, bits, G, cd, pd, ed, flag)
            torch.cuda.synchronize()
            assert_bits_equal(host_u8(cd), wc, "edge codes")
            assert_bits_equal(host_u16(pd), wp, "edge params")
            assert_bits_equal(host_f32(ed), we, "edge err")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("quant", ["zero_aware", "naive", "symmetric", "mse"])
def test_groups_zero_on_every_rank_through_every_step(echo, quant, bits):
    """Groups that are zero on every rank (+0 and -0 mixed), and groups that
    hold one constant on every rank, with no compensation: every push stores
    scale 0 for a zero group, the owner reduce decodes those peers' words and
    sums to an all-zero group, which it stores with scale 0 as well, and
    the tail decodes it; mixed with ordinary groups, bit for bit against the
    oracle at each step (the naive quantizer also stores a constant group
    with scale 0; the symmetric grid keeps its fixed zero point in the word)."""
    P = 4
    n = P * G * 18
    Sn = n // P
    flag = echo.QUANTS[quant]
    rng = np.random.default_rng(41 + bits)
    xs = []
    for r in range(P):
        v = rng.standard_normal(n).astype(np.float32)
        b = v.reshape(-1, G)
        b[0::3] = 0.0                                      # zero on every rank
        b[0::9, ::2] = -0.0                                # with negative zeros in some
        b[1::6] = 0.75                                     # one constant on every rank
        xs.append(oracle.f32_to_bf16_bits(v))
    cb = oracle.code_bytes(n, bits)
    ng = n // G
    pc_h = [np.full(cb, 0x3C, np.uint8) for _ in range(P)]
    pp_h = [np.full(2 * ng, 0x7777, np.uint16) for _ in range(P)]
    pc_d = [dev_u8(a) for a in pc_h]
    pp_d = [dev_u16(a) for a in pp_h]
    say("zero groups push", quant, bits)
    for r in range(P):
        oracle.quantize_ef(xs[r], None, n, P, r, 0, Sn, bits, G, pc_h[r], pp_h[r], None, flag)
        echo.echo_quantize_ef(dev_u16(xs[r]), None, n, P, r, 0, Sn, bits, G, pc_d[r], pp_d[r], None, flag)
    torch.cuda.synchronize()
    for r in range(P):
        assert_bits_equal(host_u8(pc_d[r]), pc_h[r], f"push codes {r}")
        assert_bits_equal(host_u16(pp_d[r]), pp_h[r], f"push params {r}")
        pushed = np.concatenate([pp_h[r][2 * (s * Sn // G):2 * ((s + 1) * Sn // G)] for s in range(P) if s != r])
        assert np.count_nonzero(pushed[0::2] == 0) >= 3 * (Sn // G) // 3       # scale 0: the zero groups
    say("zero groups reduce", quant, bits)
    sc_h = np.full(cb, 0x11, np.uint8)
    sp_h = np.full(2 * ng, 0x2222, np.uint16)
    sc_d, sp_d = dev_u8(sc_h), dev_u16(sp_h)
    for o in range(P):
        oracle.reduce_segment(xs[o], None, pc_h, pp_h, P, o, n, 0, Sn, bits, G, sc_h, sp_h, None, flag)
        echo.echo_reduce_segment(dev_u16(xs[o]), None, [None if j == o else pc_d[j] for j in range(P)],
                                 [None if j == o else pp_d[j] for j in range(P)], P, o, n, 0, Sn, bits, G,
                                 sc_d, sp_d, None, flag)
    torch.cuda.synchronize()
    assert_bits_equal(host_u8(sc_d), sc_h, "sum codes")
    assert_bits_equal(host_u16(sp_d), sp_h, "sum params")
    assert np.count_nonzero(sp_h[0::2] == 0) >= ng // 3
    for odt in (oracle.OUT_F32, oracle.OUT_BF16):
        say("zero groups gather", quant, bits, odt)
        if odt == oracle.OUT_F32:
            want, out_d = sentinel_f32(n), dev_f32(sentinel_f32(n))
        else:
            want, out_d = np.full(n, 0xBEEF, np.uint16), dev_u16(np.full(n, 0xBEEF, np.uint16))
        oracle.gather_dequant(sc_h, sp_h, n, 0, Sn, P, bits, G, want, odt)
        echo.echo_gather_dequant(sc_d, sp_d, n, 0, Sn, P, bits, G, out_d, odt)
        torch.cuda.synchronize()
        got = host_f32(out_d) if odt == oracle.OUT_F32 else host_u16(out_d)
        assert_bits_equal(got, want, "decoded output")


def search_groups(bits, group, count, seed):
    """Groups whose searched zero point differs from the closed form (chosen
    by the oracle), mixed with groups where it does not: one-decimal values
    (the shape of Fig. 4's example) and Laplace draws."""
    rng = np.random.default_rng(seed)
    moved, kept = [], []
    while len(moved) < count // 2 or len(kept) < count - count // 2:
        if rng.random() < 0.5:
            v = (rng.integers(-40, 41, size=group) / 10).astype(np.float32)
            v[rng.integers(0, group, size=group - 4)] = 0.0     # few nonzeros: the span decides
        else:
            v = (rng.laplace(size=group) * 10.0 ** rng.uniform(-3, 2)).astype(np.float32)
        _, _, zh = oracle.quantize_group(v, bits, "mse")
        _, _, zh0 = oracle.quantize_group(v, bits)
        (moved if zh != zh0 else kept).append(v)
    return moved[:count // 2] + kept[:count - count // 2]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [128, 256])
def test_zero_point_search_moves_the_zero_point(echo, bits, group):
    """The searched zero point through push and owner reduce, on groups where
    it differs from the closed form (half of them) and where it does not,
    bit for bit against the oracle."""
    P, count = 4, 32
    groups = search_groups(bits, group, count, 300 + bits + group)
    n = group * count
    Sn = n // P
    comp = np.concatenate(groups).astype(np.float32)
    x = np.zeros(n, np.uint16)
    cb = oracle.code_bytes(n, bits)
    flag = echo.QUANT_MSE
    pc_h, pp_h, pc_d, pp_d = [], [], [], []
    for rank in range(P):
        say("zero-point search push", bits, group, rank)
        wc = np.zeros(cb, np.uint8); wp = np.zeros(2 * n // group, np.uint16); we = np.zeros(n, np.float32)
        oracle.quantize_ef(x, comp, n, P, rank, 0, Sn, bits, group, wc, wp, we, flag)
        cd = dev_u8(np.zeros(cb, np.uint8)); pd = params_dev(n // group, 0); ed = dev_f32(np.zeros(n, np.float32))
        echo.echo_quantize_ef(dev_u16(x), dev_f32(comp), n, P, rank, 0, Sn, bits, group, cd, pd, ed, flag)
        torch.cuda.synchronize()
        assert_bits_equal(host_u8(cd), wc, "search codes")
        assert_bits_equal(host_u16(pd), wp, "search params")
        assert_bits_equal(host_f32(ed), we, "search err")
        pc_h.append(wc); pp_h.append(wp); pc_d.append(cd); pp_d.append(pd)
    # the owner's sum of the same groups, requantized with the search
    say("zero-point search reduce", bits, group)
    sc_h = np.zeros(cb, np.uint8); sp_h = np.zeros(2 * n // group, np.uint16)
    sc_d, sp_d = dev_u8(sc_h), dev_u16(sp_h)
    for o in range(P):
        oracle.reduce_segment(x, comp, pc_h, pp_h, P, o, n, 0, Sn, bits, group, sc_h, sp_h, None, flag)
        echo.echo_reduce_segment(dev_u16(x), dev_f32(comp), pc_d, pp_d, P, o, n, 0, Sn, bits, group, sc_d,
                                 sp_d, None, flag)
    torch.cuda.synchronize()
    assert_bits_equal(host_u8(sc_d), sc_h, "search sum codes")
    assert_bits_equal(host_u16(sp_d), sp_h, "search sum params")
