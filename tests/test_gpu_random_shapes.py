"""Seeded random shapes through the push, owner-reduce and tail entry points,
each against the oracle.

The fixed-shape tests use one message size. Here every case draws its own:
- P in 1..8 and a segment of 1..700 groups, so the kernels' blocks end at many
  different places;
- a group of 128 or 256, 4 or 8 bits, and one of the three quantizers;
- a tile inside the segment (whole groups);
- feedback off, an error output, or the negated error written in place;
- bf16 or fp32 output;
- one of four input distributions: normal, Laplace, one-sided, or mostly
  zeros (groups whose range is one-sided or empty).

Every case runs through the C ABI. Codes, parameters, errors and outputs are
compared bit for bit. Buffers start with a sentinel on both sides, so a write
outside the tile shows. Each step takes the oracle's outputs of the step
before as its inputs, so each kernel is checked on its own.
"""
import numpy as np
import pytest
import torch

import oracle
from _helpers import (assert_bits_equal, dev_f32, dev_u8, dev_u16, host_f32, host_u8, host_u16, params_dev,
                      say)

pytestmark = pytest.mark.gpu

N_CASES = 24


@pytest.fixture(scope="module")
def echo():
    from error_feedback_quant_amd import echo as e
    assert torch.cuda.is_available()
    return e


def draw(i):
    rng = np.random.default_rng(9000 + i)
    P = int(rng.integers(1, 9))
    G = int(rng.choice([128, 256]))
    groups = int(rng.integers(1, 701))
    g0 = int(rng.integers(0, groups))
    gl = int(rng.integers(1, groups - g0 + 1))
    return dict(P=P, G=G, S=groups * G, tb=g0 * G, tl=gl * G, bits=int(rng.choice([4, 8])),
                quant=str(rng.choice(["zero_aware", "naive", "symmetric", "mse"])),
                ef=str(rng.choice(["off", "err", "negated"])),
                odt=int(rng.choice([oracle.OUT_F32, oracle.OUT_BF16])),
                dist=str(rng.choice(["normal", "laplace", "one_sided", "sparse"])), seed=9100 + i)


def message(rng, n, dist):
    if dist == "normal":
        v = rng.standard_normal(n)
    elif dist == "laplace":
        v = rng.laplace(0.0, 1.0, n)
    elif dist == "one_sided":
        v = np.abs(rng.standard_normal(n)) * rng.choice([-1.0, 1.0])
    else:
        v = rng.standard_normal(n) * (rng.random(n) < 0.02)
    return oracle.f32_to_bf16_bits(v.astype(np.float32))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_shape_steps_match_oracle(echo, case):
    c = draw(case)
    P, G, S, tb, tl, bits = c["P"], c["G"], c["S"], c["tb"], c["tl"], c["bits"]
    n = P * S
    cb = oracle.code_bytes(n, bits)
    rng = np.random.default_rng(c["seed"])
    xs = [message(rng, n, c["dist"]) for _ in range(P)]
    comps = ([(rng.standard_normal(n) * 0.05).astype(np.float32) for _ in range(P)]
             if c["ef"] != "off" else [None] * P)
    flags = oracle.QUANTS[c["quant"]] | (oracle.ERR_NEGATED if c["ef"] == "negated" else 0)
    say("random shape", case, c)

    # push: every rank, its non-owned segments, inside the tile
    pc, pp = [], []
    for r in range(P):
        codes = np.full(cb, 0xAB, np.uint8)
        params = np.full(2 * n // G, 0xCDCD, np.uint16)
        err = None if c["ef"] == "off" else (comps[r].copy() if c["ef"] == "negated"
                                             else np.full(n, -7.5e-3, np.float32))
        oracle.quantize_ef(xs[r], None if comps[r] is None else comps[r].copy(), n, P, r, tb, tl, bits, G,
                           codes, params, err, flags)
        comp_d = None if comps[r] is None else dev_f32(comps[r])
        err_d = comp_d if c["ef"] == "negated" else (None if err is None else dev_f32(np.full(n, -7.5e-3, np.float32)))
        codes_d, params_d = dev_u8(np.full(cb, 0xAB, np.uint8)), params_dev(n // G)
        echo.echo_quantize_ef(dev_u16(xs[r]), comp_d, n, P, r, tb, tl, bits, G, codes_d, params_d, err_d, flags)
        torch.cuda.synchronize()
        assert_bits_equal(host_u8(codes_d), codes, f"push codes, rank {r}")
        assert_bits_equal(host_u16(params_d), params, f"push params, rank {r}")
        if err is not None:
            assert_bits_equal(host_f32(err_d), err, f"push error, rank {r}")
        pc.append(codes)
        pp.append(params)

    # owner reduce over the same tile of its segment, from the oracle's push codes
    pc_d = [dev_u8(a) for a in pc]
    pp_d = [dev_u16(a) for a in pp]
    sc = np.full(cb, 0x5A, np.uint8)
    sp = np.full(2 * n // G, 0x1234, np.uint16)
    sc_d, sp_d = dev_u8(sc.copy()), params_dev(n // G, 0x1234)
    for o in range(P):
        err = None if c["ef"] == "off" else (comps[o].copy() if c["ef"] == "negated"
                                             else np.full(n, -7.5e-3, np.float32))
        oracle.reduce_segment(xs[o], None if comps[o] is None else comps[o].copy(), pc, pp, P, o, n, tb, tl,
                              bits, G, sc, sp, err, flags)
        comp_d = None if comps[o] is None else dev_f32(comps[o])
        err_d = comp_d if c["ef"] == "negated" else (None if err is None else dev_f32(np.full(n, -7.5e-3, np.float32)))
        echo.echo_reduce_segment(dev_u16(xs[o]), comp_d, [None if j == o else pc_d[j] for j in range(P)],
                                 [None if j == o else pp_d[j] for j in range(P)], P, o, n, tb, tl, bits, G,
                                 sc_d, sp_d, err_d, flags)
        torch.cuda.synchronize()
        if err is not None:
            assert_bits_equal(host_f32(err_d), err, f"reduce error, owner {o}")
    assert_bits_equal(host_u8(sc_d), sc, "sum codes")
    assert_bits_equal(host_u16(sp_d), sp, "sum params")

    # tail: the tile of every segment, from the oracle's sum codes
    if c["odt"] == oracle.OUT_F32:
        want, out_d = np.full(n, -7.5e-3, np.float32), dev_f32(np.full(n, -7.5e-3, np.float32))
    else:
        want, out_d = np.full(n, 0xBEEF, np.uint16), dev_u16(np.full(n, 0xBEEF, np.uint16))
    oracle.gather_dequant(sc, sp, n, tb, tl, P, bits, G, want, c["odt"])
    echo.echo_gather_dequant(dev_u8(sc), dev_u16(sp), n, tb, tl, P, bits, G, out_d, c["odt"])
    torch.cuda.synchronize()
    got = host_f32(out_d) if c["odt"] == oracle.OUT_F32 else host_u16(out_d)
    assert_bits_equal(got, want, "tail output")
