"""The oracle's pins catch plausible mistakes (CPU only).

Each case below plants one mistake in a scratch copy of oracle/echo_ref.c,
builds it with the oracle's own flags, and runs the pins named beside it
against that library (through ECHO_ORACLE_LIB, in a child pytest).  Every
planted mistake must make at least one of them fail; an unmutated scratch
build must pass all of them (the control), so a broken harness cannot pass
for a caught mistake.

The mistakes are the ones a reader of the Echo paper card (Table 8, Fig. 2(a),
appendix Fig. 4) and of the PhantomByte article ("The cancellation rule")
could plausibly make when writing the oracle: in the quantizer (tie rule,
side of the zero-point add, range not widened to 0, 2^b levels instead of
2^b - 1, codes measured from the range start), in the ablations (the naive
range widened to 0, the symmetric grid over all 2^b - 1 steps), in the
zero-point search (tie rule, objective without the rounding part, the last
zero point skipped), in the call structure (wrong
segment pushed, owner's term or compensation dropped or taken from a peer,
summation order), in the compensator (sign, slow-memory input, release
taken from the updated memory or at rate 1 - beta), in decoding and packing
(off-by-one, nibble order, neighbouring group's parameters), in
the error's sign, and in the number formats (binary16 and bfloat16 ties,
missing scale clamp).
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

EX = "tests/test_oracle_exact_cases.py::"
QZ = "tests/test_oracle_quantizer.py::"
AR = "tests/test_oracle_allreduce.py::"
FM = "tests/test_oracle_formats.py::"

# (name, [(text in echo_ref.c, replacement, which occurrence)], pins expected to catch it)
MUTATIONS = [
    ("zero-aware zero point rounds half away from zero",
     [("rintf(-lo * inv)", "roundf(-lo * inv)", 0)],
     [EX + "test_zero_aware_4bit_tie_on_the_zero_point_and_codes"]),
    ("zero-aware codes round half away from zero",
     [("rintf(v[i] * inv) + (double)z", "roundf(v[i] * inv) + (double)z", 0)],
     [EX + "test_zero_aware_4bit_ties_with_an_odd_zero_point_neighbour"]),
    ("naive codes round half away from zero",
     [("rintf(v[i] * inv + zf)", "roundf(v[i] * inv + zf)", 0)],
     [EX + "test_naive_zero_point_ties"]),
    ("symmetric codes round half away from zero",
     [("rintf(v[i] * inv) + (double)mid", "roundf(v[i] * inv) + (double)mid", 0)],
     [EX + "test_symmetric_grid_ties"]),
    ("integer zero point added before rounding",
     [("(double)rintf(v[i] * inv) + (double)z", "(double)rintf(v[i] * inv + (float)z)", 0)],
     [EX + "test_zero_aware_4bit_code_ties_with_an_odd_zero_point"]),
    ("naive zero point added after rounding",
     [("rintf(v[i] * inv + zf)", "rintf(v[i] * inv) + zf", 0)],
     [EX + "test_naive_zero_point_ties"]),
    ("codes measured from the range start instead of the zero point",
     [("(double)rintf(v[i] * inv) + (double)z", "(double)rintf((v[i] - lo) * inv)", 0)],
     [QZ + "test_brute_force_one_decimal_lattice"]),
    ("zero-aware range not widened to contain 0",
     [("float lo = 0.0f, hi = 0.0f;", "float lo = v[0], hi = v[0];", 0)],
     [QZ + "test_hand_worked_groups", QZ + "test_brute_force_random_magnitudes"]),
    ("2^b levels instead of 2^b - 1",
     [("scale_bits((hi - lo) / (float)Qm)", "scale_bits((hi - lo) / (float)(Qm + 1))", 0)],
     [QZ + "test_hand_worked_groups"]),
    ("push quantizes the wrong segment",
     [("if (s == rank) continue;", "if (s == (rank + 1) % P) continue;", 0)],
     [AR + "test_sum_reveals_the_injected_error"]),
    ("owner's own term dropped from the sum",
     [("if (j == owner) {", "if (j == owner && 0) {", 0)],
     [AR + "test_sum_reveals_the_injected_error"]),
    ("owner's compensation dropped",
     [("t = own_comp ? xv + own_comp[base + i] : xv;", "t = xv;", 0)],
     [AR + "test_depth_chain_closed_form"]),
    ("owner's compensation taken from a peer",
     [("float* c = ef ? comp[o] : NULL;", "float* c = ef ? comp[(o + 1) % P] : NULL;", 0)],
     [AR + "test_depth_chain_closed_form"]),
    ("owner's sum in reverse rank order",
     [("for (int j = 0; j < P; ++j) {\n                float t;", "for (int j = P - 1; j >= 0; --j) {\n                float t;", 0),
      ("sum = (j == 0) ? t : sum + t;", "sum = (j == P - 1) ? t : sum + t;", 0)],
     [EX + "test_owner_sum_in_rank_order"]),
    ("compensation returned with the wrong sign",
     [("comp_next[i] = -(a + b);", "comp_next[i] = (a + b);", 0)],
     [AR + "test_compensator_conserves_the_error_debt"]),
    ("slow memory fed alpha*e instead of (1 - alpha)*e",
     [("float m2 = oma * e;", "float m2 = alpha * e;", 0)],
     [AR + "test_compensator_conserves_the_error_debt"]),
    ("compensation computed from the already updated slow memory",
     [("""            float b = beta * M;
            comp_next[i] = -(a + b);
            float m1 = omb * M;
            float m2 = oma * e;
            slow[i] = m1 + m2;""", """            float m1 = omb * M;
            float m2 = oma * e;
            slow[i] = m1 + m2;
            float b = beta * slow[i];
            comp_next[i] = -(a + b);""", 0)],
     [AR + "test_compensator_conserves_the_error_debt"]),
    ("slow memory released at rate 1 - beta instead of beta",
     [("float b = beta * M;", "float b = omb * M;", 0)],
     [AR + "test_compensator_conserves_the_error_debt"]),
    ("decoder off by one code",
     [("float d = (float)q - echo_ref_f16_to_f32(zero_h);", "float d = (float)(q + 1) - echo_ref_f16_to_f32(zero_h);", 0)],
     [QZ + "test_hand_worked_groups"]),
    ("nibble order swapped (pack and unpack alike)",
     [("return (i & 1) ? (byte >> 4) : (byte & 0x0F);", "return (i & 1) ? (byte & 0x0F) : (byte >> 4);", 0),
      ("if (i & 1) *byte = (uint8_t)((*byte & 0x0F) | (q << 4));",
       "if (!(i & 1)) *byte = (uint8_t)((*byte & 0x0F) | (q << 4));", 0)],
     [EX + "test_packed_nibbles_hold_the_even_element_low"]),
    ("decode reads the neighbouring group's parameters at a group's end",
     [("int64_t grp = i / g;", "int64_t grp = (i + 1) / g;", 0)],
     [AR + "test_sum_reveals_the_injected_error"]),
    ("error written as u - Q_hat(u)",
     [("float e = echo_ref_dequant(qs[i], sh, zh) - u[i];", "float e = u[i] - echo_ref_dequant(qs[i], sh, zh);", 0)],
     [AR + "test_sum_reveals_the_injected_error"]),
    ("binary16 ties rounded away from zero",
     [("(rem == half && (N & 1u))", "(rem == half)", 0)],
     [FM + "test_f16_sampled_everywhere_including_signs_and_specials"]),
    ("bfloat16 output truncated",
     [("if (rem > 0x8000u || (rem == 0x8000u && (up & 1u))) up += 1u;", "(void)rem;", 0)],
     [FM + "test_bf16_round_to_nearest_even_matches_torch"]),
    ("zero-point search keeps the larger zero point on ties",
     [("if (z == 0 || d < best) {", "if (z == 0 || d <= best) {", 0)],
     ["tests/test_oracle_quantizer_mse.py::test_hand_worked_tie_takes_the_smaller_zero_point"]),
    ("zero-point search scores the clamped codes without the rounding part",
     [("d += (c - r) * (c + r - 2.0 * (double)t);", "d += (c - r) * (c - r);", 0)],
     ["tests/test_oracle_quantizer_mse.py::test_exhaustive_exact_search_on_tiny_groups"]),
    ("naive zero point with the range widened to contain 0",
     [("float lo = v[0], hi = v[0];", "float lo = fminf(v[0], 0.0f), hi = fmaxf(v[0], 0.0f);", 0)],
     ["tests/test_oracle_quantizer_variants.py::test_brute_force_one_decimal_lattice",
      "tests/test_oracle_quantizer_variants.py::test_brute_force_random_magnitudes"]),
    ("symmetric grid scaled over 2^b - 1 levels instead of 2^(b-1) - 1",
     [("scale_bits(a / (float)Qh)", "scale_bits(a / (float)Qm)", 0)],
     ["tests/test_oracle_quantizer_variants.py::test_brute_force_one_decimal_lattice",
      "tests/test_oracle_quantizer_variants.py::test_symmetric_round_trip_and_zero"]),
    ("zero-point search stopping one short of Qm",
     [("for (int z = 0; z <= Qm; ++z) {", "for (int z = 0; z < Qm; ++z) {", 0)],
     ["tests/test_oracle_quantizer_mse.py::test_exhaustive_exact_search_on_tiny_groups"]),
    ("zero binary16 scale not clamped to 2^-24",
     [("if (sh == 0x0000u) sh = 0x0001u;", "if (0) sh = 0x0001u;", 0)],
     [QZ + "test_scale_clamps_and_all_zero_group"]),
]


def mutate(src: str, edits) -> str:
    for old, new, which in edits:
        pos = -1
        for _ in range(which + 1):
            pos = src.find(old, pos + 1)
            assert pos >= 0, f"mutation site not found: {old!r}"
        src = src[:pos] + new + src[pos + len(old):]
    return src


def build(src: str, path_c: str, path_so: str):
    with open(path_c, "w") as f:
        f.write(src)
    subprocess.run(["gcc", *oracle.CFLAGS, path_c, "-o", path_so, "-lm"], check=True,
                   capture_output=True)


def run_pins(lib: str, tests):
    env = dict(os.environ, ECHO_ORACLE_LIB=lib, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, (r.stdout or "")[-2000:] + (r.stderr or "")[-1000:]


def test_every_planted_mistake_fails_a_pin():
    src = open(oracle.SRC).read()
    with tempfile.TemporaryDirectory() as tmp:
        # control: the unmutated source, built the same way, passes every pin used below
        ctrl = os.path.join(tmp, "control.so")
        build(src, os.path.join(tmp, "control.c"), ctrl)
        all_pins = sorted({t for _, _, ts in MUTATIONS for t in ts})
        rc, out = run_pins(ctrl, all_pins)
        assert rc == 0, f"control build fails its pins:\n{out}"

        def one(k):
            name, edits, tests = MUTATIONS[k]
            so = os.path.join(tmp, f"m{k}.so")
            build(mutate(src, edits), os.path.join(tmp, f"m{k}.c"), so)
            rc, out = run_pins(so, tests)
            return name, rc, out

        with ThreadPoolExecutor(max_workers=4) as pool:
            results = list(pool.map(one, range(len(MUTATIONS))))
    survivors = [(name, rc, out) for name, rc, out in results if rc == 0 or rc in (4, 5)]
    assert not survivors, "mistakes no pin catches: " + "; ".join(f"{n} (rc {rc})" for n, rc, _ in survivors)
