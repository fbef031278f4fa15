"""Host-side checks of bench.py (CPU only): the byte formula it divides by is
the sum of the per-kernel algorithmic bytes, and the one-GPU contract."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def kernel_bytes(P, bits, group, ef_state, out_bytes):
    """Per message element per rank, kernel by kernel: the push touches the
    P-1 segments a rank does not own, the reduce its own segment (reading P-1
    peer code sets and writing one), the tail the whole message."""
    kb = bits / 8 + 4 / group
    push = (P - 1) / P * (2 + ef_state + kb)
    reduce = (2 + ef_state + (P - 1) * kb + kb) / P
    tail = kb + out_bytes
    return push + reduce + tail


@pytest.mark.parametrize("P", [1, 2, 4, 8])
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [128, 256])
def test_call_bytes_are_the_sum_of_kernel_bytes(P, bits, group):
    for ef, two, state in ((False, False, 0), (True, False, 8), (True, True, 16)):
        for out_bytes in (2, 4):
            got = bench.bytes_per_elem(P, bits, ef, out_bytes, group, two)
            assert got == pytest.approx(kernel_bytes(P, bits, group, state, out_bytes), rel=1e-12)


def test_headline_bytes():
    # 1 GiB message, P = 4, 4-bit, g = 128, feedback on, bf16 out: 13.46 B/elem/rank
    assert bench.bytes_per_elem(4, 4, True, 2) == pytest.approx(13.4609375)
    assert 4 * bench.N_1GIB * bench.bytes_per_elem(4, 4, True, 2) == 28907143168
    # the push launch of one rank: 3 * 2^27 elements
    assert 3 * (bench.N_1GIB // 4) * bench.push_bytes_per_elem(4, True) == 4240441344


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baselines_report_the_contract_fields():
    """The oracle baselines (single-threaded on a sample of every segment,
    and whole calls in host threads) carry value, unit, cores, kind and a
    sample description, on a small message here."""
    n = 4 * 64 * 256
    single = bench.cpu_baseline_sampled(4, n, 4, True, True)
    threaded = bench.cpu_baseline_threaded_full(4, n, 4, True, True, 2)
    for d in (single, threaded):
        assert set(("value", "unit", "cores", "kind", "sample", "elements_per_s")) <= set(d)
        assert d["unit"] == "GB/s" and d["kind"] == "oracle" and d["value"] > 0
    assert single["cores"] == 1 and "cpu" in single
    assert threaded["cores"] == 2


def test_two_timescale_state_bytes():
    """The fused two-timescale update reads c and M and writes c' and M':
    16 bytes of state per element instead of classic feedback's 8."""
    fused = bench.bytes_per_elem(4, 4, True, 2, 128, True)
    assert fused == pytest.approx(2 + 2 + 16 + 0.53125 * (3 - 0.25))
