"""libecho's C ABI without a GPU: the library loads, exports every function
include/echo.h declares, and rejects bad arguments on the host (these calls
return before anything would be enqueued, so no device is needed)."""
import ctypes

import pytest

from error_feedback_quant_amd import echo


def test_every_declared_function_is_exported():
    names = echo.declared_functions()
    expected = {"echo_quantize_ef", "echo_reduce_segment", "echo_gather_dequant", "echo_compensate",
                "echo_gemm_quantize_ef", "echo_allreduce_sim", "echo_allreduce_sim_workspace_bytes",
                "echo_allreduce_sim_noalloc", "echo_noalloc_scratch_bytes",
                "echo_status_str", "echo_last_hip_error"}
    assert expected <= set(names), names
    L = echo.lib()
    for nm in names:
        assert hasattr(L, nm), nm


def test_status_strings():
    L = echo.lib()
    for rc in (0, -1, -2, -3, -4, -5, -6):
        assert L.echo_status_str(rc) != b"unknown status"
    assert L.echo_status_str(123) == b"unknown status"
    assert L.echo_last_hip_error() == 0


FAKE = 1 << 20          # a 16-byte-aligned non-null address that is never dereferenced here


@pytest.fixture(autouse=True)
def _host_only():
    """These calls pass made-up pointers and rely on the host checks failing
    first; never let one reach a real device."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only argument checks (a GPU is visible)")


def rc_of(fn, *args, **kw):
    try:
        fn(*args, **kw)
        return 0
    except echo.EchoError as e:
        return e.rc


def test_quantize_ef_argument_checks():
    n, P = 4 * 1024, 4
    q = lambda **kw: rc_of(echo.echo_quantize_ef, kw.get("x", FAKE), kw.get("comp", None), kw.get("n", n),
                           kw.get("P", P), kw.get("rank", 0), kw.get("tb", 0), kw.get("tl", 128),
                           kw.get("bits", 4), kw.get("group", 128), kw.get("codes", FAKE),
                           kw.get("params", FAKE), kw.get("err", None), kw.get("flags", 0), stream=0)
    assert q(bits=3) == echo.EUNSUP
    assert q(group=64) == echo.EUNSUP
    assert q(P=0) == echo.EINVAL and q(P=9) == echo.EINVAL
    assert q(rank=4) == echo.EINVAL and q(rank=-1) == echo.EINVAL
    assert q(n=n + 128) == echo.ESHAPE and q(n=-512) == echo.ESHAPE
    assert q(tb=64) == echo.ESHAPE and q(tl=100) == echo.ESHAPE
    assert q(tb=1024, tl=128) == echo.ESHAPE          # past the segment end (S = 1024)
    big = (1 << 63) - 128                               # a multiple of 128 near INT64_MAX
    assert q(tb=big, tl=big) == echo.ESHAPE and q(tb=128, tl=big) == echo.ESHAPE
    assert q(x=None) == echo.EINVAL and q(codes=None) == echo.EINVAL
    assert q(x=FAKE + 8) == echo.EALIGN and q(comp=FAKE + 4) == echo.EALIGN
    assert q(flags=8) == echo.EINVAL and q(flags=6) == echo.EINVAL   # unknown bit; both ablations
    assert q(flags=18) == echo.EINVAL and q(flags=20) == echo.EINVAL and q(flags=32) == echo.EINVAL
    assert q(n=1 << 35, P=4) == echo.ESHAPE             # beyond the 2^34 limit
    # empty work is a successful no-op (nothing to enqueue)
    assert q(tl=0) == 0 and q(n=0, tl=0) == 0 and q(P=1, tl=128) == 0


def test_gemm_quantize_ef_argument_checks():
    M, N, K, P = 512, 256, 128, 4
    g = lambda **kw: rc_of(echo.echo_gemm_quantize_ef, kw.get("a", FAKE), kw.get("w", FAKE), kw.get("M", M),
                           kw.get("N", N), kw.get("K", K), kw.get("comp", None), kw.get("P", P),
                           kw.get("rank", 0), kw.get("bits", 4), kw.get("group", 128), kw.get("codes", FAKE),
                           kw.get("params", FAKE), kw.get("err", None), kw.get("x_out", FAKE),
                           kw.get("flags", 0), stream=0)
    assert g(bits=2) == echo.EUNSUP and g(group=64) == echo.EUNSUP
    assert g(P=0) == echo.EINVAL and g(P=9) == echo.EINVAL and g(rank=4) == echo.EINVAL
    assert g(N=N + 128) == echo.ESHAPE                # N not a multiple of 256
    assert g(K=K + 32) == echo.ESHAPE and g(K=0) == echo.ESHAPE
    assert g(M=384) == echo.ESHAPE                    # M not a multiple of 256
    assert g(M=256, P=3) == echo.ESHAPE               # M not a multiple of P
    assert g(M=-128) == echo.ESHAPE
    assert g(M=1 << 22, N=1 << 13) == echo.ESHAPE     # M * N beyond 2^34
    assert g(K=1 << 22) == echo.ESHAPE                # a 256-row operand panel would reach 2^31 bytes
    assert g(a=None) == echo.EINVAL and g(w=None) == echo.EINVAL and g(x_out=None) == echo.EINVAL
    assert g(codes=None) == echo.EINVAL
    assert g(a=FAKE + 2) == echo.EALIGN and g(err=FAKE + 4) == echo.EALIGN
    assert g(flags=32) == echo.EINVAL and g(flags=6) == echo.EINVAL and g(flags=18) == echo.EINVAL
    assert g(M=0) == 0 and g(N=0) == 0                # nothing to compute


def test_reduce_gather_compensate_argument_checks():
    n, P = 4 * 1024, 4
    peers = [FAKE] * P
    r = lambda **kw: rc_of(echo.echo_reduce_segment, FAKE, None, kw.get("pc", peers), kw.get("pp", peers),
                           kw.get("P", P), kw.get("owner", 1), n, 0, 128, kw.get("bits", 4), 128, FAKE, FAKE,
                           None, 0, stream=0)
    assert r(owner=4) == echo.EINVAL
    assert r(bits=2) == echo.EUNSUP
    assert r(pc=[FAKE, FAKE, None, FAKE]) == echo.EINVAL        # a peer's codes missing
    assert r(pc=[FAKE, FAKE, FAKE + 2, FAKE]) == echo.EALIGN
    g = lambda **kw: rc_of(echo.echo_gather_dequant, FAKE, FAKE, n, 0, 128, P, 4, 128,
                           kw.get("out", FAKE), kw.get("odt", 0), stream=0)
    assert g(odt=7) == echo.EUNSUP and g(out=None) == echo.EINVAL
    c = lambda a, b, slow: rc_of(echo.echo_compensate, FAKE, FAKE, slow, 1024, a, b, stream=0)
    assert c(0.0, 0.0, None) == echo.EINVAL          # alpha must be > 0
    assert c(0.5, 0.0, None) == echo.EINVAL          # alpha < 1 needs a slow memory
    assert c(1.0, 0.5, None) == echo.EINVAL          # beta > 0 needs a slow memory
    assert c(1.0, 0.0, FAKE) == echo.EINVAL          # and beta = 0 takes none
    assert c(1.0, 1.5, FAKE) == echo.EINVAL
    assert rc_of(echo.echo_compensate, FAKE, FAKE, None, -4, 1.0, 0.0, stream=0) == echo.ESHAPE


def test_sim_argument_checks_and_workspace_size():
    P, n = 4, 4 * 1024
    assert echo.echo_allreduce_sim_workspace_bytes(P, n, 4) == (P + 1) * (1024 * 2 + 256)  # codes + params, 256-aligned
    assert echo.echo_allreduce_sim_workspace_bytes(P, n + 1, 4) == 0
    assert echo.echo_allreduce_sim_workspace_bytes(P, n, 5) == 0

    def sim(**kw):
        a = echo.SimArgs()
        a.P, a.bits, a.group, a.tiles, a.out_dtype, a.ef = P, 4, 128, 1, 0, 0
        a.alpha, a.beta, a.n = 1.0, 0.0, n
        for r in range(P):
            a.x[r] = FAKE
            a.out[r] = FAKE
        a.workspace = FAKE
        a.workspace_bytes = echo.echo_allreduce_sim_workspace_bytes(P, n, 4)
        for k, v in kw.items():
            if k in ("x", "out", "comp", "err", "slow"):
                for r, p in enumerate(v):
                    getattr(a, k)[r] = p
            else:
                setattr(a, k, v)
        return rc_of(echo.echo_allreduce_sim, a, streams=[0])

    assert sim(tiles=0) == echo.EINVAL
    assert sim(workspace_bytes=100) == echo.EINVAL
    assert sim(out_dtype=3) == echo.EUNSUP
    assert sim(x=[FAKE, None, FAKE, FAKE]) == echo.EINVAL
    assert sim(out=[FAKE, FAKE, FAKE + 2, FAKE]) == echo.EALIGN
    assert sim(ef=1) == echo.EINVAL                                         # comp missing
    assert sim(ef=1, comp=[FAKE] * P, alpha=0.5) == echo.EINVAL             # fused form needs alpha = 1
    assert sim(ef=1, comp=[FAKE] * P, err=[FAKE, None, None, None]) == echo.EINVAL
    assert sim(ef=1, comp=[FAKE] * P, err=[FAKE] * P, alpha=0.5, beta=0.25) == echo.EINVAL  # slow missing
    assert sim(quant=6) == echo.EINVAL                                      # both ablations
    assert sim(quant=1) == echo.EINVAL                                      # not a quantizer bit
    assert sim(group=64) == echo.EUNSUP
    assert sim(n=0) == 0


def test_header_is_plain_c_and_links(tmp_path):
    """include/echo.h compiles as strict C99 with gcc, and a C program linked
    against libecho.so sees the same host-side checks."""
    import os
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = tmp_path / "abi_check"
    lib_dir = os.path.join(root, "error_feedback_quant_amd")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(root, "include"), os.path.join(root, "tests", "c", "abi_check.c"),
                    "-L", lib_dir, "-l:libecho.so", "-Wl,-rpath," + lib_dir, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_check: ok" in r.stdout


def test_noalloc_argument_checks():
    """The allocation-free call checks its arguments like echo_allreduce_sim
    (minus the workspace) and rejects a message whose workspace exceeds the
    static scratch before it touches the device."""
    P = 4
    limit = echo.echo_noalloc_scratch_bytes()
    assert limit == 64 << 20

    def sim(n, **kw):
        a = echo.SimArgs()
        a.P, a.bits, a.group, a.tiles, a.out_dtype, a.ef = P, 4, 128, 1, 1, 0
        a.alpha, a.beta, a.n = 1.0, 0.0, n
        for r in range(P):
            a.x[r] = FAKE
            a.out[r] = FAKE
        for k, v in kw.items():
            if k in ("x", "out", "comp"):
                for r, p in enumerate(v):
                    getattr(a, k)[r] = p
            else:
                setattr(a, k, v)
        return rc_of(echo.echo_allreduce_sim_noalloc, a, stream=0)

    n_big = 1 << 25
    assert echo.echo_allreduce_sim_workspace_bytes(P, n_big, 4) > limit
    assert sim(n_big) == echo.ETOOBIG
    assert sim(n_big, tiles=0) == echo.EINVAL
    assert sim(n_big, x=[FAKE, None, FAKE, FAKE]) == echo.EINVAL
    assert sim(n_big, out=[FAKE + 2, FAKE, FAKE, FAKE]) == echo.EALIGN
    assert sim(n_big, ef=1) == echo.EINVAL                  # comp missing
    assert sim(0) == 0                                      # empty message: nothing to do
