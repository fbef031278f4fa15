"""CPU oracle for Echo's error-compensated low-bit all-reduce.

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only users.  The product library never
imports this package and this package never imports the product library.

The arithmetic lives in ``echo_ref.c`` (plain single-threaded C, built with
``-O2 -ffp-contract=off -fno-fast-math``); this module only builds/loads it
and marshals numpy arrays.  Sources and readings are stated in that file:
Echo (arXiv 2610.14277) paper card -- abstract, Fig. 1, Fig. 2, Table 8 and
appendix Fig. 4 -- and the PhantomByte article on Echo, section "The
cancellation rule".

Array conventions (host memory, numpy):
  x        uint16 [n]          bfloat16 bit patterns of one rank's partial sums
  comp     float32 [n]         compensation added at the entry pass (or None)
  codes    uint8  [n*b/8]      packed codes, element i in byte i/2 (low nibble
                               when i is even) for b = 4, one byte each for b = 8
  params   uint16 [2*n/g]      per group: binary16 scale bits, binary16 zero bits
  err      float32 [n]         revealed error e = Q_hat(u) - u (or -e)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from ctypes import POINTER, c_float, c_int, c_int64, c_uint16, c_void_p

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "echo_ref.c")
LIB = os.path.join(HERE, "libecho_ref.so")
# A prebuilt checker library to load instead (the mutation test plants a
# mistake in a scratch copy of echo_ref.c and points this at its build).
LIB_OVERRIDE = os.environ.get("ECHO_ORACLE_LIB") or None

OK, EINVAL, EUNSUP, ESHAPE = 0, -1, -3, -4
ERR_NEGATED = 1
Q_NAIVE, Q_SYMMETRIC = 2, 4          # quantizer flag bits (Table 8 ablations)
X_ALL = 8                            # gemm_quantize_ef: x_out receives every segment
Q_MSE = 16                           # quantizer flag bit: zero point searched for the least squared error
QUANTS = {"zero_aware": 0, "naive": Q_NAIVE, "symmetric": Q_SYMMETRIC, "mse": Q_MSE}
OUT_F32, OUT_BF16 = 0, 1

CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
          "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    """Compile echo_ref.c into libecho_ref.so with gcc (no GPU involved).
    The compiler writes a temporary file private to this process and thread,
    which then replaces the library in one rename."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = f"{LIB}.tmp{os.getpid()}.{threading.get_ident()}"
        subprocess.run(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


_lib = None
_lib_lock = threading.Lock()


def lib():
    """The loaded oracle library, built first if missing or older than its
    source.  Safe to call from several threads at once (the chunked oracle
    runs its calls in a thread pool)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if LIB_OVERRIDE:
            L = ctypes.CDLL(LIB_OVERRIDE)
        else:
            if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                build(force=True)
            L = ctypes.CDLL(LIB)
        L.echo_ref_f32_to_f16.restype = c_uint16
        L.echo_ref_f32_to_f16.argtypes = [c_float]
        L.echo_ref_f16_to_f32.restype = c_float
        L.echo_ref_f16_to_f32.argtypes = [c_uint16]
        L.echo_ref_f32_to_f16_array.restype = None
        L.echo_ref_f32_to_f16_array.argtypes = [c_void_p, c_void_p, c_int64]
        L.echo_ref_f32_to_bf16_array.restype = None
        L.echo_ref_f32_to_bf16_array.argtypes = [c_void_p, c_void_p, c_int64]
        L.echo_ref_quantize_group.restype = c_int
        L.echo_ref_quantize_group.argtypes = [c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p]
        L.echo_ref_quantize_group_q.restype = c_int
        L.echo_ref_quantize_group_q.argtypes = [c_void_p, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p]
        L.echo_ref_dequant.restype = c_float
        L.echo_ref_dequant.argtypes = [c_int, c_uint16, c_uint16]
        L.echo_ref_quantize_ef.restype = c_int
        L.echo_ref_quantize_ef.argtypes = [c_void_p, c_void_p, c_int64, c_int, c_int, c_int64, c_int64,
                                           c_int, c_int, c_void_p, c_void_p, c_void_p, c_int]
        L.echo_ref_reduce_segment.restype = c_int
        L.echo_ref_reduce_segment.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int,
                                              c_int64, c_int64, c_int64, c_int, c_int, c_void_p,
                                              c_void_p, c_void_p, c_int]
        L.echo_ref_gather_dequant.restype = c_int
        L.echo_ref_gather_dequant.argtypes = [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_int,
                                              c_int, c_int, c_void_p, c_int]
        L.echo_ref_compensate.restype = c_int
        L.echo_ref_compensate.argtypes = [c_void_p, c_void_p, c_void_p, c_int64, c_float, c_float]
        L.echo_ref_allreduce.restype = c_int
        L.echo_ref_allreduce.argtypes = [c_int, c_int64, c_int, c_int, c_int, c_float, c_float,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                         c_void_p, c_void_p, c_int]
        _lib = L
    return _lib


class OracleError(RuntimeError):
    def __init__(self, fn, rc):
        super().__init__(f"{fn} returned {rc}")
        self.rc = rc


def _p(a):
    return None if a is None else c_void_p(a.ctypes.data)


def _need(a, dtype, n=None):
    assert a.dtype == dtype and a.flags.c_contiguous, (a.dtype, dtype)
    if n is not None:
        assert a.size >= n, (a.size, n)
    return a


def _ptr_array(arrs):
    arr = (c_void_p * len(arrs))()
    for i, a in enumerate(arrs):
        arr[i] = None if a is None else a.ctypes.data
    return arr


def _check(fn, rc):
    if rc != OK:
        raise OracleError(fn, rc)


# --- number formats ------------------------------------------------------------

def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().echo_ref_f32_to_f16_array(_p(a), _p(out), a.size)
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().echo_ref_f32_to_bf16_array(_p(a), _p(out), a.size)
    return out


def f16_bits_to_f32(h: int) -> float:
    return float(lib().echo_ref_f16_to_f32(int(h)))


# --- the quantizer -------------------------------------------------------------

def quantize_group(v, bits: int, quant: str = "zero_aware"):
    """Q_b of one group with the named quantizer ("zero_aware", "naive",
    "symmetric", "mse").  Returns (codes uint8 [g], scale_bits, zero_bits)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    q = np.zeros(v.size, dtype=np.uint8)
    sh = ctypes.c_uint16()
    zh = ctypes.c_uint16()
    mode = {"zero_aware": 0, "naive": 1, "symmetric": 2, "mse": 3}[quant]
    _check("quantize_group", lib().echo_ref_quantize_group_q(_p(v), v.size, bits, mode, _p(q),
                                                             ctypes.byref(sh), ctypes.byref(zh)))
    return q, int(sh.value), int(zh.value)


def dequant(q: int, scale_bits: int, zero_bits: int) -> float:
    return float(lib().echo_ref_dequant(int(q), int(scale_bits), int(zero_bits)))


def code_bytes(n: int, bits: int) -> int:
    return n // 2 if bits == 4 else n


# --- call-level steps (host arrays, same semantics as the GPU library) -----------

def quantize_ef(x, comp, n, P, rank, tile_begin, tile_len, bits, group, codes, params, err, flags=0):
    sane = bits in (4, 8) and group > 0 and n >= 0 and n % group == 0
    _need(x, np.uint16, n if sane else None)
    _need(codes, np.uint8, code_bytes(n, bits) if sane else None)
    _need(params, np.uint16, 2 * (n // group) if sane else None)
    if comp is not None:
        _need(comp, np.float32, n)
    if err is not None:
        _need(err, np.float32, n)
    _check("quantize_ef", lib().echo_ref_quantize_ef(_p(x), _p(comp), n, P, rank, tile_begin, tile_len,
                                                     bits, group, _p(codes), _p(params), _p(err), flags))


# --- the matmul that produces a rank's partial sums -----------------------------

def bf16_bits_to_f32(x) -> np.ndarray:
    return (np.ascontiguousarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def matmul_bf16(a, w) -> np.ndarray:
    """A rank's partial sums x = bfloat16(A W^T) of a row-parallel linear
    layer (the message of the all-reduce, paper card Fig. 2(a)): A [M, K] and
    W [N, K] are bf16 bit arrays; the products and their sum are taken in
    float64 (a library matmul), then rounded to fp32 and to bf16 (nearest
    even).  Returns the row-major message, uint16 [M*N]."""
    a64 = bf16_bits_to_f32(a).astype(np.float64)
    w64 = bf16_bits_to_f32(w).astype(np.float64)
    return f32_to_bf16_bits((a64 @ w64.T).astype(np.float32)).reshape(-1)


def gemm_quantize_ef(a, w, comp, P, rank, bits, codes, params, err, x_out, flags=0, x=None, group=128):
    """The fused matmul + entry pass as its two steps: x = matmul_bf16(A, W)
    (or the given x), then quantize_ef over the whole message (segment s =
    rows [s*M/P, (s+1)*M/P)); the rank's own rows of x go to x_out (every row
    with X_ALL).  Returns x."""
    M, N = a.shape[0], w.shape[0]
    n = M * N
    if x is None:
        x = matmul_bf16(a, w)
    quantize_ef(x, comp, n, P, rank, 0, n // P, bits, group, codes, params, err, flags & ~X_ALL)
    if flags & X_ALL:
        x_out[:] = x
    else:
        S = n // P
        x_out[rank * S:(rank + 1) * S] = x[rank * S:(rank + 1) * S]
    return x


def reduce_segment(own_x, own_comp, peer_codes, peer_params, P, owner, n, tile_begin, tile_len, bits,
                   group, sum_codes, sum_params, own_err, flags=0):
    _check("reduce_segment", lib().echo_ref_reduce_segment(
        _p(own_x), _p(own_comp), _ptr_array(peer_codes), _ptr_array(peer_params), P, owner, n,
        tile_begin, tile_len, bits, group, _p(sum_codes), _p(sum_params), _p(own_err), flags))


def gather_dequant(sum_codes, sum_params, n, tile_begin, tile_len, P, bits, group, out, out_dtype):
    _check("gather_dequant", lib().echo_ref_gather_dequant(
        _p(sum_codes), _p(sum_params), n, tile_begin, tile_len, P, bits, group, _p(out), out_dtype))


def compensate(err, comp_next, slow, n, alpha, beta):
    _check("compensate", lib().echo_ref_compensate(_p(err), _p(comp_next), _p(slow), n, alpha, beta))


def allreduce(xs, bits=4, group=128, ef=False, alpha=1.0, beta=0.0, comps=None, slows=None,
              errs=None, out_dtype=OUT_F32, want_counts=False, quant="zero_aware"):
    """One whole call over P ranks.  xs: list of uint16 [n] (bf16 bits).
    comps/slows/errs: lists of float32 [n] updated in place (ef=True).
    Returns (outs, qdepth, qwork)."""
    P = len(xs)
    n = xs[0].size
    for x in xs:
        _need(x, np.uint16, n)
    odt = np.float32 if out_dtype == OUT_F32 else np.uint16
    outs = [np.empty(n, dtype=odt) for _ in range(P)]
    qdepth = np.zeros(n, dtype=np.int32) if want_counts else None
    qwork = np.zeros(P, dtype=np.int64) if want_counts else None
    rc = lib().echo_ref_allreduce(
        P, n, bits, group, 1 if ef else 0, alpha, beta, _ptr_array(xs),
        _ptr_array(comps) if comps is not None else None,
        _ptr_array(slows) if slows is not None else None,
        _ptr_array(errs) if errs is not None else None,
        _ptr_array(outs), out_dtype, _p(qdepth), _p(qwork), QUANTS[quant])
    _check("allreduce", rc)
    return outs, qdepth, qwork


# --- depth-chain harness ([EchoCard] Fig. 1: N injection sites add their ------------
# --- all-reduce outputs to the hidden state) ----------------------------------

def depth_chain(partials, P, n, bits=4, group=128, ef=False, alpha=1.0, beta=0.0, fused=True,
                comps=None, slows=None, quant="zero_aware"):
    """Run N all-reduce calls, one per injection site, accumulating each
    call's output into a float64 hidden state h and the exact sum of all
    partials into h_exact.  `partials(site)` returns P uint16 arrays.

    Returns a dict of float64 arrays per site k:
      E     h_k - h_exact_k                     (accumulated error, [N, n])
      delta out_k - sum_j x_kj - sum_j c_kj    (error injected at site k)
      debt  sum_j (M_j - c_j) after site k      (outstanding error debt)
    and the final comps/slows.  Compensation state is created at zero unless
    passed in (carried across calls)."""
    two = ef and not fused
    if ef and comps is None:
        comps = [np.zeros(n, dtype=np.float32) for _ in range(P)]
    if two and slows is None and beta != 0.0:
        slows = [np.zeros(n, dtype=np.float32) for _ in range(P)]
    errs = [np.zeros(n, dtype=np.float32) for _ in range(P)] if two else None
    h = np.zeros(n, dtype=np.float64)
    h_exact = np.zeros(n, dtype=np.float64)
    E, delta, debt = [], [], []
    k = 0
    while True:
        xs = partials(k)
        if xs is None:
            break
        xsum = np.zeros(n, dtype=np.float64)
        for x in xs:
            xsum += (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        csum = np.zeros(n, dtype=np.float64)
        if ef:
            for c in comps:
                csum += c.astype(np.float64)
        outs, _, _ = allreduce(xs, bits=bits, group=group, ef=ef, alpha=alpha, beta=beta,
                               comps=comps, slows=slows if two else None, errs=errs, quant=quant)
        out = outs[0].astype(np.float64)
        h += out
        h_exact += xsum
        E.append(h - h_exact)
        delta.append(out - xsum - csum)
        d = np.zeros(n, dtype=np.float64)
        if ef:
            for j in range(P):
                d -= comps[j].astype(np.float64)
                if two and slows is not None:
                    d += slows[j].astype(np.float64)
        debt.append(d)
        k += 1
    return dict(E=np.array(E), delta=np.array(delta), debt=np.array(debt), comps=comps, slows=slows)
