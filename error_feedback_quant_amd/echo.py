"""Thin ctypes binding of libecho (include/echo.h), same call names.

Argument marshalling only: every step of the path runs in the HIP kernels of
libecho.so.  Tensors are passed by device pointer (``tensor.data_ptr()``);
PyTorch provides device memory and streams.  A non-zero status raises
``EchoError``.  Importing this module loads libecho.so and raises if it has
not been built -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, Structure, c_char_p, c_float, c_int, c_int64, c_size_t, c_uint16, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libecho.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "echo.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
# torch brings its own HIP runtime (libamdhip64, SONAME libamdhip64.so.7) and
# owns the device memory and streams passed to libecho, so it must be loaded
# first: libecho.so then binds to that same runtime instead of pulling a
# second copy into the process.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

OK, EINVAL, EALIGN, EUNSUP, ESHAPE, EHIP, ETOOBIG = 0, -1, -2, -3, -4, -5, -6
OUT_F32, OUT_BF16 = 0, 1
ERR_NEGATED = 1
QUANT_NAIVE, QUANT_SYMMETRIC = 2, 4
X_ALL = 8
QUANT_MSE = 16
QUANTS = {"zero_aware": 0, "naive": QUANT_NAIVE, "symmetric": QUANT_SYMMETRIC, "mse": QUANT_MSE}
MAX_P = 8


class EchoError(RuntimeError):
    def __init__(self, fn, rc):
        msg = _lib.echo_status_str(rc).decode()
        if rc == EHIP:
            msg += f" (hipError {_lib.echo_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [{rc}]")
        self.rc = rc


class SimArgs(Structure):
    """Mirror of echo_sim_args."""
    _fields_ = [
        ("P", c_int), ("bits", c_int), ("group", c_int), ("tiles", c_int),
        ("out_dtype", c_int), ("ef", c_int), ("quant", c_int), ("alpha", c_float), ("beta", c_float),
        ("n", c_int64),
        ("x", c_void_p * MAX_P), ("comp", c_void_p * MAX_P), ("slow", c_void_p * MAX_P),
        ("err", c_void_p * MAX_P), ("out", c_void_p * MAX_P),
        ("workspace", c_void_p), ("workspace_bytes", c_size_t),
    ]


_lib.echo_status_str.restype = c_char_p
_lib.echo_status_str.argtypes = [c_int]
_lib.echo_last_hip_error.restype = c_int
_lib.echo_last_hip_error.argtypes = []
_lib.echo_quantize_ef.restype = c_int
_lib.echo_quantize_ef.argtypes = [c_void_p, c_void_p, c_int64, c_int, c_int, c_int64, c_int64, c_int, c_int,
                                  c_void_p, c_void_p, c_void_p, c_int, c_void_p]
_lib.echo_reduce_segment.restype = c_int
_lib.echo_reduce_segment.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int64, c_int64,
                                     c_int64, c_int, c_int, c_void_p, c_void_p, c_void_p, c_int, c_void_p]
_lib.echo_gather_dequant.restype = c_int
_lib.echo_gather_dequant.argtypes = [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_int, c_int, c_int,
                                     c_void_p, c_int, c_void_p]
_lib.echo_compensate.restype = c_int
_lib.echo_compensate.argtypes = [c_void_p, c_void_p, c_void_p, c_int64, c_float, c_float, c_void_p]
_lib.echo_gemm_quantize_ef.restype = c_int
_lib.echo_gemm_quantize_ef.argtypes = [c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int, c_int,
                                       c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_void_p]
_lib.echo_allreduce_sim_workspace_bytes.restype = c_size_t
_lib.echo_allreduce_sim_workspace_bytes.argtypes = [c_int, c_int64, c_int, c_int]
_lib.echo_allreduce_sim.restype = c_int
_lib.echo_allreduce_sim.argtypes = [POINTER(SimArgs), c_void_p, c_int]
_lib.echo_allreduce_sim_noalloc.restype = c_int
_lib.echo_allreduce_sim_noalloc.argtypes = [POINTER(SimArgs), c_void_p]
_lib.echo_noalloc_scratch_bytes.restype = c_size_t
_lib.echo_noalloc_scratch_bytes.argtypes = []


def lib():
    return _lib


def declared_functions():
    """Function names declared in include/echo.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(echo_[a-z_0-9]+)\s*\(", text, re.M)))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn, rc):
    if rc != OK:
        raise EchoError(fn, rc)


def echo_quantize_ef(x, comp, n, P, rank, tile_begin, tile_len, bits, group, codes, params, err,
                     flags=0, stream=None):
    _check("echo_quantize_ef", _lib.echo_quantize_ef(
        _ptr(x), _ptr(comp), n, P, rank, tile_begin, tile_len, bits, group, _ptr(codes), _ptr(params),
        _ptr(err), flags, _stream(stream)))


def echo_gemm_quantize_ef(a, w, M, N, K, comp, P, rank, bits, group, codes, params, err, x_out, flags=0,
                          stream=None):
    _check("echo_gemm_quantize_ef", _lib.echo_gemm_quantize_ef(
        _ptr(a), _ptr(w), M, N, K, _ptr(comp), P, rank, bits, group, _ptr(codes), _ptr(params), _ptr(err),
        _ptr(x_out), flags, _stream(stream)))


def echo_reduce_segment(own_x, own_comp, peer_codes, peer_params, P, owner, n, tile_begin, tile_len, bits,
                        group, sum_codes, sum_params, own_err, flags=0, stream=None):
    pc = (c_void_p * max(P, 1))(*[_ptr(t) for t in peer_codes])
    pp = (c_void_p * max(P, 1))(*[_ptr(t) for t in peer_params])
    _check("echo_reduce_segment", _lib.echo_reduce_segment(
        _ptr(own_x), _ptr(own_comp), pc, pp, P, owner, n, tile_begin, tile_len, bits, group,
        _ptr(sum_codes), _ptr(sum_params), _ptr(own_err), flags, _stream(stream)))


def echo_gather_dequant(sum_codes, sum_params, n, tile_begin, tile_len, P, bits, group, out, out_dtype,
                        stream=None):
    _check("echo_gather_dequant", _lib.echo_gather_dequant(
        _ptr(sum_codes), _ptr(sum_params), n, tile_begin, tile_len, P, bits, group, _ptr(out), out_dtype,
        _stream(stream)))


def echo_compensate(err, comp_next, slow, n, alpha, beta, stream=None):
    _check("echo_compensate", _lib.echo_compensate(
        _ptr(err), _ptr(comp_next), _ptr(slow), n, alpha, beta, _stream(stream)))


def echo_allreduce_sim_workspace_bytes(P, n, bits, group=128):
    return int(_lib.echo_allreduce_sim_workspace_bytes(P, n, bits, group))


def make_sim_args(xs, outs, workspace, bits=4, group=128, tiles=1, out_dtype=OUT_F32, ef=False,
                  alpha=1.0, beta=0.0, comps=None, slows=None, errs=None, workspace_bytes=None,
                  quant="zero_aware"):
    """Fill an echo_sim_args from lists of tensors (one per simulated rank)."""
    P = len(xs)
    a = SimArgs()
    a.P, a.bits, a.group, a.tiles, a.out_dtype, a.ef = P, bits, group, tiles, out_dtype, 1 if ef else 0
    a.quant = QUANTS[quant]
    a.alpha, a.beta = alpha, beta
    a.n = xs[0].numel() if P else 0
    for r in range(P):
        a.x[r] = _ptr(xs[r])
        a.out[r] = _ptr(outs[r])
        a.comp[r] = _ptr(comps[r]) if comps is not None else None
        a.slow[r] = _ptr(slows[r]) if slows is not None else None
        a.err[r] = _ptr(errs[r]) if errs is not None else None
    a.workspace = _ptr(workspace)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    a.workspace_bytes = workspace_bytes
    return a


def echo_allreduce_sim(args: SimArgs, streams=None):
    """streams: None (torch's current stream only) or a list of torch streams / handles."""
    if streams is None:
        arr, ns = (c_void_p * 1)(_stream(None)), 1
    else:
        arr, ns = (c_void_p * len(streams))(*[_stream(s) for s in streams]), len(streams)
    _check("echo_allreduce_sim", _lib.echo_allreduce_sim(ctypes.byref(args), arr, ns))


def echo_allreduce_sim_noalloc(args: SimArgs, stream=None):
    """The allocation-free call: args.workspace is ignored; every stage runs
    on `stream` (a torch stream or handle; None = torch's current stream)."""
    _check("echo_allreduce_sim_noalloc", _lib.echo_allreduce_sim_noalloc(ctypes.byref(args), _stream(stream)))


def echo_noalloc_scratch_bytes() -> int:
    return int(_lib.echo_noalloc_scratch_bytes())
