"""Shared helpers for the GPU parity tests (marshalling between numpy host
arrays for the oracle and torch device tensors for libecho)."""
import sys

import numpy as np
import torch

import oracle

DEV = "cuda:0"


def say(*a):
    """Name the case before each GPU step (flushed, so a crash still shows it)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint8)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.float32)


def params_dev(n_groups: int, fill: int = 0xCDCD) -> torch.Tensor:
    """Device buffer for n_groups echo_qparam words (two uint16 each)."""
    return dev_u16(np.full(2 * n_groups, fill, dtype=np.uint16))


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    g = np.ascontiguousarray(got).view(np.uint8)
    w = np.ascontiguousarray(want).view(np.uint8)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    if not np.array_equal(g, w):
        bad = np.nonzero(g != w)[0]
        raise AssertionError(f"{what}: {bad.size} bytes differ, first at byte {bad[0]}")


def assert_f32_parity(got: np.ndarray, want: np.ndarray, what: str, rel: float = 1e-6):
    """fp32 results: within max relative error 1e-6 (floored at the smallest
    normal), and report how many are bit-identical."""
    g = got.astype(np.float64)
    w = want.astype(np.float64)
    both_nan = np.isnan(g) & np.isnan(w)
    err = np.abs(g - w)
    tol = rel * np.maximum(np.abs(w), 2.0 ** -126)
    bad = (~both_nan) & (err > tol)
    if bad.any():
        i = int(np.nonzero(bad)[0][0])
        raise AssertionError(f"{what}: {int(bad.sum())} values beyond 1e-6 rel; first at {i}: {got[i]!r} vs {want[i]!r}")


def bf16_bits_to_f64(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_bf16(n, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return oracle.f32_to_bf16_bits((rng.standard_normal(n) * scale).astype(np.float32))


def chunk_slices(P: int, S: int, a: int, b: int):
    """The element range [a, b) of every segment of a message with P segments
    of S elements.  Concatenated in segment order they form a mini message
    whose segment s is that range of segment s, so ownership is kept."""
    return [slice(s * S + a, s * S + b) for s in range(P)]


def gather_chunk(arr: np.ndarray, sl) -> np.ndarray:
    return np.concatenate([arr[q] for q in sl])


def oracle_by_chunks(xs, comps, P, L, out_dtype, workers, visit, bits=4, slows=None, alpha=1.0,
                     beta=0.0, quant="zero_aware", group=128):
    """The oracle's whole call over a message of P segments, computed as
    independent calls on mini messages made of the same L-element range of
    every segment.  Feedback is on when `comps` is given (classic, written
    in place, for alpha = 1 and beta = 0; otherwise two-timescale with the
    slow memories `slows`), else off.  Quantization, the owner's sum and the
    feedback act per group and per element, and every range holds whole
    groups, so the results are those of one call on the whole message.  The
    calls run in `workers` host threads (the oracle's C entry point releases
    the GIL).  `comps` and `slows` are the state before the call and are
    left untouched.  visit(slices, outs, comps_after, slows_after) runs in
    the worker for each chunk and returns None or a description of the
    first mismatch; the first such description is returned."""
    from concurrent.futures import ThreadPoolExecutor

    n = xs[0].size
    S = n // P
    assert S % L == 0 and L % group == 0

    def one(a):
        sl = chunk_slices(P, S, a, a + L)
        xm = [gather_chunk(x, sl) for x in xs]
        cm = [gather_chunk(c, sl) for c in comps] if comps is not None else None
        sm = [gather_chunk(m, sl) for m in slows] if slows is not None else None
        outs, _, _ = oracle.allreduce(xm, bits=bits, group=group, ef=comps is not None, alpha=alpha, beta=beta,
                                      comps=cm, slows=sm, out_dtype=out_dtype, quant=quant)
        return visit(sl, outs, cm, sm)

    with ThreadPoolExecutor(max_workers=workers) as pool:
        for res in pool.map(one, range(0, S, L)):
            if res is not None:
                return res
    return None


def host_workers(cap: int = 16) -> int:
    import os
    try:
        return max(1, min(cap, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(cap, os.cpu_count() or 1))
