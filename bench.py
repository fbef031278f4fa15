"""Benchmark: one simulated Echo all-reduce call on one MI355X, 1 GiB messages.

A step is one echo_allreduce_sim call over P simulated ranks: push quantize
with the compensation added in the entry pass, owner reduce, tail decode, and
the compensator update (classic error feedback: -e written in place).  The
headline runs the tile-staged schedule: each segment is split into 4 tiles
whose stages overlap on two HIP streams (the push of tile t + 1 beside the
owner reduce of tile t, the tail of tile t after it), ordered by events.  The
same call with the stages back to back on one stream (one tile) is reported
beside it.  Inputs: 2^29 bfloat16 elements per rank, Laplace(0, 1), resident
in HBM before timing starts.

value = algorithmic bytes of the call / time, in GB/s (10^9 B/s), where the
algorithmic bytes per message element per rank are
    B = 2 + o + 8*ef + k_b * (3 - 1/P),  k_b = b/8 + 4/128
(bf16 in, output o bytes, compensation read + write, codes and per-group
parameters written by the push, read by the owner, written once by the
owner, read by every rank's tail).  Each simulated rank does its own reads.
elements/s counts the P*n elements the call all-reduces.

Also printed (same JSON line):
  roofline      the dominant kernel (push quantize of one rank over whole
                segments, as the back-to-back schedule launches it):
                algorithmic bytes per launch / its mean launch time from HIP
                events on its stream, against 8 TB/s; traffic from the
                committed rocprofv3 counter summary if it was taken on the
                current kernel source.
  serial        the same call with the stages back to back on one stream.
  p8            the same measurement at P = 8 (staged and serial), with its
                own roofline.
  configs       per-call throughput of the other workloads: a single call of
                64 x 1024 per rank (latency, cache-resident), the depth-chain
                call (2048 x 4096, feedback on and off), the 8-bit chain call
                (4096 x 1024, on and off) and the training call (2^27 per
                rank, two-timescale compensator, fused and as a separate
                update pass).
  cpu_baseline  the CPU oracle (single thread) on 1/64 of every segment of
                the 1 GiB message, scaled to the whole call.
  cpu_baselines the rest of the oracle's timing plan: single-threaded calls
                of the other workloads and of P = 8, and the whole 1 GiB call
                as independent calls on ranges of every segment in host
                threads, at P = 4 and 8; with the host's CPU count and model.
  variants      the same call with Table 8's ablation quantizers (naive zero
                point, symmetric grid), with groups of 256, and with the zero
                point searched for the least squared error.
  modes         the same call with feedback off, with fp32 output, with
                the two-timescale compensator fused into push and reduce
                (B then counts 16 bytes of state traffic instead of 8), and
                with the other code width (8-bit codes: k_b = 1.03125), each
                in the headline's schedule and back to back (`serial`).
  tp_block      one rank's row-parallel matmul with the entry pass fused in
                its epilogue (echo_gemm_quantize_ef) against hipBLASLt +
                echo_quantize_ef, at the Llama-3-8B down projection (TP = 4),
                with an MFMA roofline; and the two-timescale update run
                beside the next matmul against back to back.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
G = 128
N_1GIB = 1 << 29
METRIC = "fused quant/reduce/gather GB/s and % of HBM peak per call, 1 GB msg, P=4/8"
STAGED_TILES, STAGED_STREAMS = 4, 2


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("echo_kernels.hpp", "echo_api.hip"):
        with open(os.path.join(ROOT, "error_feedback_quant_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def bytes_per_elem(P, bits, ef, out_bytes, group=G, two_timescale=False):
    """Algorithmic bytes per message element per rank.  Classic feedback
    reads c and writes -e in place (8 B); the two-timescale update, fused into
    the push and the reduce, reads c and M and writes c' and M' (16 B)."""
    kb = bits / 8 + 4 / group
    state = (16 if two_timescale else 8) if ef else 0
    return 2 + out_bytes + state + kb * (3 - 1 / P)


def push_bytes_per_elem(bits, ef):
    return 2 + (8 if ef else 0) + bits / 8 + 4 / G


def committed_traffic(P, n):
    """HBM traffic per push launch (whole segments) from
    profiles/push_quantize_onegb_counters.json, if those counters were taken
    on the current kernel source and shape."""
    path = os.path.join(ROOT, "profiles", "push_quantize_onegb_counters.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        key = f"P{P}_tiles1_n{n}"
        if d.get("kernel_source_hash") != kernel_source_hash() or key not in d.get("push", {}):
            return None
        return d["push"][key]["hbm_bytes_per_launch"]
    except Exception:
        return None


def schedule_name(tiles, nstreams):
    if (tiles, nstreams) == (1, 1):
        return "push, reduce and tail back to back on one stream (one tile per segment)"
    if nstreams == 2:
        return (f"{tiles} tiles per segment staged across 2 HIP streams: the push of tile t+1 runs beside "
                f"the owner reduce of tile t, the tail of tile t follows on the push stream; events order each tile")
    return f"{tiles} tiles per segment staged across {nstreams} HIP streams (push, reduce, tail on their own)"


def run_case(echo, torch, inputs, P, n, bits, tiles, nstreams, steps, warmup, out_bf16, ef, time_kernel=True,
             quant="zero_aware", group=G, alpha=1.0, beta=0.0, xs=None, unfused=False):
    """Time `steps` calls of echo_allreduce_sim.  xs: the ranks' bf16 inputs
    on the device (default: the 1 GiB Laplace workload's draw).  unfused:
    errors go to err buffers and echo_compensate runs as its own pass."""
    dev = "cuda:0"
    two = ef and (alpha != 1.0 or beta != 0.0)
    if xs is None:
        xs = [inputs.laplace(r, n, device=dev) for r in range(P)]
    comps = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(P)] if ef else None
    slows = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(P)] if two else None
    errs = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(P)] if (ef and unfused) else None
    odt = torch.int16 if out_bf16 else torch.float32
    outs = [torch.empty(n, dtype=odt, device=dev) for _ in range(P)]
    ws = torch.empty(echo.echo_allreduce_sim_workspace_bytes(P, n, bits, group), dtype=torch.uint8, device=dev)
    main = torch.cuda.current_stream()
    streams = [main] + [torch.cuda.Stream() for _ in range(nstreams - 1)]
    args = echo.make_sim_args(xs, outs, ws, bits=bits, tiles=tiles, group=group,
                              out_dtype=echo.OUT_BF16 if out_bf16 else echo.OUT_F32, ef=ef, comps=comps,
                              quant=quant, alpha=alpha, beta=beta, slows=slows, errs=errs)
    for _ in range(warmup):
        echo.echo_allreduce_sim(args, streams=streams)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # one event between consecutive calls: per-call times for the median and
    # the minimum, and the first-to-last span for the whole run
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(main)
    for i in range(steps):
        echo.echo_allreduce_sim(args, streams=streams)
        evs[i + 1].record(main)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = evs[0].elapsed_time(evs[-1])
    ms_per_step = max(wall * 1e3, ev_ms) / steps
    per_call = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    call_ms = {"median": round(per_call[steps // 2], 4), "min": round(per_call[0], 4)}

    B = bytes_per_elem(P, bits, ef, 2 if out_bf16 else 4, group, two)
    if ef and unfused:
        B += 8                         # e written by the call and read back by the update pass
    res = dict(value=P * n * B / (ms_per_step * 1e-3) / 1e9, ms_per_step=ms_per_step, bytes_per_call=P * n * B,
               B=B, call_ms=call_ms, elements_per_s=P * n / (ms_per_step * 1e-3),
               wall_ms_per_step=wall * 1e3 / steps, event_ms_per_step=ev_ms / steps)
    if time_kernel:
        res["roofline"] = push_roofline(echo, torch, xs, comps, ws, P, n, bits, ef)
    del xs, comps, slows, errs, outs, ws, args
    torch.cuda.empty_cache()
    return res


def push_roofline(echo, torch, xs, comps, ws, P, n, bits, ef):
    """The dominant kernel, push quantize of one rank over whole segments
    (the launch the back-to-back schedule makes), timed with events on the
    stream it is launched on; codes and params go to the workspace's first
    rank slots."""
    S = n // P
    reps = max(8, 2 * P)
    main = torch.cuda.current_stream()
    cb = n // 2 if bits == 4 else n
    codes_t, params_t = ws, ws[((cb + 255) // 256) * 256 * P:]

    def push(r):
        echo.echo_quantize_ef(xs[r], comps[r] if ef else None, n, P, r, 0, S, bits, G,
                              codes_t, params_t, comps[r] if ef else None,
                              echo.ERR_NEGATED if ef else 0, stream=main)

    for r in range(P):     # warm
        push(r)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(main)
    for i in range(reps):
        push(i % P)
    e1.record(main)
    torch.cuda.synchronize()
    push_ms = e0.elapsed_time(e1) / reps
    push_bytes = (P - 1) * S * push_bytes_per_elem(bits, ef)
    achieved = push_bytes / (push_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": committed_traffic(P, n),
            "kernel": "echo::push_kernel (echo_quantize_ef), one rank over whole segments",
            "launch_elements": (P - 1) * S, "algorithmic_bytes_per_launch": int(push_bytes),
            "mean_launch_ms": round(push_ms, 4)}


def leg(r, extra=None):
    d = {"value": round(r["value"], 1), "unit": "GB/s", "ms_per_step": round(r["ms_per_step"], 4),
         "frac_of_peak": round(r["value"] / HBM_PEAK_GBS, 4), "elements_per_s": float(f"{r['elements_per_s']:.4g}"),
         "call_ms": r["call_ms"], "bytes_per_elem_per_rank": round(r["B"], 5)}
    if extra:
        d.update(extra)
    return d


def graph_call_latency(echo, torch, xs, calls=50, replays=7):
    """Device-side time per call of a small workload: `calls` consecutive
    calls of echo_allreduce_sim_noalloc (the allocation-free form; one tile,
    so one launch each at this size) captured in one HIP graph and replayed,
    so that no host work sits between the calls.  The compensation carries
    from call to call as in eager use."""
    dev = "cuda:0"
    P, n = len(xs), xs[0].numel()
    comps = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(P)]
    outs = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(P)]
    a = echo.make_sim_args(xs, outs, None, bits=4, tiles=1, out_dtype=echo.OUT_BF16, ef=True, comps=comps,
                           workspace_bytes=0)
    echo.echo_allreduce_sim_noalloc(a)    # an eager call first looks up the scratch's device address
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            echo.echo_allreduce_sim_noalloc(a)
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    per_call = []
    for _ in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main)
        g.replay()
        e1.record(main)
        torch.cuda.synchronize()
        per_call.append(e0.elapsed_time(e1) / calls)
    del g
    per_call.sort()
    return {"calls_per_graph": calls, "replays": replays, "call_us_median": round(per_call[replays // 2] * 1e3, 2),
            "call_us_min": round(per_call[0] * 1e3, 2),
            "what": "calls captured in one HIP graph (echo_allreduce_sim_noalloc) and replayed: no host work between calls"}


def config_legs(echo, torch, inputs):
    """Per-call throughput of the single-call, depth-chain, 8-bit-chain and
    training workloads (one call each, inputs of the workload's recipe),
    back to back on one stream."""
    dev = "cuda:0"
    out = {}
    P = 4
    xs = [inputs.single(r).to(dev) for r in range(P)]
    n = xs[0].numel()
    r = run_case(echo, torch, inputs, P, n, 4, 1, 1, 200, 20, True, True, time_kernel=False, xs=xs)
    out["single_call_64x1024"] = leg(r, {"P": P, "n": n, "bits": 4, "ef": "classic", "cache_resident": True,
                                         "latency_us_median": round(r["call_ms"]["median"] * 1e3, 1),
                                         "graph_replay": graph_call_latency(echo, torch, xs)})
    sigma = inputs.chain_channel_scale(device=dev)
    for ef in (True, False):
        xs = [inputs.chain(r, 0, sigma_h=sigma, device=dev) for r in range(P)]
        n = xs[0].numel()
        r = run_case(echo, torch, inputs, P, n, 4, 1, 1, 50, 10, True, ef, time_kernel=False, xs=xs)
        out[f"chain_2048x4096_ef_{'on' if ef else 'off'}"] = leg(r, {"P": P, "n": n, "bits": 4})
    for ef in (True, False):
        xs = [inputs.chain8(r, 0, device=dev) for r in range(P)]
        n = xs[0].numel()
        r = run_case(echo, torch, inputs, P, n, 8, 1, 1, 50, 10, True, ef, time_kernel=False, xs=xs)
        out[f"chain8_4096x1024_ef_{'on' if ef else 'off'}"] = leg(r, {"P": P, "n": n, "bits": 8})
    n = 32 * 4096 * 1024
    for unfused in (False, True):
        xs = [inputs.training(r, 0, 0, False, n, device=dev) for r in range(P)]
        r = run_case(echo, torch, inputs, P, n, 4, 1, 1, 10, 3, True, True, time_kernel=False, xs=xs,
                     alpha=0.5, beta=0.25, unfused=unfused)
        name = "training_2^27_two_timescale_" + ("update_pass" if unfused else "fused")
        out[name] = leg(r, {"P": P, "n": n, "bits": 4, "alpha": 0.5, "beta": 0.25,
                            "update": "separate echo_compensate pass after the call (e written, then read)"
                            if unfused else "fused into push and reduce"})
    torch.cuda.empty_cache()
    return out


def tp_block(echo, torch, inputs, reps=10, beside_runs=5):
    """One rank's row-parallel matmul and entry pass at the Llama-3-8B MLP down
    projection with TP = 4 (4096 tokens, hidden 4096, K = 14336/4), random
    weights: the fused echo_gemm_quantize_ef against torch.matmul (hipBLASLt)
    followed by echo_quantize_ef, same compensation and outputs; and the
    two-timescale update (echo_compensate) run beside the next matmul (the
    gate/up projection, N = 2*14336/4) on a second stream, against running
    the two back to back, repeated to show the spread of the hidden part."""
    shp = inputs.SHAPES["tpblock"]
    M, N, K, P = shp["tokens"], shp["hidden"], shp["k"], shp["P"]
    n = M * N
    dev = "cuda:0"
    a16, w16 = inputs.tp_operands(1, M, N, K, "normal", device=dev)
    comp = torch.zeros(n, dtype=torch.float32, device=dev)
    codes = torch.empty(n // 2, dtype=torch.uint8, device=dev)
    params = torch.empty(2 * n // 128, dtype=torch.int16, device=dev)
    x_out = torch.empty(n, dtype=torch.int16, device=dev)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    main = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(main)
        for _ in range(reps):
            fn()
        e1.record(main)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3          # microseconds

    fused = lambda: echo.echo_gemm_quantize_ef(a16, w16, M, N, K, comp, P, 1, 4, 128, codes, params, comp,
                                               x_out, echo.ERR_NEGATED, stream=main)
    gemm_only = lambda: echo.echo_gemm_quantize_ef(a16, w16, M, N, K, None, 1, 0, 4, 128, codes, params, None,
                                                   x_out, 0, stream=main)
    lib = lambda: torch.matmul(a16.view(torch.bfloat16), w16.view(torch.bfloat16).t(), out=y)
    push = lambda: echo.echo_quantize_ef(y.view(torch.int16), comp, n, P, 1, 0, n // P, 4, 128, codes, params,
                                         comp, echo.ERR_NEGATED, stream=main)
    t_fused = timed(fused)
    t_gemm = timed(gemm_only)
    t_lib = timed(lib)
    t_push = timed(push)
    t_lib_push = timed(lambda: (lib(), push()))
    flop = 2.0 * M * N * K

    N2 = 2 * 14336 // P
    w2 = (torch.randn(N2, N, device=dev) * N ** -0.5).to(torch.bfloat16)
    z = torch.empty(M, N2, dtype=torch.bfloat16, device=dev)
    err = torch.randn(n, device=dev) * 1e-2
    slow = torch.zeros(n, device=dev)
    side = torch.cuda.Stream()
    nxt = lambda: torch.matmul(y, w2.t(), out=z)
    upd = lambda s: echo.echo_compensate(err, comp, slow, n, 0.5, 0.25, stream=s)

    def beside():
        ev = torch.cuda.Event()
        ev.record(main)
        side.wait_event(ev)
        nxt()
        upd(side)
        ev2 = torch.cuda.Event()
        ev2.record(side)
        main.wait_event(ev2)

    runs = []
    for _ in range(beside_runs):
        t_next = timed(nxt)
        t_upd = timed(lambda: upd(main))
        t_serial = timed(lambda: (nxt(), upd(main)))
        t_beside = timed(beside)
        hidden = (t_serial - t_beside) / t_upd if t_upd > 0 else 0.0
        runs.append({"next_matmul_us": round(t_next, 1), "update_us": round(t_upd, 1),
                     "serial_us": round(t_serial, 1), "beside_us": round(t_beside, 1),
                     "hidden_fraction": round(hidden, 3)})
    hid = sorted(r["hidden_fraction"] for r in runs)
    out = {
        "shape": {"M": M, "N": N, "K": K, "P": P, "bits": 4, "ef": "classic, -e in place"},
        "fused_us": round(t_fused, 1),
        "gemm_alone_us": round(t_gemm, 1),
        "hipblaslt_gemm_us": round(t_lib, 1),
        "push_alone_us": round(t_push, 1),
        "hipblaslt_gemm_plus_push_us": round(t_lib_push, 1),
        "roofline": {"bound": "mfma", "achieved": round(flop / t_fused / 1e6, 1), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(flop / t_fused / 1e6 / 2500.0, 4),
                     "kernel": "echo::gemm256_push_kernel (echo_gemm_quantize_ef)"},
        "gemm_alone_tflops": round(flop / t_gemm / 1e6, 1),
        "hipblaslt_tflops": round(flop / t_lib / 1e6, 1),
        "update_beside_next_matmul": {"runs": runs, "hidden_fraction_median": hid[len(hid) // 2],
                                      "hidden_fraction_range": [hid[0], hid[-1]]},
    }
    del a16, w16, comp, codes, params, x_out, y, w2, z, err, slow
    torch.cuda.empty_cache()
    return out


def device_copy_gbs(torch, reps=10):
    """A plain 1 GiB device-to-device copy (hipMemcpyAsync through torch),
    counted as read + write bytes: a measured second denominator beside the
    8 TB/s peak."""
    src = torch.empty(N_1GIB // 2, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * src.numel() * 4 / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


# ------------------------------------------------------------- CPU baselines --

def _oracle_call(P, xs, bits, ef, out_bf16):
    """One whole oracle call over host arrays; returns seconds."""
    import numpy as np
    import oracle
    comps = [np.zeros(xs[0].size, np.float32) for _ in range(P)] if ef else None
    odt = oracle.OUT_BF16 if out_bf16 else oracle.OUT_F32
    t0 = time.perf_counter()
    oracle.allreduce(xs, bits=bits, ef=ef, comps=comps, out_dtype=odt)
    return time.perf_counter() - t0


def _rate(P, n_per_rank, bits, ef, out_bf16, seconds, cores, sample, extra=None):
    B = bytes_per_elem(P, bits, ef, 2 if out_bf16 else 4)
    d = {"value": round(P * n_per_rank * B / seconds / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
         "sample": sample, "seconds_per_call": round(seconds, 4),
         "elements_per_s": float(f"{P * n_per_rank / seconds:.4g}")}
    if extra:
        d.update(extra)
    return d


def onegb_sample(P, L, base=1 << 22):
    """Host inputs for a 1 GiB-workload sample of P segments of L elements:
    Laplace(0,1) draws from the workload's CPU generator (base elements per
    rank, repeated to length; the oracle's work does not depend on the
    values)."""
    import numpy as np
    from error_feedback_quant_amd import inputs
    xs = []
    for r in range(P):
        b = inputs.as_numpy_u16(inputs.laplace(r, min(base, P * L), device="cpu", chunk=1 << 22))
        reps = -(-(P * L) // b.size)
        xs.append(np.ascontiguousarray(np.tile(b, reps)[:P * L]))
    return xs


def cpu_baseline_sampled(P, n, bits, out_bf16, ef, den=64):
    """The oracle, single-threaded, on 1/den of every segment of the 1 GiB
    message (tiles are independent, so the work scales exactly), reported
    for the whole call."""
    S = n // P
    L = S // den // G * G
    xs = onegb_sample(P, L)
    dt = _oracle_call(P, xs, bits, ef, out_bf16) * (S / L)
    return _rate(P, n, bits, ef, out_bf16, dt, 1,
                 f"one call on 1/{den} of every segment ({P}x{L} elements per rank, Laplace(0,1)), "
                 f"single-threaded, scaled x{S // L} to the 2^29-element call, P={P}",
                 {"cpu": host_cpu_model()})


def cpu_baseline_threaded_full(P, n, bits, out_bf16, ef, workers):
    """The whole 1 GiB call as independent oracle calls on mini messages made
    of the same range of every segment (groups and elements are independent),
    in `workers` host threads (the oracle's C entry point releases the GIL)."""
    import numpy as np
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    S = n // P
    xs = onegb_sample(P, S)
    chunk = min(1 << 18, S)
    assert S % chunk == 0
    odt = oracle.OUT_BF16 if out_bf16 else oracle.OUT_F32

    def one(a0):
        xm = [np.concatenate([x[s * S + a0:s * S + a0 + chunk] for s in range(P)]) for x in xs]
        cm = [np.zeros(P * chunk, np.float32) for _ in range(P)] if ef else None
        oracle.allreduce(xm, bits=bits, ef=ef, comps=cm, out_dtype=odt)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=workers) as pool:
        list(pool.map(one, range(0, S, chunk)))
    dt = time.perf_counter() - t0
    del xs
    return _rate(P, n, bits, ef, out_bf16, dt, workers,
                 f"the whole 2^29-element call at P={P} as {S // chunk} independent calls on {chunk}-element "
                 f"ranges of every segment, {workers} threads")


def cpu_baselines(out_bf16=True):
    """The oracle's timing plan beside the GPU numbers: single-threaded calls
    of the single-call (whole), depth-chain and 8-bit-chain workloads (one
    call each), the 1 GiB call at P = 8 (sampled, scaled), and the whole
    1 GiB call in host threads at P = 4 and 8."""
    from error_feedback_quant_amd import inputs
    P = 4
    res = {"nproc": os.cpu_count(), "threads_available": host_threads(1 << 30), "cpu": host_cpu_model()}
    xs = [inputs.as_numpy_u16(inputs.single(r)) for r in range(P)]
    dt = _oracle_call(P, xs, 4, True, out_bf16)
    res["single_call_64x1024"] = _rate(P, xs[0].size, 4, True, out_bf16, dt, 1, "one whole call, single-threaded")
    sigma = inputs.chain_channel_scale()
    for ef in (True, False):
        xs = [inputs.as_numpy_u16(inputs.chain(r, 0, sigma_h=sigma)) for r in range(P)]
        dt = _oracle_call(P, xs, 4, ef, out_bf16)
        res[f"chain_2048x4096_ef_{'on' if ef else 'off'}"] = _rate(P, xs[0].size, 4, ef, out_bf16, dt, 1,
                                                                   "one whole call, single-threaded")
    for ef in (True, False):
        xs = [inputs.as_numpy_u16(inputs.chain8(r, 0)) for r in range(P)]
        dt = _oracle_call(P, xs, 8, ef, out_bf16)
        res[f"chain8_4096x1024_ef_{'on' if ef else 'off'}"] = _rate(P, xs[0].size, 8, ef, out_bf16, dt, 1,
                                                                    "one whole call, single-threaded")
    res["onegb_p8_sampled"] = cpu_baseline_sampled(8, N_1GIB, 4, out_bf16, True)
    workers = host_threads()
    for Pt in (4, 8):
        res[f"onegb_p{Pt}_threaded_whole_call"] = cpu_baseline_threaded_full(Pt, N_1GIB, 4, out_bf16, True, workers)
    return res


def host_threads(cap: int = 16) -> int:
    """Worker threads for the threaded oracle: the CPUs this process may run
    on, at most `cap`."""
    try:
        return max(1, min(cap, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(cap, os.cpu_count() or 1))


def host_cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--P", type=int, default=4)
    ap.add_argument("--bits", type=int, default=4, choices=[4, 8])
    ap.add_argument("--tiles", type=int, default=STAGED_TILES)
    ap.add_argument("--streams", type=int, default=STAGED_STREAMS)
    ap.add_argument("--no-serial", action="store_true", help="skip the back-to-back schedule leg")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the Table 8 quantizer/group-size legs")
    ap.add_argument("--out", choices=["bf16", "f32"], default="bf16")
    ap.add_argument("--no-ef", action="store_true")
    ap.add_argument("--no-modes", action="store_true",
                    help="skip the feedback-off, fp32-output, two-timescale and 8-bit legs")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload call legs")
    ap.add_argument("--no-p8", action="store_true", help="skip the P=8 leg")
    ap.add_argument("--no-tp", action="store_true", help="skip the fused matmul + entry pass leg")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one plain 1 GiB device copy (counter calibration)")
    a = ap.parse_args()

    if a.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (the P ranks are simulated on it); "
              f"--gpus {a.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: one process, one GPU; not for torch.distributed launch", file=sys.stderr)
        sys.exit(2)

    import torch
    from error_feedback_quant_amd import echo, inputs
    assert torch.cuda.is_available(), "no GPU visible"

    out_bf16 = a.out == "bf16"
    ef = not a.no_ef
    main_res = run_case(echo, torch, inputs, a.P, N_1GIB, a.bits, a.tiles, a.streams, a.steps, a.warmup,
                        out_bf16, ef, time_kernel=False)
    serial = None
    roof = None
    if not a.no_serial:
        rs = run_case(echo, torch, inputs, a.P, N_1GIB, a.bits, 1, 1, a.steps, a.warmup, out_bf16, ef)
        roof = rs.pop("roofline")
        serial = leg(rs, {"tiles": 1, "streams": 1, "schedule": schedule_name(1, 1)})
    variants = None
    if not a.no_variants:
        variants = {}
        for name, quant, group in (("naive_zero_point", "naive", G), ("symmetric_grid", "symmetric", G),
                                   ("zero_aware_g256", "zero_aware", 256), ("searched_zero_point", "mse", G)):
            rv = run_case(echo, torch, inputs, a.P, N_1GIB, a.bits, a.tiles, a.streams, max(5, a.steps // 3),
                          a.warmup, out_bf16, ef, time_kernel=False, quant=quant, group=group)
            variants[name] = leg(rv)
    modes = None
    if not a.no_modes:
        # the same call with feedback off, with fp32 output, with the
        # two-timescale compensator (alpha = 0.5, beta = 0.25) fused into the
        # push and the reduce, and with 8-bit codes
        modes = {}
        other_bits = 8 if a.bits == 4 else 4
        for name, m_ef, m_bf16, alpha, beta, m_bits in (
                ("ef_off", False, out_bf16, 1.0, 0.0, a.bits),
                ("f32_out", ef, False, 1.0, 0.0, a.bits),
                ("two_timescale", True, out_bf16, 0.5, 0.25, a.bits),
                (f"bits{other_bits}", ef, out_bf16, 1.0, 0.0, other_bits)):
            rm = run_case(echo, torch, inputs, a.P, N_1GIB, m_bits, a.tiles, a.streams, max(5, a.steps // 3),
                          a.warmup, m_bf16, m_ef, time_kernel=False, alpha=alpha, beta=beta)
            extra = {"tiles": a.tiles, "streams": a.streams, "schedule": schedule_name(a.tiles, a.streams)}
            if not a.no_serial and (a.tiles, a.streams) != (1, 1):
                # the same mode back to back: with feedback off every stage is
                # short, and the staged pipeline's launch and event costs weigh more
                rms = run_case(echo, torch, inputs, a.P, N_1GIB, m_bits, 1, 1, max(5, a.steps // 3), a.warmup,
                               m_bf16, m_ef, time_kernel=False, alpha=alpha, beta=beta)
                extra["serial"] = leg(rms, {"tiles": 1, "streams": 1, "schedule": schedule_name(1, 1)})
            modes[name] = leg(rm, extra)
    p8 = None
    if not a.no_p8 and a.P != 8:
        r8 = run_case(echo, torch, inputs, 8, N_1GIB, a.bits, a.tiles, a.streams, max(5, a.steps // 2),
                      a.warmup, out_bf16, ef, time_kernel=False)
        r8s = run_case(echo, torch, inputs, 8, N_1GIB, a.bits, 1, 1, max(5, a.steps // 2), a.warmup, out_bf16, ef)
        roof8 = r8s.pop("roofline")
        p8 = leg(r8, {"tiles": a.tiles, "streams": a.streams, "schedule": schedule_name(a.tiles, a.streams),
                      "roofline": roof8,
                      "serial": leg(r8s, {"tiles": 1, "streams": 1, "schedule": schedule_name(1, 1)})})
    configs = None if a.no_configs else config_legs(echo, torch, inputs)
    copy_gbs = device_copy_gbs(torch)
    tp = None if a.no_tp else tp_block(echo, torch, inputs)
    if a.calib_copy:
        src = torch.empty(N_1GIB, dtype=torch.int16, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cpu = cpu_plan = None
    if not a.no_cpu:
        cpu = cpu_baseline_sampled(a.P, N_1GIB, a.bits, out_bf16, ef)
        cpu_plan = cpu_baselines(out_bf16)

    line = {
        "metric": METRIC,
        "value": round(main_res["value"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"1 GiB message: 2^29 bf16 elements per rank, Laplace(0,1), P={a.P} simulated ranks",
            "P": a.P, "bits": a.bits, "group": G, "tiles": a.tiles, "streams": a.streams,
            "schedule": schedule_name(a.tiles, a.streams),
            "ef": "classic error feedback (alpha=1), -e written in place" if ef else "off",
            "out": a.out, "bytes_per_elem_per_rank": round(main_res["B"], 5),
            "bytes_per_call": int(main_res["bytes_per_call"]),
            "frac_of_peak": round(main_res["value"] / HBM_PEAK_GBS, 4),
            "elements_per_s": float(f"{main_res['elements_per_s']:.4g}"),
            "call_ms": main_res["call_ms"],
            "device_copy_gbs": round(copy_gbs, 1),
            "frac_of_device_copy": round(main_res["value"] / copy_gbs, 4),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "serial": serial,
        "p8": p8,
        "configs": configs,
        "cpu_baselines": cpu_plan,
        "variants": variants,
        "modes": modes,
        "tp_block": tp,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
