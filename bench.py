"""Benchmark: one simulated Echo all-reduce call on one MI355X, 1 GiB messages.

A step is one echo_allreduce_sim call over P simulated ranks: push quantize
with the compensation added in the entry pass, owner reduce, tail decode, and
the compensator update (classic error feedback: -e written in place).  The
headline schedule runs the stages back to back on one stream (one tile per
segment), the fastest schedule on a single GPU; the same call with each
segment split into 4 tiles staggered across 4 HIP streams is reported beside
it ("staged").  Inputs: 2^29 bfloat16 elements per rank, Laplace(0, 1),
resident in HBM before timing starts.

value = algorithmic bytes of the call / time, in GB/s (10^9 B/s), where the
algorithmic bytes per message element per rank are
    B = 2 + o + 8*ef + k_b * (3 - 1/P),  k_b = b/8 + 4/128
(bf16 in, output o bytes, compensation read + write, codes and per-group
parameters written by the push, read by the owner, written once by the
owner, read by every rank's tail).  Each simulated rank does its own reads.

Also printed (same JSON line):
  roofline      the dominant kernel (push quantize): algorithmic bytes per
                launch / its mean launch time from HIP events on its stream,
                against 8 TB/s; traffic from the committed rocprofv3 counter
                summary if it was taken on the current kernel source.
  cpu_baseline  the CPU oracle (single thread) on a bounded sample of the same
                workload: 1/4 of every segment's groups, same byte formula.
  cpu_baseline_threaded
                the same sample as independent calls on ranges of every
                segment, in up to 16 host threads.
  staged        the same call with tiles staggered across streams.
  variants      the same call with Table 8's ablation quantizers (naive zero
                point, symmetric grid) and with groups of 256.
  modes         the same call with feedback off, with fp32 output, with
                the two-timescale compensator fused into push and reduce
                (B then counts 16 bytes of state traffic instead of 8), and
                with the other code width (8-bit codes: k_b = 1.03125).
  tp_block      one rank's row-parallel matmul with the entry pass fused in
                its epilogue (echo_gemm_quantize_ef) against hipBLASLt +
                echo_quantize_ef, at the Llama-3-8B down projection (TP = 4),
                with an MFMA roofline; and the two-timescale update run
                beside the next matmul against back to back.
  config        also carries the per-call median and minimum (HIP events
                between consecutive calls) and a plain 1 GiB device copy's
                bandwidth as a measured second denominator.
  p8            the same measurement at P = 8.
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


def committed_traffic(P, tiles, n):
    """HBM traffic per push launch from profiles/push_quantize_onegb_counters.json,
    if those counters were taken on the current kernel source and shape."""
    path = os.path.join(ROOT, "profiles", "push_quantize_onegb_counters.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        key = f"P{P}_tiles{tiles}_n{n}"
        if d.get("kernel_source_hash") != kernel_source_hash() or key not in d.get("push", {}):
            return None
        return d["push"][key]["hbm_bytes_per_launch"]
    except Exception:
        return None


def run_case(echo, torch, inputs, P, n, bits, tiles, nstreams, steps, warmup, out_bf16, ef, time_kernel=True,
             quant="zero_aware", group=G, alpha=1.0, beta=0.0):
    dev = "cuda:0"
    two = ef and (alpha != 1.0 or beta != 0.0)
    xs = [inputs.laplace(r, n, device=dev) for r in range(P)]
    comps = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(P)] if ef else None
    slows = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(P)] if two else None
    odt = torch.int16 if out_bf16 else torch.float32
    outs = [torch.empty(n, dtype=odt, device=dev) for _ in range(P)]
    ws = torch.empty(echo.echo_allreduce_sim_workspace_bytes(P, n, bits, group), dtype=torch.uint8, device=dev)
    main = torch.cuda.current_stream()
    streams = [main] + [torch.cuda.Stream() for _ in range(nstreams - 1)]
    args = echo.make_sim_args(xs, outs, ws, bits=bits, tiles=tiles, group=group,
                              out_dtype=echo.OUT_BF16 if out_bf16 else echo.OUT_F32, ef=ef, comps=comps,
                              quant=quant, alpha=alpha, beta=beta, slows=slows)
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
    value = P * n * B / (ms_per_step * 1e-3) / 1e9
    if not time_kernel:
        del xs, comps, slows, outs, ws
        torch.cuda.empty_cache()
        return dict(value=value, ms_per_step=ms_per_step, bytes_per_call=P * n * B, B=B, call_ms=call_ms)

    # dominant kernel: the push of one rank over one tile, timed with events on
    # the stream it is launched on (the sim launches the same kernel, same size)
    S = n // P
    gps = S // G
    tile_groups = -(-gps // min(tiles, gps))
    tile_len = tile_groups * G
    reps = max(8, 2 * P)
    # codes and params of this timing go to the workspace's first rank slots
    cb = n // 2 if bits == 4 else n
    codes_t, params_t = ws, ws[((cb + 255) // 256) * 256 * P:]

    def push(r):
        echo.echo_quantize_ef(xs[r], comps[r] if ef else None, n, P, r, 0, tile_len, bits, G,
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
    push_bytes = (P - 1) * tile_len * push_bytes_per_elem(bits, ef)
    achieved = push_bytes / (push_ms * 1e-3) / 1e9
    traffic = committed_traffic(P, tiles, n)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": "echo::push_kernel (echo_quantize_ef)", "launch_elements": (P - 1) * tile_len,
            "algorithmic_bytes_per_launch": int(push_bytes), "mean_launch_ms": round(push_ms, 4)}
    del xs, comps, slows, outs, ws
    torch.cuda.empty_cache()
    return dict(value=value, ms_per_step=ms_per_step, bytes_per_call=P * n * B, B=B, roofline=roof,
                wall_ms_per_step=wall * 1e3 / steps, event_ms_per_step=ev_ms / steps, call_ms=call_ms)


def tp_block(echo, torch, inputs, reps=10):
    """One rank's row-parallel matmul and entry pass at the Llama-3-8B MLP down
    projection with TP = 4 (4096 tokens, hidden 4096, K = 14336/4), random
    weights: the fused echo_gemm_quantize_ef against torch.matmul (hipBLASLt)
    followed by echo_quantize_ef, same compensation and outputs; and the
    two-timescale update (echo_compensate) run beside the next matmul (the
    gate/up projection, N = 2*14336/4) on a second stream, against running
    the two back to back."""
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

    t_next = timed(nxt)
    t_upd = timed(lambda: upd(main))
    t_serial = timed(lambda: (nxt(), upd(main)))
    t_beside = timed(beside)
    out = {
        "shape": {"M": M, "N": N, "K": K, "P": P, "bits": 4, "ef": "classic, -e in place"},
        "fused_us": round(t_fused, 1),
        "gemm_alone_us": round(t_gemm, 1),
        "hipblaslt_gemm_us": round(t_lib, 1),
        "hipblaslt_gemm_plus_push_us": round(t_lib_push, 1),
        "roofline": {"bound": "mfma", "achieved": round(flop / t_fused / 1e6, 1), "peak": 2500.0,
                     "unit": "TFLOP/s", "frac": round(flop / t_fused / 1e6 / 2500.0, 4),
                     "kernel": "echo::gemm256_push_kernel (echo_gemm_quantize_ef)"},
        "gemm_alone_tflops": round(flop / t_gemm / 1e6, 1),
        "hipblaslt_tflops": round(flop / t_lib / 1e6, 1),
        "update_beside_next_matmul": {"next_matmul_us": round(t_next, 1), "update_us": round(t_upd, 1),
                                      "serial_us": round(t_serial, 1), "beside_us": round(t_beside, 1)},
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


def cpu_baseline(P, n, bits, out_bf16, ef, frac_den=4):
    """The oracle (single-threaded C) on a bounded sample of the workload:
    a message 1/frac_den the size (every segment shortened alike), drawn from
    the same Laplace(0,1) recipe, timed over one whole call; then the same
    sample in host threads.  Returns (single-threaded, threaded)."""
    import numpy as np
    import oracle
    from error_feedback_quant_amd import inputs
    S = n // P
    L = S // frac_den // G * G            # sampled elements per segment
    # each rank's sample: P segments of L elements from the same Laplace(0,1)
    # generator (the CPU generator's stream; the distribution is the workload's)
    sample = [inputs.as_numpy_u16(inputs.laplace(r, P * L, device="cpu", chunk=1 << 24)) for r in range(P)]
    m = sample[0].size
    comps = [np.zeros(m, np.float32) for _ in range(P)] if ef else None
    odt = oracle.OUT_BF16 if out_bf16 else oracle.OUT_F32
    t0 = time.perf_counter()
    oracle.allreduce(sample, bits=bits, ef=ef, comps=comps, out_dtype=odt)
    dt = time.perf_counter() - t0
    B = bytes_per_elem(P, bits, ef, 2 if out_bf16 else 4)
    single = {"value": round(P * m * B / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
              "sample": f"one call on {m} of {n} elements per rank (1/{frac_den} of every segment, "
                        f"same distribution), P={P}, {dt:.2f} s single-threaded",
              "cpu": host_cpu_model()}
    # the same call as independent calls on mini messages made of the same
    # range of every segment (groups and elements are independent), one per
    # worker thread at a time; the oracle's C entry point releases the GIL
    from concurrent.futures import ThreadPoolExecutor
    workers = host_threads()
    chunk = max(G, (L // (8 * workers)) // G * G)
    comps = [np.zeros(m, np.float32) for _ in range(P)] if ef else None

    def one(a0):
        b0 = min(L, a0 + chunk)
        xm = [np.concatenate([x[s * L + a0:s * L + b0] for s in range(P)]) for x in sample]
        cm = [np.concatenate([c[s * L + a0:s * L + b0] for s in range(P)]) for c in comps] if ef else None
        oracle.allreduce(xm, bits=bits, ef=ef, comps=cm, out_dtype=odt)

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=workers) as pool:
        list(pool.map(one, range(0, L, chunk)))
    dtt = time.perf_counter() - t0
    threaded = {"value": round(P * m * B / dtt / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
                "sample": f"the same sample as {-(-L // chunk)} independent calls on ranges of {chunk} elements "
                          f"of every segment, {workers} threads, {dtt:.2f} s"}
    return single, threaded


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
    ap.add_argument("--tiles", type=int, default=1)
    ap.add_argument("--streams", type=int, default=1)
    ap.add_argument("--staged-tiles", type=int, default=4)
    ap.add_argument("--staged-streams", type=int, default=4)
    ap.add_argument("--no-staged", action="store_true", help="skip the staged-schedule leg")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the Table 8 quantizer/group-size legs")
    ap.add_argument("--out", choices=["bf16", "f32"], default="bf16")
    ap.add_argument("--no-ef", action="store_true")
    ap.add_argument("--no-modes", action="store_true",
                    help="skip the feedback-off, fp32-output and two-timescale legs")
    ap.add_argument("--no-p8", action="store_true", help="skip the P=8 leg")
    ap.add_argument("--no-tp", action="store_true", help="skip the fused matmul + entry pass leg")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
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
                        out_bf16, ef)
    staged = None
    if not a.no_staged:
        rs = run_case(echo, torch, inputs, a.P, N_1GIB, a.bits, a.staged_tiles, a.staged_streams,
                      max(5, a.steps // 2), a.warmup, out_bf16, ef, time_kernel=False)
        staged = {"tiles": a.staged_tiles, "streams": a.staged_streams, "value": round(rs["value"], 1),
                  "ms_per_step": round(rs["ms_per_step"], 4), "frac_of_peak": round(rs["value"] / HBM_PEAK_GBS, 4)}
    variants = None
    if not a.no_variants:
        variants = {}
        for name, quant, group in (("naive_zero_point", "naive", G), ("symmetric_grid", "symmetric", G),
                                   ("zero_aware_g256", "zero_aware", 256)):
            rv = run_case(echo, torch, inputs, a.P, N_1GIB, a.bits, a.tiles, a.streams, max(5, a.steps // 3),
                          a.warmup, out_bf16, ef, time_kernel=False, quant=quant, group=group)
            variants[name] = {"value": round(rv["value"], 1), "ms_per_step": round(rv["ms_per_step"], 4),
                              "frac_of_peak": round(rv["value"] / HBM_PEAK_GBS, 4)}
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
            modes[name] = {"value": round(rm["value"], 1), "ms_per_step": round(rm["ms_per_step"], 4),
                           "bytes_per_elem_per_rank": round(rm["B"], 5),
                           "frac_of_peak": round(rm["value"] / HBM_PEAK_GBS, 4)}
    copy_gbs = device_copy_gbs(torch)
    tp = None if a.no_tp else tp_block(echo, torch, inputs)
    p8 = None
    if not a.no_p8 and a.P != 8:
        r8 = run_case(echo, torch, inputs, 8, N_1GIB, a.bits, a.tiles, a.streams, max(5, a.steps // 2),
                      a.warmup, out_bf16, ef)
        p8 = {"value": round(r8["value"], 1), "ms_per_step": round(r8["ms_per_step"], 4),
              "frac_of_peak": round(r8["value"] / HBM_PEAK_GBS, 4), "roofline": r8["roofline"]}
    if a.calib_copy:
        src = torch.empty(N_1GIB, dtype=torch.int16, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cpu = cpu_threaded = None
    if not a.no_cpu:
        cpu, cpu_threaded = cpu_baseline(a.P, N_1GIB, a.bits, out_bf16, ef)

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
            "schedule": ("push, reduce and tail back to back on one stream, the fastest on one GPU; "
                         "the tile-staged multi-stream schedule is reported under 'staged'")
                        if (a.tiles, a.streams) == (1, 1) else "tile-staged across streams",
            "ef": "classic error feedback (alpha=1), -e written in place" if ef else "off",
            "out": a.out, "bytes_per_elem_per_rank": round(main_res["B"], 5),
            "bytes_per_call": int(main_res["bytes_per_call"]),
            "frac_of_peak": round(main_res["value"] / HBM_PEAK_GBS, 4),
            "call_ms": main_res["call_ms"],
            "device_copy_gbs": round(copy_gbs, 1),
            "frac_of_device_copy": round(main_res["value"] / copy_gbs, 4),
        },
        "roofline": main_res["roofline"],
        "cpu_baseline": cpu,
        "cpu_baseline_threaded": cpu_threaded,
        "staged": staged,
        "variants": variants,
        "modes": modes,
        "p8": p8,
        "tp_block": tp,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
