"""Benchmark of the TANGO / WANGO block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode] [--no-pages]
                    [--no-backward] [--no-three-set] [--no-configs]

One step runs every part of the block forward once at T = 8192 tokens:
  * TANGO, bf16 compute, B = 1, T = 8192, d = 512, F = 2048, q/k width 128,
    scale 10, the shared block applied 4 times (projection, full-prefix
    aggregation, output projection, four times over);
  * WANGO, bf16 compute, B = 1, T = 8192, same widths as two heads of 64,
    window 256, prefix-scan chunk 128, one application (projection, running-sum
    scan, window band + combine, output projection).
Inputs are seeded synthetic tensors already resident in HBM.  The value is
sequence tokens per second: (8192 + 8192) tokens / step time.

Alongside, with HIP events on the launch stream:
  * roofline: the TANGO aggregation kernel (the dominant one), useful MFMA
    flops 2 * (causal pairs) * (q/k width + F) per launch over its mean
    launch time: five batches of back-to-back launches, one event pair per
    batch on the launch stream (an event pair around every launch would add
    the dispatch latency, about 10 us, to each), the fastest and slowest batch
    beside it; against 2.5 PFLOP/s dense bf16;
  * roofline_scan: the WANGO running-sum scan (two launches), algorithmic
    HBM bytes (q, k, g read once; n_old, z_old written once) over its mean
    time, against 8 TB/s, timed the same way with a cold cache: the launches
    cycle through 8 copies of the scan's inputs and outputs, so every launch
    reads data the others have evicted from the 256 MB Infinity Cache (the
    warm-cache time, one copy over and over, is reported beside it);
  * ceilings: what the vendor's kernels reach here -- a 1 GiB device copy and
    a square 8192^3 bf16 GEMM (torch.matmul) -- as context for the fractions
    of the published peaks (off the measured path);
  * gemm_reference: context for the projection and output GEMMs -- the
    vendor library (torch.matmul) on plain bf16 GEMMs of the same shapes next
    to this build's stage calls (off the measured path);
  * other_configs: the TANGO B = 8, T = 2048 block and the WANGO B = 2,
    T = 65,536, window 512 stack of 8 applications, as tokens per second of
    the whole forward, with the long stack's scan per application (cold:
    each launch moves 1.68 GB) against 8 TB/s;
  * decode: one autoregressive decode step (every layer) at position 8192 of
    the decode workloads -- TANGO, 16 sequences, 4 stacked layers each with its
    own key/gate cache; WANGO, 64 sequences, window 256 -- as decoded tokens
    per second, and the algorithmic HBM bytes of the step (weights, the state
    each layer must touch, x and out) over its median time against 8 TB/s;
  * pages_geometry: one forward (4 applications) of the block in the pages'
    own geometry at T = 8192 (16 heads of 32, F = 28,480, window and block
    64), with the block's operation count as the pages tally it (Table 5
    without the vocabulary projection) per second;
  * three_set: the TANGO stack with three gated-projection sets (widths 704,
    640 and 704 for the first, middle and last of 8 applications) through the
    single call tango_stack_fwd, as tokens per second and per-application
    speed against the one-set block (F = 2048);
  * backward: the TANGO aggregation's backward pass at the same T = 8192
    shape (dq, dk, dg, dtheta from dgbar; the forward that saves the
    denominators runs once, untimed), with its algorithmic flops
    2 * pairs * (2 F + 3 * q/k width) per second against 2.5 PFLOP/s;
  * backward_wango: the WANGO aggregation's backward pass at the WANGO shape
    above (two heads of 64, window 256, chunk 128), with the algorithmic
    flops of wango_backward_flops;
  * cpu_baseline: the float64 CPU oracle on a bounded sample of the same work
    (one of the four TANGO applications, scaled by 4, plus the WANGO block).
The "traffic" of the two rooflines is the HBM traffic per launch measured by
rocprofv3 counters (FETCH_SIZE and WRITE_SIZE, scaled by what they read for a
plain copy of known size, which --copy-calibration runs), read from
profiles/hbm_traffic_t8192.md; it is reported only while the sha256 of the
kernel's sources still matches the one recorded there, else null.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12    # MI355X HBM3E

TANGO = "tango_bf16_t8192_r4"
WANGO = "wango_bf16_t8192_w256"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the part reaches its sustained clock some 40 ms into a run of these steps (about 30
    # steps); the default warm-up covers that, so that the timed steps see the sustained rate
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-loops", type=int, default=None,
                    help="launches per roofline measurement (default: --steps, at most 20)")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step measurement")
    ap.add_argument("--no-pages", action="store_true", help="skip the pages'-geometry forward")
    ap.add_argument("--no-backward", action="store_true", help="skip the aggregation backward")
    ap.add_argument("--no-three-set", action="store_true", help="skip the three-set stack")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the B=8 T=2048 TANGO and B=2 T=65536 WANGO workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (for counter calibration)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_t8192.md")
KERNEL_SOURCES = {
    "agg_kernel": ["agg_kernels.hip", "common.hpp", "kernels.hpp"],
    "scan": ["scan_kernels.hip", "common.hpp", "kernels.hpp"],
}


def source_hash(key: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[key]:
        with open(os.path.join(ROOT, "cross_token_gated_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(key: str):
    """HBM bytes per launch recorded for `key`, or None if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    for line in lines:
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 5 and cells[0] == key:
            try:
                return float(cells[4]) if cells[1] == source_hash(key) else None
            except ValueError:
                return None
    return None


def tango_flops(w) -> float:
    pairs = w.B * w.T * (w.T + 1) // 2
    return 2.0 * pairs * (w.n_heads * w.head_dim + w.d_gate)


def scan_bytes(w) -> float:
    """Algorithmic HBM bytes of the running-sum scan: query and key features
    read once (2 x H*d_h, bf16), gates read once (F, bf16), n_old written once
    (F, float32), z_old written once (H, float32), per token."""
    hd = w.n_heads * w.head_dim
    return float(w.B * w.T * (2 * hd * 2 + w.d_gate * 2 + w.d_gate * 4 + w.n_heads * 4))


def host_cpu() -> dict:
    """The host's CPU model (from /proc/cpuinfo), the threads this process may
    run on, and the BLAS numpy calls (library, version, threads)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = {"library": "unknown", "version": None, "threads": None}
    try:
        import numpy  # noqa: F401  (loads the BLAS that threadpoolctl then reports)
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = {"library": i.get("internal_api"), "version": i.get("version"),
                        "threads": i.get("num_threads"), "architecture": i.get("architecture")}
                break
    except Exception:  # noqa: BLE001
        pass
    return {"cpu_model": model, "affinity_threads": len(os.sched_getaffinity(0)), "blas": blas}


def cpu_baseline(wt, wg) -> dict:
    """The float64 oracle, untuned, on a bounded sample of the step."""
    import numpy as np

    import oracle.tango_oracle as O
    from cross_token_gated_amd import workload as wl
    from tests import helpers as H

    info = host_cpu()
    cores = info["blas"]["threads"] or info["affinity_threads"]
    # one TANGO application (timed x repeats) plus the WANGO application,
    # repeated until about 10 s of host time have passed; the mean is reported
    cases = []
    for w, scale in ((wt, wt.repeats), (wg, 1)):
        inp = wl.make_inputs(w)
        cases.append((np.asarray(inp.h[0], dtype=np.float64), H.oracle_params(inp), H.oracle_config(w), scale))
    step_secs, spent, runs = 0.0, 0.0, 0
    while runs == 0 or (spent < 10.0 and runs < 8):
        secs = 0.0
        for h, p, cfg, scale in cases:
            t0 = time.perf_counter()
            O.block_sequence(h, p, cfg)
            dt = time.perf_counter() - t0
            spent += dt
            secs += dt * scale
        step_secs += secs
        runs += 1
    secs = step_secs / runs
    tokens = wt.tokens + wg.tokens
    return {"value": tokens / secs, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": info["cpu_model"], "blas": info["blas"], "affinity_threads": info["affinity_threads"],
            "sample": (f"one of the {wt.repeats} TANGO T={wt.T} applications (time x{wt.repeats}) "
                       f"plus the WANGO T={wg.T} application, float64 numpy, mean of {runs} runs "
                       f"({spent:.1f} s of host time); {secs:.1f} s for one step")}


def _align256(n: int) -> int:
    return (n + 255) // 256 * 256


def decode_bytes(w, es: int, io_es: int) -> float:
    """Algorithmic HBM bytes of one decode step over all layers: the weights
    once per layer, the state each layer must touch (TANGO: keys and gates of
    positions 0..p read, the new row written; WANGO: S read and written, the
    window's and the leaving token's keys and gates read, the new row
    written), x read and out written."""
    p = w.T - 1
    HD, F, d = w.n_heads * w.head_dim, w.d_gate, w.d_model
    weights = ((2 * F + 2 * HD) * d + d * F) * es
    row = (HD + F) * es
    if w.mode == "tango":
        state = w.B * (p + 1) * row + w.B * row
    else:
        state = 2 * w.B * w.n_heads * w.head_dim * (F // w.n_heads) * 4 + w.B * (w.window + 2) * row
    return float(w.repeats * (weights + state + 2 * w.B * d * io_es))


def pages_block_macs(w) -> float:
    """MACs of w.repeats block applications as the pages count them ([TANGO]
    §3 and Table 5): linear projections T(2dF + 2dHd_h + Fd); pairs over the
    full T x T grid for TANGO, 3W pairs per token plus the running-sum update
    and read-out 2 d_h F per token for WANGO.  The output vocabulary
    projection that Table 5 adds is not part of the block and is left out."""
    T, d, F, H, dh = w.T, w.d_model, w.d_gate, w.n_heads, w.head_dim
    linear = T * (2 * d * F + 2 * d * H * dh + F * d)
    if w.mode == "tango":
        pairs = T * T * (H * dh + F)
    else:
        pairs = T * 3 * w.window * (H * dh + F) + T * 2 * dh * F
    return float(w.repeats * (linear + pairs))


def pages_bench(steps: int, warmup: int, dev, stream) -> dict:
    """One forward (all 4 applications) of the pages' geometry at T = 8192:
    16 heads of 32, F = 28,480, window and prefix-sum block 64."""
    import torch

    from cross_token_gated_amd import api
    from cross_token_gated_amd import workload as wl
    from cross_token_gated_amd.device import block_weights, dev_tensor

    out = {}
    for name, w in wl.PAGES_WORKLOADS.items():
        inp = wl.make_inputs(w)
        bw = block_weights(w, inp, dev)
        x = dev_tensor(inp.h, w.io, dev)
        ping, pong = torch.empty_like(x), torch.empty_like(x)
        shape = api.shape_of(x, bw, w.rope_base, w.rms_eps, w.operand_parts)
        n = (api.tango_workspace_size(shape) if w.mode == "tango"
             else api.wango_workspace_size(shape, w.window, w.head_dim, w.chunk))
        ws = api.workspace(n, dev)

        def fwd():
            src = x
            for r in range(w.repeats):
                dst = ping if r % 2 == 0 else pong
                if w.mode == "tango":
                    api.tango_block_fwd(src, bw, out=dst, ws=ws, rope_base=w.rope_base, rms_eps=w.rms_eps, operand_parts=w.operand_parts,
                                        stream=stream)
                else:
                    api.wango_block_fwd(src, bw, w.window, w.head_dim, w.chunk, out=dst, ws=ws,
                                        rope_base=w.rope_base, rms_eps=w.rms_eps, operand_parts=w.operand_parts, stream=stream)
                src = dst

        for _ in range(warmup):
            fwd()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            fwd()
            b.record(stream)
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ev)
        ms = t[steps // 2] if steps % 2 else 0.5 * (t[steps // 2 - 1] + t[steps // 2])
        macs = pages_block_macs(w)
        out[name] = {"ms_per_forward": ms, "tokens_per_s": w.tokens / (ms * 1e-3),
                     "applications": w.repeats, "pages_block_macs": macs,
                     "pages_macs_per_s": macs / (ms * 1e-3)}
        print(f"[bench] pages geometry {name}: {ms:.2f} ms per forward ({w.repeats} applications), "
              f"{w.tokens / (ms * 1e-3):.0f} tokens/s, {macs / (ms * 1e-3) / 1e12:.0f} T MAC/s of the pages' "
              f"count", file=sys.stderr, flush=True)
        del ws, x, ping, pong
        torch.cuda.empty_cache()
    return out


def configs_bench(steps: int, warmup: int, dev, stream, timed_batches) -> dict:
    """The other two block workloads at full size: TANGO B = 8, T = 2048 (one
    application) and WANGO B = 2, T = 65,536, window 512, eight shared
    applications -- tokens per second of the whole forward (mean over batches
    of back-to-back forwards).  For the long WANGO workload also its
    running-sum scan per application, launched back to back: each launch moves
    1.68 GB, so the previous one has evicted its inputs from the 256 MB
    Infinity Cache and every launch reads from HBM; algorithmic bytes over the
    mean launch time against 8 TB/s."""
    import torch

    from cross_token_gated_amd import api
    from cross_token_gated_amd import workload as wl
    from cross_token_gated_amd.device import block_weights, dev_tensor

    out = {}
    for name in ("tango_bf16_b8_t2048", "wango_bf16_b2_t65536_w512_r8"):
        w = wl.WORKLOADS[name]
        inp = wl.make_inputs(w)
        bw = block_weights(w, inp, dev)
        x = dev_tensor(inp.h, w.io, dev)
        ping, pong = torch.empty_like(x), torch.empty_like(x)
        shape = api.shape_of(x, bw, w.rope_base, w.rms_eps, w.operand_parts)
        n = (api.tango_workspace_size(shape) if w.mode == "tango"
             else api.wango_workspace_size(shape, w.window, w.head_dim, w.chunk))
        ws = api.workspace(n, dev)

        def fwd():
            src = x
            for r in range(w.repeats):
                dst = ping if r % 2 == 0 else pong
                if w.mode == "tango":
                    api.tango_block_fwd(src, bw, out=dst, ws=ws, rope_base=w.rope_base, rms_eps=w.rms_eps, operand_parts=w.operand_parts,
                                        stream=stream)
                else:
                    api.wango_block_fwd(src, bw, w.window, w.head_dim, w.chunk, out=dst, ws=ws,
                                        rope_base=w.rope_base, rms_eps=w.rms_eps, operand_parts=w.operand_parts, stream=stream)
                src = dst

        for _ in range(warmup):
            fwd()
        ms, ms_lo, ms_hi = timed_batches(fwd, steps, 3)
        rec = {"ms_per_forward": ms, "ms_batch_min": ms_lo, "ms_batch_max": ms_hi,
               "tokens_per_s": w.tokens / (ms * 1e-3),
               "applications": w.repeats, "B": w.B, "T": w.T, "d_gate": w.d_gate,
               "heads": w.n_heads, "head_dim": w.head_dim}
        msg = f"[bench] {name}: {ms:.3f} ms per forward, {w.tokens / (ms * 1e-3):.0f} tokens/s"
        if w.mode == "wango":
            M = w.B * api.padded_len(w.T)
            HD = w.n_heads * w.head_dim
            gp = torch.empty(M * w.d_gate, dtype=torch.bfloat16, device=dev)
            v = torch.empty(M, w.d_gate, dtype=api.v_dtype(shape), device=dev)
            qh = torch.empty(M, HD, dtype=torch.bfloat16, device=dev)
            kh = torch.empty(M, HD, dtype=torch.bfloat16, device=dev)
            fq = torch.empty(M, HD, dtype=torch.bfloat16, device=dev)
            fk = torch.empty(M * HD, dtype=torch.bfloat16, device=dev)
            api.wango_stage_proj(shape, bw, x, gp, v, qh, kh, fq, fk, ws=ws, stream=stream)
            del v, qh, kh
            n_old = torch.empty(M * w.d_gate, dtype=torch.float32, device=dev)
            z_old = torch.empty(M, w.n_heads, dtype=torch.float32, device=dev)
            scan = lambda: api.wango_stage_scan(shape, w.window, w.chunk, fq, fk, gp, n_old, z_old,  # noqa: E731
                                                ws, stream=stream)
            sms, smin, smax = timed_batches(scan, steps, 3)
            sb = scan_bytes(w)
            rec["scan"] = {"bound": "hbm", "bytes_per_launch": sb, "ms_per_launch": sms,
                           "ms_batch_min": smin, "ms_batch_max": smax,
                           "achieved": sb / (sms * 1e-3) / 1e9, "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                           "frac": sb / (sms * 1e-3) / PEAK_HBM_BYTES,
                           "cache": "cold: each launch moves 1.68 GB, over 6x the Infinity Cache"}
            msg += (f"; scan {sms * 1e3:.0f} us per application ({sb / 1e6:.0f} MB, "
                    f"{100 * rec['scan']['frac']:.1f}% of HBM peak)")
            del gp, fq, fk, n_old, z_old
        out[name] = rec
        print(msg, file=sys.stderr, flush=True)
        del ws, x, ping, pong
        torch.cuda.empty_cache()
    return out


def gemm_reference(steps: int, dev, stream, timed_batches, ours: dict) -> dict:
    """Context for the two GEMM kernels, outside the timed step: the vendor
    library's dense bf16 GEMM (torch.matmul, i.e. hipBLASLt) on plain products
    of the same shapes -- the projection with its two-part activation operand
    stacked along K (8192 x 1024 times 1024 x 4352), the output product
    likewise (8192 x 4096 times 4096 x 512) -- with the weights stored [N, K]
    as the library takes them, next to this build's kernels on the same shapes
    (which also do their epilogues: SiLU and the packed gate layout, RoPE and
    unit length; the gated product and the residual).  None of this is on the
    measured path."""
    import torch

    out = {}
    for name, (M, K, N) in (("projection", (8192, 1024, 4352)), ("output", (8192, 4096, 512))):
        A = torch.randn(M, K, device=dev, dtype=torch.bfloat16)
        Wt = torch.randn(N, K, device=dev, dtype=torch.bfloat16)
        C = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
        ms, _, _ = timed_batches(lambda: torch.matmul(A, Wt.t(), out=C), steps, 3)
        flops = 2.0 * M * N * K
        out[name] = {"shape_mkn": [M, K, N], "library_ms": ms,
                     "library_frac_of_bf16_peak": flops / (ms * 1e-3) / PEAK_BF16_FLOPS,
                     "this_build_ms": ours[name],
                     "this_build_frac_of_bf16_peak": flops / (ours[name] * 1e-3) / PEAK_BF16_FLOPS}
        print(f"[bench] {name} GEMM shape {M}x{K}x{N}: library {ms * 1e3:.1f} us "
              f"({100 * out[name]['library_frac_of_bf16_peak']:.1f}% of peak), this build {ours[name] * 1e3:.1f} us",
              file=sys.stderr, flush=True)
        del A, Wt, C
    return out


def ceilings(dev, stream, timed_batches) -> dict:
    """What the vendor's own kernels reach on this part, as context for the
    fractions of the published peaks: a plain device copy of 1 GiB (torch
    copy_: 1 GiB read, 1 GiB written, cold by size against the 256 MB Infinity
    Cache) and a square bf16 GEMM (8192^3, torch.matmul -> hipBLASLt).  Off the
    measured path."""
    import torch

    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ms_c, _, _ = timed_batches(lambda: dst.copy_(src), 10, 3)
    del src, dst
    m = 8192
    A = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    Bm = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    C = torch.empty(m, m, device=dev, dtype=torch.bfloat16)
    ms_g, _, _ = timed_batches(lambda: torch.matmul(A, Bm, out=C), 10, 3)
    del A, Bm, C
    copy_gbs = 2 * 4 * n / (ms_c * 1e-3) / 1e9
    gemm_tf = 2.0 * m ** 3 / (ms_g * 1e-3) / 1e12
    out = {"copy_1gib": {"ms": ms_c, "GB_per_s": copy_gbs, "frac_of_hbm_peak": copy_gbs * 1e9 / PEAK_HBM_BYTES},
           "gemm_bf16_8192": {"ms": ms_g, "TFLOP_per_s": gemm_tf,
                              "frac_of_bf16_peak": gemm_tf * 1e12 / PEAK_BF16_FLOPS}}
    print(f"[bench] ceilings: device copy {copy_gbs:.0f} GB/s ({100 * out['copy_1gib']['frac_of_hbm_peak']:.1f}% of "
          f"the HBM peak), bf16 GEMM 8192^3 {gemm_tf:.0f} TFLOP/s "
          f"({100 * out['gemm_bf16_8192']['frac_of_bf16_peak']:.1f}% of the bf16 peak)", file=sys.stderr, flush=True)
    return out


def three_set_bench(steps: int, warmup: int, dev, stream, ms_one_set_app: float) -> dict:
    """The three-set TANGO stack at T = 8192 (eight applications; gate widths
    704, 640, 704 for the first, middle and last applications) through the one
    C call tango_stack_fwd, against the one-set block (F = 2048) per
    application."""
    import torch

    from cross_token_gated_amd import api
    from cross_token_gated_amd import workload as wl
    from cross_token_gated_amd.device import block_weights, dev_tensor

    out = {}
    for name, sw in wl.STACK_WORKLOADS.items():
        inps = wl.make_stack_inputs(sw)
        sets = [block_weights(sw.set_workload(k), inps[k], dev) for k in range(len(sw.widths))]
        w = sw.base
        x = dev_tensor(inps[0].h, w.io, dev)
        y = torch.empty_like(x)
        shapes = [api.shape_of(x, b, w.rope_base, w.rms_eps, w.operand_parts) for b in sets]
        ws = api.workspace(api.tango_stack_workspace_size(shapes), dev)

        def fwd():
            api.tango_stack_fwd(x, sets, sw.schedule, out=y, ws=ws, rope_base=w.rope_base,
                                rms_eps=w.rms_eps, operand_parts=w.operand_parts, stream=stream)

        for _ in range(warmup):
            fwd()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            fwd()
            b.record(stream)
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ev)
        ms = t[steps // 2] if steps % 2 else 0.5 * (t[steps // 2 - 1] + t[steps // 2])
        n = len(sw.schedule)
        out[name] = {"ms_per_forward": ms, "tokens_per_s": sw.tokens / (ms * 1e-3), "applications": n,
                     "widths": list(sw.widths), "schedule": list(sw.schedule),
                     "ms_per_application": ms / n,
                     "speedup_per_application_vs_one_set_f2048": ms_one_set_app / (ms / n)}
        print(f"[bench] three-set stack {name}: {ms:.3f} ms per forward ({n} applications), "
              f"{sw.tokens / (ms * 1e-3):.0f} tokens/s, {ms_one_set_app / (ms / n):.2f}x the one-set "
              f"block per application", file=sys.stderr, flush=True)
        del ws, x, y
        torch.cuda.empty_cache()
    return out


def backward_bench(steps: int, warmup: int, dev, stream) -> dict:
    """Backward pass of the TANGO aggregation at the T = 8192 bench shape (one
    head of 128, F = 2048, bf16): the forward that saves the denominators is
    run once; the backward (all its kernels) is timed, median of `steps`."""
    import numpy as np
    import torch

    from cross_token_gated_amd import api
    from cross_token_gated_amd import layouts as lay
    from cross_token_gated_amd import workload as wl

    c = wl.BACKWARD_SHAPE
    T, F, Hh, dh = c["T"], c["F"], c["H"], c["dh"]
    Tp = lay.padded_len(T)
    q, k, g, dg_in = wl.aggregate_inputs(T, F, Hh, dh, c["seed"])
    bf = torch.bfloat16
    qd = torch.from_numpy(lay.pad_rows(q.reshape(1, T, Hh * dh), Tp).reshape(Tp, Hh * dh)).to(dev).to(bf)
    kd = torch.from_numpy(lay.pad_rows(k.reshape(1, T, Hh * dh), Tp).reshape(Tp, Hh * dh)).to(dev).to(bf)
    gp = torch.from_numpy(lay.pack_gates(lay.pad_rows(g[None], Tp)).reshape(-1)).to(dev).to(bf)
    dgbar = torch.from_numpy(lay.pad_rows(dg_in[None], Tp).reshape(Tp, F)).to(dev).to(bf)
    theta = torch.full((Hh,), math.log(10.0), dtype=torch.float32, device=dev)
    shape = api.make_shape(1, T, 512, F, Hh, dh, bf)
    gbar = torch.empty((Tp, F), dtype=bf, device=dev)
    den = torch.empty((Tp, Hh), dtype=torch.float32, device=dev)
    wsf = api.workspace(api.tango_workspace_size(shape), dev)
    api.tango_aggregate_fwd_train(shape, theta, None, qd, kd, gp, gbar, den, wsf, stream=stream)
    dq = torch.empty((Tp, Hh * dh), dtype=torch.float32, device=dev)
    dk = torch.empty_like(dq)
    dg = torch.empty((Tp, F), dtype=bf, device=dev)
    dth = torch.empty((Hh,), dtype=torch.float32, device=dev)
    wsb = api.workspace(api.tango_aggregate_bwd_workspace_size(shape), dev)

    def bwd():
        api.tango_aggregate_bwd(shape, theta, None, qd, kd, gp, gbar, den, dgbar, dq, dk, dg, dth, None, wsb,
                                stream=stream)

    for _ in range(warmup):
        bwd()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        bwd()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    ms = t[steps // 2] if steps % 2 else 0.5 * (t[steps // 2 - 1] + t[steps // 2])
    pairs = T * (T + 1) / 2
    # algorithmic work of the gradients: dg and u.g over F per pair, s, dq, dk over d_h
    flops = 2.0 * pairs * Hh * (2 * F // Hh + 3 * dh)
    achieved = flops / (ms * 1e-3)
    out = {"workload": "tango_aggregate_bwd_bf16_t8192_f2048_h1", "ms_per_backward": ms,
           "tokens_per_s": T / (ms * 1e-3),
           "roofline": {"kernel": "whole aggregation backward (prep, reversed aggregation, dq, dk, finish)",
                        "bound": "mfma", "achieved": achieved / 1e12, "peak": PEAK_BF16_FLOPS / 1e12,
                        "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_FLOPS, "flops_per_backward": flops}}
    print(f"[bench] backward tango_aggregate_bwd T=8192 F=2048: {ms:.3f} ms, {achieved / 1e12:.0f} TFLOP/s "
          f"({achieved / PEAK_BF16_FLOPS * 100:.1f}% of bf16 peak)", file=sys.stderr, flush=True)
    del wsf, wsb
    torch.cuda.empty_cache()
    return out


def wango_backward_flops(T: int, F: int, H: int, dh: int, W: int) -> float:
    """Algorithmic flops of the WANGO aggregation backward: per head, every
    window pair forms u.g and its dg term over the head's F/H gate columns and
    s, dq, dk over d_h (2 (2 F/H + 3 d_h) each); the older prefix is linear:
    per position the two state sums and their two read-outs (d_h x F/H each
    way) and the state update and read-out of dg, 12 d_h F/H in all."""
    fh = F // H
    pairs = sum(min(i + 1, W) for i in range(T))
    return float(H * (2 * pairs * (2 * fh + 3 * dh) + 12 * T * dh * fh))


def wango_backward_bench(steps: int, warmup: int, dev, stream) -> dict:
    """Backward pass of the WANGO aggregation at the T = 8192 WANGO bench shape
    (two heads of 64, F = 2048, window 256, chunk 128, bf16): the forward that
    saves the denominators runs once; the backward is timed, median of `steps`."""
    import torch

    from cross_token_gated_amd import api
    from cross_token_gated_amd import workload as wl
    from cross_token_gated_amd import layouts as lay

    c = wl.WANGO_BACKWARD_SHAPE
    T, F, Hh, dh, W, C = c["T"], c["F"], c["H"], c["dh"], c["window"], c["chunk"]
    Tp = lay.padded_len(T)
    q, k, g, dg_in = wl.aggregate_inputs(T, F, Hh, dh, c["seed"])
    bf = torch.bfloat16
    qd = torch.from_numpy(lay.pad_rows(q.reshape(1, T, Hh * dh), Tp)).to(dev).to(bf)
    kd = torch.from_numpy(lay.pad_rows(k.reshape(1, T, Hh * dh), Tp)).to(dev).to(bf)
    gp = torch.from_numpy(lay.pack_gates(lay.pad_rows(g[None], Tp)).reshape(-1)).to(dev).to(bf)
    dgbar = torch.from_numpy(lay.pad_rows(dg_in[None], Tp)).to(dev).to(bf)
    theta = torch.full((Hh,), math.log(10.0), dtype=torch.float32, device=dev)
    shape = api.make_shape(1, T, 512, F, Hh, dh, bf)
    gbar = torch.empty((Tp, F), dtype=bf, device=dev)
    den = torch.empty((Tp, Hh), dtype=torch.float32, device=dev)
    wsf = api.workspace(api.wango_aggregate_fwd_train_workspace_size(shape, W, C), dev)
    api.wango_aggregate_fwd_train(shape, W, C, theta, None, qd, kd, gp, gbar, den, wsf, stream=stream)
    dq = torch.empty((Tp, Hh * dh), dtype=torch.float32, device=dev)
    dk = torch.empty_like(dq)
    dg = torch.empty((Tp, F), dtype=bf, device=dev)
    dth = torch.empty((Hh,), dtype=torch.float32, device=dev)
    wsb = api.workspace(api.wango_aggregate_bwd_workspace_size(shape, W, C), dev)

    def bwd():
        api.wango_aggregate_bwd(shape, W, C, theta, None, qd, kd, gp, gbar, den, dgbar, dq, dk, dg, dth, None,
                                wsb, stream=stream)

    for _ in range(warmup):
        bwd()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        bwd()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    ms = t[steps // 2] if steps % 2 else 0.5 * (t[steps // 2 - 1] + t[steps // 2])
    flops = wango_backward_flops(T, F, Hh, dh, W)
    achieved = flops / (ms * 1e-3)
    out = {"workload": "wango_aggregate_bwd_bf16_t8192_f2048_h2_w256", "ms_per_backward": ms,
           "tokens_per_s": T / (ms * 1e-3),
           "roofline": {"kernel": "whole WANGO aggregation backward", "bound": "mfma",
                        "achieved": achieved / 1e12, "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                        "frac": achieved / PEAK_BF16_FLOPS, "flops_per_backward": flops}}
    print(f"[bench] backward wango_aggregate_bwd T=8192 F=2048 W=256: {ms:.3f} ms, "
          f"{achieved / 1e12:.0f} TFLOP/s ({achieved / PEAK_BF16_FLOPS * 100:.1f}% of bf16 peak)",
          file=sys.stderr, flush=True)
    del wsf, wsb
    torch.cuda.empty_cache()
    return out


def decode_bench(steps: int, warmup: int, dev, stream) -> dict:
    """One decode step (every layer) at position T - 1 of the decode workloads,
    timed with HIP events.  The state is filled with synthetic content of the
    right kind (unit keys, SiLU gates, positive running sums) rather than by
    decoding 8192 positions first: every decode kernel does the same work
    whatever the values (the parity tests decode real prefixes)."""
    import torch

    from cross_token_gated_amd import api
    from cross_token_gated_amd import workload as wl
    from cross_token_gated_amd.device import TORCH_DTYPE, block_weights

    out = {}
    for name, w in wl.DECODE_WORKLOADS.items():
        inp = wl.make_inputs(w.scaled(T=1))          # weights and one input row per sequence
        bw = block_weights(w, inp, dev)
        io = TORCH_DTYPE[w.io]
        es, io_es = (2 if w.dtype == "bf16" else 4), (2 if w.io == "bf16" else 4)
        cap = w.T if w.mode == "tango" else 1
        shape = api.decode_shape(w.B, cap, bw, io, w.d_model, w.rope_base, w.rms_eps)
        if w.mode == "tango":
            ns, nw = api.tango_decode_state_size(shape), api.tango_decode_workspace_size(shape)
            rows = w.T
        else:
            ns = api.wango_decode_state_size(shape, w.window, w.head_dim)
            nw = api.wango_decode_workspace_size(shape, w.window, w.head_dim)
            rows = w.window + 1
        HD, F = w.n_heads * w.head_dim, w.d_gate
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.seed)
        states = []
        for _ in range(w.repeats):
            st = torch.empty(ns, dtype=torch.uint8, device=dev)
            kb = w.B * rows * HD * es
            k = st[:kb].view(TORCH_DTYPE[w.dtype]).view(w.B * rows, w.n_heads, w.head_dim)
            g = st[_align256(kb):_align256(kb) + w.B * rows * F * es].view(TORCH_DTYPE[w.dtype]).view(w.B * rows, F)
            for r0 in range(0, w.B * rows, 8192):
                r1 = min(w.B * rows, r0 + 8192)
                kk = torch.randn(r1 - r0, w.n_heads, w.head_dim, device=dev, generator=gen)
                k[r0:r1] = torch.nn.functional.normalize(kk, dim=-1).to(k.dtype)
                g[r0:r1] = torch.nn.functional.silu(torch.randn(r1 - r0, F, device=dev, generator=gen)).to(g.dtype)
            if w.mode == "wango":
                so = _align256(_align256(kb) + w.B * rows * F * es)
                ne = w.B * w.n_heads * w.head_dim * (F // w.n_heads)
                st[so:so + ne * 4].view(torch.float32).copy_(
                    torch.rand(ne, device=dev, generator=gen) * (w.T - w.window) * 0.02)
                zo = _align256(so + ne * 4)
                nz = w.B * 2 * w.n_heads * w.head_dim
                st[zo:zo + nz * 4].view(torch.float32).copy_(
                    torch.rand(nz, device=dev, generator=gen) * (w.T - w.window) * 0.02)
            states.append(st)
        ws = api.workspace(nw, dev)
        x = torch.randn(w.B, w.d_model, device=dev, generator=gen).to(io)
        y = torch.empty_like(x)
        pos = torch.full((w.B,), w.T - 1, dtype=torch.int32, device=dev)

        def step():
            cur, nxt = x, y
            for r in range(w.repeats):
                if w.mode == "tango":
                    api.tango_decode_step(shape, bw, pos, cur, nxt, states[r], ws, stream)
                else:
                    api.wango_decode_step(shape, bw, w.window, w.head_dim, pos, cur, nxt, states[r], ws,
                                          stream)
                cur, nxt = nxt, cur

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ev)
        ms = t[steps // 2] if steps % 2 else 0.5 * (t[steps // 2 - 1] + t[steps // 2])
        nbytes = decode_bytes(w, es, io_es)
        ach = nbytes / (ms * 1e-3)
        out[name] = {
            "tokens_per_s": w.B / (ms * 1e-3), "ms_per_step": ms, "sequences": w.B, "position": w.T - 1,
            "layers": w.repeats, "window": w.window or None,
            "roofline": {"kernel": "whole decode step (row prep, projections, aggregation, output) x layers",
                         "bound": "hbm", "achieved": ach / 1e9, "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                         "frac": ach / PEAK_HBM_BYTES, "bytes_per_step": nbytes}}
        print(f"[bench] decode {name}: {ms * 1e3:.1f} us/step, {w.B / (ms * 1e-3):.0f} tokens/s, "
              f"{ach / 1e9:.0f} GB/s ({100 * ach / PEAK_HBM_BYTES:.1f}% of HBM peak)", file=sys.stderr, flush=True)
        del states, ws
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the block forward on one sequence batch needs no collectives)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from cross_token_gated_amd import api
    from cross_token_gated_amd import workload as wl
    from cross_token_gated_amd.device import block_weights, dev_f32, dev_tensor

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    wt, wg = wl.WORKLOADS[TANGO], wl.WORKLOADS[WANGO]
    it, ig = wl.make_inputs(wt), wl.make_inputs(wg)
    bt, bg = block_weights(wt, it), block_weights(wg, ig)
    xt = dev_tensor(it.h, wt.io)
    xg = dev_tensor(ig.h, wg.io)
    ping, pong, outg = torch.empty_like(xt), torch.empty_like(xt), torch.empty_like(xg)
    st = api.shape_of(xt, bt, wt.rope_base, wt.rms_eps, wt.operand_parts)
    sg = api.shape_of(xg, bg, wg.rope_base, wg.rms_eps, wg.operand_parts)
    ws_t = api.workspace(api.tango_workspace_size(st), dev)
    ws_g = api.workspace(api.wango_workspace_size(sg, wg.window, wg.head_dim, wg.chunk), dev)
    stream = torch.cuda.current_stream()

    def step():
        src = xt
        for r in range(wt.repeats):            # x -> ping -> pong -> ping -> pong
            dst = ping if r % 2 == 0 else pong
            api.tango_block_fwd(src, bt, out=dst, ws=ws_t, rope_base=wt.rope_base,
                                rms_eps=wt.rms_eps, operand_parts=wt.operand_parts, stream=stream)
            src = dst
        api.wango_block_fwd(xg, bg, wg.window, wg.head_dim, wg.chunk, out=outg, ws=ws_g,
                            rope_base=wg.rope_base, rms_eps=wg.rms_eps, operand_parts=wg.operand_parts, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = e0.elapsed_time(e1) / args.steps
    tokens = wt.tokens + wg.tokens
    print(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step (host wall {1e3 * wall / args.steps:.3f})",
          file=sys.stderr, flush=True)

    # ---- per-workload breakdown and the dominant kernels, same stream ----
    loops = args.kernel_loops or min(args.steps, 20)
    Tp = api.padded_len(wt.T)
    M = wt.B * Tp
    F, HD = wt.d_gate, wt.n_heads * wt.head_dim
    gp = torch.empty(M * F, dtype=torch.bfloat16, device=dev)
    v = torch.empty(M, F, dtype=api.v_dtype(st), device=dev)
    qh = torch.empty(M, HD, dtype=torch.bfloat16, device=dev)
    kh = torch.empty(M, HD, dtype=torch.bfloat16, device=dev)
    gbar = torch.empty(M, F, dtype=torch.bfloat16, device=dev)
    api.tango_stage_proj(st, bt, xt, gp, v, qh, kh, ws=ws_t, stream=stream)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def timed_batches(fn, n, batches):
        """Mean launch time of fn over `batches` batches of n back-to-back
        launches, one event pair around each batch on the launch stream (events
        around single launches would add the dispatch latency, ~10 us, to each):
        (mean over all launches, fastest batch mean, slowest batch mean)."""
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(batches)]
        for a, b in ev:
            a.record(stream)
            for _ in range(n):
                fn()
            b.record(stream)
        torch.cuda.synchronize()
        t = [a.elapsed_time(b) / n for a, b in ev]
        return sum(t) / batches, min(t), max(t)

    def tango_only():
        src = xt
        for r in range(wt.repeats):
            dst = ping if r % 2 == 0 else pong
            api.tango_block_fwd(src, bt, out=dst, ws=ws_t, stream=stream, operand_parts=wt.operand_parts)
            src = dst

    ms_tango = timed(tango_only, loops)
    ms_wango = timed(lambda: api.wango_block_fwd(xg, bg, wg.window, wg.head_dim, wg.chunk, out=outg,
                                                 ws=ws_g, stream=stream, operand_parts=wg.operand_parts),
                     loops)
    n_batches = 5
    ms_agg, agg_min, agg_max = timed_batches(
        lambda: api.tango_stage_aggregate(st, bt.theta, None, qh, kh, gp, gbar, ws_t, stream=stream),
        loops, n_batches)
    # WANGO scan inputs (two heads of 64).  For the cold-cache time the scan
    # cycles through NCOPY copies of its inputs and outputs: between two uses of
    # one copy the other copies move about 7 x 105 MB through the memory system,
    # more than twice the 256 MB Infinity Cache, so every launch reads its inputs
    # from HBM, and the launches still run back to back between one event pair.
    NCOPY = 8
    Mg = wg.B * api.padded_len(wg.T)
    HDg = wg.n_heads * wg.head_dim
    gpg = torch.empty(Mg * wg.d_gate, dtype=torch.bfloat16, device=dev)
    vg = torch.empty(Mg, wg.d_gate, dtype=api.v_dtype(sg), device=dev)
    qg = torch.empty(Mg, HDg, dtype=torch.bfloat16, device=dev)
    kg = torch.empty(Mg, HDg, dtype=torch.bfloat16, device=dev)
    fqg = torch.empty(Mg, HDg, dtype=torch.bfloat16, device=dev)
    fkg = torch.empty(Mg * HDg, dtype=torch.bfloat16, device=dev)
    api.wango_stage_proj(sg, bg, xg, gpg, vg, qg, kg, fqg, fkg, ws=ws_g, stream=stream)
    copies = [(fqg, fkg, gpg)] + [(fqg.clone(), fkg.clone(), gpg.clone()) for _ in range(NCOPY - 1)]
    outs_s = [(torch.empty(Mg * wg.d_gate, dtype=torch.float32, device=dev),
               torch.empty(Mg, wg.n_heads, dtype=torch.float32, device=dev)) for _ in range(NCOPY)]
    turn = [0]

    def scan_cold():
        k = turn[0] % NCOPY
        turn[0] += 1
        fq_k, fk_k, gp_k = copies[k]
        api.wango_stage_scan(sg, wg.window, wg.chunk, fq_k, fk_k, gp_k, outs_s[k][0], outs_s[k][1], ws_g,
                             stream=stream)

    def scan_warm():
        api.wango_stage_scan(sg, wg.window, wg.chunk, fqg, fkg, gpg, outs_s[0][0], outs_s[0][1], ws_g,
                             stream=stream)

    ms_scan_warm, _, _ = timed_batches(scan_warm, loops, n_batches)
    ms_scan, scan_min, scan_max = timed_batches(scan_cold, loops, n_batches)
    del copies, outs_s

    agg_flops = tango_flops(wt)
    achieved = agg_flops / (ms_agg * 1e-3)
    sbytes = scan_bytes(wg)
    s_ach = sbytes / (ms_scan * 1e-3)
    result = {
        "metric": "block fwd tokens/s at T=8192 (TANGO & WANGO); % MFMA peak / % HBM peak",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) activations, N(0,1/fan_in) weights, rounded to bf16",
        "config": {"workload": "tango_t8192_x4+wango_t8192_w256",
                   "tango": {"B": wt.B, "T": wt.T, "d_model": wt.d_model, "d_gate": wt.d_gate,
                             "qk_dim": HD, "heads": wt.n_heads, "repeats": wt.repeats},
                   "wango": {"B": wg.B, "T": wg.T, "d_model": wg.d_model, "d_gate": wg.d_gate,
                             "qk_dim": HDg, "heads": wg.n_heads, "window": wg.window,
                             "phi_dim": wg.head_dim, "chunk": wg.chunk},
                   "residual_dtype": "f32",
                   "gemm_operand_parts": {"tango": wt.operand_parts, "wango": wg.operand_parts},
                   "parallelism": "single GPU"},
        "per_workload": {
            TANGO: {"tokens_per_s": wt.tokens / (ms_tango * 1e-3), "ms": ms_tango,
                    "ms_per_application": ms_tango / wt.repeats},
            WANGO: {"tokens_per_s": wg.tokens / (ms_wango * 1e-3), "ms": ms_wango},
        },
        "roofline": {"kernel": "agg_kernel (TANGO aggregation, T=8192)", "bound": "mfma",
                     "achieved": achieved / 1e12, "peak": PEAK_BF16_FLOPS / 1e12, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_FLOPS, "traffic": recorded_traffic("agg_kernel"),
                     "flops_per_launch": agg_flops, "ms_per_launch": ms_agg,
                     "ms_batch_min": agg_min, "ms_batch_max": agg_max,
                     "launches": loops * n_batches,
                     "time_basis": f"mean launch time over {n_batches} batches of {loops} back-to-back launches, "
                                   "one event pair per batch on the launch stream"},
        "roofline_scan": {"kernel": "WANGO running-sum scan (2 launches, T=8192)", "bound": "hbm",
                          "achieved": s_ach / 1e9, "peak": PEAK_HBM_BYTES / 1e9, "unit": "GB/s",
                          "frac": s_ach / PEAK_HBM_BYTES, "traffic": recorded_traffic("scan"),
                          "bytes_per_launch": sbytes, "ms_per_launch": ms_scan,
                          "ms_batch_min": scan_min, "ms_batch_max": scan_max,
                          "launches": loops * n_batches,
                          "time_basis": f"mean launch time over {n_batches} batches of {loops} back-to-back launches, "
                                        "one event pair per batch on the launch stream",
                          "cache": f"cold: the launches cycle through {NCOPY} copies of the inputs and outputs "
                                   f"(about {NCOPY * sbytes / 1e6:.0f} MB, over 3x the 256 MB Infinity Cache)",
                          "ms_per_launch_warm_cache": ms_scan_warm},
    }
    print(f"[bench] tango {ms_tango:.3f} ms, wango {ms_wango:.3f} ms, aggregation {ms_agg:.3f} ms "
          f"({result['roofline']['frac'] * 100:.1f}% of bf16 peak), scan {ms_scan:.4f} ms "
          f"({result['roofline_scan']['frac'] * 100:.1f}% of HBM peak)", file=sys.stderr, flush=True)
    if args.copy_calibration:
        # a plain device copy of known size: 2^28 bytes read, 2^28 bytes written
        src = torch.ones(1 << 26, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    # this build's projection (row prep + projection GEMM with its epilogue) and
    # output GEMM on the T = 8192 TANGO shapes, for the library comparison
    vt = torch.empty(M, F, dtype=api.v_dtype(st), device=dev)
    vt.copy_(v)
    ms_proj, _, _ = timed_batches(lambda: api.tango_stage_proj(st, bt, xt, gp, v, qh, kh, ws=ws_t, stream=stream),
                                  loops, 3)
    ms_out, _, _ = timed_batches(lambda: api.tango_stage_out(st, bt.w_o, xt, gbar, vt, ping, stream=stream),
                                 loops, 3)
    result["gemm_reference"] = gemm_reference(loops, dev, stream, timed_batches,
                                              {"projection": ms_proj, "output": ms_out})
    result["ceilings"] = ceilings(dev, stream, timed_batches)
    if not args.no_configs:
        result["other_configs"] = configs_bench(min(loops, 5), 1, dev, stream, timed_batches)
    if not args.no_decode:
        result["decode"] = decode_bench(loops, min(args.warmup, 3), dev, stream)
    if not args.no_pages:
        result["pages_geometry"] = pages_bench(min(loops, 5), 1, dev, stream)
    if not args.no_three_set:
        result["three_set"] = three_set_bench(min(loops, 10), 1, dev, stream, ms_tango / wt.repeats)
    if not args.no_backward:
        result["backward"] = backward_bench(loops, min(args.warmup, 3), dev, stream)
        result["backward_wango"] = wango_backward_bench(loops, min(args.warmup, 3), dev, stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wt, wg)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
