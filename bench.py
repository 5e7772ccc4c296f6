#!/usr/bin/env python3
"""KDA forward (prefill) throughput on one MI355X.

One step = one kda_fwd call over the whole workload (all heads, all
sequences), inputs resident in HBM.  Default workload: 16 packed sequences,
65,536 tokens, H = 32, d = 128, bf16 q/k/v/o, fp32 g and beta, bf16 initial
and final states.  The T = 8192 single-sequence prefill is timed as well and
reported under "secondary".  Prints one JSON line on stdout; progress goes to
stderr.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]

Also timed, each with its own roofline: the 4 x 32K continuation workload
(fp32 states) and the T = 1M long-context workload (under "other_workloads";
the latter's oracle runs on 4 heads, "cpu_baseline_long_context").
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA fwd prefill tokens/s (H=32,d=128) at T=8K and 64K varlen; % of roofline"
# the sources of the measured kernels: the fused kernel body and its launch / tail kernel
KERNEL_SRCS = [os.path.join(ROOT, "linear_attention_kda_amd", "csrc", f)
               for f in ("kda_fwd_core.h", "kda_fwd_kernel.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_fwd_traffic.json")
KERNEL_NAME = "kda_fwd call: kda_fwd_kernel + kda_tail_kernel (scan, fix-up)"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_sha() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def state_bytes_of(dtype_name):
    return {None: 0, "bf16": 2, "fp32": 4}[dtype_name]


def time_workload(wid: int, steps: int, warmup: int, copies: int = 1):
    """Time `steps` kda_fwd calls on workload `wid` after `warmup` untimed ones.

    With copies > 1 the calls rotate over that many copies of the inputs and
    outputs, so that a working set smaller than the 256 MB Infinity Cache is
    not served from it on the next call."""
    import torch

    from linear_attention_kda_amd import binding, perfmodel
    from linear_attention_kda_amd.workloads import make_inputs

    x = make_inputs(wid, "cuda")
    w = x["workload"]
    dev = x["q"].device
    N, H = w.num_states, w.H
    sdt = {"bf16": torch.bfloat16, "fp32": torch.float32}
    sets = []
    for c in range(copies):
        xi = x if c == 0 else {k: (v.clone() if torch.is_tensor(v) else v) for k, v in x.items()}
        final = torch.empty(N, H, 128, 128, dtype=sdt[w.final_state], device=dev) \
            if w.final_state else None
        sets.append((xi, final, torch.empty_like(x["v"])))

    def step(i):
        xi, final, out = sets[i % copies]
        binding.fwd(xi["q"], xi["k"], xi["v"], xi["g"], xi["beta"], xi["scale"],
                    initial_state=xi["initial_state"], final_state=final,
                    cu_seqlens=xi["cu_seqlens"], out=out)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # The timed region holds the K calls and nothing else: an event pair around
    # every call would add two markers, ~9 us of device time, per call.
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    kernel_ms = total_ms / steps
    # the spread of single calls, from K more calls with an event pair each
    # (these include the markers' cost)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record()
        step(i)
        ends[i].record()
    torch.cuda.synchronize()
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    tokens = w.tokens
    nbytes = perfmodel.workload_bytes(tokens, H, N, state_bytes_of(w.init_state),
                                      state_bytes_of(w.final_state))
    flops = perfmodel.workload_flops(tokens, H)
    res = dict(
        workload=w, tokens=tokens, N=N, H=H, total_ms=total_ms, wall_s=wall,
        ms_per_step=total_ms / steps, kernel_ms=kernel_ms,
        kernel_ms_median=statistics.median(launch_ms), kernel_ms_min=min(launch_ms),
        kernel_ms_max=max(launch_ms),
        tokens_per_s=tokens * steps / (total_ms * 1e-3),
        bytes_per_launch=nbytes, flops_per_launch=flops,
        achieved_gbs=nbytes / (kernel_ms * 1e-3) / 1e9,
        achieved_tflops=flops / (kernel_ms * 1e-3) / 1e12,
        lengths=x["lengths"], copies=copies,
    )
    res["hbm_frac"] = res["achieved_gbs"] / perfmodel.HBM_PEAK_GBS
    res["mfma_frac"] = res["achieved_tflops"] / perfmodel.BF16_PEAK_TFLOPS
    del sets
    return res, x, None


def workload_line(r):
    """The JSON object of a timed workload other than the headline one."""
    from linear_attention_kda_amd import perfmodel
    w = r["workload"]
    return {"workload": w.name, "value": r["tokens_per_s"], "unit": "tokens/s",
            "ms_per_step": r["ms_per_step"], "kernel_ms": r["kernel_ms"],
            "single_call_ms_range": [r["kernel_ms_min"], r["kernel_ms_max"]],
            "input_copies": r["copies"], "state_dtype": w.final_state,
            "roofline": {"bound": "hbm", "achieved": r["achieved_gbs"],
                         "peak": perfmodel.HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": r["hbm_frac"], "traffic": None,
                         "algorithmic_bytes": r["bytes_per_launch"]},
            "mfma_frac": r["mfma_frac"]}


def input_copies(wid: int) -> int:
    """Two input copies when one set would fit twice in the 256 MB Infinity Cache's reach
    (the T = 8K workload's 406 MB), one otherwise."""
    from linear_attention_kda_amd import perfmodel
    from linear_attention_kda_amd.workloads import WORKLOADS
    w = WORKLOADS[wid]
    nbytes = perfmodel.workload_bytes(w.tokens, w.H, w.num_states, state_bytes_of(w.init_state),
                                      state_bytes_of(w.final_state))
    return 2 if nbytes < (1 << 30) else 1


def measured_traffic(wid: int):
    """HBM bytes per launch from committed rocprofv3 counters, if still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_sha() or t.get("workload") != wid:
        return None
    return float(t["fetch_bytes_per_launch"]) + float(t["write_bytes_per_launch"])


def host_sample(x, heads: int):
    """The first `heads` heads of workload tensors x, copied to the host (for the oracle)."""
    w = x["workload"]
    hs = list(range(min(heads, w.H)))
    init = x["initial_state"]
    s = {k: x[k][:, :, hs].cpu() for k in ("q", "k", "v", "g", "beta")}
    s.update(workload=w, heads=len(hs), scale=x["scale"],
             initial_state=None if init is None else init[:, hs].cpu(),
             cu_seqlens=None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu())
    return s


def cpu_baseline(s, min_seconds: float = 10.0, max_passes: int = 1 << 30):
    """The fp64 oracle, as it stands, on a host sample of a workload (host_sample)."""
    from oracle import oracle
    w = s["workload"]
    nh = s["heads"]
    args = [s[k] for k in ("q", "k", "v", "g", "beta")]
    threads = oracle.max_threads()
    col_block = 16
    tasks = w.num_states * nh * (128 // col_block)
    # Whole passes over the sample until at least min_seconds of CPU work.
    passes, dt = 0, 0.0
    while passes == 0 or (dt < min_seconds and passes < max_passes):
        t0 = time.perf_counter()
        oracle.fwd(*args, s["scale"], s["initial_state"], cu_seqlens=s["cu_seqlens"],
                   col_block=col_block)
        dt += time.perf_counter() - t0
        passes += 1
    head_tokens = passes * w.tokens * nh
    tokens_equiv = head_tokens / w.H  # all-head-equivalent tokens
    res = dict(value=tokens_equiv / dt, unit="tokens/s", cores=min(threads, tasks),
               nproc=os.cpu_count(), kind="oracle",
               sample=(f"{w.name}: {passes} pass(es) over all {w.tokens} tokens of "
                       f"{nh} of {w.H} heads ({dt:.1f} s); value scaled to all heads"))
    if nh < w.H:
        res["head_tokens_per_s"] = head_tokens / dt
        res["heads_run"] = nh
    return res


def decode_bench(steps: int, warmup: int, N: int = 256, H: int = 32, d: int = 128):
    """One decode step for N sequences x H heads of size d with fp32 states: HBM-bound
    on the state."""
    import torch

    from linear_attention_kda_amd import binding, perfmodel
    from linear_attention_kda_amd.workloads import random_inputs

    x = random_inputs(N, 1, H, d, d, seed=1300, device="cuda", init_state="fp32")
    one = {k: x[k][:, 0].contiguous() for k in ("q", "k", "v", "g", "beta")}
    S = x["initial_state"]
    out = torch.empty(N, H, d, dtype=torch.bfloat16, device="cuda")

    def step():
        binding.decode(one["q"], one["k"], one["v"], one["g"], one["beta"], S, x["scale"], out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # per (sequence, head): state read + write (fp32), q/k/v/o bf16, g fp32, beta
    nbytes = N * H * (2 * d * d * 4 + 4 * d * 2 + d * 4 + 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tag = "" if d == 128 else f" d={d}"
    log(f"[bench] decode{tag} N={N} H={H} fp32 state: {ms * 1e3:.1f} us/step, {gbs:.0f} GB/s "
        f"({100 * gbs / perfmodel.HBM_PEAK_GBS:.1f}% of HBM peak)")
    return {"workload": f"decode step N={N} sequences H={H}{tag} fp32 state", "unit": "steps/s",
            "value": 1e3 / ms, "us_per_step": ms * 1e3, "tokens_per_s": N * 1e3 / ms,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": perfmodel.HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": gbs / perfmodel.HBM_PEAK_GBS, "traffic": None,
                         "kernel": "kda_decode_kernel", "algorithmic_bytes": nbytes}}


def gdn_bench(wid: int, steps: int, warmup: int):
    """The scalar-gate forward (kda_gdn_fwd) on workload `wid`'s tensors, with the
    first channel of the per-channel gate as the gate of each token and head."""
    import torch

    from linear_attention_kda_amd import binding, perfmodel
    from linear_attention_kda_amd.workloads import make_inputs

    x = make_inputs(wid, "cuda")
    w = x["workload"]
    gs = x["g"][..., 0].contiguous()
    N, H = w.num_states, w.H
    sdt = {"bf16": torch.bfloat16, "fp32": torch.float32}
    final = torch.empty(N, H, 128, 128, dtype=sdt[w.final_state], device="cuda") \
        if w.final_state else None
    out = torch.empty_like(x["v"])

    def step():
        binding.gdn_fwd(x["q"], x["k"], x["v"], gs, x["beta"], x["scale"],
                        initial_state=x["initial_state"], final_state=final,
                        cu_seqlens=x["cu_seqlens"], out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = perfmodel.workload_bytes(w.tokens, H, N, state_bytes_of(w.init_state),
                                      state_bytes_of(w.final_state), scalar_gate=True)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] gdn {w.name}: {ms:.3f} ms, {w.tokens / ms / 1e3:.2f} M tokens/s, "
        f"{gbs:.0f} GB/s ({100 * gbs / perfmodel.HBM_PEAK_GBS:.1f}% of HBM peak)")
    return {"workload": f"scalar gate (Gated DeltaNet), {w.name}", "unit": "tokens/s",
            "value": w.tokens / (ms * 1e-3), "ms_per_step": ms,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": perfmodel.HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": gbs / perfmodel.HBM_PEAK_GBS, "traffic": None,
                         "kernel": "kda_gdn_fwd call", "algorithmic_bytes": nbytes}}


def dim_bench(wid: int, d: int, steps: int, warmup: int):
    """kda_fwd at head dimension d (64 or 256) on workload `wid`'s shape: the same
    lengths, heads and state dtype, inputs drawn with the same recipe at size d."""
    import torch

    from linear_attention_kda_amd import binding, perfmodel
    from linear_attention_kda_amd.workloads import WORKLOADS, random_inputs, varlen_lengths

    w = WORKLOADS[wid]
    lengths = None
    if w.n_seqs:
        gen = torch.Generator(device="cpu")
        gen.manual_seed(w.seed)
        lengths = varlen_lengths(w.n_seqs, w.T, gen)
    x = random_inputs(w.B, w.T, w.H, d, d, seed=w.seed + 7919 + d, device="cuda",
                      g_lo=w.g_lo, g_hi=w.g_hi, init_state=w.init_state, lengths=lengths)
    N, H = w.num_states, w.H
    sdt = {"bf16": torch.bfloat16, "fp32": torch.float32}
    final = torch.empty(N, H, d, d, dtype=sdt[w.final_state], device="cuda") \
        if w.final_state else None
    out = torch.empty_like(x["v"])

    def step():
        binding.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"],
                    initial_state=x["initial_state"], final_state=final,
                    cu_seqlens=x["cu_seqlens"], out=out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = perfmodel.workload_bytes(w.tokens, H, N, state_bytes_of(w.init_state),
                                      state_bytes_of(w.final_state), d=d)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] d={d} {w.name}: {ms:.3f} ms, {w.tokens / ms / 1e3:.2f} M tokens/s, "
        f"{gbs:.0f} GB/s ({100 * gbs / perfmodel.HBM_PEAK_GBS:.1f}% of HBM peak)")
    return {"workload": f"head dim {d}, {w.name}", "head_dim": d, "unit": "tokens/s",
            "value": w.tokens / (ms * 1e-3), "ms_per_step": ms,
            "workspace_bytes": (binding.plan(N, w.T, H, bool(w.n_seqs), 0)[2] if d == 64
                                else binding.dim_workspace_bytes(N, w.tokens, H, d)),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": perfmodel.HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": gbs / perfmodel.HBM_PEAK_GBS, "traffic": None,
                         "kernel": ("kda_fwd call at d=64: kda_fwd_kernel<1, false, 64>" if d == 64 else
                                    "kda_fwd call at d=%d: dim_prep_kernel + dim_state_kernel" % d),
                         "algorithmic_bytes": nbytes}}


def bwd_bench(wid: int, steps: int, warmup: int):
    """The backward pass (kda_bwd) on workload `wid` with seeded upstream gradients."""
    import torch

    from linear_attention_kda_amd import binding, perfmodel
    from linear_attention_kda_amd.workloads import make_inputs

    x = make_inputs(wid, "cuda")
    w = x["workload"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1400 + wid)
    do = torch.randn(x["v"].shape, generator=gen, device="cuda").to(torch.bfloat16)

    def step():
        binding.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["scale"],
                    initial_state=x["initial_state"], cu_seqlens=x["cu_seqlens"])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # per token-head: q, k, v, dO bf16, g fp32, beta read; dq, dk, dv, dg fp32, dbeta written;
    # per (sequence, head): the initial state read and its gradient written (fp32)
    N, H = w.num_states, w.H
    nbytes = w.tokens * H * (4 * 128 * 2 + 128 * 4 + 4 + 4 * 128 * 4 + 4) \
        + (perfmodel.state_bytes(N, H, state_bytes_of(w.init_state)) if w.init_state else 0) \
        + perfmodel.state_bytes(N, H, 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] bwd {w.name}: {ms:.3f} ms, {w.tokens / ms / 1e3:.2f} M tokens/s, "
        f"{gbs:.0f} GB/s ({100 * gbs / perfmodel.HBM_PEAK_GBS:.1f}% of HBM peak)")
    return {"workload": f"backward, {w.name}", "unit": "tokens/s", "value": w.tokens / (ms * 1e-3),
            "ms_per_step": ms,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": perfmodel.HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": gbs / perfmodel.HBM_PEAK_GBS, "traffic": None,
                         "kernel": "kda_bwd call", "algorithmic_bytes": nbytes}}


def counter_run(wid: int, target: str = "fwd"):
    """Launch sequence profiled by the hardware-counter passes.

    The copy moves exactly 1 GiB in each direction, so its FETCH_SIZE /
    WRITE_SIZE readings give the factor that turns a counter reading into
    bytes.  Then two launches of `target` on workload `wid`: the d = 128
    forward (fwd), the scalar-gate forward (gdn), the forward at head
    dimension 64 or 256 (dim64, dim256) or the backward (bwd)."""
    import torch

    from linear_attention_kda_amd import binding
    from linear_attention_kda_amd.workloads import WORKLOADS, make_inputs, random_inputs, varlen_lengths

    a = torch.rand(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    sdt = {"bf16": torch.bfloat16, "fp32": torch.float32}
    if target in ("dim64", "dim256"):
        d = int(target[3:])
        w = WORKLOADS[wid]
        lengths = None
        if w.n_seqs:
            gen = torch.Generator(device="cpu")
            gen.manual_seed(w.seed)
            lengths = varlen_lengths(w.n_seqs, w.T, gen)
        x = random_inputs(w.B, w.T, w.H, d, d, seed=w.seed + 7919 + d, device="cuda",
                          g_lo=w.g_lo, g_hi=w.g_hi, init_state=w.init_state, lengths=lengths)
    else:
        d = 128
        x = make_inputs(wid, "cuda")
        w = x["workload"]
    final = torch.empty(w.num_states, w.H, d, d, dtype=sdt[w.final_state],
                        device="cuda") if w.final_state else None
    out = torch.empty_like(x["v"])
    gs = x["g"][..., 0].contiguous() if target == "gdn" else None
    do = None
    if target == "bwd":
        gen = torch.Generator(device="cuda")
        gen.manual_seed(1400 + wid)
        do = torch.randn(x["v"].shape, generator=gen, device="cuda").to(torch.bfloat16)
    for _ in range(2):
        if target == "bwd":
            binding.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["scale"],
                        initial_state=x["initial_state"], cu_seqlens=x["cu_seqlens"])
        else:
            fn = binding.gdn_fwd if target == "gdn" else binding.fwd
            fn(x["q"], x["k"], x["v"], gs if target == "gdn" else x["g"], x["beta"], x["scale"],
               initial_state=x["initial_state"], final_state=final,
               cu_seqlens=x["cu_seqlens"], out=out)
    torch.cuda.synchronize()
    log(f"[bench] counter run done: 2 copies of 1 GiB, 2 launches of {target} on {w.name}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--secondary", type=int, default=1,
                    help="second workload timed and reported under 'secondary' (-1: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step line")
    ap.add_argument("--no-gdn", action="store_true", help="skip the scalar-gate line")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward line")
    ap.add_argument("--no-dims", action="store_true", help="skip the head dim 64 / 256 lines")
    ap.add_argument("--bwd-workload", type=int, default=1)
    ap.add_argument("--also", type=int, nargs="*", default=[3, 4],
                    help="further workloads timed with their own lines (default: 3 4)")
    ap.add_argument("--cpu-heads", type=int, default=32)
    ap.add_argument("--counter-target", default="fwd",
                    choices=["fwd", "gdn", "dim64", "dim256", "bwd"],
                    help="what --counters launches (on --workload)")
    ap.add_argument("--counters", action="store_true",
                    help="untimed run for hardware-counter passes: a 1 GiB device copy "
                         "(the calibration kernel) twice, then two launches of the workload")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the KDA forward pass splits across GPUs by "
              "heads and sequences with no communication, so a single GPU's share at its "
              "real shape is the whole measurement; --gpus must be 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a HIP GPU", file=sys.stderr)
        sys.exit(2)
    from linear_attention_kda_amd import binding, perfmodel
    binding.load_library()

    if args.counters:
        counter_run(args.workload, args.counter_target)
        return

    # The card runs ~15% slower for the first ~25 calls of a sustained load while its
    # clock and power management settle; the lines that are not the headline run first,
    # so the T = 8K and 64K varlen lines are timed in the steady state.  Each line still
    # does exactly its own warmup and timed steps.
    # the other full-size workloads: 4 x 32K continuation (fp32 states), T = 1M
    others = []
    cpu_long = None
    long_sample = None
    for wid in args.also:
        if wid in (args.workload, args.secondary):
            continue
        st = args.steps if wid != 4 else max(3, args.steps // 5)
        wu = args.warmup if wid != 4 else 1
        log(f"[bench] workload {wid}, warmup {wu}, steps {st}")
        r3, x3, _ = time_workload(wid, st, wu, copies=input_copies(wid))
        w3 = r3["workload"]
        log(f"[bench] {w3.name}: {r3['kernel_ms']:.3f} ms, {r3['tokens_per_s'] / 1e6:.2f} M "
            f"tokens/s, {100 * r3['hbm_frac']:.1f}% of HBM peak")
        others.append(workload_line(r3))
        if wid == 4 and not args.no_cpu_baseline:
            long_sample = host_sample(x3, 4)  # timed after the GPU lines
        del x3

    decode = None
    decode_dims = None
    if not args.no_decode:
        decode = decode_bench(max(args.steps, 20), args.warmup)
        decode_dims = [decode_bench(max(args.steps, 20), args.warmup, d=d) for d in (64, 256)]

    gdn = None
    if not args.no_gdn:
        gdn = gdn_bench(args.workload, args.steps, args.warmup)

    dims = None
    if not args.no_dims:
        dims = [dim_bench(args.workload, d, args.steps, args.warmup) for d in (64, 256)]

    bwd = None
    if not args.no_bwd:
        bwd = bwd_bench(args.bwd_workload, max(5, args.steps // 4), 2)

    secondary = None
    if args.secondary >= 0 and args.secondary != args.workload:
        log(f"[bench] secondary workload {args.secondary}")
        r2, x2, _ = time_workload(args.secondary, args.steps, args.warmup,
                                  copies=input_copies(args.secondary))
        w2 = r2["workload"]
        log(f"[bench] {w2.name}: {r2['kernel_ms']:.3f} ms ({r2['copies']} input copies), "
            f"{r2['tokens_per_s'] / 1e6:.2f} M tokens/s, {100 * r2['hbm_frac']:.1f}% of HBM peak")
        secondary = workload_line(r2)
        del x2

    log(f"[bench] workload {args.workload}, warmup {args.warmup}, steps {args.steps}")
    r, x, _ = time_workload(args.workload, args.steps, args.warmup)
    w = r["workload"]
    log(f"[bench] {w.name}: {r['ms_per_step']:.3f} ms/step, kernel {r['kernel_ms']:.3f} ms, "
        f"{r['tokens_per_s'] / 1e6:.2f} M tokens/s, {r['achieved_gbs']:.0f} GB/s "
        f"({100 * r['hbm_frac']:.1f}% of HBM peak)")
    wg, ns, wsb = binding.plan(r["N"], w.T, r["H"], varlen=bool(w.n_seqs))
    traffic = measured_traffic(args.workload)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_heads} heads of {w.name}")
        cpu = cpu_baseline(host_sample(x, args.cpu_heads))
        log(f"[bench] cpu baseline {cpu['value']:.1f} tokens/s on {cpu['cores']} threads "
            f"({cpu['nproc']} host cpus)")
    if long_sample is not None:
        # the long-context oracle on 4 heads, one pass over all 1M tokens
        log(f"[bench] cpu baseline: oracle on 4 heads of {long_sample['workload'].name}")
        cpu_long = cpu_baseline(long_sample, min_seconds=0.0, max_passes=1)
        log(f"[bench] cpu baseline {cpu_long['head_tokens_per_s']:.1f} head-tokens/s "
            f"(4 of 32 heads) on {cpu_long['cores']} threads")

    line = {
        "metric": METRIC,
        "value": r["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": r["tokens"], "sequences": r["N"],
                   "lengths": r["lengths"], "heads": r["H"], "head_dim": 128, "chunk": 64,
                   "state_dtype": w.final_state, "global_batch": w.B, "seq_len": w.T,
                   "parallelism": "single GPU", "workgroups": wg, "value_splits": ns,
                   "workspace_bytes": wsb},
        "roofline": {"bound": "hbm", "achieved": r["achieved_gbs"],
                     "peak": perfmodel.HBM_PEAK_GBS, "unit": "GB/s", "frac": r["hbm_frac"],
                     "traffic": traffic, "kernel": KERNEL_NAME,
                     "algorithmic_bytes": r["bytes_per_launch"],
                     "kernel_ms": r["kernel_ms"],
                     "single_call_ms_range": [r["kernel_ms_min"], r["kernel_ms_max"]]},
        "mfma": {"achieved": r["achieved_tflops"], "peak": perfmodel.BF16_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": r["mfma_frac"],
                 "flops_model": "6Td^2+3TCd+TC^2 per head"},
        "secondary": secondary,
        "other_workloads": others,
        "decode": decode,
        "decode_head_dims": decode_dims,
        "gdn": gdn,
        "head_dims": dims,
        "bwd": bwd,
        "cpu_baseline": cpu,
        "cpu_baseline_long_context": cpu_long,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
