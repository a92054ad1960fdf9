"""Benchmark of the chunked-prefill attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
  prefill workloads -- every chunk of the prompt(s): finish Q (norm, RoPE) and
                       append K/V (norm, RoPE) to the cache in one call, then
                       causal attention of the chunk;
  decode workload   -- finish q and append k/v at ctx-1 (one call), attention
                       over the context with probabilities.
Inputs are resident in HBM before timing starts.  The timed steps replay a
HIP graph of one step (the chunk loop is launch-bound at small chunks); the
graph was checked against eager execution by the test suite.

Prints ONE JSON line.  The headline workload is the 128K-token YaRN
prefill (64 query / 8 KV heads, chunks of 2048), the largest configuration;
the line also carries the smaller prefill workloads (`prefill_small`) and the
decode batch (`decode`) as sub-objects.  `value` is the whole-step
throughput (algorithmic FLOP/s for prefill, K/V bytes read per second for
decode); `roofline` is the attention call measured per launch with HIP events
on its stream, against the published peak and against the peak measured on
the same GPU in the same run (`calibration`: a matrix-core loop on random
operands, `measured_peak`, and on constant ones, `measured_peak_const`, and a
streaming read); `cpu_baseline` is the CPU oracle timed on a bounded sample
of the same workload on this host.  The decode line also carries
`importance`: the per-position importance call (sum over heads of the step's
probabilities), timed per launch after the step, outside it; and
`without_probs`: the same attention call with no probabilities asked for,
timed per launch (the K/V read path alone, next to the step's full rate).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s (% MFMA peak); decode KV-read GB/s (% HBM peak)"
PEAK_MFMA_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
PEAK_VALU_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4_yarn_128k")
    ap.add_argument("--no-decode", action="store_true", help="skip the secondary decode line")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the smaller prefill sub-lines (c1, c3)")
    ap.add_argument("--no-calib", action="store_true", help="skip the measured-peak calibration")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--eager", action="store_true", help="time eager launches, not a graph")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (counter calibration)")
    return ap.parse_args()


def kernel_code_hash():
    """Hash of the built library's GPU code (its .hip_fatbin section): recorded
    counter traffic is only reported while the kernels it was taken on are
    unchanged.  Edits that leave the machine code alone (comments, host-side
    code) keep the record."""
    import hashlib
    import struct
    from chunked_prefill_causal_rope_amd import api
    data = open(api.LIB_PATH, "rb").read()
    if data[:4] != b"\x7fELF" or data[4] != 2:
        return None
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    secs = [struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize) for i in range(shnum)]
    names = secs[shstrndx][4]
    for sec in secs:
        name = data[names + sec[0]: data.index(b"\0", names + sec[0])]
        if name == b".hip_fatbin":
            return hashlib.sha256(data[sec[4]: sec[4] + sec[5]]).hexdigest()[:16]
    return None


def recorded_traffic(workload):
    """HBM bytes per launch of the attention call from the committed counter
    record (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or None when there
    is no record for this workload or the kernels changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    code = kernel_code_hash()
    if code is None or rec.get("kernel_code_hash") != code:
        return None
    w = rec.get("workloads", {}).get(workload)
    return None if w is None else w.get("bytes_per_launch")


def step_flops(w, run, i):
    """Algorithmic causal FLOPs of one chunk call: 4*hd per (row, head, key)."""
    from chunked_prefill_causal_rope_amd import workloads as wl
    b = run.steps[i]["batch"]
    # rows at positions s..s+n-1 see p+1 keys each (at most window)
    tot = sum(wl.keys_read(s, n, w.window) for s, n in zip(b.starts, b.lens))
    return 4.0 * w.head_dim * w.n_heads * tot


def time_launches(torch, calls, stream):
    """Per-launch durations (ms) of `calls`, each bracketed by HIP events on
    `stream`; the GPU is first held by a spin so every launch is queued
    back to back and no host gap lands inside a bracket."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in calls]
    with torch.cuda.stream(stream):
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(20_000_000)
        for (e0, e1), fn in zip(evs, calls):
            e0.record(stream)
            fn()
            e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def graph_of(torch, fn, stream):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            fn()
    torch.cuda.synchronize()
    return g


def time_steps(torch, step_fn, steps, warmup, eager, stream):
    if eager:
        run = step_fn
    else:
        g = graph_of(torch, step_fn, stream)
        run = g.replay
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            run()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    return (t1 - t0) / steps


# ------------------------------------------------------------------ CPU baseline

def _cores(threads):
    """The oracle's thread count next to the host's core counts.  The oracle
    runs at most 16 threads: on a one-GPU machine that is the process's CPU share,
    whatever the host reports."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cores": threads, "threads": threads, "host_cores": os.cpu_count(),
            "affinity_cores": affinity}


def sample_rows(w, lengths, n_fixed_rows=512, seed=None):
    """The seeded (sequence, position, head) sample of a large prefill
    workload: for prompt 0, position 0, the first and last rows of 8 chunks
    spread over the prompt and the final row, each with the first, the last
    and two random heads; the rest random rows of any prompt (position
    uniform in the prompt, head uniform)."""
    import numpy as np
    rng = np.random.default_rng(w.seed if seed is None else seed)
    n0 = lengths[0]
    n_ch = -(-n0 // w.chunk)
    fixed_pos = {0, n0 - 1}
    for c in np.linspace(0, n_ch - 1, 8).round().astype(int):
        fixed_pos.add(int(c) * w.chunk)
        fixed_pos.add(min(n0, (int(c) + 1) * w.chunk) - 1)
    rows = []
    for p in sorted(fixed_pos):
        for h in (0, w.n_heads - 1, int(rng.integers(w.n_heads)), int(rng.integers(w.n_heads))):
            rows.append((0, p, h))
    rows = list(dict.fromkeys(rows))
    while len(rows) < n_fixed_rows:
        b = int(rng.integers(len(lengths)))
        rows.append((b, int(rng.integers(lengths[b])), int(rng.integers(w.n_heads))))
    return rows, rng


def cpu_baseline_prefill_sampled(w, d, budget_s):
    """The oracle, as it stands, on a seeded sample of (sequence, position,
    head) rows of a workload too large to run whole on the CPU: 512 rows
    (sample_rows), then further random rows while the time budget lasts.
    The keys each sampled sequence needs are finished (norm, RoPE, rounding)
    by the oracle first; that time is included.  Reports the algorithmic FLOP
    rate of the sample and the full workload's time extrapolated from it."""
    import numpy as np

    import oracle
    from chunked_prefill_causal_rope_amd import workloads as wl
    f = (oracle.yarn_inv_freq(w.rd, w.base, *w.yarn) if w.yarn is not None
         else oracle.rope_inv_freq(w.rd, w.base))
    store = oracle.STORE_BF16 if w.dtype == "bf16" else oracle.STORE_F32
    lengths, cu = d["lengths"], d["cu_seq"]
    threads = oracle.default_threads()
    G = w.n_heads // w.n_kv
    rows, rng = sample_rows(w, lengths)
    t_start = time.perf_counter()
    caches = {}

    def cache_of(b):
        if b not in caches:
            n = lengths[b]
            kn = dict(norm_style=w.norm_style, eps=w.norm_eps,
                      norm_w=d["k_norm_w"].numpy()) if w.norm_style else {}
            k = oracle.finish_heads(d["k"][cu[b]:cu[b] + n].float().numpy(), np.arange(n), f, w.rd,
                                    w.rope_scale, store=store, **kn)
            caches[b] = (np.ascontiguousarray(k.transpose(1, 0, 2)),
                         np.ascontiguousarray(d["v"][cu[b]:cu[b] + n].float().numpy()
                                              .astype(np.float64).transpose(1, 0, 2)))
        return caches[b]

    t_prep = 0.0
    flops = 0.0
    done = 0
    batch = 64
    i = 0
    while True:
        if i >= len(rows):
            if time.perf_counter() - t_start >= budget_s:
                break
            for _ in range(batch):
                b = int(rng.integers(len(lengths)))
                rows.append((b, int(rng.integers(lengths[b])), int(rng.integers(w.n_heads))))
        chunk_rows = rows[i:i + batch]
        i += len(chunk_rows)
        tp = time.perf_counter()
        for b, _, _ in chunk_rows:
            cache_of(b)
        t_prep += time.perf_counter() - tp
        qn = dict(norm_style=w.norm_style, eps=w.norm_eps,
                  norm_w=d["q_norm_w"].numpy()) if w.norm_style else {}
        # rows of one (sequence, KV head) go to the oracle together, each as
        # a one-head query row at its own position (threads over rows)
        groups = {}
        for b, p, h in chunk_rows:
            groups.setdefault((b, h // G), []).append((p, h))
        for (b, g), items in groups.items():
            kc, vc = caches[b]
            pos = np.array([p for p, _ in items])
            qraw = np.stack([d["q"][cu[b] + p, h:h + 1].float().numpy() for p, h in items])
            q = oracle.finish_heads(qraw, pos, f, w.rd, w.rope_scale, store=store, **qn)
            oracle.attend(q, kc[g:g + 1], vc[g:g + 1], pos, w.scale, n_threads=threads,
                          window=w.window)
            for p in pos:
                keys = min(p + 1, w.window) if w.window > 0 else p + 1
                flops += 4.0 * w.head_dim * float(keys)
                done += 1
        if done >= 512 and time.perf_counter() - t_start >= budget_s:
            break
    dt = time.perf_counter() - t_start
    total = wl.prefill_flops(w, lengths)
    t_attend = dt - t_prep
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", **_cores(threads), "kind": "oracle",
            "sample": f"{done} seeded (sequence, position, head) rows of {w.name} (position 0, first "
                      f"and last rows of 8 chunks and the final row of prompt 0, then random rows); "
                      f"f64 oracle incl. the RoPE of the keys they read ({t_prep:.1f} s) and of "
                      f"their queries; {dt:.1f} s",
            "sample_flop": flops,
            "extrapolated_full_s": round(t_prep + t_attend * total / max(flops, 1.0), 1),
            "extrapolated": True}


def cpu_baseline_prefill(w, d, budget_s):
    """The oracle, as it stands, on the last chunks of the first prompt (the
    costliest rows), walking backwards until about budget_s seconds of CPU
    work; reports its algorithmic FLOP rate in TFLOP/s."""
    import numpy as np

    import oracle
    f = (oracle.yarn_inv_freq(w.rd, w.base, *w.yarn) if w.yarn is not None
         else oracle.rope_inv_freq(w.rd, w.base))
    store = oracle.STORE_BF16 if w.dtype == "bf16" else oracle.STORE_F32
    n = d["lengths"][0]
    threads = oracle.default_threads()
    norm = dict(norm_style=w.norm_style, eps=w.norm_eps)
    t_start = time.perf_counter()
    flops = 0.0
    rows = 0
    chunks = 0
    passes = 0
    # walk back from the prompt's end; a prompt shorter than the budget is
    # walked again from scratch (RoPE of the keys included) until it is spent
    while time.perf_counter() - t_start < budget_s:
        passes += 1
        c_end = n
        kc = vc = None
        while c_end > 0 and time.perf_counter() - t_start < budget_s:
            c0 = max(0, c_end - w.chunk)
            if kc is None:
                kn = dict(norm, norm_w=d["k_norm_w"].numpy()) if w.norm_style else {}
                k = oracle.finish_heads(d["k"][:c_end].float().numpy(), np.arange(c_end), f, w.rd,
                                        w.rope_scale, store=store, **kn)
                kc = np.ascontiguousarray(k.transpose(1, 0, 2))
                vc = np.ascontiguousarray(d["v"][:c_end].float().numpy().astype(np.float64)
                                          .transpose(1, 0, 2))
            qn = dict(norm, norm_w=d["q_norm_w"].numpy()) if w.norm_style else {}
            pos = np.arange(c0, c_end)
            q = oracle.finish_heads(d["q"][c0:c_end].float().numpy(), pos, f, w.rd, w.rope_scale,
                                    store=store, **qn)
            oracle.attend(q, kc, vc, pos, w.scale, n_threads=threads, window=w.window)
            keys = np.minimum(pos + 1, w.window) if w.window > 0 else pos + 1
            flops += 4.0 * w.head_dim * w.n_heads * float(np.sum(keys))
            rows += c_end - c0
            chunks += 1
            c_end = c0
    dt = time.perf_counter() - t_start
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", **_cores(threads), "kind": "oracle",
            "sample": _prefill_sample(chunks, rows, n, w) + f", f64 oracle incl. K/Q RoPE, {dt:.1f} s"}


def _prefill_sample(chunks, rows, n, w):
    n_ch = -(-n // w.chunk)
    if chunks < n_ch:
        return f"last {chunks} chunk(s) ({rows} positions x {w.n_heads} heads) of prompt 0"
    whole, rest = divmod(chunks, n_ch)
    return (f"{whole} whole pass(es) over prompt 0 ({n} positions x {w.n_heads} heads, {n_ch} chunks)"
            + (f" and its last {rest} chunk(s) once more" if rest else ""))


def cpu_baseline_decode(w, d, budget_s):
    import numpy as np

    import oracle
    f = oracle.rope_inv_freq(w.rd, w.base)
    threads = oracle.default_threads()
    t_start = time.perf_counter()
    nbytes = 0.0
    seqs = 0
    for b, c in enumerate(d["ctx"]):
        if time.perf_counter() - t_start >= budget_s:
            break
        pos = np.array([c - 1])
        kc = d["k_cache"][b, :, :c].float().cpu().numpy().astype(np.float64)
        vc = d["v_cache"][b, :, :c].float().cpu().numpy().astype(np.float64)
        kc[:, c - 1] = oracle.finish_heads(d["k"][b:b + 1].float().cpu().numpy(), pos, f, w.rd,
                                           store=oracle.STORE_BF16)[0]
        vc[:, c - 1] = d["v"][b].float().cpu().numpy()
        q = oracle.finish_heads(d["q"][b:b + 1].float().cpu().numpy(), pos, f, w.rd,
                                store=oracle.STORE_BF16)
        oracle.attend(q, kc, vc, pos, w.scale, want_probs=True, n_threads=threads, window=w.window)
        nbytes += 2.0 * (min(c, w.window) if w.window > 0 else c) * w.n_kv * w.head_dim * 2
        seqs += 1
    dt = time.perf_counter() - t_start
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", **_cores(threads), "kind": "oracle",
            "sample": f"{seqs} of {len(d['ctx'])} sequences (all heads, with probabilities), "
                      f"f64 oracle, {dt:.1f} s"}


# ------------------------------------------------------------------ measured peaks

def calibrate(torch, stream):
    """Measured peaks of this GPU in this run: a loop of bf16 32x32x16 matrix
    products (two workgroups of 4 waves per CU, four independent accumulators
    per wave), once on hashed random operands (data like the kernels': the
    part's clock under load falls with the operands' switching activity) and
    once on small constants (the highest rate it sustains), and a streaming
    read of 4 GiB with 16-byte nontemporal loads (each workgroup a contiguous
    share of 128, 256 or 512 KB, the best kept); the best of 5 launches each,
    timed with events on `stream`.  Each matrix loop launch runs ~7-10 ms,
    five in a row, so the clock settles."""
    from chunked_prefill_causal_rope_amd import api
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nwg = 2 * cus
    out = torch.empty(nwg * 4, dtype=torch.float32, device="cuda")
    iters = 65536
    rates = {}
    for random_operands in (True, False):
        flop = [0.0]

        def mf():
            flop[0] = api.calibrate_mfma(nwg, iters, out, random_operands)
        with torch.cuda.stream(stream):
            mf()
        ms = min(time_launches(torch, [mf] * 5, stream))
        rates[random_operands] = (flop[0] / (ms * 1e-3) / 1e12, ms)
    mfma_tflops, ms = rates[True]
    src = torch.empty(1 << 30, dtype=torch.int32, device="cuda")     # 4 GiB, contents irrelevant
    best = None
    for share_kb in (128, 256, 512):                                  # contiguous bytes per workgroup
        nwr = (4 << 30) // (share_kb << 10)
        rout = torch.empty(nwr * 4, dtype=torch.int32, device="cuda")
        nbytes = [0]

        def rd():
            nbytes[0] = api.calibrate_read(src, nwr, rout)
        with torch.cuda.stream(stream):
            rd()
        ms_r = min(time_launches(torch, [rd] * 5, stream))
        if best is None or ms_r < best[0]:
            best = (ms_r, nbytes[0], share_kb)
    ms_r, nb, share_kb = best
    nbytes = [nb]
    read_gbs = nb / (ms_r * 1e-3) / 1e9
    del src
    torch.cuda.synchronize()
    return {"mfma_bf16_tflops": round(mfma_tflops, 1), "mfma_kernel": "attn_calibrate_mfma",
            "mfma_operands": "hashed random bf16", "mfma_ms": round(ms, 4),
            "mfma_bf16_tflops_const": round(rates[False][0], 1), "mfma_ms_const": round(rates[False][1], 4),
            "hbm_read_gbs": round(read_gbs, 1),
            "read_kernel": "attn_calibrate_read", "read_bytes": nbytes[0], "read_ms": round(ms_r, 4),
            "read_share_kb": share_kb, "compute_units": cus}


def bare_with_measured_peak(bare, calib):
    """The decode line's probability-free sub-line, with the measured read peak."""
    if calib is None:
        return bare
    bare = dict(bare)
    bare["frac_measured"] = round(bare["kv_read_gbs"] / calib["hbm_read_gbs"], 4)
    return bare


def with_measured_peak(roof, calib):
    """Add the fraction of the peak measured in this run to a roofline."""
    if calib is None:
        return roof
    peak = calib["mfma_bf16_tflops"] if roof["bound"] == "mfma" else calib["hbm_read_gbs"]
    roof = dict(roof)
    roof["measured_peak"] = peak
    roof["frac_measured"] = round(roof["achieved"] / peak, 4)
    if roof["bound"] == "mfma":
        roof["measured_peak_const"] = calib["mfma_bf16_tflops_const"]
        roof["frac_measured_const"] = round(roof["achieved"] / calib["mfma_bf16_tflops_const"], 4)
    return roof


# ------------------------------------------------------------------ workloads

def bench_prefill(torch, w, args, stream):
    from chunked_prefill_causal_rope_amd import runner, workloads as wl
    dev = "cuda"
    d = wl.gen_prefill(w, device=dev)
    run = runner.ChunkedPrefill(w, d, device=dev)
    n_steps = len(run.steps)
    total_flops = wl.prefill_flops(w, d["lengths"])
    sec = time_steps(torch, run.run_all, args.steps, args.warmup, args.eager, stream)
    value = total_flops / sec / 1e12
    # dominant kernel: the attention call, per launch, with the cache filled
    per_launch = []
    for _ in range(2):
        per_launch = time_launches(torch, [lambda i=i: run.attend_step(i) for i in range(n_steps)],
                                   stream)
    flops = [step_flops(w, run, i) for i in range(n_steps)]
    avg_ms = sum(per_launch) / n_steps
    achieved = sum(flops) / (sum(per_launch) * 1e-3) / 1e12
    # calls that split the key range (the library then launches its combine
    # kernel too): those whose plan asks for a workspace
    from chunked_prefill_causal_rope_amd import api
    split_calls = sum(1 for s in run.steps
                      if api.prefill_workspace_bytes(s["batch"], w.n_heads, w.n_kv, w.head_dim) > 0)
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_BF16_TFLOPS, 4),
            "traffic": recorded_traffic(w.name),
            # 256-row items run the ping-pong kernel, 128-row ones the key-split kernel
            "kernel": "attn_prefill_chunk (prefill_pp_kernel or prefill_bf16_ks_kernel"
                      + (" + prefill_combine_kernel" if split_calls else "") + ")",
            "launches": n_steps, "avg_launch_ms": round(avg_ms, 4),
            "flop_per_launch": round(sum(flops) / n_steps), "split_calls": split_calls}
    cfg = {"workload": w.name, "n_heads": w.n_heads, "n_kv": w.n_kv, "head_dim": w.head_dim,
           "n_seq": w.n_seq, "tokens": sum(d["lengths"]), "chunk": w.chunk,
           "chunks": n_steps, "rotary_dim": w.rd, "yarn": w.yarn is not None,
           "qk_norm": bool(w.norm_style), "graph": not args.eager,
           **({"window": w.window} if w.window else {})}
    out = {"metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic", "config": cfg,
           "roofline": roof}
    return out, d


def decode_bytes(w, ctx):
    # K and V of the keys read once per KV group (the last `window` with a
    # window, plus the earlier queries' extra key for a multi-token step);
    # the probability rows are written whole (zeros before the window)
    span = lambda c: min(c, w.window + w.new_tokens - 1) if w.window > 0 else c
    kv = 2.0 * sum(span(c) for c in ctx) * w.n_kv * w.head_dim * 2
    probs = 4.0 * sum(ctx) * w.n_heads if w.want_probs else 0.0
    small = len(ctx) * w.new_tokens * w.n_heads * w.head_dim * (2 + 4)
    return kv, kv + probs + small


def bench_decode(torch, w, args, stream):
    from chunked_prefill_causal_rope_amd import runner, workloads as wl
    d = wl.gen_decode(w, device="cuda")
    # several new tokens per sequence (a verify) go through the prefill call
    step = (runner.VerifyStep if w.new_tokens > 1 else runner.DecodeStep)(w, d, device="cuda")
    sec = time_steps(torch, step.run, args.steps, args.warmup, args.eager, stream)
    kv, alg = decode_bytes(w, d["ctx"])
    per_launch = []
    for _ in range(2):
        per_launch = time_launches(torch, [step.attend] * max(3, args.steps), stream)
    avg_ms = sum(per_launch) / len(per_launch)
    achieved = alg / (avg_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": recorded_traffic(w.name),
            "kernel": ("attn_prefill_chunk" if w.new_tokens > 1 else "attn_decode")
                      + " (decode_split_kernel + decode_combine_kernel)",
            "avg_launch_ms": round(avg_ms, 4), "bytes_per_launch": alg,
            "kv_read_gbs": round(kv / (avg_ms * 1e-3) / 1e9, 1)}
    out = {"metric": "decode KV-read GB/s", "value": round(kv / sec / 1e9, 1), "unit": "GB/s",
           "ms_per_step": round(sec * 1e3, 4), "workload": w.name,
           "config": {"n_seq": w.n_seq, "n_heads": w.n_heads, "n_kv": w.n_kv,
                      "head_dim": w.head_dim, "ctx_total": sum(d["ctx"]),
                      **({"new_tokens": w.new_tokens} if w.new_tokens > 1 else {}),
                      "probs": w.want_probs, **({"window": w.window} if w.window else {})},
           "roofline": roof}
    if w.want_probs:
        # per-position importance of the step (sum over heads of the
        # probabilities): a separate call after the decode, not part of the
        # step above; its algorithmic bytes are the probabilities read once
        # and the importance vector read and written
        from chunked_prefill_causal_rope_amd import api
        imp = torch.zeros((w.n_seq, step.max_ctx), dtype=torch.float32, device="cuda")
        call = lambda: api.decode_importance(step.probs, step.ctx, step.max_ctx, imp)
        for _ in range(2):
            per = time_launches(torch, [call] * max(3, args.steps), stream)
        imp_ms = sum(per) / len(per)
        imp_bytes = 4.0 * sum(d["ctx"]) * (w.n_heads + 2)
        out["importance"] = {"kernel": "attn_decode_importance (decode_importance_kernel)",
                             "avg_launch_ms": round(imp_ms, 4), "bytes_per_launch": imp_bytes,
                             "achieved_gbs": round(imp_bytes / (imp_ms * 1e-3) / 1e9, 1),
                             "frac": round(imp_bytes / (imp_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        if w.new_tokens == 1:
            # the same batch and call with probs = NULL: the K/V read path on
            # its own, so the cost of the probabilities' writes shows apart
            bare = runner.DecodeStep(w.replace(want_probs=False), d, device="cuda")
            bare.finish_and_append()
            for _ in range(2):
                per = time_launches(torch, [bare.attend] * max(3, args.steps), stream)
            bare_ms = sum(per) / len(per)
            out["without_probs"] = {"kernel": "attn_decode, probs NULL (decode_split_kernel + decode_combine_kernel)",
                                    "avg_launch_ms": round(bare_ms, 4), "bytes_per_launch": kv,
                                    "kv_read_gbs": round(kv / (bare_ms * 1e-3) / 1e9, 1),
                                    "frac": round(kv / (bare_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    return out, d


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by KV head or by sequence with no exchange; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from chunked_prefill_causal_rope_amd import workloads as wl
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration // 4
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 4 * n, "kernel_code_hash": kernel_code_hash()}))
        return
    stream = torch.cuda.Stream()
    calib = None if args.no_calib else calibrate(torch, stream)
    w = wl.CONFIGS[args.workload]
    if w.decode:
        res, d = bench_decode(torch, w, args, stream)
        res = {"metric": METRIC, "value": res["value"], "unit": "GB/s", "n_gpus": 1,
               "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
               "data": "synthetic", "config": dict(res["config"], workload=w.name),
               "roofline": with_measured_peak(res["roofline"], calib),
               **({"importance": res["importance"]} if "importance" in res else {}),
               **({"without_probs": bare_with_measured_peak(res["without_probs"], calib)}
                  if "without_probs" in res else {})}
        # the decode baseline covers one new token over a full-length cache
        if not args.no_cpu and w.new_tokens == 1 and not w.ring:
            res["cpu_baseline"] = cpu_baseline_decode(w, d, args.cpu_seconds)
    else:
        res, d = bench_prefill(torch, w, args, stream)
        res["roofline"] = with_measured_peak(res["roofline"], calib)
        if not args.no_cpu:
            from chunked_prefill_causal_rope_amd import workloads as wl_
            dc = {k: (v.cpu() if hasattr(v, "cpu") else v) for k, v in d.items()}
            del d
            # whole chunks of the oracle for the small workloads; a row sample
            # (time extrapolated) where the oracle would take hours
            big = wl_.prefill_flops(w, dc["lengths"]) > 5e11
            res["cpu_baseline"] = (cpu_baseline_prefill_sampled(w, dc, args.cpu_seconds) if big
                                   else cpu_baseline_prefill(w, dc, args.cpu_seconds))
            del dc
        else:
            del d
        if not args.no_extra and args.workload == "c4_yarn_128k":
            subs = {}
            for name in ("c1_llama_prefill", "c3_qwen_varlen"):
                torch.cuda.empty_cache()
                sub, dd = bench_prefill(torch, wl.CONFIGS[name], args, stream)
                del dd
                subs[name] = {"value": sub["value"], "unit": sub["unit"],
                              "ms_per_step": sub["ms_per_step"], "config": sub["config"],
                              "roofline": with_measured_peak(sub["roofline"], calib)}
            res["prefill_small"] = subs
        if not args.no_decode:
            torch.cuda.empty_cache()
            dec, _ = bench_decode(torch, wl.CONFIGS["c2_decode"], args, stream)
            dec["roofline"] = with_measured_peak(dec["roofline"], calib)
            if "without_probs" in dec:
                dec["without_probs"] = bare_with_measured_peak(dec["without_probs"], calib)
            res["decode"] = dec
    if calib is not None:
        res["calibration"] = calib
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
