"""Benchmark of the MiTA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one full mita_forward call (pool, landmark scoring with shared
values and top-k, routing, bucketing, joint-softmax attention) over one batch
of synthetic inputs already resident in HBM.  The headline workload is the
N = 1M long sequence (B=1, H=2, d=64, m=k=512, s=1); the N = 64K and 256K
shapes are timed the same way and reported beside it, and so is the
training step (forward_train + backward) of the headline workload.  Prints
one JSON line.

The roofline of the dominant kernel uses the per-stage durations measured
with HIP events on the launch stream during the timed steps, against the
spec-sheet peak and against the peak this GPU sustains on a pure
matrix-core loop or a plain copy (measured at the start of the run); its HBM traffic
comes from committed rocprofv3 counter summaries (profiles/) when they were
taken on the current kernel sources, else null.  The CPU baseline times the
fp64 oracle on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from efficient_long_sequence_amd.configs import HEADLINE, LONG, WORKLOADS  # noqa: E402

METRIC = "MiTA fwd tokens/s (B·H·N) at N=64K/256K/1M; % of HBM and MFMA peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
COPY_FETCH_FACTOR_DEFAULT = 2.0  # see profiles/: FETCH_SIZE reads half of a plain copy's bytes


# sources of the forward pass's kernels and host plan (the backward and the
# dense baseline live in files of their own and do not change them)
FORWARD_SOURCES = ("api.cpp", "pool.hip", "score.hip", "route.hip", "attend.hip", "resident.hip",
                   "mita_dev.h", "mita_plan.h", "tile.h")


def sources_sha() -> str:
    """Hash of the forward pass's sources: counter figures are only reported
    for the kernels they were measured on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "efficient_long_sequence_amd", "csrc")
    for f in FORWARD_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def algorithmic(w, stage: str):
    """Algorithmic flops and compulsory HBM bytes of one launch of a stage's
    kernel (the method's own work and traffic), and the design-overhead bytes
    the kernel moves beyond them.

    score:  every landmark row against every key: one logit and one value sum
            of length d (4 d N m flops); reads K and V once and Q~, writes v~.
            Overhead: reported as 0 here; the kernel also writes the split-N
            partials of v~ (B H m C (d + 4) fp32, C key chunks from the launch
            plan, 36 MB at N = 1M) and the score records of the candidate
            filter (data-dependent), which the measured traffic includes.
    route:  every query against every landmark: the routing score, which is
            also the shared logit, and the shared value sum (4 d N m flops);
            reads Q, Q~ and v~, writes the routes.  Overhead: the shared part
            of each query's softmax, handed to the attention kernel (fp16 row
            and two fp32 per query for bf16 inputs; fp32 row for fp32).
    attend: every query against the k raw entries of each of its s experts
            (4 d N s k flops); reads Q, the m*k gathered key and value rows,
            the expert index lists and the permutation, writes O.  Overhead:
            the shared part read back (and, for s >= 2, every later slot's
            partial written and read again).
    """
    es = 2 if w.dtype == "bf16" else 4
    part = (w.d * 2 + 8) if w.dtype == "bf16" else (w.d * 4 + 8)
    BH, N, d, m, k, s = w.B * w.H, w.N, w.d, w.m, w.k, w.s
    if stage == "score":
        flops = 4.0 * d * N * m * BH
        byts = BH * (2 * N * d * es + m * d * es + m * d * 4)
        over = 0.0
    elif stage == "route":
        flops = 4.0 * d * N * m * BH
        byts = BH * (N * d * es + 2 * m * d * es + N * s * 4)
        over = BH * N * part
    elif stage == "attend":
        flops = 4.0 * d * N * s * k * BH
        byts = BH * (N * d * es + 2 * m * k * d * es + m * k * 4 + s * N * 4 + N * d * es)
        over = BH * N * part * (1 + 2 * (s - 1))
    else:
        return None, None, None
    return flops, float(byts), float(over)


def make_device_inputs(w):
    import torch
    from efficient_long_sequence_amd import synth
    Q, K, V = synth.make_from_workload(w)
    out = []
    for x in (Q, K, V):
        if w.dtype == "bf16":
            bits = synth.f32_to_bf16_bits(x)
            out.append(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda())
        else:
            out.append(torch.from_numpy(x).cuda())
    return (Q, K, V), out


def time_workload(w, steps: int, warmup: int, variant: str = "paper", k: int | None = None, inputs=None):
    import torch
    from efficient_long_sequence_amd import mita
    host, (q, kk, v) = make_device_inputs(w) if inputs is None else inputs
    k = w.k if k is None else k
    pool = (w.grid_h, w.grid_w, w.land_h, w.land_w)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    ws = torch.empty(mita.workspace_bytes(q.dtype, w.B, w.H, w.N, w.d, pool, k, w.s), dtype=torch.uint8,
                     device=q.device)
    out = torch.empty_like(q)
    for _ in range(warmup):
        mita.forward(q, kk, v, pool, k, w.s, workspace=ws, out=out, variant=variant)

    def calls(events):
        for i in range(steps):
            mita.forward(q, kk, v, pool, k, w.s, workspace=ws, out=out, events=events[i], variant=variant)

    def collect(events):
        stages, per_call = {}, []
        for ev in events:
            ms_all = ev.elapsed_ms()
            per_call.append(sum(ms_all.values()))
            for name, ms in ms_all.items():
                stages[name] = stages.get(name, 0.0) + ms / steps
            ev.close()
        return stages, per_call

    # stage breakdown: the same K calls with an event pair around every stage
    # (the records between the small kernels cost a few microseconds each, so
    # this pass is not the timed one)
    events = [mita.Events() for _ in range(steps)]
    calls(events)
    torch.cuda.synchronize()
    stages, per_call = collect(events)
    # timed region: event pairs around the three heavy kernels only (the
    # roofline's kernel times come from here)
    events = [mita.Events(stages=HEAVY_STAGES) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    calls(events)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    heavy, _ = collect(events)
    # per-call device time (sum of the call's stage event pairs on its stream)
    call_ms = dict(median=float(np.median(per_call)), min=float(np.min(per_call)), max=float(np.max(per_call)))
    # device memory of one call: the caller's tensors (Q, K, V, O) and the workspace, and the allocator's peak
    memory = dict(tensor_bytes=4 * q.numel() * q.element_size(), workspace_bytes=ws.numel(),
                  peak_allocated_bytes=int(torch.cuda.max_memory_allocated()))
    return dict(seconds=dt, memory=memory, ms_per_step=1e3 * dt / steps, tokens_per_s=w.tokens * steps / dt, stages=stages,
                heavy=heavy, call_ms=call_ms, tokens_per_s_median_call=w.tokens / (call_ms["median"] * 1e-3),
                host=host, q=q, k=kk, v=v, pool=pool, ws=ws)


HEAVY_STAGES = ("score", "route", "attend")


STAGE_KERNEL = {"score": "k_score", "route": "k_route_shared", "attend": "k_expert"}


MEASURED_PEAKS = {}  # filled once per run by mita.probe_peaks()


def roofline_of(w, stages: dict, stage: str, traffic):
    flops, byts, over = algorithmic(w, stage)
    sec = stages[stage] * 1e-3
    peak_f = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / byts > ridge:
        r = dict(bound="mfma", achieved=flops / sec / 1e12, peak=peak_f, unit="TFLOP/s")
    else:
        r = dict(bound="hbm", achieved=byts / sec / 1e9, peak=PEAK_HBM_GBS, unit="GB/s")
    r["frac"] = r["achieved"] / r["peak"]
    r["traffic"] = traffic
    # the same against what this GPU sustains on a pure matrix-core loop or a
    # plain copy (bf16 only: the probe runs bf16 MFMA)
    pm = MEASURED_PEAKS.get("mfma_bf16_tflops" if r["bound"] == "mfma" else "hbm_copy_gbs")
    if pm and (r["bound"] == "hbm" or w.dtype == "bf16"):
        r["peak_measured"] = pm
        r["frac_measured"] = r["achieved"] / pm
    # and against the best rate of the bare online-softmax step these kernels
    # are built on (d = 64 bf16, any of the probed launch shapes)
    step = MEASURED_PEAKS.get("step_bf16_tflops")
    if step and r["bound"] == "mfma" and w.dtype == "bf16" and w.d == 64:
        r["step_ceiling"] = max(step.values())
        r["frac_of_step_ceiling"] = r["achieved"] / r["step_ceiling"]
    r.update(kernel=STAGE_KERNEL[stage], kernel_ms=stages[stage], alg_flops=flops, alg_bytes=byts,
             flop_per_byte=flops / byts, overhead_bytes=over,
             hbm_gbs_alg=byts / sec / 1e9, mfma_tflops_alg=flops / sec / 1e12,
             mfma_frac=flops / sec / 1e12 / peak_f, hbm_frac=byts / sec / 1e9 / PEAK_HBM_GBS)
    return r


def roofline(w, stages: dict):
    """Roofline of the dominant kernel, plus the other two heavy kernels."""
    heavy = [s for s in HEAVY_STAGES if stages.get(s, 0.0) > 0]
    dom = max(heavy, key=lambda s: stages[s])
    r = roofline_of(w, stages, dom, measured_traffic(w, dom))
    r["others"] = {s: {k2: v for k2, v in roofline_of(w, stages, s, measured_traffic(w, s)).items()
                       if k2 in ("bound", "achieved", "frac", "unit", "kernel", "kernel_ms", "traffic",
                                 "mfma_frac", "hbm_frac", "overhead_bytes")}
                   for s in heavy if s != dom}
    return r


def measured_traffic(w, stage: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on this workload and on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("sources_sha") != sources_sha():
        return None
    ent = rec.get("kernels", {}).get(f"{STAGE_KERNEL[stage]}:{w.name}")
    return None if not ent else ent.get("bytes_per_launch")


def ingest(trace_dir: str, fetch_dir: str, write_dir: str, workload: str, command: str, log: str | None = None):
    """Turn rocprofv3 output (kernel-trace stats, FETCH_SIZE and WRITE_SIZE
    counter runs of the same command with --copy-calib-mib) into the committed
    text summaries under profiles/.  `log`: the traced run's stdout, whose
    JSON line holds bench.py's own event times of the heavy kernels, set
    beside the trace's durations of the same (timed) launches."""
    import csv
    import glob

    def rows(d, pat):
        out = []
        for f in glob.glob(os.path.join(d, "**", pat), recursive=True):
            out += list(csv.DictReader(open(f)))
        return out

    def short(name):
        n = name.split("(")[0]
        for key in ("k_score", "k_expert", "k_route_shared", "k_route", "k_attend", "k_final", "k_pool_short", "k_pool",
                    "k_scatter", "k_est", "k_tau", "k_scan", "k_topk_small", "k_fallback"):
            if f"{len(key)}{key}I" in n or n.endswith(key) or f"::{key}" in n or f"{len(key)}{key}E" in n:
                return key
        return n[:48]

    stats = rows(trace_dir, "*kernel_stats.csv")
    counters = {}
    for kind, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        acc = {}
        for r in rows(d, "*counter_collection.csv"):
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        counters[kind] = acc
    copy = [k for k in counters["FETCH_SIZE"] if "copyBuffer" in k]
    calib = {}
    if copy:
        n_kib = None
        for kind in ("FETCH_SIZE", "WRITE_SIZE"):
            v = counters[kind][copy[0]][0]
            calib[kind] = v
    mib = int(command.split("--copy-calib-mib")[1].split()[0]) if "--copy-calib-mib" in command else 0
    f_fac = (mib * 1024 / calib["FETCH_SIZE"]) if calib.get("FETCH_SIZE") else COPY_FETCH_FACTOR_DEFAULT
    w_fac = (mib * 1024 / calib["WRITE_SIZE"]) if calib.get("WRITE_SIZE") else 1.0
    kern = {}
    for name, vals in counters["FETCH_SIZE"].items():
        key = short(name)
        if key.startswith("k_"):
            fetch = sum(vals) / len(vals) * 1024 * f_fac
            wv = counters["WRITE_SIZE"].get(name, [0.0])
            write = sum(wv) / len(wv) * 1024 * w_fac
            kern[f"{key}:{workload}"] = dict(fetch_bytes=fetch, write_bytes=write, bytes_per_launch=fetch + write)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    # one record for every workload profiled on the current sources: the
    # entries of other workloads are kept when they were taken on these sources
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = dict(sources_sha=sources_sha(), kernels={}, commands={}, factors={})
    if os.path.exists(path):
        with open(path) as f:
            old = json.load(f)
        if old.get("sources_sha") == rec["sources_sha"] and "commands" in old:
            rec = old
    rec["kernels"] = {k2: v for k2, v in rec["kernels"].items() if not k2.endswith(":" + workload)}
    rec["kernels"].update(kern)
    rec["commands"][workload] = command
    rec["factors"][workload] = dict(fetch_factor=f_fac, write_factor=w_fac)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# rocprofv3 kernel trace and HBM traffic: mita_forward, {workload}", "",
             "Command (run from /tmp, TMPDIR=/tmp, repository at $R):", "",
             f"    rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- {command}",
             f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o run -- {command}",
             f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o run -- {command}", "",
             f"Counter calibration (plain {mib} MiB device copy in the same run): FETCH_SIZE x{f_fac:.3f}, "
             f"WRITE_SIZE x{w_fac:.3f}.", f"Kernel sources hash: {sources_sha()}.", "",
             "| kernel | calls | avg us | % time | HBM fetch MB | HBM write MB |", "|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        key = short(r["Name"])
        t = kern.get(f"{key}:{workload}", {})
        lines.append(f"| {key} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} | "
                     f"{t.get('fetch_bytes', 0) / 1e6:.1f} | {t.get('write_bytes', 0) / 1e6:.1f} |")
    if log:
        with open(log) as f:
            js = [json.loads(x) for x in f if x.startswith("{")]
        if js:
            rl = js[-1]["roofline"]
            live = {rl["kernel"]: rl["kernel_ms"]}
            live.update({v["kernel"]: v["kernel_ms"] for v in rl.get("others", {}).values()})
            steps = int(js[-1]["steps"])
            launches = {}
            for r in sorted(rows(trace_dir, "*kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"])):
                key = short(r["Kernel_Name"])
                if key in live:
                    launches.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
            lines += ["", "Agreement with `bench.py`'s own HIP events in the same traced run (its timed region is "
                      f"the last {steps} calls):", "",
                      "| kernel | bench.py events, timed calls (ms) | trace, same launches (ms) | trace, all launches (ms) |",
                      "|---|---|---|---|"]
            for key, ms in live.items():
                d = launches.get(key, [])
                if d:
                    lines.append(f"| {key} | {ms:.3f} | {sum(d[-steps:]) / len(d[-steps:]):.3f} | "
                                 f"{sum(d) / len(d):.3f} |")
            lines += ["", "The tracer lengthens each launch by a few percent; the kernel times of an untraced "
                      "`bench.py` run are in its JSON line (`roofline.kernel_ms`)."]
    with open(os.path.join(ROOT, "profiles", f"mita_forward_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_baseline(w, run):
    """Time the fp64 oracle on a bounded sample of the same workload.

    Sample: head 0.  Pooling runs in full; landmark scoring, top-k and shared
    values run on 1/3 of the landmark rows; routing and the joint softmax on
    1/3 of the queries (with the GPU's expert lists and shared values as
    inputs, which the oracle's cost does not depend on): about ten seconds of
    CPU work at N = 1M.  Each part's time is scaled by its sampling factor and
    summed over the B*H heads.
    """
    import torch
    from oracle import mita_oracle as mo
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    from efficient_long_sequence_amd import mita
    Q, K, V = (x[0, 0].astype(np.float64) for x in run["host"])
    _, dbg = mita.forward(run["q"], run["k"], run["v"], run["pool"], w.k, w.s, debug=True)
    torch.cuda.synchronize()
    I_gpu = dbg.topk[0, 0].cpu().numpy().astype(np.int64)
    Vt_gpu = dbg.vtilde[0, 0].cpu().numpy().astype(np.float64)
    fr, fq = 3, 3
    t0 = time.perf_counter()
    Qt = mo.landmarks(Q, w.grid_h, w.grid_w, w.land_h, w.land_w, w.dtype)
    t_pool = time.perf_counter() - t0
    rows = np.arange(0, w.m, fr)
    t0 = time.perf_counter()
    for r0 in range(0, rows.size, 32):
        rr = rows[r0:r0 + 32]
        S = mo.landmark_scores(Qt, K, rows=rr)
        mo.topk(S, w.k)
        mo.shared_values(S, V)
        del S
    t_rows = time.perf_counter() - t0
    qs = np.arange(0, w.N, fq)
    t0 = time.perf_counter()
    e, R = mo.route(Q[qs], Qt, w.s)
    mo.attend(Q[qs], K, V, Qt, Vt_gpu, I_gpu, e, R=R)
    t_query = time.perf_counter() - t0
    est_head = t_pool + t_rows * (w.m / rows.size) + t_query * (w.N / qs.size)
    measured = t_pool + t_rows + t_query
    est_total = est_head * w.B * w.H
    return dict(value=w.tokens / est_total, unit="tokens/s", cores=int(threads), kind="oracle",
                sample=(f"{w.name} head 0: pooling in full, scoring/top-k/shared values on "
                        f"{rows.size}/{w.m} landmark rows, routing and joint softmax on "
                        f"{qs.size}/{w.N} queries; {measured:.1f}s measured, scaled to "
                        f"{est_total:.1f}s for all {w.B * w.H} heads"))


# The pages' long-sequence throughput test (MiTA tutorial, ch.7, "LRA and
# synthetic long sequences"; paper section 4.3, Fig. 5): a three-layer model
# of width 128, m*k ~ N/4, batch chosen per length, speed-up of MiTA over full
# attention.  Points: (N, m = k, batch); the speed-ups the pages report (on an
# RTX 4090 with FlashAttention as the dense baseline) are context only.
E2E_POINTS = [(16384, 64, 16), (65536, 128, 4), (262144, 256, 1), (1048576, 512, 1)]
E2E_PAGES_SPEEDUP = {16384: 4.7, 65536: 19.0, 262144: 56.0, 1048576: 159.0}


def e2e(points, reps_mita: int = 5, reps_dense: int = 2):
    """Forward throughput of a 3-layer, width-128 Transformer (2 heads of 64,
    pre-LayerNorm blocks, GELU MLP of width 512, random bf16 weights) with
    MiTA attention (mita_forward) and with dense attention (our own
    mita_dense_attention kernel); projections, norms and the MLP are library
    calls shared by both.  Returns one dict per point."""
    import torch
    import torch.nn.functional as F
    from efficient_long_sequence_amd import mita
    dim, H, d, layers, hidden = 128, 2, 64, 3, 512
    g = torch.Generator(device="cuda").manual_seed(0)

    def w(i, o):
        return (torch.randn(i, o, device="cuda", generator=g) * (1.0 / i ** 0.5)).to(torch.bfloat16).contiguous()

    params = [dict(wqkv=w(dim, 3 * dim), wo=w(dim, dim), w1=w(dim, hidden), w2=w(hidden, dim)) for _ in range(layers)]

    def run_model(x, attend):
        B, N, _ = x.shape
        for P in params:
            h = F.layer_norm(x, (dim,))
            qkv = (h @ P["wqkv"]).view(B, N, 3, H, d).permute(2, 0, 3, 1, 4).contiguous()
            o = attend(qkv[0], qkv[1], qkv[2])
            x = x + o.permute(0, 2, 1, 3).reshape(B, N, dim) @ P["wo"]
            h = F.layer_norm(x, (dim,))
            x = x + F.gelu(h @ P["w1"]) @ P["w2"]
        return x

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps

    out = []
    for N, mk, B in points:
        x = torch.randn(B, N, dim, device="cuda", generator=g).to(torch.bfloat16)
        pool = (1, N, 1, mk)
        ws = torch.empty(mita.workspace_bytes(torch.bfloat16, B, H, N, d, pool, mk, 1), dtype=torch.uint8,
                         device="cuda")
        mita_attn = lambda q, k, v: mita.forward(q, k, v, pool, mk, 1, workspace=ws)
        t_mita = timed(lambda: run_model(x, mita_attn), reps_mita)
        t_dense = timed(lambda: run_model(x, mita.dense_attention), reps_dense)
        q = torch.randn(B, H, N, d, device="cuda", generator=g).to(torch.bfloat16)
        ta_mita = timed(lambda: mita_attn(q, q, q), reps_mita)
        ta_dense = timed(lambda: mita.dense_attention(q, q, q), reps_dense)
        out.append(dict(N=N, batch=B, m=mk, k=mk, s=1, model_tokens_per_s_mita=B * N / t_mita,
                        model_tokens_per_s_dense=B * N / t_dense, speedup_model=t_dense / t_mita,
                        attention_ms_mita=1e3 * ta_mita, attention_ms_dense=1e3 * ta_dense,
                        speedup_attention=ta_dense / ta_mita,
                        dense_attention_tflops=4.0 * B * H * N * N * d / ta_dense * 1e-12,
                        pages_reported_speedup=E2E_PAGES_SPEEDUP.get(N)))
        print(json.dumps(out[-1]), file=sys.stderr, flush=True)
        del x, ws, q
        torch.cuda.empty_cache()
    return out


def ablation(steps: int, warmup: int):
    """The pages' ablation with matched entries per query (republication,
    "LRA" section): MiTA (m shared + s k routed entries) against routing only
    (s k' routed entries, k' = k + m / s), on the long workloads."""
    import torch
    out = []
    for name in LONG:
        w = WORKLOADS[name]
        inputs = make_device_inputs(w)
        kk = w.k + w.m // w.s
        full = time_workload(w, steps, warmup, inputs=inputs)
        routed = time_workload(w, steps, warmup, variant="routed", k=kk, inputs=inputs)
        out.append(dict(workload=name, entries_per_query=w.m + w.s * w.k, mita_tokens_per_s=full["tokens_per_s"],
                        routed_only_k=kk, routed_only_tokens_per_s=routed["tokens_per_s"],
                        speedup_of_shared_branch=routed["ms_per_step"] / full["ms_per_step"],
                        mita_stages_ms=full["stages"], routed_only_stages_ms=routed["stages"]))
        del inputs, full, routed
        torch.cuda.empty_cache()
    return out


def time_graph(w, run, steps: int) -> float:
    """Tokens/s of the same forward captured once in a HIP graph
    (torch.cuda.CUDAGraph) and replayed `steps` times: the launch cost
    removed, which is what bounds the small shapes."""
    import torch
    from efficient_long_sequence_amd import mita
    q, kk, v, pool, ws = run["q"], run["k"], run["v"], run["pool"], run["ws"]
    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mita.forward(q, kk, v, pool, w.k, w.s, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mita.forward(q, kk, v, pool, w.k, w.s, workspace=ws, out=out)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    del g
    return w.tokens * steps / dt


def backward_flops(w, k: int | None = None) -> float:
    """Matrix-core flops of one backward pass (2 flops per multiply-add):
    joint softmax at the landmarks (S, dP, dq~, dv~ over m N pairs), routed
    keys (S, dP, dk, dv over N s k pairs), shared-value keys (the same four
    over N m pairs), shared-value landmarks (S, dP, dq~ over m N) and queries
    (S, dP, dq over N (m + s k)): d N (28 m + 14 s k) per head."""
    k = w.k if k is None else k
    return 2.0 * w.B * w.H * w.d * w.N * (14 * w.m + 7 * w.s * k)


def time_backward(w, steps: int, warmup: int, variant: str = "paper"):
    """forward_train and backward of one workload, timed with torch events on
    the launch stream (the library enqueues on torch's current stream)."""
    import torch
    from efficient_long_sequence_amd import mita, synth
    _, (q, kk, v) = make_device_inputs(w)
    pool = (w.grid_h, w.grid_w, w.land_h, w.land_w)
    g = torch.from_numpy(synth.make_grad(w.B, w.H, w.N, w.d, w.dtype, w.seed)).cuda().to(q.dtype)
    ws_f = torch.empty(mita.workspace_bytes(q.dtype, w.B, w.H, w.N, w.d, pool, w.k, w.s), dtype=torch.uint8,
                       device="cuda")
    ws_b = torch.empty(mita.backward_workspace_bytes(q.dtype, w.B, w.H, w.N, w.d, pool, w.k, w.s),
                       dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        O, sv = mita.forward_train(q, kk, v, pool, w.k, w.s, variant=variant, workspace=ws_f)
        mita.backward(q, kk, v, O, g, pool, w.k, w.s, sv, variant=variant, workspace=ws_b)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        O, sv = mita.forward_train(q, kk, v, pool, w.k, w.s, variant=variant, workspace=ws_f)
        e[1].record()
        mita.backward(q, kk, v, O, g, pool, w.k, w.s, sv, variant=variant, workspace=ws_b)
        e[2].record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    fwd = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    bwd = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    fl = backward_flops(w)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    return dict(workload=w.name, variant=variant, train_step_tokens_per_s=w.tokens * steps / dt,
                ms_per_step=1e3 * dt / steps, forward_train_ms=fwd, backward_ms=bwd,
                backward_tflops=fl / (bwd * 1e-3) * 1e-12, backward_frac_of_mfma_peak=fl / (bwd * 1e-3) * 1e-12 / peak)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE, choices=list(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", action="store_true", help="time only --workload")
    ap.add_argument("--ingest", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summaries from rocprofv3 output of the same command")
    ap.add_argument("--ingest-command", default="")
    ap.add_argument("--ingest-log", default=None, help="stdout of the traced run (its JSON line)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (calibrates HBM byte counters)")
    ap.add_argument("--e2e", action="store_true",
                    help="instead: the three-layer, width-128 model with MiTA vs dense attention at 16K-1M")
    ap.add_argument("--e2e-max-n", type=int, default=1 << 20, help="largest sequence length of --e2e")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the measured-peak probes (profiling runs: keeps their kernels out of the trace)")
    ap.add_argument("--backward", action="store_true",
                    help="instead: training step (forward_train + backward) of --workload (all long ones unless --only)")
    ap.add_argument("--ablation", action="store_true",
                    help="instead: MiTA against the routing-only variant with matched entries per query")
    args = ap.parse_args()
    if args.ingest:
        ingest(*args.ingest, workload=args.workload, command=args.ingest_command, log=args.ingest_log)
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU; --gpus {args.gpus} is not supported "
              "(every head is independent: a multi-GPU run would shard heads with no communication)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    if args.backward:
        names = [args.workload] if args.only else LONG
        pts = []
        for name in names:
            pts.append(time_backward(WORKLOADS[name], args.steps, args.warmup))
            print(json.dumps(pts[-1]), file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
        print(json.dumps(dict(metric="MiTA training step (forward_train + backward) tokens/s", unit="tokens/s",
                              n_gpus=1, dtype="bf16", data="synthetic", points=pts)), flush=True)
        return
    if args.ablation:
        print(json.dumps(dict(metric="MiTA vs routing-only forward tokens/s, entries per query matched",
                              unit="tokens/s", n_gpus=1, dtype="bf16", data="synthetic",
                              points=ablation(args.steps, args.warmup))), flush=True)
        return
    if args.e2e:
        pts = [p for p in E2E_POINTS if p[0] <= args.e2e_max_n]
        print(json.dumps(dict(metric="3-layer width-128 model forward tokens/s, MiTA vs dense attention",
                              unit="tokens/s", n_gpus=1, dtype="bf16", data="synthetic, random weights",
                              points=e2e(pts))), flush=True)
        return
    w = WORKLOADS[args.workload]
    if not args.no_probe:
        from efficient_long_sequence_amd import mita as _mita
        MEASURED_PEAKS.update(_mita.probe_peaks())
        torch.cuda.empty_cache()
    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    run = time_workload(w, args.steps, args.warmup)
    others = []
    if not args.only:
        # every other bf16 workload (the long ones the metric names, then the
        # vision-shaped and s = 2 ones); the tiny fp32 case is for parity only
        rest = [n for n in LONG if n != w.name] + [n for n in WORKLOADS
                                                   if n not in LONG and n != w.name and WORKLOADS[n].dtype == "bf16"]
        for name in rest:
            wo = WORKLOADS[name]
            r = time_workload(wo, args.steps, args.warmup)
            others.append(dict(workload=name, tokens_per_s=r["tokens_per_s"], ms_per_step=r["ms_per_step"],
                               call_ms=r["call_ms"], stages_ms=r["stages"], roofline=roofline(wo, r["heavy"]),
                               memory=r["memory"], tokens_per_s_graph=time_graph(wo, r, args.steps)))
            del r
            torch.cuda.empty_cache()
    # the same calls replayed from one captured HIP graph (launch cost removed)
    graph_value = time_graph(w, run, args.steps)
    train = None
    if not args.only:
        # the backward pass of the same workload (forward_train + backward), reported beside the forward
        try:
            train = time_backward(w, 5, 2)
        except Exception as exc:  # keep the forward line even if this extra measurement fails
            train = dict(error=f"{type(exc).__name__}: {exc}")
        torch.cuda.empty_cache()
    e2e_pts = abl = None
    if not args.only:
        # the pages' end-to-end comparison with dense attention at 16K-1M
        # (the dense model forward at 1M takes about 4 s: one timed run) and
        # the routing-only ablation, beside the forward
        try:
            e2e_pts = e2e(E2E_POINTS, reps_mita=3, reps_dense=1)
        except Exception as exc:
            e2e_pts = dict(error=f"{type(exc).__name__}: {exc}")
        torch.cuda.empty_cache()
        try:
            abl = ablation(5, 2)
        except Exception as exc:
            abl = dict(error=f"{type(exc).__name__}: {exc}")
        torch.cuda.empty_cache()
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, run)
    line = dict(
        metric=METRIC, value=run["tokens_per_s"], unit="tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=run["ms_per_step"], higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype=w.dtype, data="synthetic",
        config=dict(workload=w.name, B=w.B, H=w.H, N=w.N, d=w.d, m=w.m, k=w.k, s=w.s,
                    pool=f"{w.grid_h}x{w.grid_w} tokens -> {w.land_h}x{w.land_w} landmarks",
                    values=f"{w.kind}, {w.n_clusters} clusters, seed {w.seed}"),
        roofline=roofline(w, run["heavy"]), cpu_baseline=cpu, stages_ms=run["stages"],
        call_ms=run["call_ms"], tokens_per_s_median_call=run["tokens_per_s_median_call"],
        tokens_per_s_graph=graph_value,
        measured_peaks=dict(MEASURED_PEAKS), memory=run["memory"],
        other_workloads=others, training_step=train, end_to_end=e2e_pts, ablation_routing_only=abl,
    )
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
