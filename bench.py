"""Benchmark of the GQE attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--cpu-seconds S]

A step is one gqe_attn_fwd call over the whole layer (router, permutation,
sparse Q, dense K/V, causal attention, weighted slot, output projection) on
one batch of seeded synthetic input already resident in HBM. The default
workload is the 32K-token long-context layer (B=1, T=32768, D=1024, G=8, M=2,
k=1, d_h=64, bf16). Prints ONE JSON line with tokens/s, the attention kernel's
MFMA roofline fraction (timed live with HIP events on the library's stream),
the speedup over dense 16q/8kv GQA built from the same kernels, the training
step (forward that keeps its state + backward, with the attention backward's
MFMA rate), a decode step (16 sequences over a dense KV cache of the
workload's length, with the cache read's HBM rate), the chip's sustained
matrix-core rate from a register-only MFMA load (the published peak assumes a
clock the power limit does not hold), and the fp64 oracle timed on the host's
cores (a baseline only).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GQE attn fwd tokens/s at T=32K + MFMA util %; speedup vs dense GQA 16q/8kv"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (fp32 layers run fp32 MFMA)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_traffic.json")
ATTN_SRC = os.path.join(ROOT, "sparse_moe_attention_amd", "csrc", "attention.hpp")
DECODE_SRC = os.path.join(ROOT, "sparse_moe_attention_amd", "csrc", "decode.hpp")


def attn_flops(s, heads: int) -> float:
    """Algorithmic flops of one attention launch: 2 products of 2*d flops per
    (query, key) pair of the causal lower triangle (diagonal included)."""
    return heads * s.B * 4.0 * s.d * s.T * (s.T + 1) / 2.0


def active_heads(s) -> int:
    """Attention heads per token: the routed picks plus the shared head unless the merge drops it."""
    return s.G * s.k + (0 if getattr(s, "variant", "full") == "no_shared" else 1)


def layer_flops(s) -> float:
    per_tok = (2 * s.D * s.G * s.M + 2 * s.D * active_heads(s) * s.d + 4 * s.D * s.G * s.d
               + 2 * s.slots * s.d * s.D + 2 * s.G * s.k * s.d)
    return s.N * per_tok + attn_flops(s, active_heads(s))


def attn_bwd_flops(s, heads: int) -> float:
    """Algorithmic flops of the attention backward: five products of 2*d flops
    per causal (query, key) pair (scores recomputed, dP, dV, dK, dQ), i.e.
    2.5 times the forward's."""
    return 2.5 * attn_flops(s, heads)


def layer_leg(gq, torch, s, dv, steps, warmup, mk_events, with_gqa=True):
    """gqe_attn_fwd on one workload: W warmup steps, then K timed steps with
    HIP events around the attention kernel in every step (on the library's
    stream), one extra isolated step for the per-stage breakdown, and the dense
    GQA layer (all G*M heads) on the same tensors."""
    dt = s.torch_dtype()
    shape = gq.shape_from(s)
    out = torch.empty(s.N, s.D, dtype=dt, device="cuda")
    ws = torch.empty(gq.gqe_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    dcode = gq.GQE_F32 if s.dtype == "f32" else gq.GQE_BF16
    A0, A1 = 5, 6                    # events before / after the attention stage

    def fwd(arr=None):
        gq.gqe_attn_fwd_timed(shape, dv["x"], dv["Wr"], dv["br"], dv["Wq"], dv["Wk"], dv["Wv"], dv["Wq_sh"],
                              dv["Wo"], out, arr, ws=ws)

    for _ in range(warmup):
        fwd()
    step_ev = []
    for _ in range(steps):
        e = mk_events(2)
        arr = [None] * (gq.GQE_N_STAGES + 1)
        arr[A0], arr[A1] = e
        step_ev.append((e, gq.event_array(arr)))
    t0, t1 = mk_events(2)
    torch.cuda.synchronize()
    wall = time.perf_counter()
    t0.record()
    for _, arr in step_ev:
        fwd(arr)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall
    ms_step = t0.elapsed_time(t1) / steps
    attn_ms = sum(e[0].elapsed_time(e[1]) for e, _ in step_ev) / steps

    # one fully instrumented step for the per-stage breakdown (outside the timed region)
    evs = mk_events(gq.GQE_N_STAGES + 1)
    torch.cuda.synchronize()
    fwd(gq.event_array(evs))
    torch.cuda.synchronize()
    stage_ms = {n: round(evs[i].elapsed_time(evs[i + 1]), 4) for i, n in enumerate(gq.GQE_STAGE_NAMES)}
    del ws, out

    gqa = None
    if with_gqa:
        wsg = torch.empty(gq.gqa_workspace_bytes(s.B, s.T, s.D, s.Hq, s.G, s.d, dcode), dtype=torch.uint8,
                          device="cuda")
        og = torch.empty(s.N, s.D, dtype=dt, device="cuda")

        def gfwd(arr=None):
            gq.gqa_attn_fwd_timed(s.B, s.T, s.D, s.Hq, s.G, s.d, dcode, dv["x"], dv["Wq"], dv["Wk"], dv["Wv"],
                                  dv["Wo_gqa"], og, arr, ws=wsg)

        for _ in range(warmup):
            gfwd()
        gev = []
        for _ in range(steps):
            e = mk_events(2)
            arr = [None] * (gq.GQA_N_STAGES + 1)
            arr[1], arr[2] = e
            gev.append((e, gq.event_array(arr)))
        g0, g1 = mk_events(2)
        torch.cuda.synchronize()
        g0.record()
        for _, arr in gev:
            gfwd(arr)
        g1.record()
        torch.cuda.synchronize()
        gqa_ms = g0.elapsed_time(g1) / steps
        gqa_attn_ms = sum(e[0].elapsed_time(e[1]) for e, _ in gev) / steps
        gqa = {"tokens_per_s": s.N / (gqa_ms / 1e3), "ms_per_step": gqa_ms, "attention_ms": gqa_attn_ms,
               "heads": f"{s.Hq}q/{s.G}kv", "speedup_gqe_over_gqa": gqa_ms / ms_step,
               "attention_speedup": gqa_attn_ms / attn_ms}
        del wsg, og
    peak = PEAK_F32_TFLOPS if s.dtype == "f32" else PEAK_BF16_TFLOPS
    fl = attn_flops(s, active_heads(s))
    achieved = fl / (attn_ms / 1e3) / 1e12
    return {"tokens_per_s": s.N / (ms_step / 1e3), "ms_per_step": ms_step, "steps": steps, "warmup": warmup,
            "attention_ms": attn_ms, "attn_tflops": achieved, "attn_frac": achieved / peak,
            "layer_mfma_frac": layer_flops(s) / (ms_step / 1e3) / 1e12 / peak, "stage_ms": stage_ms,
            "gqa_baseline": gqa, "wall_s_timed_region": wall}


OTHER_STEPS = {1: 50, 2: 50, 3: 20, 4: 20, 5: 3}


def other_configs(gq, torch, headline: int, warmup: int, mk_events):
    """The other workloads at one GPU, each timed like the headline (fewer steps
    at 1M tokens); reported beside the headline, never as its value."""
    from workloads import CONFIG_NAMES, config_inputs
    res = {}
    for cid in sorted(OTHER_STEPS):
        if cid == headline:
            continue
        s, inp = config_inputs(cid)
        dv = {k: (v.cuda().contiguous() if v is not None else None) for k, v in inp.items()}
        del inp
        r = layer_leg(gq, torch, s, dv, OTHER_STEPS[cid], min(warmup, 1) if cid == 5 else warmup, mk_events)
        r["workload"] = CONFIG_NAMES[cid]
        res[f"config{cid}"] = r
        del dv
        torch.cuda.empty_cache()
        print(f"[bench] config {cid}: {r['tokens_per_s']:.4g} tokens/s, attention frac {r['attn_frac']:.3f}",
              file=sys.stderr, flush=True)
    return res


def train_leg(gq, torch, s, dv, steps, warmup, mk_events):
    """Training step = gqe_attn_fwd_train + gqe_attn_bwd on the same inputs
    (dout seeded, resident in HBM). Returns the record's "backward" object."""
    from workloads import make_grad_output
    shape = gq.shape_from(s)
    wst = torch.empty(gq.gqe_train_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    out = torch.empty(s.N, s.D, dtype=torch.bfloat16, device="cuda")
    dout = make_grad_output(s, seed=3000).cuda()
    g = {k: torch.empty_like(dv[k[1:]] if k != "dx" else dv["x"], dtype=torch.float32) for k in gq.BWD_GRADS}
    dbr = torch.empty(s.G * s.M, dtype=torch.float32, device="cuda")
    aux = torch.empty(1, dtype=torch.float32, device="cuda")
    coef = 0.01

    def step(events=None):
        gq.gqe_attn_fwd_train(shape, dv["x"], dv["Wr"], dv["br"], dv["Wq"], dv["Wk"], dv["Wv"], dv["Wq_sh"],
                              dv["Wo"], out, wst)
        gq.gqe_attn_bwd(shape, dv["x"], dv["Wr"], dv["Wq"], dv["Wk"], dv["Wv"], dv["Wq_sh"], dv["Wo"], dout,
                        coef, g, wst, dbr=dbr, aux_loss=aux, events=events)

    for _ in range(warmup):
        step()
    # events around the two attention-backward kernels of every timed step
    D0, D1, D2 = 3, 4, 5
    ev = []
    for _ in range(steps):
        e = mk_events(3)
        arr = [None] * (gq.GQE_BWD_N_STAGES + 1)
        arr[D0], arr[D1], arr[D2] = e
        ev.append((e, gq.event_array(arr)))
    t0, t1 = mk_events(2)
    torch.cuda.synchronize()
    t0.record()
    for _, arr in ev:
        step(arr)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    dkdv_ms = sum(e[0].elapsed_time(e[1]) for e, _ in ev) / steps
    dq_ms = sum(e[1].elapsed_time(e[2]) for e, _ in ev) / steps
    evs = mk_events(gq.GQE_BWD_N_STAGES + 1)
    torch.cuda.synchronize()
    step(gq.event_array(evs))
    torch.cuda.synchronize()
    stage_ms = {n: round(evs[i].elapsed_time(evs[i + 1]), 4) for i, n in enumerate(gq.GQE_BWD_STAGE_NAMES)}
    heads = active_heads(s)
    fl = attn_bwd_flops(s, heads)
    tf = fl / ((dkdv_ms + dq_ms) / 1e3) / 1e12
    return {"tokens_per_s": s.N / (ms / 1e3), "ms_per_step": ms, "what": "gqe_attn_fwd_train + gqe_attn_bwd",
            "bwd_stage_ms": stage_ms, "attn_bwd_ms": {"dkdv": dkdv_ms, "dq": dq_ms},
            "attn_bwd_algorithmic_flops": fl, "attn_bwd_tflops": tf, "attn_bwd_frac": tf / PEAK_BF16_TFLOPS,
            "aux_coef": coef}


DECODE_B = 16


def decode_leg(gq, torch, s, dv, steps, warmup, mk_events, cid):
    """One decode step per sequence over a dense KV cache: B = 16 sequences
    with T - 1 cached positions each (the new token at T - 1), the layer of
    the workload otherwise. Synthetic bf16 caches. Returns the record's
    "decode_step" object with the attention-over-cache kernel's HBM rate."""
    import dataclasses
    from workloads import Shape, make_inputs
    B, T = DECODE_B, s.T
    ds = Shape(B=B, T=T, D=s.D, G=s.G, M=s.M, k=s.k, d=s.d, router_bias=s.router_bias,
               shared_kv_group=s.shared_kv_group)
    tok = make_inputs(dataclasses.replace(ds, T=1), seed=4000)
    w = {k: (v.cuda() if v is not None else None) for k, v in tok.items()}
    gen = torch.Generator(device="cuda").manual_seed(4001)
    kc = torch.randn(ds.G, B, T, ds.d, device="cuda", generator=gen).to(torch.bfloat16)
    vtc = torch.randn(ds.G, ds.d, B * T, device="cuda", generator=gen).to(torch.bfloat16)
    pos = torch.full((B,), T - 1, dtype=torch.int32, device="cuda")
    sh = gq.shape_from(ds)
    ws = torch.empty(gq.gqe_decode_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, ds.D, dtype=torch.bfloat16, device="cuda")

    def step(ev=None):
        gq.gqe_decode_step(sh, pos, w["x"], w["Wr"], w["br"], w["Wq"], w["Wk"], w["Wv"], w["Wq_sh"], w["Wo"], kc,
                           vtc, out, ws, events=ev)

    for _ in range(warmup):
        step()
    n = max(steps, 20)
    ev = [mk_events(gq.GQE_DECODE_N_STAGES + 1) for _ in range(n)]
    t0, t1 = mk_events(2)
    torch.cuda.synchronize()
    t0.record()
    for e in ev:
        step(gq.event_array(e))
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / n
    stage = [sum(e[i].elapsed_time(e[i + 1]) for e in ev) / n for i in range(gq.GQE_DECODE_N_STAGES)]
    attn_ms = stage[1]
    kv_bytes = 2.0 * B * ds.G * T * ds.d * 2          # every cached key and value read once
    gbs = kv_bytes / (attn_ms * 1e-3) / 1e9
    return {"tokens_per_s": B / (ms / 1e3), "ms_per_step": ms,
            "workload": f"{B} sequences x {T - 1} cached positions, one new token each, D{ds.D} G{ds.G} "
                        f"M{ds.M} k{ds.k} d{ds.d} bf16",
            "stage_ms": {nm: round(v, 4) for nm, v in zip(gq.GQE_DECODE_STAGE_NAMES, stage)},
            "attn_roofline": {"bound": "hbm", "kernel": "attn_decode_kernel", "achieved": gbs, "peak": 8000.0,
                              "unit": "GB/s", "frac": gbs / 8000.0,
                              "traffic": measured_traffic(f"decode_config{cid}", DECODE_SRC),
                              "algorithmic_bytes_per_launch": kv_bytes, "avg_launch_ms": attn_ms}}


def mfma_probe_leg(gq, torch, mk_events, launches: int = 5):
    """The sustained bf16 matrix-core rate of this chip: gqe_mfma_probe keeps
    every SIMD issuing 16x16x32 bf16 products from registers (no memory
    traffic) for several milliseconds per launch, long enough to reach the
    clock the power limit holds. The implied clock assumes one product per
    SIMD every 16 cycles (1024 flops per SIMD per cycle, 1024 SIMDs)."""
    wgs, iters = 256 * 8, 8000
    out = torch.empty(wgs, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(2):
        gq.gqe_mfma_probe(wgs, iters, out)
    e0, e1 = mk_events(2)
    e0.record(stream)
    for _ in range(launches):
        gq.gqe_mfma_probe(wgs, iters, out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("gqe_mfma_probe: non-finite checksum")
    fl = wgs * 4 * iters * 8 * 16384.0
    tf = fl / (ms / 1e3) / 1e12
    return {"kernel": "mfma_probe_kernel", "tflops": tf, "frac_of_published": tf / PEAK_BF16_TFLOPS,
            "implied_clock_ghz": tf * 1e12 / (1024 * 1024) / 1e9, "avg_launch_ms": ms}


def source_sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(key: str, src: str):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary (entry `key`), if it was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get(key)
    if not entry or entry.get("src_sha") != source_sha(src):
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(s, inp, target_s: float):
    """The fp64 oracle on the host's cores, on a bounded sample of the same
    layer: the dense per-token work (routing of all tokens, K/V projections)
    runs in full; the per-row work (routed and shared queries, attention over
    the whole causal prefix, slots, Wo) runs on R stratified rows and is
    scaled by N/R. Returns the estimated whole-layer tokens/s."""
    import numpy as np
    import oracle.gqe_oracle as go
    from workloads import sample_rows, to_f64
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(p.get("num_threads", 1)) for p in threadpool_info()) if threadpool_info() else 1
    except Exception:
        cores = os.cpu_count() or 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next(ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name"))
    except (OSError, StopIteration):
        pass
    f = {k: to_f64(v) for k, v in inp.items()}
    t = time.perf_counter()
    go.route(f["x"], f["Wr"], f.get("br"), s.G, s.M, s.k)
    go.project(f["x"], f["Wk"])
    go.project(f["x"], f["Wv"])
    t_fixed = time.perf_counter() - t
    # calibrate the row count on a small sample, then fill the time budget
    r0 = 16
    t = time.perf_counter()
    go.gqe_rows(f, s.G, s.M, s.k, s.d, s.B, s.T, sample_rows(s, r0, 7), shared_kv_group=s.shared_kv_group, variant=s.variant)
    per_row = max((time.perf_counter() - t - t_fixed) / r0, 1e-6)
    R = int(min(s.N, max(r0, (target_s - t_fixed) / per_row)))
    rows = sample_rows(s, R, 11)
    t = time.perf_counter()
    go.gqe_rows(f, s.G, s.M, s.k, s.d, s.B, s.T, rows, shared_kv_group=s.shared_kv_group, variant=s.variant)
    t_rows = time.perf_counter() - t
    per_row = max((t_rows - t_fixed) / len(rows), 1e-9)
    est = t_fixed + s.N * per_row
    return {
        "value": s.N / est, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model,
        "host_cpus_visible": os.cpu_count(),
        "sample": (f"fp64 numpy oracle: routing + K/V projection of all {s.N} tokens in full "
                   f"({t_fixed:.2f} s), then {len(rows)} stratified rows of the full layer over their whole "
                   f"causal prefix ({t_rows:.2f} s incl. the dense part again), per-row cost scaled to N; "
                   f"estimated full-layer time {est:.1f} s"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=25.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gqa", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the training-step (forward + backward) leg")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other workloads (reported under \"configs\")")
    ap.add_argument("--variant", default="full", choices=["full", "weighted_concat", "hard_concat", "no_shared"],
                    help="merge of the picked experts: the layer, or one of the pages' ablations")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times): the reference that scales "
                         "rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the GQE forward runs on a single MI355X here; "
              "run it with --gpus 1 (sharding over several GPUs is not built).",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "dispatches": 3}), flush=True)
        return
    import sparse_moe_attention_amd as gq
    from workloads import CONFIG_NAMES, config_inputs

    gq.load()
    torch.cuda.set_device(0)
    s, inp = config_inputs(args.config)
    if args.variant != "full":
        # the ablations' Wo has one slot fewer; its leading columns serve
        s = dataclasses.replace(s, variant=args.variant)
        inp = dict(inp, Wo=inp["Wo"][:, :s.slots * s.d].contiguous())
    steps = args.steps if args.steps is not None else {1: 50, 2: 50, 3: 20, 4: 20, 5: 3}[args.config]
    dv = {k: (v.cuda().contiguous() if v is not None else None) for k, v in inp.items()}
    def mk_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record()
        return evs

    lay = layer_leg(gq, torch, s, dv, steps, args.warmup, mk_events, with_gqa=not args.no_gqa)
    ms_step, attn_ms, wall = lay["ms_per_step"], lay["attention_ms"], lay["wall_s_timed_region"]
    stage_ms, gqa = lay["stage_ms"], lay["gqa_baseline"]

    bwd = None
    if not args.no_backward and s.dtype == "bf16" and s.variant == "full":
        bwd = train_leg(gq, torch, s, dv, steps, args.warmup, mk_events)

    dec = None
    if not args.no_decode and s.dtype == "bf16" and s.variant == "full" and s.T % 32 == 0:
        dec = decode_leg(gq, torch, s, dv, steps, args.warmup, mk_events, args.config)

    others = None
    if not args.no_configs and s.variant == "full":
        del dv
        torch.cuda.empty_cache()
        others = other_configs(gq, torch, args.config, args.warmup, mk_events)

    probe = mfma_probe_leg(gq, torch, mk_events)
    peak = PEAK_F32_TFLOPS if s.dtype == "f32" else PEAK_BF16_TFLOPS
    fl = attn_flops(s, active_heads(s))
    achieved = fl / (attn_ms / 1e3) / 1e12
    if s.dtype == "bf16":
        probe["attn_frac_of_sustained"] = achieved / probe["tflops"]
    traffic = measured_traffic(f"config{args.config}", ATTN_SRC)
    rec = {
        "metric": METRIC,
        "value": s.N / (ms_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.dtype == "bf16" else "f32",
        "data": "synthetic (seeded randn inputs and random-init weights of the layer's shape)",
        "config": {"workload": CONFIG_NAMES[args.config] + ("" if s.variant == "full" else f", {s.variant} merge"),
                   "B": s.B, "T": s.T, "D": s.D, "G": s.G, "M": s.M, "k": s.k, "d_h": s.d,
                   "shared_kv_group": s.shared_kv_group, "variant": s.variant, "tokens_per_step": s.N},
        "roofline": {"bound": "mfma", "kernel": "attn_fwd_kernel", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": traffic,
                     "algorithmic_flops_per_launch": fl, "avg_launch_ms": attn_ms},
        "layer_mfma_frac": layer_flops(s) / (ms_step / 1e3) / 1e12 / peak,
        "mfma_sustained": probe,
        "stage_ms": stage_ms,
        "gqa_baseline": gqa,
        "training_step": bwd,
        "decode_step": dec,
        "configs": others,
        "wall_s_timed_region": wall,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(s, inp, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
