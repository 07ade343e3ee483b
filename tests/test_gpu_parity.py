"""GPU parity of libgqe.so against the fp64 oracle, through the C ABI.

Per stage: router logits (fp32 vs fp64), idx (bit-exact except near-tie
rows), w, per-expert counts, merged slots, and the layer output. Every
layer up to 32K tokens (the small edge shapes and the four workloads that fit
the fp64 oracle whole) is compared element by element over the whole tensor;
the 1M-token layer and the long-shape cases on sampled rows that the oracle
computes one by one.
"""
from __future__ import annotations

import dataclasses
import os
import time

import numpy as np
import pytest
import torch

import oracle.gqe_oracle as go
import sparse_moe_attention_amd as gq
from tests import harness as H
from workloads import CONFIGS, Shape, config_inputs, make_inputs, sample_rows

pytestmark = pytest.mark.gpu

# Shapes that span several tiles, ragged tails and the degenerate cases.
CASES = {
    "ragged_bias_k2": Shape(B=3, T=200, D=128, G=3, M=3, k=2, d=32, router_bias=True, shared_kv_group=1),
    "fp32_k3_of_4": Shape(B=2, T=77, D=64, G=2, M=4, k=3, d=64, dtype="f32"),
    "single_token": Shape(B=2, T=1, D=64, G=2, M=2, k=1, d=64),
    "one_group": Shape(B=1, T=300, D=192, G=1, M=4, k=2, d=64),
    "one_expert": Shape(B=1, T=130, D=64, G=4, M=1, k=1, d=32),
    "all_experts": Shape(B=2, T=150, D=128, G=2, M=3, k=3, d=64),
    "multi_tile": Shape(B=2, T=1000, D=256, G=8, M=2, k=1, d=64),
    "wide_pool": Shape(B=1, T=260, D=128, G=4, M=16, k=4, d=32, router_bias=True),
    "max_pool_256_experts": Shape(B=2, T=131, D=64, G=4, M=64, k=3, d=32, router_bias=True, shared_kv_group=3),
    "many_short_sequences": Shape(B=33, T=37, D=64, G=2, M=2, k=1, d=64),
    # 9 regular KV streams and one or two shared-head tiles per level: some
    # levels have more streams homed on an XCD than slots landing on it.
    "many_groups": Shape(B=1, T=300, D=128, G=10, M=4, k=4, d=32),
    # Wo contracts over (G*k + 2)*d = 96 columns: the GEMM's last K step is partial.
    "partial_k_step": Shape(B=2, T=230, D=128, G=1, M=2, k=1, d=32, router_bias=True),
}

# Dense GQA layers (Hq = G*M query heads over G KV groups). 3 sequences x 3
# groups = 9 KV streams: the attention grid's placement then has to hand some
# streams to slots away from their home XCD.
GQA_CASES = {
    "gqa_9_streams": Shape(B=3, T=600, D=128, G=3, M=2, k=1, d=32),
    "gqa_ragged_f32": Shape(B=2, T=333, D=64, G=1, M=4, k=1, d=64, dtype="f32"),
    "gqa_wide": Shape(B=1, T=515, D=256, G=5, M=3, k=1, d=64),
    # 3 heads x 32: the output projection contracts over 96 columns (partial last K step).
    "gqa_partial_k_step": Shape(B=2, T=190, D=64, G=1, M=3, k=1, d=32),
}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load()
    torch.cuda.set_device(0)


def check_routing(s, f, dv, tag):
    """gqe_route against the oracle; returns (GPU idx, GPU w, oracle routing, near-tie mask)."""
    logits_ref, sel_ref, w_ref = H.oracle_routing(f, s)
    near = H.near_tie_rows(logits_ref, s)
    o = H.alloc_outputs(s)
    lg = torch.empty(s.N, s.G * s.M, dtype=torch.float32, device="cuda")
    counts = torch.empty(s.G * s.M, dtype=torch.int32, device="cuda")
    gq.gqe_route(gq.shape_from(s), dv["x"], dv["Wr"], dv["br"], o["idx"], o["w"], lg, counts)
    torch.cuda.synchronize()
    lg_n = lg.cpu().numpy().astype(np.float64)
    lerr = np.abs(lg_n - logits_ref) / np.maximum(1.0, np.abs(logits_ref))
    assert lerr.max() <= H.LOGIT_REL, (tag, "logits", lerr.max())
    idx = o["idx"].cpu().numpy()
    w = o["w"].cpu().numpy().astype(np.float64)
    bad = (idx != sel_ref).any(axis=(1, 2))
    assert not (bad & ~near).any(), (tag, "idx mismatch off near-ties", np.nonzero(bad & ~near)[0][:10])
    ok = ~bad
    werr = np.abs(w[ok] - w_ref[ok]).max() if ok.any() else 0.0
    assert werr <= H.W_ABS, (tag, "w", werr)
    e = (idx.reshape(s.N, s.G, s.k) + (np.arange(s.G) * s.M)[None, :, None]).reshape(-1)
    assert (counts.cpu().numpy() == np.bincount(e, minlength=s.G * s.M)).all(), (tag, "counts")
    assert (counts.cpu().numpy().sum() == s.N * s.G * s.k)
    return idx, w, (logits_ref, sel_ref, w_ref), near, bad


@pytest.mark.parametrize("name", sorted(CASES))
def test_small_layer_full_parity(name):
    layer_parity(CASES[name], name, seed=7 + len(name))


# The pages' merge ablations on two of the shapes above (one with the shared
# head on group 1, one spanning several attention tiles).
VARIANT_CASES = [(v, base) for v in ("weighted_concat", "hard_concat", "no_shared")
                 for base in ("ragged_bias_k2", "multi_tile")]


@pytest.mark.parametrize("variant,base", VARIANT_CASES, ids=[f"{v}-{b}" for v, b in VARIANT_CASES])
def test_variant_full_parity(variant, base):
    layer_parity(dataclasses.replace(CASES[base], variant=variant), f"{variant}/{base}", seed=31 + len(base))


def layer_parity(s, name, seed):
    inp = make_inputs(s, seed=seed)
    f = H.f64_inputs(inp)
    dv = H.to_device(inp)
    print(f"[case {name}] {s}", flush=True)
    idx, w, (lref, sref, wref), near, bad = check_routing(s, f, dv, name)
    ref = go.gqe_forward(f, s.G, s.M, s.k, s.d, s.B, s.T, shared_kv_group=s.shared_kv_group, variant=s.variant)

    # Full path: idx_out must equal gqe_route's, out must match on every row
    # whose routing agrees with the oracle.
    o = H.alloc_outputs(s)
    H.run_gqe(s, dv, o)
    torch.cuda.synchronize()
    assert (o["idx"].cpu().numpy() == idx).all()
    assert (o["w"].cpu().numpy() == w.astype(np.float32)).all()
    got = H.np32(o["out"])
    keep = ~bad
    err, bound = H.out_error(got[keep], ref["out"][keep])
    assert err <= bound, (name, "out", err, bound)

    # Routed path with the oracle's routing injected: slots and out on every row.
    out2 = torch.empty_like(o["out"])
    slots = torch.empty(s.N, s.slots * s.d, dtype=s.torch_dtype(), device="cuda")
    H.run_gqe_routed(s, dv, torch.from_numpy(sref.astype(np.int32)).cuda(),
                     torch.from_numpy(wref.astype(np.float32)).cuda(), out2, slots)
    torch.cuda.synchronize()
    err, bound = H.out_error(H.np32(slots), ref["C"])
    assert err <= bound, (name, "slots", err, bound)
    err, bound = H.out_error(H.np32(out2), ref["out"])
    assert err <= bound, (name, "routed out", err, bound)


@pytest.mark.parametrize("name", sorted(GQA_CASES))
def test_small_gqa_full_parity(name):
    s = GQA_CASES[name]
    inp = make_inputs(s, seed=11 + len(name))
    f = H.f64_inputs(inp)
    dv = H.to_device(inp)
    print(f"[gqa case {name}] {s}", flush=True)
    ga = go.gqa_forward(dict(x=f["x"], Wq=f["Wq"], Wk=f["Wk"], Wv=f["Wv"], Wo=f["Wo_gqa"]),
                        s.G, s.Hq, s.d, s.B, s.T)
    og = torch.empty(s.N, s.D, dtype=s.torch_dtype(), device="cuda")
    H.run_gqa(s, dv, og)
    torch.cuda.synchronize()
    err, bound = H.out_error(H.np32(og), ga["out"])
    assert err <= bound, (name, err, bound)


# Threads for the oracle's per-head attentions on the large layers (results
# are bit-identical to the serial loop; the box gives one GPU 16 host cores).
ORACLE_WORKERS = max(1, min(16, os.cpu_count() or 1))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_config_full_parity(cid):
    """Every configuration that fits the fp64 oracle whole (up to 32K tokens),
    over the whole tensor: routing as in check_routing; the full path's output
    on every row whose routing agrees with the oracle (near-tie rows may
    differ); then the oracle's routing injected into the routed path, whose
    merged slots C and output are compared on every row."""
    s, inp = config_inputs(cid)
    print(f"[config {cid}] {s}", flush=True)
    f = H.f64_inputs(inp)
    dv = H.to_device(inp)
    idx, w, (lref, sref, wref), near, bad = check_routing(s, f, dv, f"config{cid}")
    o = H.alloc_outputs(s)
    H.run_gqe(s, dv, o)
    out2 = torch.empty_like(o["out"])
    slots = torch.empty(s.N, s.slots * s.d, dtype=s.torch_dtype(), device="cuda")
    H.run_gqe_routed(s, dv, torch.from_numpy(sref.astype(np.int32)).cuda(),
                     torch.from_numpy(wref.astype(np.float32)).cuda(), out2, slots)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ref = go.gqe_forward(f, s.G, s.M, s.k, s.d, s.B, s.T, shared_kv_group=s.shared_kv_group,
                         workers=ORACLE_WORKERS)
    print(f"[config {cid}] oracle {time.perf_counter() - t0:.1f} s on {ORACLE_WORKERS} threads", flush=True)
    assert (ref["idx"] == sref).all()
    got = H.np32(o["out"])
    err, bound = H.out_error(got[~bad], ref["out"][~bad])
    print(f"[config {cid}] out max err {err:.3e} bound {bound:.3e}; near-tie rows {int(near.sum())}, "
          f"mismatched {int(bad.sum())}", flush=True)
    assert err <= bound
    err, bound = H.out_error(H.np32(slots), ref["C"])
    print(f"[config {cid}] routed slots max err {err:.3e} bound {bound:.3e}", flush=True)
    assert err <= bound, ("routed slots", err, bound)
    err, bound = H.out_error(H.np32(out2), ref["out"])
    assert err <= bound, ("routed out", err, bound)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_config_gqa_full_parity(cid):
    """The dense GQA baseline (all G*M heads) on the same tensors, whole tensor."""
    s, inp = config_inputs(cid)
    print(f"[config {cid} gqa] {s}", flush=True)
    f = H.f64_inputs(inp)
    dv = H.to_device(inp)
    og = torch.empty(s.N, s.D, dtype=s.torch_dtype(), device="cuda")
    H.run_gqa(s, dv, og)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ga = go.gqa_forward(dict(x=f["x"], Wq=f["Wq"], Wk=f["Wk"], Wv=f["Wv"], Wo=f["Wo_gqa"]),
                        s.G, s.Hq, s.d, s.B, s.T, workers=ORACLE_WORKERS)
    err, bound = H.out_error(H.np32(og), ga["out"])
    print(f"[config {cid} gqa] oracle {time.perf_counter() - t0:.1f} s; out max err {err:.3e} bound {bound:.3e}",
          flush=True)
    assert err <= bound, ("gqa", err, bound)


@pytest.mark.timeout(600)
def test_config5_sampled_parity():
    """The 1M-token layer: routing of every token, outputs on 64 sampled rows
    (t = 0, t = T-1 and 62 stratified rows) that the oracle streams one by one."""
    cid, n_rows = 5, 64
    s, inp = config_inputs(cid)
    print(f"[config {cid}] {s}", flush=True)
    f = H.f64_inputs(inp)
    dv = H.to_device(inp)
    del inp
    idx, w, (lref, sref, wref), near, bad = check_routing(s, f, dv, f"config{cid}")
    rows = sample_rows(s, n_rows, seed=1000 + cid)
    ref = go.gqe_rows(f, s.G, s.M, s.k, s.d, s.B, s.T, rows)
    o = H.alloc_outputs(s)
    H.run_gqe(s, dv, o)
    torch.cuda.synchronize()
    got = H.np32(o["out"][torch.from_numpy(rows).cuda()])
    keep = ~bad[rows]
    err, bound = H.out_error(got[keep], ref["out"][keep])
    print(f"[config {cid}] sampled out max err {err:.3e} bound {bound:.3e}; near-tie rows "
          f"{int(near.sum())}, mismatched {int(bad.sum())}", flush=True)
    assert err <= bound
    # routed path with the oracle's routing
    out2 = torch.empty_like(o["out"])
    H.run_gqe_routed(s, dv, torch.from_numpy(sref.astype(np.int32)).cuda(),
                     torch.from_numpy(wref.astype(np.float32)).cuda(), out2)
    torch.cuda.synchronize()
    got2 = H.np32(out2[torch.from_numpy(rows).cuda()])
    err, bound = H.out_error(got2, ref["out"])
    assert err <= bound, ("routed", err, bound)


# Sequences past 256K tokens take the long-context attention tile shape
# (8 waves x 32 rows, 128-key tiles); the 1M-token workload above covers it at
# d = 64 with T a multiple of the tile. These add a ragged T (a partial last
# key tile and row tile), d = 32, k = 2 with the shared head on group 1, two
# sequences, and the dense GQA layer, on sampled rows that include the last
# rows of each sequence.
LONG_CASES = {
    "long_ragged_d32_k2": Shape(B=2, T=262144 + 1037, D=64, G=2, M=3, k=2, d=32, router_bias=True,
                                shared_kv_group=1),
    "long_ragged_d64": Shape(B=1, T=262144 + 4099, D=64, G=3, M=2, k=1, d=64),
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", sorted(LONG_CASES))
def test_long_shape_sampled_parity(name):
    s = LONG_CASES[name]
    print(f"[long case {name}] {s}", flush=True)
    inp = make_inputs(s, seed=77 + len(name))
    f = H.f64_inputs(inp)
    dv = H.to_device(inp)
    del inp
    idx, w, (lref, sref, wref), near, bad = check_routing(s, f, dv, name)
    tails = [b * s.T + t for b in range(s.B) for t in (s.T - 1, s.T - 2, s.T - 129, s.T - 1037)]
    rows = np.unique(np.concatenate([sample_rows(s, 48, seed=2000 + len(name)), np.array(tails, dtype=np.int64)]))
    ref = go.gqe_rows(f, s.G, s.M, s.k, s.d, s.B, s.T, rows, shared_kv_group=s.shared_kv_group)
    o = H.alloc_outputs(s)
    H.run_gqe(s, dv, o)
    torch.cuda.synchronize()
    got = H.np32(o["out"][torch.from_numpy(rows).cuda()])
    keep = ~bad[rows]
    err, bound = H.out_error(got[keep], ref["out"][keep])
    print(f"[long case {name}] sampled out max err {err:.3e} bound {bound:.3e}; mismatched {int(bad.sum())}",
          flush=True)
    assert np.isfinite(got).all() and err <= bound
    gref = go.gqa_rows(dict(x=f["x"], Wq=f["Wq"], Wk=f["Wk"], Wv=f["Wv"], Wo=f["Wo_gqa"]),
                       s.G, s.Hq, s.d, s.B, s.T, rows)
    og = torch.empty_like(o["out"])
    H.run_gqa(s, dv, og)
    torch.cuda.synchronize()
    err, bound = H.out_error(H.np32(og[torch.from_numpy(rows).cuda()]), gref["out"])
    assert err <= bound, ("gqa", err, bound)
