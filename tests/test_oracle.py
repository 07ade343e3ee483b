"""Pins for the fp64 oracle (CPU only).

Every oracle function is checked against something other than itself:
brute force on tiny inputs (pure-Python loops), closed forms, library routines
(scipy's softmax, torch's scaled_dot_product_attention in fp64 on the CPU),
invariants the pages state, and reductions to GQA / MQA / MHA. The planted-
mistake tests at the end patch plausible bugs into the oracle and check that a
pin fails for each.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle.gqe_oracle as go

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_layer(rng, B, T, D, G, M, k, d, bias=False):
    s = 1.0 / math.sqrt(D)
    inp = dict(
        x=rng.standard_normal((B * T, D)),
        Wr=rng.standard_normal((G * M, D)) * s,
        br=(rng.standard_normal(G * M) * math.sqrt(0.5)) if bias else None,
        Wq=rng.standard_normal((G * M * d, D)) * s,
        Wk=rng.standard_normal((G * d, D)) * s,
        Wv=rng.standard_normal((G * d, D)) * s,
        Wq_sh=rng.standard_normal((d, D)) * s,
        Wo=rng.standard_normal((D, (G * k + 2) * d)) * s,
        Wo_gqa=rng.standard_normal((D, G * M * d)) * s,
    )
    return inp


def sdpa_causal(q, k, v):
    """torch's attention routine in fp64 on the CPU. q,k,v [B,H,T,d]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True).numpy()


# ----------------------------------------------------------------------------
# Pins (each raises AssertionError on failure; the planted-mistake tests reuse them)
# ----------------------------------------------------------------------------
def pin_topk_brute_force():
    """Top-k against enumeration of every ordered k-tuple of distinct experts:
    the chosen tuple is the lexicographic maximum of ((logit, -m) per position)."""
    rng = np.random.default_rng(1)
    for M in (1, 2, 3, 4):
        for k in range(1, M + 1):
            G, N = 3, 40
            # quantised logits give many exact ties
            logits = rng.integers(-2, 3, size=(N, G * M)).astype(np.float64) * 0.5
            sel = go.select_topk(logits, G, M, k)
            for n in range(N):
                for g in range(G):
                    z = logits[n, g * M:(g + 1) * M]
                    best = max(itertools.permutations(range(M), k),
                               key=lambda tup: tuple((z[m], -m) for m in tup))
                    assert tuple(sel[n, g]) == best, (M, k, n, g, z, sel[n, g], best)


def pin_group_softmax_scipy():
    rng = np.random.default_rng(2)
    G, M = 4, 3
    logits = rng.standard_normal((17, G * M)) * 3
    p = go.group_softmax(logits, G, M)
    ref = scipy.special.softmax(logits.reshape(17, G, M), axis=2)
    assert np.allclose(p, ref, rtol=0, atol=1e-15)


def pin_route_tiny_brute_force():
    """Weights from scratch with math.exp loops: w = p_sel / sum of all picks."""
    rng = np.random.default_rng(3)
    G, M, k, D, N = 3, 4, 2, 8, 6
    x = rng.standard_normal((N, D))
    Wr = rng.standard_normal((G * M, D))
    br = rng.standard_normal(G * M)
    logits, p, sel, w = go.route(x, Wr, br, G, M, k)
    for n in range(N):
        picks = []
        for g in range(G):
            z = [sum(x[n, i] * Wr[g * M + m, i] for i in range(D)) + br[g * M + m] for m in range(M)]
            zmax = max(z)
            e = [math.exp(v - zmax) for v in z]
            tot = sum(e)
            order = sorted(range(M), key=lambda m: (-z[m], m))[:k]
            assert list(sel[n, g]) == order
            picks.append([e[m] / tot for m in order])
        denom = sum(sum(r) for r in picks)
        for g in range(G):
            for r in range(k):
                assert abs(w[n, g, r] - picks[g][r] / denom) < 1e-14


def pin_route_uniform_router():
    """Wr = 0: every expert ties, so sel = (0..k-1) and w = 1/(G*k)."""
    rng = np.random.default_rng(4)
    for (G, M, k) in [(2, 2, 1), (8, 2, 1), (8, 4, 2), (3, 5, 5)]:
        x = rng.standard_normal((9, 16))
        _, _, sel, w = go.route(x, np.zeros((G * M, 16)), None, G, M, k)
        assert (sel == np.arange(k)[None, None, :]).all()
        assert np.allclose(w, 1.0 / (G * k), rtol=0, atol=1e-15)


def pin_route_single_expert():
    """M = 1: the only expert is always chosen, each group's p is 1, w = 1/G."""
    rng = np.random.default_rng(5)
    G = 5
    x = rng.standard_normal((7, 16))
    _, p, sel, w = go.route(x, rng.standard_normal((G, 16)), None, G, 1, 1)
    assert (sel == 0).all() and np.allclose(p, 1.0) and np.allclose(w, 1.0 / G, atol=1e-15)


def pin_route_invariants():
    rng = np.random.default_rng(6)
    G, M, k = 8, 4, 2
    x = rng.standard_normal((300, 64))
    _, p, sel, w = go.route(x, rng.standard_normal((G * M, 64)) / 8, rng.standard_normal(G * M), G, M, k)
    assert np.allclose(w.sum(axis=(1, 2)), 1.0, atol=1e-14)
    assert (w > 0).all()
    for r1 in range(k):
        for r2 in range(r1 + 1, k):
            assert (sel[:, :, r1] != sel[:, :, r2]).all()
    assert np.allclose(p.sum(axis=2), 1.0, atol=1e-14)


def pin_attention_brute_force():
    """Full T x T masked softmax with pure-Python loops, T <= 16."""
    rng = np.random.default_rng(7)
    for (B, T, d) in [(1, 1, 4), (2, 5, 3), (1, 16, 8)]:
        q, k, v = (rng.standard_normal((B, T, d)) for _ in range(3))
        out = go.causal_attention(q, k, v, q_block=3)
        for b in range(B):
            for t in range(T):
                sc = [sum(q[b, t, i] * k[b, s, i] for i in range(d)) / math.sqrt(d) for s in range(T)]
                allowed = [sc[s] for s in range(t + 1)]
                mx = max(allowed)
                e = [math.exp(a - mx) for a in allowed]
                z = sum(e)
                for i in range(d):
                    ref = sum(e[s] * v[b, s, i] for s in range(t + 1)) / z
                    assert abs(out[b, t, i] - ref) < 1e-12, (b, t, i)


def pin_attention_sdpa():
    """Against torch's fp64 scaled_dot_product_attention (causal), ragged q blocks."""
    rng = np.random.default_rng(8)
    B, T, d = 2, 100, 16
    q, k, v = (rng.standard_normal((B, T, d)) for _ in range(3))
    ref = sdpa_causal(q[:, None], k[:, None], v[:, None])[:, 0]
    for qb in (7, 64, 512):
        assert np.allclose(go.causal_attention(q, k, v, q_block=qb), ref, rtol=0, atol=1e-12)


def pin_attention_closed_forms():
    rng = np.random.default_rng(9)
    B, T, d = 2, 33, 8
    v = rng.standard_normal((B, T, d))
    # T = 1: the only key is the query itself, O = V[0]
    one = go.causal_attention(rng.standard_normal((B, 1, d)), rng.standard_normal((B, 1, d)), v[:, :1])
    assert np.allclose(one, v[:, :1], atol=1e-15)
    # q = 0: uniform weights over the prefix, O[t] = mean(V[0..t])
    zero = go.causal_attention(np.zeros((B, T, d)), rng.standard_normal((B, T, d)), v, q_block=5)
    prefix = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None]
    assert np.allclose(zero, prefix, atol=1e-13)


def _layer(inp, B, T, G, M, k, d, s0=0):
    return go.gqe_forward(inp, G, M, k, d, B, T, shared_kv_group=s0, q_block=16)


def pin_layer_causality():
    rng = np.random.default_rng(10)
    B, T, D, G, M, k, d = 1, 40, 32, 2, 3, 2, 8
    inp = rand_layer(rng, B, T, D, G, M, k, d)
    a = _layer(inp, B, T, G, M, k, d)
    cut = 17
    inp2 = dict(inp)
    inp2["x"] = inp["x"].copy()
    inp2["x"][cut:] += rng.standard_normal(inp["x"][cut:].shape)
    b = _layer(inp2, B, T, G, M, k, d)
    assert np.allclose(a["out"][:cut], b["out"][:cut], rtol=0, atol=1e-13)
    assert not np.allclose(a["out"][cut:], b["out"][cut:])


def pin_layer_batch_independence():
    rng = np.random.default_rng(11)
    B, T, D, G, M, k, d = 3, 20, 32, 2, 2, 1, 8
    inp = rand_layer(rng, B, T, D, G, M, k, d)
    full = _layer(inp, B, T, G, M, k, d)
    for b in range(B):
        one = dict(inp)
        one["x"] = inp["x"][b * T:(b + 1) * T]
        single = _layer(one, 1, T, G, M, k, d)
        assert np.allclose(full["out"][b * T:(b + 1) * T], single["out"], rtol=0, atol=1e-13)


def pin_reduction_to_gqa():
    """k = M with a uniform router and Wo = [Wo_gqa | 0 | 0] is dense GQA."""
    rng = np.random.default_rng(12)
    for (B, T, D, G, M, d) in [(2, 24, 32, 2, 2, 8), (1, 30, 48, 3, 4, 16), (1, 9, 16, 1, 3, 4)]:
        k = M
        inp = rand_layer(rng, B, T, D, G, M, k, d)
        inp["Wr"] = np.zeros_like(inp["Wr"])
        inp["Wo"] = np.concatenate([inp["Wo_gqa"], np.zeros((D, 2 * d))], axis=1)
        e = _layer(inp, B, T, G, M, k, d)
        a = go.gqa_forward(dict(x=inp["x"], Wq=inp["Wq"], Wk=inp["Wk"], Wv=inp["Wv"], Wo=inp["Wo_gqa"]),
                           G, G * M, d, B, T, q_block=16)
        assert np.allclose(e["out"], a["out"], rtol=0, atol=1e-12)
        assert np.allclose(e["C"][:, :G * M * d], a["C"], rtol=0, atol=1e-13)


def pin_gqa_vs_sdpa_endpoints():
    """GQA against torch SDPA with K/V repeated per group, including the MQA
    (one KV group) and MHA (one head per group) endpoints."""
    rng = np.random.default_rng(13)
    B, T, D, d = 2, 21, 24, 8
    for (G, Hq) in [(1, 4), (4, 4), (2, 6)]:
        x = rng.standard_normal((B * T, D))
        Wq = rng.standard_normal((Hq * d, D)) / 5
        Wk = rng.standard_normal((G * d, D)) / 5
        Wv = rng.standard_normal((G * d, D)) / 5
        Wo = rng.standard_normal((D, Hq * d)) / 5
        r = go.gqa_forward(dict(x=x, Wq=Wq, Wk=Wk, Wv=Wv, Wo=Wo), G, Hq, d, B, T, q_block=8)
        q = (x @ Wq.T).reshape(B, T, Hq, d).transpose(0, 2, 1, 3)
        k = (x @ Wk.T).reshape(B, T, G, d).transpose(0, 2, 1, 3)
        v = (x @ Wv.T).reshape(B, T, G, d).transpose(0, 2, 1, 3)
        k = np.repeat(k, Hq // G, axis=1)
        v = np.repeat(v, Hq // G, axis=1)
        o = sdpa_causal(np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v))
        C = o.transpose(0, 2, 1, 3).reshape(B * T, Hq * d)
        assert np.allclose(r["C"], C, rtol=0, atol=1e-12)
        assert np.allclose(r["out"], C @ Wo.T, rtol=0, atol=1e-12)


def pin_slots_closed_form():
    """Wq = Wq_sh = 0: every head attends uniformly over its prefix, so hard slot
    (g,r) = prefix mean pm_g of V_g whatever the routing, the weighted slot =
    sum_g (sum_r w[n,g,r]) pm_g with a live (biased, random) router, and the
    shared slot = pm of the shared head's group."""
    rng = np.random.default_rng(14)
    B, T, D, G, M, k, d = 1, 12, 16, 3, 3, 2, 4
    inp = rand_layer(rng, B, T, D, G, M, k, d, bias=True)
    inp["Wq"] = np.zeros_like(inp["Wq"])
    inp["Wq_sh"] = np.zeros_like(inp["Wq_sh"])
    s0 = 2
    r = _layer(inp, B, T, G, M, k, d, s0=s0)
    w = r["w"]
    assert w.std() > 1e-3                      # the weights really vary
    V = (inp["x"] @ inp["Wv"].T).reshape(T, G, d)
    pm = np.cumsum(V, axis=0) / np.arange(1, T + 1)[:, None, None]     # [T,G,d]
    C = r["C"]
    for g in range(G):
        for rr in range(k):
            c0 = (g * k + rr) * d
            assert np.allclose(C[:, c0:c0 + d], pm[:, g], atol=1e-13)
    expect = np.einsum("tg,tgd->td", w.sum(axis=2), pm)
    assert np.allclose(C[:, G * k * d:(G * k + 1) * d], expect, atol=1e-13)
    assert np.allclose(C[:, (G * k + 1) * d:], pm[:, s0], atol=1e-13)


def pin_hard_slot_rank_order():
    """k = 2 of M = 4 with constant offsets br = (0, 2, 0, 5) and Wr = 0: every
    token picks expert 3 then expert 1, so hard slot r=0 is expert 3's head and
    r=1 expert 1's, i.e. dense GQA heads g*M+3 and g*M+1."""
    rng = np.random.default_rng(15)
    B, T, D, G, M, k, d = 1, 10, 16, 2, 4, 2, 4
    inp = rand_layer(rng, B, T, D, G, M, k, d)
    inp["Wr"] = np.zeros_like(inp["Wr"])
    inp["br"] = np.tile(np.array([0.0, 2.0, 0.0, 5.0]), G)
    r = _layer(inp, B, T, G, M, k, d)
    assert (r["idx"] == np.array([3, 1])[None, None, :]).all()
    a = go.gqa_forward(dict(x=inp["x"], Wq=inp["Wq"], Wk=inp["Wk"], Wv=inp["Wv"], Wo=inp["Wo_gqa"]),
                       G, G * M, d, B, T)
    Cg = a["C"].reshape(B * T, G * M, d)
    for g in range(G):
        assert np.allclose(r["C"][:, (g * k + 0) * d:(g * k + 1) * d], Cg[:, g * M + 3], atol=1e-13)
        assert np.allclose(r["C"][:, (g * k + 1) * d:(g * k + 2) * d], Cg[:, g * M + 1], atol=1e-13)


def pin_expert_permutation_invariance():
    """Relabelling the experts of each group (Wq blocks together with router rows)
    changes idx but not the layer's output."""
    rng = np.random.default_rng(16)
    B, T, D, G, M, k, d = 1, 15, 16, 2, 3, 2, 4
    inp = rand_layer(rng, B, T, D, G, M, k, d, bias=True)
    base = _layer(inp, B, T, G, M, k, d)
    perm = np.array([2, 0, 1])
    inp2 = dict(inp)
    inp2["Wq"] = inp["Wq"].reshape(G, M, d, D)[:, perm].reshape(G * M * d, D)
    inp2["Wr"] = inp["Wr"].reshape(G, M, D)[:, perm].reshape(G * M, D)
    inp2["br"] = inp["br"].reshape(G, M)[:, perm].reshape(G * M)
    other = _layer(inp2, B, T, G, M, k, d)
    assert np.allclose(base["out"], other["out"], rtol=0, atol=1e-13)
    assert (perm[other["idx"]] == base["idx"]).all()


def pin_linearity_in_Wo():
    rng = np.random.default_rng(17)
    B, T, D, G, M, k, d = 1, 11, 16, 2, 2, 1, 4
    inp = rand_layer(rng, B, T, D, G, M, k, d)
    a = _layer(inp, B, T, G, M, k, d)["out"]
    inp2 = dict(inp)
    W2 = rng.standard_normal(inp["Wo"].shape)
    inp2["Wo"] = 2.0 * inp["Wo"] - 3.0 * W2
    b = _layer(inp2, B, T, G, M, k, d)["out"]
    inp3 = dict(inp)
    inp3["Wo"] = W2
    c = _layer(inp3, B, T, G, M, k, d)["out"]
    assert np.allclose(b, 2.0 * a - 3.0 * c, atol=1e-12)


def pin_active_heads_pages():
    """The pages' main setting activates 8 routed + 1 shared = 9 of 16 query heads."""
    with open(os.path.join(GOLDEN, "pages_structural.json")) as f:
        gold = json.load(f)
    G, M, k = gold["kv_groups"], gold["experts_per_group"], gold["k"]
    assert G * M == gold["query_heads"]
    rng = np.random.default_rng(18)
    x = rng.standard_normal((64, 32))
    _, _, sel, _ = go.route(x, rng.standard_normal((G * M, 32)), None, G, M, k)
    act = go.active_heads(sel)
    assert (act == gold["active_query_heads"]).all()
    frac = act[0] / gold["query_heads"]
    tol = gold["rounding_tolerance"]
    assert abs(frac - gold["active_fraction_approx"]) <= tol
    assert abs((1 - frac) - gold["saving_fraction_approx"]) <= tol


def pin_rows_mode():
    """The streamed sampled-row oracle against the full oracle (ragged chunks)."""
    rng = np.random.default_rng(19)
    B, T, D, G, M, k, d = 2, 96, 32, 2, 3, 2, 8
    inp = rand_layer(rng, B, T, D, G, M, k, d, bias=True)
    full = _layer(inp, B, T, G, M, k, d, s0=1)
    rows = np.array([0, 1, 50, 95, 96, 130, 191])
    part = go.gqe_rows(inp, G, M, k, d, B, T, rows, shared_kv_group=1, kv_chunk=23)
    assert np.allclose(part["C"], full["C"][rows], rtol=0, atol=1e-12)
    assert np.allclose(part["out"], full["out"][rows], rtol=0, atol=1e-12)
    assert (part["idx"] == full["idx"]).all()
    ga = dict(x=inp["x"], Wq=inp["Wq"], Wk=inp["Wk"], Wv=inp["Wv"], Wo=inp["Wo_gqa"])
    gf = go.gqa_forward(ga, G, G * M, d, B, T)
    gp = go.gqa_rows(ga, G, G * M, d, B, T, rows, kv_chunk=31)
    assert np.allclose(gp["out"], gf["out"][rows], rtol=0, atol=1e-12)


def pin_variants_against_full():
    """The ablations' merges against the full layer's slots: hard concat and
    no-shared are the full merge with one slot dropped; the weighted concat's
    scaled hard slots, summed and divided by the sum of the pick probabilities,
    give the full layer's renormalised weighted slot; the no-shared variant
    never reads Wq_sh."""
    rng = np.random.default_rng(23)
    B, T, D, G, M, k, d = 2, 33, 32, 3, 3, 2, 8
    inp = rand_layer(rng, B, T, D, G, M, k, d, bias=True)
    GK, N = G * k, B * T
    full = _layer(inp, B, T, G, M, k, d)
    for variant in ("weighted_concat", "hard_concat", "no_shared"):
        Wo = inp["Wo"][:, :go.variant_slots(G, k, variant) * d]
        v = go.gqe_forward(dict(inp, Wo=Wo), G, M, k, d, B, T, q_block=16, variant=variant)
        assert v["C"].shape == (N, (GK + 1) * d)
        assert np.allclose(v["out"], v["C"] @ Wo.T, rtol=0, atol=1e-12)
        hard = full["C"][:, :GK * d]
        if variant == "hard_concat":
            assert np.array_equal(v["C"], np.concatenate([hard, full["C"][:, (GK + 1) * d:]], axis=1))
        if variant == "no_shared":
            assert np.array_equal(v["C"], full["C"][:, :(GK + 1) * d])
            nosh = go.gqe_forward(dict(inp, Wo=Wo, Wq_sh=np.full_like(inp["Wq_sh"], np.nan)), G, M, k, d, B, T,
                                  q_block=16, variant=variant)
            assert np.array_equal(nosh["out"], v["out"])
        if variant == "weighted_concat":
            pp = v["w"]                                           # per-group probabilities of the picks
            assert np.allclose(pp, np.take_along_axis(full["p"], full["idx"], axis=2), rtol=0, atol=0)
            scaled = v["C"][:, :GK * d].reshape(N, GK, d)
            wsum = scaled.sum(axis=1) / pp.reshape(N, GK).sum(axis=1, keepdims=True)
            assert np.allclose(wsum, full["C"][:, GK * d:(GK + 1) * d], rtol=1e-12, atol=1e-14)
            assert np.array_equal(v["C"][:, GK * d:], full["C"][:, (GK + 1) * d:])
            # each slot is its hard slot times one probability in (0, 1]
            ratio = scaled / hard.reshape(N, GK, d)
            assert np.allclose(ratio, pp.reshape(N, GK, 1), rtol=1e-12)
            assert (pp > 0).all() and (pp <= 1).all()


def pin_threaded_heads_identical():
    """workers > 1 (heads on a thread pool, used for the large layers) returns
    bit-identical arrays to the serial loop, for GQE (k = 2, shared head on
    group 1, ragged query blocks) and for dense GQA."""
    rng = np.random.default_rng(29)
    B, T, D, G, M, k, d = 2, 45, 32, 3, 3, 2, 8
    inp = rand_layer(rng, B, T, D, G, M, k, d, bias=True)
    a = go.gqe_forward(inp, G, M, k, d, B, T, shared_kv_group=1, q_block=16)
    b = go.gqe_forward(inp, G, M, k, d, B, T, shared_kv_group=1, q_block=16, workers=4)
    for key in ("C", "out", "Qr", "w"):
        assert np.array_equal(a[key], b[key]), key
    ga = dict(x=inp["x"], Wq=inp["Wq"], Wk=inp["Wk"], Wv=inp["Wv"], Wo=inp["Wo_gqa"])
    assert np.array_equal(go.gqa_forward(ga, G, G * M, d, B, T, q_block=16)["out"],
                          go.gqa_forward(ga, G, G * M, d, B, T, q_block=16, workers=5)["out"])


PINS = [
    pin_threaded_heads_identical,
    pin_topk_brute_force, pin_group_softmax_scipy, pin_route_tiny_brute_force,
    pin_route_uniform_router, pin_route_single_expert, pin_route_invariants,
    pin_attention_brute_force, pin_attention_sdpa, pin_attention_closed_forms,
    pin_layer_causality, pin_layer_batch_independence, pin_reduction_to_gqa,
    pin_gqa_vs_sdpa_endpoints, pin_slots_closed_form, pin_hard_slot_rank_order,
    pin_expert_permutation_invariance, pin_linearity_in_Wo, pin_active_heads_pages,
    pin_rows_mode, pin_variants_against_full,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# Planted mistakes: each variant breaks the oracle in one plausible way; at
# least one pin must fail for each.
# ----------------------------------------------------------------------------
def _topk_ties_high(logits, G, M, k):
    z = logits.reshape(-1, G, M)
    m_index = np.broadcast_to(np.arange(M), z.shape)
    return np.lexsort((-m_index, -z), axis=-1)[..., :k]


def _renorm_per_group(p, sel):
    picked = np.take_along_axis(p, sel, axis=2)
    return picked / picked.sum(axis=2, keepdims=True)


def _softmax_global(logits, G, M):
    z = logits - logits.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).reshape(-1, G, M)


def _attention_no_diagonal(q, k, v, q_block=512):
    B, T, d = q.shape
    out = np.empty_like(q)
    for b in range(B):
        s = q[b] @ k[b].T / np.sqrt(d)
        allowed = np.arange(T)[None, :] < np.arange(T)[:, None]
        allowed[0, 0] = True
        s = np.where(allowed, s, -np.inf)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        out[b] = e / e.sum(axis=1, keepdims=True) @ v[b]
    return out


def _attention_unscaled(q, k, v, q_block=512):
    return go.__dict__["_orig_attention"](q * np.sqrt(q.shape[-1]), k, v, q_block)


def _attention_noncausal(q, k, v, q_block=512):
    B, T, d = q.shape
    out = np.empty_like(q)
    for b in range(B):
        s = q[b] @ k[b].T / np.sqrt(d)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        out[b] = e / e.sum(axis=1, keepdims=True) @ v[b]
    return out


def _assemble_swapped(O, wsum, O_sh):
    N = O.shape[0]
    return np.concatenate([O.reshape(N, -1), O_sh, wsum], axis=1)


def _assemble_rank_reversed(O, wsum, O_sh):
    N = O.shape[0]
    return np.concatenate([O[:, :, ::-1].reshape(N, -1), wsum, O_sh], axis=1)


def _weighted_slot_unweighted(O, w):
    return O.mean(axis=(1, 2))


_orig_assemble_variant = go.assemble_variant


def _assemble_variant_renormalised(O, w, p_pick, O_sh, variant):
    """Weighted concatenation that scales by the renormalised w instead of p."""
    return _orig_assemble_variant(O, w, w if variant == "weighted_concat" else p_pick, O_sh, variant)


def _pick_probs_rank_shifted(p, sel):
    return np.take_along_axis(p, np.roll(sel, 1, axis=2), axis=2)


MUTANTS = {
    "topk_ties_to_high_index": ("select_topk", _topk_ties_high),
    "renormalise_per_group": ("renormalize", _renorm_per_group),
    "softmax_over_all_groups": ("group_softmax", _softmax_global),
    "attention_excludes_diagonal": ("causal_attention", _attention_no_diagonal),
    "attention_without_scale": ("causal_attention", _attention_unscaled),
    "attention_not_causal": ("causal_attention", _attention_noncausal),
    "weighted_and_shared_swapped": ("assemble_slots", _assemble_swapped),
    "hard_slots_in_reverse_rank": ("assemble_slots", _assemble_rank_reversed),
    "weighted_slot_ignores_w": ("weighted_slot", _weighted_slot_unweighted),
    "weighted_concat_uses_renormalised_w": ("assemble_variant", _assemble_variant_renormalised),
    "pick_probabilities_of_wrong_rank": ("pick_probs", _pick_probs_rank_shifted),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(go.__dict__, "_orig_attention", go.causal_attention)
    monkeypatch.setattr(go, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
