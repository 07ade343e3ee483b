"""Pins for the fp64 decode-step oracle (CPU only).

* a decode step at position t with the cache holding the prefix's own keys
  and values equals row t of the prefill oracle (a causal layer decoded token
  by token computes what the whole-sequence pass does), with different
  positions per sequence;
* an empty cache (position 0): every head's output is the new token's value
  (a softmax over one key);
* a tiny random cache against pure-Python loops (math.exp);
* planted mistakes (new token not attended, an extra cached row attended,
  shared head on the wrong group) each fail a pin.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle.gqe_decode as gd
import oracle.gqe_oracle as go

from .test_oracle import rand_layer


def _prefix_caches(fwd, B, T, G, d):
    """Per-sequence K/V of every position from the prefill oracle, as [B, G, T, d]."""
    K = fwd["K"].reshape(B, T, G, d).transpose(0, 2, 1, 3)
    V = fwd["V"].reshape(B, T, G, d).transpose(0, 2, 1, 3)
    return K, V


def pin_decode_equals_prefill_rows():
    rng = np.random.default_rng(11)
    B, T, D, G, M, k, d, s0 = 3, 13, 24, 3, 3, 2, 8, 1
    inp = rand_layer(rng, B, T, D, G, M, k, d, bias=True)
    fwd = go.gqe_forward(inp, G, M, k, d, B, T, shared_kv_group=s0, q_block=4)
    Kc, Vc = _prefix_caches(fwd, B, T, G, d)
    for pos in ([0, 5, 12], [12, 12, 12], [7, 1, 3]):
        rows = [b * T + pos[b] for b in range(B)]
        step = dict(inp, x=inp["x"][rows])
        dec = gd.gqe_decode(step, Kc, Vc, pos, G, M, k, d, shared_kv_group=s0)
        np.testing.assert_array_equal(dec["idx"], fwd["idx"][rows])
        np.testing.assert_allclose(dec["w"], fwd["w"][rows], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dec["C"], fwd["C"][rows], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dec["out"], fwd["out"][rows], rtol=1e-10, atol=1e-12)
        # the appended K/V are the prefill's projections at pos[b]
        for b in range(B):
            np.testing.assert_allclose(dec["K_new"][b], Kc[b, :, pos[b]], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(dec["V_new"][b], Vc[b, :, pos[b]], rtol=1e-12, atol=1e-14)


def pin_empty_cache():
    rng = np.random.default_rng(12)
    B, D, G, M, k, d = 2, 16, 2, 2, 1, 4
    inp = rand_layer(rng, B, 1, D, G, M, k, d)
    garbage = rng.standard_normal((B, G, 5, d)) * 1e3          # never read at pos 0
    dec = gd.gqe_decode(inp, garbage, garbage, [0, 0], G, M, k, d)
    for b in range(B):
        for g in range(G):
            for r in range(k):
                np.testing.assert_allclose(dec["O"][b, g, r], dec["V_new"][b, g], rtol=1e-12)
        np.testing.assert_allclose(dec["O_sh"][b], dec["V_new"][b, 0], rtol=1e-12)


def pin_tiny_brute_force():
    rng = np.random.default_rng(13)
    B, D, G, M, k, d, L = 2, 8, 2, 3, 2, 4, 6
    inp = rand_layer(rng, B, 1, D, G, M, k, d, bias=True)
    Kc = rng.standard_normal((B, G, L, d))
    Vc = rng.standard_normal((B, G, L, d))
    pos = [4, 2]
    dec = gd.gqe_decode(inp, Kc, Vc, pos, G, M, k, d, shared_kv_group=1)
    x = inp["x"]
    for b in range(B):
        for g in range(G):
            kn = [sum(x[b][i] * inp["Wk"][g * d + c][i] for i in range(D)) for c in range(d)]
            vn = [sum(x[b][i] * inp["Wv"][g * d + c][i] for i in range(D)) for c in range(d)]
            keys = [list(Kc[b, g, j]) for j in range(pos[b])] + [kn]
            vals = [list(Vc[b, g, j]) for j in range(pos[b])] + [vn]
            heads = [("r", r) for r in range(k)] + ([("sh", 0)] if g == 1 else [])
            for kind, r in heads:
                if kind == "r":
                    m = int(dec["idx"][b, g, r])
                    wq = inp["Wq"][(g * M + m) * d:(g * M + m + 1) * d]
                else:
                    wq = inp["Wq_sh"]
                q = [sum(x[b][i] * wq[c][i] for i in range(D)) for c in range(d)]
                sc = [sum(q[c] * kk[c] for c in range(d)) / math.sqrt(d) for kk in keys]
                mx = max(sc)
                e = [math.exp(v - mx) for v in sc]
                o = [sum(e[j] * vals[j][c] for j in range(len(keys))) / sum(e) for c in range(d)]
                got = dec["O"][b, g, r] if kind == "r" else dec["O_sh"][b]
                np.testing.assert_allclose(got, o, rtol=1e-10, atol=1e-12)


PINS = [pin_decode_equals_prefill_rows, pin_empty_cache, pin_tiny_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------
def _attend_without_self(q, keys, vals):
    if len(keys) > 1:
        keys, vals = keys[:-1], vals[:-1]
    s = keys @ q / np.sqrt(q.shape[0])
    p = np.exp(s - s.max())
    return (p / p.sum()) @ vals


def _decode_one_row_too_many(inp, k_cache, v_cache, pos, G, M, k, d, shared_kv_group=0):
    return _orig_decode(inp, k_cache, v_cache, [int(p) + 1 for p in pos], G, M, k, d, shared_kv_group)


def _decode_shared_on_group0(inp, k_cache, v_cache, pos, G, M, k, d, shared_kv_group=0):
    return _orig_decode(inp, k_cache, v_cache, pos, G, M, k, d, 0)


_orig_decode = gd.gqe_decode

MUTANTS = {
    "new_token_not_attended": ("_attend", _attend_without_self),
    "cache_row_past_pos_attended": ("gqe_decode", _decode_one_row_too_many),
    "shared_head_on_group_0": ("gqe_decode", _decode_shared_on_group0),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(gd, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
