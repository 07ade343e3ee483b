"""Plain fp64 CPU oracle for one decode step of the GQE layer.

TEST INFRASTRUCTURE ONLY, like gqe_oracle: only tests/ and bench.py's
cpu_baseline leg may import it; the HIP library never does.

One new token per sequence attends over that sequence's dense KV cache plus
itself. GQE keeps the K/V projections, and so the KV cache, of the underlying
GQA model unchanged: only the query side is sparse ("Grouped Query Experts"
explainer, technical summary, "Architecture and routing"; FrontiersMind GQE
article, part 4). The step is the layer of gqe_oracle applied to the new
token, with the causal attention reading the cached keys and values of the
earlier positions:

  routing, Q of the picked experts and the shared head  (as in gqe_forward)
  K_new = x Wk^T, V_new = x Wv^T                         (appended at pos[b])
  O[b,g,r] = softmax_j(q . K[b,g,j] / sqrt(d)) V[b,g,j], j = 0 .. pos[b]
  C = [hard slots | weighted slot | shared slot], out = C Wo^T

Reading where the pages are silent: they describe the cache only as dense and
unchanged; positions are per sequence (pos[b] cached keys precede the new
token), and nothing else (no positional encoding) enters the attention.
"""
from __future__ import annotations

import numpy as np

from . import gqe_oracle as go

__all__ = ["gqe_decode"]


def _attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """softmax(q . keys^T / sqrt(d)) vals for one query over all given keys."""
    s = keys @ q / np.sqrt(q.shape[0])
    s = s - s.max()
    p = np.exp(s)
    return (p / p.sum()) @ vals


def gqe_decode(inp: dict, k_cache: np.ndarray, v_cache: np.ndarray, pos, G: int, M: int, k: int, d: int,
               shared_kv_group: int = 0) -> dict:
    """inp: x [B, D] (the new tokens) and the layer's weights as in gqe_forward.
    k_cache, v_cache [B, G, L, d]: positions < pos[b] of sequence b are valid.
    Returns out [B, D], idx, w, the appended K_new / V_new [B, G, d] and C."""
    x = inp["x"]
    B = x.shape[0]
    logits, p, sel, w = go.route(x, inp["Wr"], inp.get("br"), G, M, k)
    Wq = inp["Wq"].reshape(G, M, d, -1)
    K_new = go.project(x, inp["Wk"]).reshape(B, G, d)
    V_new = go.project(x, inp["Wv"]).reshape(B, G, d)
    Q_sh = go.project(x, inp["Wq_sh"])
    O = np.zeros((B, G, k, d))
    O_sh = np.zeros((B, d))
    for b in range(B):
        n = int(pos[b])
        for g in range(G):
            keys = np.concatenate([k_cache[b, g, :n], K_new[b, g][None]])
            vals = np.concatenate([v_cache[b, g, :n], V_new[b, g][None]])
            for r in range(k):
                q = x[b] @ Wq[g, sel[b, g, r]].T
                O[b, g, r] = _attend(q, keys, vals)
            if g == shared_kv_group:
                O_sh[b] = _attend(Q_sh[b], keys, vals)
    C = go.assemble_slots(O, go.weighted_slot(O, w), O_sh)
    return dict(logits=logits, idx=sel, w=w, K_new=K_new, V_new=V_new, O=O, O_sh=O_sh, C=C,
                out=go.project(C, inp["Wo"]))
