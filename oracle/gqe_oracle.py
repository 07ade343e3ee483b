"""Plain fp64 CPU oracle for the Grouped Query Experts (GQE) attention forward pass.

TEST INFRASTRUCTURE ONLY. This module exists to check the HIP library. Only
tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import or
call it. The product path (the gfx950 kernels, the C ABI and its Python binding)
never imports it and has no CPU fallback.

It is written from the pages' description of the layer, step by step, in numpy
float64 with no blocking or fusion beyond what each step states. Sources
(cited by title and section):

  [GQE-x]  "Grouped Query Experts: Mixture-of-Experts on GQA Self-Attention",
           gist.science explainer of arXiv 2606.20945 (Chinese, Italian and
           Spanish editions), technical summary: "Architecture and routing",
           "Training and loss", "Experimental results".
  [GQE-n]  FrontiersMind GQE news article (animattoys.com), part 4 (the forward
           workflow: groups, router, output integration, shared head), part 5
           (router learning), part 6 (experiments).
  [GQA-w]  aiboss88.com wiki "What is Grouped-Query Attention", section
           "Mechanism" (GQA generalizes MQA; MHA and MQA are its endpoints).

Readings where the pages are silent:
  * the router is linear in the token's features, x @ Wr.T, plus an optional
    per-expert offset br; softmax is taken per group over its M experts;
  * top-k orders the experts by descending logit, ties to the lower index;
  * the renormalisation runs over all G*k picks of the token, so the weights
    of one token sum to 1 and feed one extra output slot;
  * attention is causal with the diagonal included, scale 1/sqrt(d), no
    positional encoding; each batch element is an independent sequence;
  * the shared head has its own query projection and reads the K/V of group
    shared_kv_group (0 by default);
  * the merged output is [hard slots g-major, rank-minor | weighted | shared],
    then multiplied by Wo.T;
  * the ablations' weighted concatenation scales each hard slot by its pick's
    per-group softmax probability (not renormalised).

All pins live in tests/test_oracle.py; every function here is pinned there.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "router_logits", "group_softmax", "select_topk", "renormalize", "route",
    "project", "causal_attention", "weighted_slot", "assemble_slots",
    "VARIANTS", "variant_slots", "pick_probs", "assemble_variant",
    "gqe_forward", "gqa_forward", "gqe_rows", "gqa_rows", "active_heads",
]


# ----------------------------------------------------------------------------
# Step 1: the router. [GQE-x] "Architecture and routing" (conditional
# activation: per token, a sparse subset of k experts from every group);
# [GQE-n] part 4 (a lightweight scorer looks at the current token's features
# and scores every expert of every group, then keeps the best k).
# ----------------------------------------------------------------------------
def router_logits(x: np.ndarray, Wr: np.ndarray, br: np.ndarray | None = None) -> np.ndarray:
    """l[n, g*M+m] = x[n] . Wr[g*M+m] (+ br[g*M+m]).  x [N,D], Wr [G*M,D] -> [N,G*M]."""
    logits = x @ Wr.T
    if br is not None:
        logits = logits + br[None, :]
    return logits


def group_softmax(logits: np.ndarray, G: int, M: int) -> np.ndarray:
    """Router probabilities: softmax over the M experts of each group. -> [N,G,M]."""
    z = logits.reshape(-1, G, M)
    z = z - z.max(axis=2, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=2, keepdims=True)


def select_topk(logits: np.ndarray, G: int, M: int, k: int) -> np.ndarray:
    """The k best experts of each group, best first, ties to the lower index.

    [GQE-n] part 4 ranks the scores from high to low and activates the top k.
    Returns sel [N,G,k] (expert index m inside the group).
    """
    z = logits.reshape(-1, G, M)
    m_index = np.broadcast_to(np.arange(M), z.shape)
    # np.lexsort: the last key is the primary one -> descending logit, then ascending m.
    order = np.lexsort((m_index, -z), axis=-1)
    return order[..., :k].astype(np.int64)


def renormalize(p: np.ndarray, sel: np.ndarray) -> np.ndarray:
    """Weights of the selected experts, renormalised over all G*k picks of a token.

    [GQE-x] "Architecture and routing" (renormalised weighted sum with the
    router probabilities); [GQE-n] part 4 (one extra output: a weighted average
    of all selected experts). Returns w [N,G,k] with sum over (g, r) equal to 1.
    """
    picked = np.take_along_axis(p, sel, axis=2)             # [N,G,k]
    total = picked.sum(axis=(1, 2), keepdims=True)           # [N,1,1]
    return picked / total


def route(x, Wr, br, G, M, k):
    """Steps 1-4 of the routing: logits, per-group softmax, top-k, renormalisation."""
    logits = router_logits(x, Wr, br)
    p = group_softmax(logits, G, M)
    sel = select_topk(logits, G, M, k)
    w = renormalize(p, sel)
    return logits, p, sel, w


# ----------------------------------------------------------------------------
# Step 2: projections. [GQE-x] "Architecture and routing" (dense KV path: K/V
# projections stay dense; only the selected experts compute Q); [GQE-n] part 4
# (each expert owns its query projection matrix; experts of one group read the
# same K/V).
# ----------------------------------------------------------------------------
def project(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """y = x @ W.T for an [out, in] weight."""
    return x @ W.T


# ----------------------------------------------------------------------------
# Step 3: causal attention of one head over one group's K/V.
# [GQE-n] part 4 (every selected expert runs its own attention).
# ----------------------------------------------------------------------------
def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_block: int = 512) -> np.ndarray:
    """O[b,t] = sum_{s<=t} softmax_s(q[b,t].k[b,s] / sqrt(d)) v[b,s].

    q, k, v: [B,T,d]. The softmax row of query t runs over keys 0..t of its
    own sequence. Query blocks only bound memory; each row's softmax is taken
    over the whole row at once.
    """
    B, T, d = q.shape
    scale = 1.0 / np.sqrt(d)
    out = np.empty_like(q)
    for b in range(B):
        for t0 in range(0, T, q_block):
            t1 = min(T, t0 + q_block)
            s = (q[b, t0:t1] @ k[b, :t1].T) * scale
            allowed = np.arange(t1)[None, :] <= np.arange(t0, t1)[:, None]
            s = np.where(allowed, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            out[b, t0:t1] = (e / e.sum(axis=1, keepdims=True)) @ v[b, :t1]
    return out


# ----------------------------------------------------------------------------
# Steps 4-5: output construction and the output projection.
# [GQE-x] "Architecture and routing" (hard concatenation of the k outputs per
# group; renormalised weighted sum; always-on shared head); [GQE-n] part 4
# (the three parts are merged, then projected).
# ----------------------------------------------------------------------------
def weighted_slot(O: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Wsum[n] = sum_{g,r} w[n,g,r] O[n,g,r].  O [N,G,k,d], w [N,G,k] -> [N,d]."""
    return np.einsum("ngr,ngrd->nd", w, O)


def assemble_slots(O: np.ndarray, wsum: np.ndarray, O_sh: np.ndarray) -> np.ndarray:
    """C[n] = [O[n,0,0..k-1], ..., O[n,G-1,0..k-1], Wsum[n], O_sh[n]]  -> [N,(G*k+2)*d]."""
    N = O.shape[0]
    return np.concatenate([O.reshape(N, -1), wsum, O_sh], axis=1)


# ----------------------------------------------------------------------------
# The pages' ablations of the merge. [GQE-n] part 6 compares the full layer
# with a weighted concatenation that has no renormalised weighted-sum slot
# (the router's scores weight the expert outputs directly) and with a pure hard
# concatenation (no weighting at all); [GQE-x] "Experimental results" reports
# removing the renormalised slot or the shared head. Readings: "the router's
# scores" are each pick's per-group softmax probability, not renormalised;
# every variant keeps the other parts of the merge and the slot order.
# ----------------------------------------------------------------------------
VARIANTS = ("full", "weighted_concat", "hard_concat", "no_shared")


def variant_slots(G: int, k: int, variant: str = "full") -> int:
    """d-wide slots of the merged output: G*k hard slots plus the weighted and
    shared slots that the variant keeps."""
    return G * k + (2 if variant == "full" else 1)


def pick_probs(p: np.ndarray, sel: np.ndarray) -> np.ndarray:
    """p_pick[n,g,r] = p[n, g, sel[n,g,r]]: the router probability of each pick."""
    return np.take_along_axis(p, sel, axis=2)


def assemble_variant(O: np.ndarray, w: np.ndarray, p_pick: np.ndarray, O_sh, variant: str) -> np.ndarray:
    """Merged slots of each variant (O [N,G,k,d], w and p_pick [N,G,k], O_sh [N,d]):
      full             [O | sum w O | O_sh]
      weighted_concat  [p_pick * O | O_sh]
      hard_concat      [O | O_sh]
      no_shared        [O | sum w O]"""
    N = O.shape[0]
    if variant == "full":
        return assemble_slots(O, weighted_slot(O, w), O_sh)
    if variant == "weighted_concat":
        return np.concatenate([(O * p_pick[..., None]).reshape(N, -1), O_sh], axis=1)
    if variant == "hard_concat":
        return np.concatenate([O.reshape(N, -1), O_sh], axis=1)
    if variant == "no_shared":
        return np.concatenate([O.reshape(N, -1), weighted_slot(O, w)], axis=1)
    raise ValueError(f"unknown variant {variant!r}")


def _routed_queries(x: np.ndarray, Wq: np.ndarray, sel: np.ndarray) -> np.ndarray:
    """Qr[n,g,r] = x[n] . Wq[g, sel[n,g,r]].T, computed expert by expert over the
    tokens that picked it (no query is formed for an expert a token skipped).
    Wq [G,M,d,D], sel [N,G,k] -> [N,G,k,d]."""
    G, M, d, _ = Wq.shape
    N, _, k = sel.shape
    Qr = np.zeros((N, G, k, d))
    for g in range(G):
        for r in range(k):
            for m in range(M):
                pick = sel[:, g, r] == m
                if pick.any():
                    Qr[pick, g, r] = x[pick] @ Wq[g, m].T
    return Qr


def _map_heads(fn, jobs, workers: int):
    """[fn(*job) for job in jobs], on a pool of `workers` threads when workers > 1.

    The heads are independent computations and each one runs the same numpy
    calls either way, so the results are bit-identical to the serial loop; the
    threads only let several heads' large array operations (which release the
    interpreter lock) run at once on the big layers."""
    if workers <= 1 or len(jobs) <= 1:
        return [fn(*j) for j in jobs]
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(lambda j: fn(*j), jobs))


def gqe_forward(inp: dict, G: int, M: int, k: int, d: int, B: int, T: int,
                shared_kv_group: int = 0, q_block: int = 512, variant: str = "full",
                workers: int = 1) -> dict:
    """The whole GQE layer in fp64. inp holds float64 arrays x, Wr, br (or None),
    Wq [G*M*d,D], Wk [G*d,D], Wv [G*d,D], Wq_sh [d,D], Wo [D, variant_slots*d].

    Expert e = g*M + m owns rows e*d .. e*d+d-1 of Wq. The returned w is the
    weight the variant applies to each pick: p_pick for the weighted
    concatenation, the renormalised w otherwise. workers > 1 runs the
    per-head attentions on that many threads (same results).
    """
    x = inp["x"]
    N = x.shape[0]
    logits, p, sel, w = route(x, inp["Wr"], inp.get("br"), G, M, k)

    Wq = inp["Wq"].reshape(G, M, d, -1)
    K = project(x, inp["Wk"]).reshape(B, T, G, d)
    V = project(x, inp["Wv"]).reshape(B, T, G, d)

    # Q only for the selected experts: Qr[n,g,r] = x[n] . Wq[g, sel[n,g,r]].T
    Qr = _routed_queries(x, Wq, sel)
    Q_sh = project(x, inp["Wq_sh"])

    # One attention per routed (g, r) head slot, then the shared head.
    jobs = [(Qr[:, g, r].reshape(B, T, d), K[:, :, g], V[:, :, g], q_block) for g in range(G) for r in range(k)]
    s0 = shared_kv_group
    if variant != "no_shared":
        jobs.append((Q_sh.reshape(B, T, d), K[:, :, s0], V[:, :, s0], q_block))
    res = _map_heads(causal_attention, jobs, workers)
    O = np.empty((N, G, k, d))
    for g in range(G):
        for r in range(k):
            O[:, g, r] = res[g * k + r].reshape(N, d)
    O_sh = res[G * k].reshape(N, d) if variant != "no_shared" else None

    p_pick = pick_probs(p, sel)
    C = assemble_variant(O, w, p_pick, O_sh, variant)
    out = project(C, inp["Wo"])
    return dict(logits=logits, p=p, idx=sel, w=(p_pick if variant == "weighted_concat" else w), Qr=Qr,
                Q_sh=Q_sh, K=K.reshape(N, G, d), V=V.reshape(N, G, d), C=C, out=out)


def gqa_forward(inp: dict, G: int, Hq: int, d: int, B: int, T: int, q_block: int = 512,
                workers: int = 1) -> dict:
    """Dense GQA: every query head on every token, head h on KV group h // (Hq/G).

    [GQA-w] "Mechanism": query heads split into groups sharing one K/V head.
    inp: x, Wq [Hq*d,D], Wk, Wv [G*d,D], Wo [D,Hq*d]. workers as in gqe_forward.
    """
    x = inp["x"]
    N = x.shape[0]
    per = Hq // G
    Q = project(x, inp["Wq"]).reshape(B, T, Hq, d)
    K = project(x, inp["Wk"]).reshape(B, T, G, d)
    V = project(x, inp["Wv"]).reshape(B, T, G, d)
    res = _map_heads(causal_attention, [(Q[:, :, h], K[:, :, h // per], V[:, :, h // per], q_block)
                                        for h in range(Hq)], workers)
    O = np.empty((N, Hq, d))
    for h in range(Hq):
        O[:, h] = res[h].reshape(N, d)
    C = O.reshape(N, Hq * d)
    return dict(Q=Q.reshape(N, Hq, d), C=C, out=project(C, inp["Wo"]))


def active_heads(sel: np.ndarray) -> np.ndarray:
    """Query heads a token activates: its G*k routed experts plus the shared head."""
    N, G, k = sel.shape
    distinct = np.array([len({(g, int(sel[n, g, r])) for g in range(G) for r in range(k)})
                         for n in range(N)])
    return distinct + 1


# ----------------------------------------------------------------------------
# Sampled-row mode: full routing, outputs for a few rows only, with K/V
# streamed over key chunks (online softmax in fp64). Same arithmetic as above
# up to fp64 rounding order.
# ----------------------------------------------------------------------------
def _rows_attention(x, heads, Wk, Wv, G, d, B, T, rows, kv_chunk):
    """For each sampled row n=(b,t) and each head (q vector, KV group), stream
    keys s=0..t of sequence b in chunks and return O [n_rows, H, d]."""
    n_rows = len(rows)
    H = heads[0].shape[1]
    bs, ts = rows // T, rows % T
    m = np.full((n_rows, H), -np.inf)
    l = np.zeros((n_rows, H))
    acc = np.zeros((n_rows, H, d))
    scale = 1.0 / np.sqrt(d)
    qv, grp = heads                                            # qv [n_rows,H,d]; grp [H]
    for b in np.unique(bs):
        mine = np.nonzero(bs == b)[0]
        t_max = int(ts[mine].max())
        for c0 in range(0, t_max + 1, kv_chunk):
            c1 = min(t_max + 1, c0 + kv_chunk)
            xc = x[b * T + c0: b * T + c1]
            Kc = project(xc, Wk).reshape(-1, G, d)
            Vc = project(xc, Wv).reshape(-1, G, d)
            for i in mine:
                if ts[i] < c0:
                    continue
                hi = min(c1, int(ts[i]) + 1) - c0
                for hh in range(H):
                    g = grp[hh]
                    s = (Kc[:hi, g] @ qv[i, hh]) * scale            # [hi]
                    m_new = max(m[i, hh], s.max())
                    corr = np.exp(m[i, hh] - m_new)
                    e = np.exp(s - m_new)
                    l[i, hh] = l[i, hh] * corr + e.sum()
                    acc[i, hh] = acc[i, hh] * corr + e @ Vc[:hi, g]
                    m[i, hh] = m_new
    return acc / l[:, :, None]


def gqe_rows(inp: dict, G: int, M: int, k: int, d: int, B: int, T: int, rows,
             shared_kv_group: int = 0, kv_chunk: int = 65536, variant: str = "full") -> dict:
    """Routing for every token; slots C and out only for the given rows."""
    rows = np.asarray(rows, dtype=np.int64)
    x = inp["x"]
    logits, p, sel, w = route(x, inp["Wr"], inp.get("br"), G, M, k)
    xr = x[rows]
    Wq = inp["Wq"].reshape(G, M, d, -1)
    q = np.empty((len(rows), G * k + 1, d))
    q[:, :G * k] = _routed_queries(xr, Wq, sel[rows]).reshape(len(rows), G * k, d)
    grp = np.empty(G * k + 1, dtype=np.int64)
    grp[:G * k] = np.repeat(np.arange(G), k)
    q[:, G * k] = project(xr, inp["Wq_sh"])
    grp[G * k] = shared_kv_group
    O_all = _rows_attention(x, (q, grp), inp["Wk"], inp["Wv"], G, d, B, T, rows, kv_chunk)
    O = O_all[:, :G * k].reshape(len(rows), G, k, d)
    p_pick = pick_probs(p, sel)
    C = assemble_variant(O, w[rows], p_pick[rows], O_all[:, G * k], variant)
    return dict(logits=logits, p=p, idx=sel, w=(p_pick if variant == "weighted_concat" else w), rows=rows,
                C=C, out=project(C, inp["Wo"]))


def gqa_rows(inp: dict, G: int, Hq: int, d: int, B: int, T: int, rows, kv_chunk: int = 65536) -> dict:
    """Dense GQA outputs for the given rows only (K/V streamed)."""
    rows = np.asarray(rows, dtype=np.int64)
    x = inp["x"]
    q = project(x[rows], inp["Wq"]).reshape(len(rows), Hq, d)
    grp = np.arange(Hq) // (Hq // G)
    O = _rows_attention(x, (q, grp), inp["Wk"], inp["Wv"], G, d, B, T, rows, kv_chunk)
    C = O.reshape(len(rows), Hq * d)
    return dict(rows=rows, C=C, out=project(C, inp["Wo"]))
