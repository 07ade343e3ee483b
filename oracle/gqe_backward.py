"""Plain fp64 CPU oracle for the backward pass of the GQE attention layer.

TEST INFRASTRUCTURE ONLY, like gqe_oracle: only tests/ (and bench.py's
cpu_baseline leg) may import it; the HIP library never does.

Gradients of a loss L = <dout, out> + L_aux through the full layer of
gqe_oracle.gqe_forward, written out from the chain rule step by step in
float64. Sources (title and section):

  [GQE-x]  "Grouped Query Experts: Mixture-of-Experts on GQA Self-Attention",
           gist.science explainer, technical summary: "Architecture and
           routing" (the routed hard concatenation carries no routing
           gradient; the renormalised weighted sum is the differentiable path
           to the router), "Training and loss" (a load-balancing auxiliary loss
           spreads each group's tokens over its experts).
  [GQE-n]  FrontiersMind GQE article, part 5 (the weighted-sum slot is the
           router's learning signal; an auxiliary balancing loss keeps the
           router from always picking the same experts).

Readings where the pages are silent or garbled:
  * the top-k selection is piecewise constant: no gradient flows through idx;
  * the auxiliary loss is the usual fraction-times-mean-probability form,
    per group and averaged over groups:
        L_aux = coef * (1/G) * sum_g M * sum_m f[g,m] * P[g,m],
    f[g,m] = share of group g's N*k picks that went to expert m,
    P[g,m] = mean over tokens of the router probability p[n,g,m];
    f is a count and carries no gradient. The pages give no formula.

Every function here is pinned in tests/test_oracle_backward.py.
"""
from __future__ import annotations

import numpy as np

from . import gqe_oracle as go

__all__ = [
    "attention_backward", "renormalize_backward", "scatter_picks", "group_softmax_backward",
    "load_balance_loss", "gqe_backward", "gqe_backward_rows",
]


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dO: np.ndarray, q_block: int = 512):
    """Gradients of O = causal_attention(q, k, v) (scale 1/sqrt(d)) against dO.

    With P the row softmax of S = q k^T / sqrt(d): dV = P^T dO, dP = dO V^T,
    dS = P * (dP - rowsum(dP * P)), dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d).
    q, k, v, dO [B,T,d] -> (dq, dk, dv)."""
    B, T, d = q.shape
    scale = 1.0 / np.sqrt(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for t0 in range(0, T, q_block):
            t1 = min(T, t0 + q_block)
            s = (q[b, t0:t1] @ k[b, :t1].T) * scale
            allowed = np.arange(t1)[None, :] <= np.arange(t0, t1)[:, None]
            s = np.where(allowed, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            P = e / e.sum(axis=1, keepdims=True)
            do = dO[b, t0:t1]
            dv[b, :t1] += P.T @ do
            dP = do @ v[b, :t1].T
            dS = P * (dP - (dP * P).sum(axis=1, keepdims=True))
            dq[b, t0:t1] = (dS @ k[b, :t1]) * scale
            dk[b, :t1] += (dS.T @ q[b, t0:t1]) * scale
    return dq, dk, dv


def renormalize_backward(p_pick: np.ndarray, w: np.ndarray, dw: np.ndarray) -> np.ndarray:
    """w = p_pick / S with S the sum over the token's G*k picks:
    dp_pick = (dw - sum(dw * w)) / S.  [N,G,k] arrays."""
    S = p_pick.sum(axis=(1, 2), keepdims=True)
    return (dw - (dw * w).sum(axis=(1, 2), keepdims=True)) / S


def scatter_picks(dp_pick: np.ndarray, sel: np.ndarray, M: int) -> np.ndarray:
    """[N,G,k] values at the picked experts -> [N,G,M] (zero for the others;
    the picks of one group are distinct experts)."""
    N, G, k = sel.shape
    out = np.zeros((N, G, M))
    np.put_along_axis(out, sel, dp_pick, axis=2)
    return out


def group_softmax_backward(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """Through p = softmax over each group's M logits: dz = p * (dp - sum(p * dp))."""
    return p * (dp - (p * dp).sum(axis=2, keepdims=True))


def load_balance_loss(p: np.ndarray, sel: np.ndarray, coef: float):
    """The auxiliary load-balancing loss (reading above) and its gradient in p.
    p [N,G,M], sel [N,G,k] -> (loss, dL/dp [N,G,M])."""
    N, G, M = p.shape
    k = sel.shape[2]
    f = np.stack([np.bincount(sel[:, g, :].ravel(), minlength=M) for g in range(G)]) / (N * k)
    Pbar = p.mean(axis=0)
    loss = coef * float((M * (f * Pbar).sum(axis=1)).mean())
    dp = np.broadcast_to(coef * M * f / (N * G), p.shape).copy()
    return loss, dp


def gqe_backward(inp: dict, fwd: dict, dout: np.ndarray, G: int, M: int, k: int, d: int, B: int, T: int,
                 shared_kv_group: int = 0, aux_coef: float = 0.0, q_block: int = 512) -> dict:
    """Gradients of <dout, out> + L_aux for the full layer, given the forward's
    dict (gqe_forward with the same inputs). Returns dx, dWr, dbr, dWq, dWk,
    dWv, dWq_sh, dWo, aux_loss, and the intermediate dC, dO, dw, dQr, dQ_sh,
    dK, dV, dlogits."""
    x = inp["x"]
    N, D = x.shape
    GK = G * k
    C, w, sel, p = fwd["C"], fwd["w"], fwd["idx"], fwd["p"]

    # out = C Wo^T
    dWo = dout.T @ C
    dC = dout @ inp["Wo"]
    dCh = dC[:, :GK * d].reshape(N, G, k, d)
    dCw = dC[:, GK * d:(GK + 1) * d]
    dCsh = dC[:, (GK + 1) * d:]

    # C = [O | sum w O | O_sh]
    O = C[:, :GK * d].reshape(N, G, k, d)
    dO = dCh + w[..., None] * dCw[:, None, None, :]
    dw = np.einsum("ngrd,nd->ngr", O, dCw)

    # attention of every routed head and of the shared head
    K = fwd["K"].reshape(B, T, G, d)
    V = fwd["V"].reshape(B, T, G, d)
    dK = np.zeros((B, T, G, d))
    dV = np.zeros((B, T, G, d))
    dQr = np.zeros((N, G, k, d))
    for g in range(G):
        for r in range(k):
            dq, dk_, dv_ = attention_backward(fwd["Qr"][:, g, r].reshape(B, T, d), K[:, :, g], V[:, :, g],
                                              dO[:, g, r].reshape(B, T, d), q_block)
            dQr[:, g, r] = dq.reshape(N, d)
            dK[:, :, g] += dk_
            dV[:, :, g] += dv_
    s0 = shared_kv_group
    dq, dk_, dv_ = attention_backward(fwd["Q_sh"].reshape(B, T, d), K[:, :, s0], V[:, :, s0],
                                      dCsh.reshape(B, T, d), q_block)
    dQ_sh = dq.reshape(N, d)
    dK[:, :, s0] += dk_
    dV[:, :, s0] += dv_

    # projections: Qr[n,g,r] = x[n] Wq[g,sel]^T, Q_sh = x Wq_sh^T, K = x Wk^T, V = x Wv^T
    Wq = inp["Wq"].reshape(G, M, d, D)
    dWq = np.zeros_like(Wq)
    dx = np.zeros_like(x)
    for g in range(G):
        for r in range(k):
            for m in range(M):
                pick = sel[:, g, r] == m
                if pick.any():
                    dWq[g, m] += dQr[pick, g, r].T @ x[pick]
                    dx[pick] += dQr[pick, g, r] @ Wq[g, m]
    dWq_sh = dQ_sh.T @ x
    dx += dQ_sh @ inp["Wq_sh"]
    dKf = dK.reshape(N, G * d)
    dVf = dV.reshape(N, G * d)
    dWk = dKf.T @ x
    dWv = dVf.T @ x
    dx += dKf @ inp["Wk"] + dVf @ inp["Wv"]

    # router: w = renormalised picked probabilities of the per-group softmax
    p_pick = go.pick_probs(p, sel)
    dp = scatter_picks(renormalize_backward(p_pick, w, dw), sel, M)
    aux, dp_aux = load_balance_loss(p, sel, aux_coef)
    dlogits = group_softmax_backward(p, dp + dp_aux).reshape(N, G * M)
    dWr = dlogits.T @ x
    dbr = dlogits.sum(axis=0)
    dx += dlogits @ inp["Wr"]

    return dict(dx=dx, dWr=dWr, dbr=dbr, dWq=dWq.reshape(G * M * d, D), dWk=dWk, dWv=dWv, dWq_sh=dWq_sh,
                dWo=dWo, aux_loss=aux, dC=dC, dO=dO, dw=dw, dQr=dQr, dQ_sh=dQ_sh,
                dK=dKf, dV=dVf, dlogits=dlogits)


def gqe_backward_rows(inp: dict, rows, dout_rows: np.ndarray, G: int, M: int, k: int, d: int, B: int, T: int,
                      shared_kv_group: int = 0) -> dict:
    """The gradients of gqe_backward when dout is zero on every token except
    `rows` (dout_rows [len(rows), D] holds theirs) and there is no balancing
    loss, computed row by row, so that sequences far longer than the full
    oracle can hold are checked: only the given rows' attention enters
    (their causal prefixes in full), every key and value of those prefixes
    receives its dK, dV contribution, and the projections then sum over all
    tokens. Same formulas as gqe_backward: dV = P^T dO, dS = P * (dP -
    rowsum(dP * P)), dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d); the slots'
    split dO = dC_hard + w dC_weighted, dw = <O, dC_weighted>; the router
    through the renormalisation and the group softmax. Returns dx [N,D], dWr,
    dbr, dWq, dWk, dWv, dWq_sh, dWo and the forward's picks of the rows."""
    rows = np.asarray(rows, dtype=np.int64)
    x = inp["x"]
    N, D = x.shape
    GK = G * k
    scale = 1.0 / np.sqrt(d)
    xr = x[rows]
    logits, p, sel, w = go.route(xr, inp["Wr"], inp.get("br"), G, M, k)

    K = go.project(x, inp["Wk"]).reshape(N, G, d)
    V = go.project(x, inp["Wv"]).reshape(N, G, d)
    Wq = inp["Wq"].reshape(G, M, d, D)
    nR = len(rows)
    # query of every (row, head): routed heads (g, r), then the shared head
    q = np.zeros((nR, GK + 1, d))
    grp = np.empty(GK + 1, dtype=np.int64)
    for g in range(G):
        for r in range(k):
            grp[g * k + r] = g
            for i in range(nR):
                q[i, g * k + r] = xr[i] @ Wq[g, sel[i, g, r]].T
    q[:, GK] = go.project(xr, inp["Wq_sh"])
    grp[GK] = shared_kv_group

    # forward attention of the rows, kept for the backward
    P = {}
    O = np.zeros((nR, GK + 1, d))
    for i, n in enumerate(rows):
        b, t = divmod(int(n), T)
        keys = slice(b * T, b * T + t + 1)
        for h in range(GK + 1):
            s_ = (K[keys, grp[h]] @ q[i, h]) * scale
            e = np.exp(s_ - s_.max())
            P[i, h] = e / e.sum()
            O[i, h] = P[i, h] @ V[keys, grp[h]]
    C = np.concatenate([O[:, :GK].reshape(nR, GK * d), np.einsum("ngr,ngrd->nd", w, O[:, :GK].reshape(nR, G, k, d)),
                        O[:, GK]], axis=1)

    dWo = dout_rows.T @ C
    dC = dout_rows @ inp["Wo"]
    dCw = dC[:, GK * d:(GK + 1) * d]
    dO = np.zeros((nR, GK + 1, d))
    dO[:, :GK] = dC[:, :GK * d].reshape(nR, GK, d) + w.reshape(nR, GK)[..., None] * dCw[:, None, :]
    dO[:, GK] = dC[:, (GK + 1) * d:]
    dw = np.einsum("nhd,nd->nh", O[:, :GK], dCw).reshape(nR, G, k)

    dK = np.zeros((N, G, d))
    dV = np.zeros((N, G, d))
    dq = np.zeros((nR, GK + 1, d))
    for i, n in enumerate(rows):
        b, t = divmod(int(n), T)
        keys = slice(b * T, b * T + t + 1)
        for h in range(GK + 1):
            g = grp[h]
            Ph = P[i, h]
            dV[keys, g] += np.outer(Ph, dO[i, h])
            dP = V[keys, g] @ dO[i, h]
            dS = Ph * (dP - (dP * Ph).sum())
            dq[i, h] = (dS @ K[keys, g]) * scale
            dK[keys, g] += np.outer(dS, q[i, h]) * scale

    dx = np.zeros_like(x)
    dWq = np.zeros_like(Wq)
    for g in range(G):
        for r in range(k):
            for i in range(nR):
                m = sel[i, g, r]
                dWq[g, m] += np.outer(dq[i, g * k + r], xr[i])
                dx[rows[i]] += dq[i, g * k + r] @ Wq[g, m]
    dWq_sh = dq[:, GK].T @ xr
    dx[rows] += dq[:, GK] @ inp["Wq_sh"]
    dKf = dK.reshape(N, G * d)
    dVf = dV.reshape(N, G * d)
    dWk = dKf.T @ x
    dWv = dVf.T @ x
    dx += dKf @ inp["Wk"] + dVf @ inp["Wv"]

    p_pick = go.pick_probs(p, sel)
    dp = scatter_picks(renormalize_backward(p_pick, w, dw), sel, M)
    dlogits = group_softmax_backward(p, dp).reshape(nR, G * M)
    dWr = dlogits.T @ xr
    dbr = dlogits.sum(axis=0)
    dx[rows] += dlogits @ inp["Wr"]
    return dict(dx=dx, dWr=dWr, dbr=dbr, dWq=dWq.reshape(G * M * d, D), dWk=dWk, dWv=dWv, dWq_sh=dWq_sh,
                dWo=dWo, idx=sel, rows=rows)
