"""Pins for the fp64 backward oracle (CPU only).

The gradients are checked against things other than themselves: central finite
differences of the forward oracle (the whole layer, one random direction per
parameter, routing held fixed), torch autograd through torch's own attention and
softmax routines in fp64, closed-form invariants (the renormalisation is scale
invariant; a softmax is shift invariant), the pages' statement that the router
learns only through the weighted slot, and a pure-Python count for the
auxiliary loss. Planted mistakes at the end must each fail a pin.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle.gqe_backward as gb
import oracle.gqe_oracle as go

from .test_oracle import rand_layer

PARAMS = ("x", "Wr", "br", "Wq", "Wk", "Wv", "Wq_sh", "Wo")
GRAD = dict(x="dx", Wr="dWr", br="dbr", Wq="dWq", Wk="dWk", Wv="dWv", Wq_sh="dWq_sh", Wo="dWo")


def scipy_softmax(z):
    return scipy.special.softmax(z, axis=2)


def _loss(inp, dout, G, M, k, d, B, T, s0, coef, q_block):
    f = go.gqe_forward(inp, G, M, k, d, B, T, shared_kv_group=s0, q_block=q_block)
    aux, _ = gb.load_balance_loss(f["p"], f["idx"], coef)
    return float((dout * f["out"]).sum()) + aux, f["idx"]


def _fd_case(seed, B, T, D, G, M, k, d, s0, coef, q_block, h=1e-5, rtol=2e-7):
    rng = np.random.default_rng(seed)
    inp = rand_layer(rng, B, T, D, G, M, k, d, bias=True)
    inp.pop("Wo_gqa")
    N = B * T
    dout = rng.standard_normal((N, D))
    fwd = go.gqe_forward(inp, G, M, k, d, B, T, shared_kv_group=s0, q_block=q_block)
    g = gb.gqe_backward(inp, fwd, dout, G, M, k, d, B, T, shared_kv_group=s0, aux_coef=coef, q_block=q_block)
    _, sel0 = _loss(inp, dout, G, M, k, d, B, T, s0, coef, q_block)
    for name in PARAMS:
        v = rng.standard_normal(inp[name].shape)
        pts = []
        for sgn in (1.0, -1.0):
            pert = dict(inp)
            pert[name] = inp[name] + sgn * h * v
            L, sel = _loss(pert, dout, G, M, k, d, B, T, s0, coef, q_block)
            assert np.array_equal(sel, sel0), "routing flipped under the finite-difference step"
            pts.append(L)
        fd = (pts[0] - pts[1]) / (2 * h)
        an = float((g[GRAD[name]] * v).sum())
        assert abs(fd - an) <= rtol * max(1.0, abs(fd)), (name, fd, an)


# ----------------------------------------------------------------------------
# Pins
# ----------------------------------------------------------------------------
def pin_layer_finite_differences():
    """Every parameter's gradient against central differences of the forward,
    at a shape that spans several query blocks, k > 1, a biased router, the
    shared head on a non-zero group and a non-zero auxiliary coefficient."""
    _fd_case(3, B=2, T=20, D=16, G=2, M=3, k=2, d=8, s0=1, coef=0.3, q_block=8)
    _fd_case(4, B=1, T=9, D=12, G=3, M=2, k=1, d=4, s0=0, coef=0.0, q_block=512)


def pin_attention_torch_autograd():
    """attention_backward against autograd through torch's attention routine
    (fp64, CPU), with the query blocking of the oracle shorter than T."""
    rng = np.random.default_rng(5)
    B, T, d = 2, 37, 8
    q, k, v, do = (rng.standard_normal((B, T, d)) for _ in range(4))
    tq, tk, tv = (torch.from_numpy(a[:, None]).requires_grad_() for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    o.backward(torch.from_numpy(do[:, None]))
    dq, dk, dv = gb.attention_backward(q, k, v, do, q_block=16)
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, t.grad.numpy()[:, 0], rtol=1e-10, atol=1e-12)


def pin_softmax_torch_autograd():
    """group_softmax_backward against autograd through torch.softmax."""
    rng = np.random.default_rng(6)
    z = torch.from_numpy(rng.standard_normal((11, 3, 4))).requires_grad_()
    dp = rng.standard_normal((11, 3, 4))
    p = torch.softmax(z, dim=2)
    p.backward(torch.from_numpy(dp))
    np.testing.assert_allclose(gb.group_softmax_backward(p.detach().numpy(), dp), z.grad.numpy(),
                               rtol=1e-12, atol=1e-14)


def pin_gradient_invariants():
    """w depends on p_pick only through its direction, so dp_pick is orthogonal
    to p_pick; a softmax ignores a shift of its logits, so dz sums to zero per
    group."""
    rng = np.random.default_rng(7)
    p_pick = rng.uniform(0.05, 1.0, (13, 3, 2))
    w = p_pick / p_pick.sum(axis=(1, 2), keepdims=True)
    dp = gb.renormalize_backward(p_pick, w, rng.standard_normal(p_pick.shape))
    np.testing.assert_allclose((dp * p_pick).sum(axis=(1, 2)), 0.0, atol=1e-13)
    p = scipy_softmax(rng.standard_normal((13, 3, 4)))
    dz = gb.group_softmax_backward(p, rng.standard_normal(p.shape))
    np.testing.assert_allclose(dz.sum(axis=2), 0.0, atol=1e-13)


def pin_router_learns_only_through_weighted_slot():
    """With the weighted slot's Wo columns zero and no auxiliary loss, the hard
    concatenation and the shared head pass no gradient to the router; with the
    columns non-zero they do."""
    rng = np.random.default_rng(8)
    B, T, D, G, M, k, d = 1, 12, 10, 2, 3, 2, 4
    inp = rand_layer(rng, B, T, D, G, M, k, d, bias=True)
    dout = rng.standard_normal((B * T, D))
    fwd = go.gqe_forward(inp, G, M, k, d, B, T)
    g = gb.gqe_backward(inp, fwd, dout, G, M, k, d, B, T)
    assert np.abs(g["dWr"]).max() > 1e-6
    inp["Wo"] = inp["Wo"].copy()
    inp["Wo"][:, G * k * d:(G * k + 1) * d] = 0.0
    fwd = go.gqe_forward(inp, G, M, k, d, B, T)
    g = gb.gqe_backward(inp, fwd, dout, G, M, k, d, B, T)
    assert np.abs(g["dWr"]).max() == 0.0 and np.abs(g["dbr"]).max() == 0.0


def pin_load_balance_loss_count():
    """The auxiliary loss value against a pure-Python count of the picks; a
    router that spreads picks and probability evenly (f = mean p = 1/M for
    every expert) scores exactly coef."""
    rng = np.random.default_rng(9)
    N, G, M, k = 17, 2, 4, 2
    p = scipy_softmax(rng.standard_normal((N, G, M)))
    sel = np.stack([np.stack([rng.permutation(M)[:k] for _ in range(G)]) for _ in range(N)])
    total = 0.0
    for g in range(G):
        for m in range(M):
            cnt = sum(1 for n in range(N) for r in range(k) if sel[n, g, r] == m)
            mean_p = sum(p[n, g, m] for n in range(N)) / N
            total += M * (cnt / (N * k)) * mean_p
    loss, _ = gb.load_balance_loss(p, sel, 0.7)
    assert math.isclose(loss, 0.7 * total / G, rel_tol=1e-12)
    # perfectly balanced: every expert picked equally often, uniform probabilities
    M, k, N = 4, 2, 8
    sel = np.array([[[(2 * n) % M, (2 * n + 1) % M]] for n in range(N)])
    loss, _ = gb.load_balance_loss(np.full((N, 1, M), 1.0 / M), sel, 1.0)
    assert math.isclose(loss, 1.0, rel_tol=1e-12)


def pin_rows_backward_against_full():
    """The row-by-row backward (dout zero outside a few rows, no balancing
    loss) against the full-matrix backward on the same inputs: two shapes,
    one with k = 2, a biased router, two sequences and the shared head on
    group 1; rows at both sequences' ends, their starts and the middle. Then
    finite differences of the forward oracle along random directions, with
    dout zero outside the rows."""
    for seed, (B, T, D, G, M, k, d, s0) in ((41, (2, 37, 24, 3, 3, 2, 8, 1)), (43, (1, 70, 16, 2, 2, 1, 8, 0))):
        rng = np.random.default_rng(seed)
        inp = rand_layer(rng, B, T, D, G, M, k, d, bias=True)
        inp.pop("Wo_gqa")
        N = B * T
        rows = np.array(sorted({0, T - 1, N - 1, N - 3, T // 2, N - T}))
        dout = np.zeros((N, D))
        dout[rows] = rng.standard_normal((len(rows), D))
        fwd = go.gqe_forward(inp, G, M, k, d, B, T, shared_kv_group=s0, q_block=16)
        full = gb.gqe_backward(inp, fwd, dout, G, M, k, d, B, T, shared_kv_group=s0, aux_coef=0.0, q_block=16)
        part = gb.gqe_backward_rows(inp, rows, dout[rows], G, M, k, d, B, T, shared_kv_group=s0)
        assert (part["idx"] == fwd["idx"][rows]).all()
        for name in PARAMS:
            a, b = part[GRAD[name]], full[GRAD[name]]
            assert np.allclose(a, b, rtol=1e-9, atol=1e-12 * max(1.0, np.abs(b).max())), name
        h = 1e-5
        for name in PARAMS:
            v = rng.standard_normal(inp[name].shape)
            Ls = []
            for sgn in (1.0, -1.0):
                pert = dict(inp)
                pert[name] = inp[name] + sgn * h * v
                f = go.gqe_forward(pert, G, M, k, d, B, T, shared_kv_group=s0, q_block=16)
                assert np.array_equal(f["idx"], fwd["idx"])
                Ls.append(float((dout * f["out"]).sum()))
            fd = (Ls[0] - Ls[1]) / (2 * h)
            an = float((part[GRAD[name]] * v).sum())
            assert abs(fd - an) <= 2e-7 * max(1.0, abs(fd)), (name, fd, an)


PINS = [pin_layer_finite_differences, pin_attention_torch_autograd, pin_softmax_torch_autograd,
        pin_gradient_invariants, pin_router_learns_only_through_weighted_slot, pin_load_balance_loss_count,
        pin_rows_backward_against_full]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# Planted mistakes: each must fail at least one pin
# ----------------------------------------------------------------------------
_orig = dict(attention_backward=gb.attention_backward, renormalize_backward=gb.renormalize_backward,
             group_softmax_backward=gb.group_softmax_backward, load_balance_loss=gb.load_balance_loss,
             scatter_picks=gb.scatter_picks)


def _attn_no_rowsum(q, k, v, dO, q_block=512):
    """dS = P * dP (drops the rowsum term)."""
    B, T, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        s = q[b] @ k[b].T / math.sqrt(d)
        s = np.where(np.tri(T, dtype=bool), s, -np.inf)
        P = np.exp(s - s.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        dv[b] = P.T @ dO[b]
        dS = P * (dO[b] @ v[b].T)
        dq[b] = dS @ k[b] / math.sqrt(d)
        dk[b] = dS.T @ q[b] / math.sqrt(d)
    return dq, dk, dv


def _attn_dk_unscaled(q, k, v, dO, q_block=512):
    dq, dk, dv = _orig["attention_backward"](q, k, v, dO, q_block)
    return dq, dk * math.sqrt(q.shape[2]), dv


def _renorm_no_projection(p_pick, w, dw):
    return dw / p_pick.sum(axis=(1, 2), keepdims=True)


def _softmax_bwd_identity(p, dp):
    return p * dp


def _aux_grad_without_M(p, sel, coef):
    loss, dp = _orig["load_balance_loss"](p, sel, coef)
    return loss, dp / p.shape[2]


def _scatter_rank_reversed(dp_pick, sel, M):
    return _orig["scatter_picks"](dp_pick[:, :, ::-1], sel, M)


MUTANTS = {
    "attention_drops_rowsum": ("attention_backward", _attn_no_rowsum),
    "attention_dk_unscaled": ("attention_backward", _attn_dk_unscaled),
    "renormalisation_not_projected": ("renormalize_backward", _renorm_no_projection),
    "softmax_jacobian_diagonal_only": ("group_softmax_backward", _softmax_bwd_identity),
    "aux_gradient_drops_M": ("load_balance_loss", _aux_grad_without_M),
    "router_gradient_to_wrong_rank": ("scatter_picks", _scatter_rank_reversed),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(gb, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
