"""Helpers for the GPU parity tests and the benchmark's checks.

Inputs come from workloads.py (seeded), the GPU path runs through the ctypes
binding of libgqe.so, expected values come from the fp64 oracle. The two
sides share only the input generator.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle.gqe_oracle as go
import sparse_moe_attention_amd as gq
from workloads import Shape, to_f64

# Acceptance bars.
OUT_REL, OUT_ABS = 1e-2, 1e-3          # max|err| <= 1e-2 * max|ref| + 1e-3
LOGIT_REL = 1e-5                       # |err| <= 1e-5 * max(1, |l|)
W_ABS = 1e-6                           # routing weights
NEAR_TIE = 1e-4                        # top-k margin below which either routing is correct


def to_device(inp: dict, dev="cuda") -> dict:
    return {k: (v.to(dev).contiguous() if v is not None else None) for k, v in inp.items()}


def f64_inputs(inp: dict) -> dict:
    return {k: to_f64(v) for k, v in inp.items()}


def oracle_routing(f: dict, s: Shape, chunk: int = 65536):
    """Oracle routing of every token, in token chunks (routing is per token).
    w is the weight the shape's merge variant applies to each pick."""
    logits, sel, w = [], [], []
    for n0 in range(0, s.N, chunk):
        lg, p, se, ww = go.route(f["x"][n0:n0 + chunk], f["Wr"], f.get("br"), s.G, s.M, s.k)
        logits.append(lg)
        sel.append(se)
        w.append(go.pick_probs(p, se) if s.variant == "weighted_concat" else ww)
    return np.concatenate(logits), np.concatenate(sel), np.concatenate(w)


def near_tie_rows(logits: np.ndarray, s: Shape, thr: float = NEAR_TIE) -> np.ndarray:
    """Tokens where some group's top-k decision is within thr: the gap between
    consecutive sorted logits at ranks r, r+1 for r < min(k, M-1)."""
    N = logits.shape[0]
    if s.M == 1:
        return np.zeros(N, dtype=bool)
    z = -np.sort(-logits.reshape(N, s.G, s.M), axis=2)
    R = min(s.k, s.M - 1)
    gaps = z[:, :, :R] - z[:, :, 1:R + 1]
    return (gaps < thr).any(axis=(1, 2))


def out_error(got: np.ndarray, ref: np.ndarray):
    err = float(np.abs(got - ref).max())
    bound = OUT_REL * float(np.abs(ref).max()) + OUT_ABS
    return err, bound


def alloc_outputs(s: Shape, dev="cuda"):
    dt = s.torch_dtype()
    return dict(
        out=torch.empty(s.N, s.D, dtype=dt, device=dev),
        idx=torch.empty(s.N, s.G, s.k, dtype=torch.int32, device=dev),
        w=torch.empty(s.N, s.G, s.k, dtype=torch.float32, device=dev),
    )


def run_gqe(s: Shape, d: dict, o: dict, ws=None):
    gq.gqe_attn_fwd(gq.shape_from(s), d["x"], d["Wr"], d["br"], d["Wq"], d["Wk"], d["Wv"], d["Wq_sh"],
                    d["Wo"], o["out"], o["idx"], o["w"], ws=ws)


def run_gqe_routed(s: Shape, d: dict, idx, w, out, slots=None, ws=None):
    gq.gqe_attn_fwd_routed(gq.shape_from(s), d["x"], d["Wq"], d["Wk"], d["Wv"], d["Wq_sh"], d["Wo"],
                           idx, w, out, slots, ws=ws)


def run_gqa(s: Shape, d: dict, out, ws=None):
    dt = gq.GQE_F32 if s.dtype == "f32" else gq.GQE_BF16
    gq.gqa_attn_fwd(s.B, s.T, s.D, s.Hq, s.G, s.d, dt, d["x"], d["Wq"], d["Wk"], d["Wv"], d["Wo_gqa"], out,
                    ws=ws)


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
