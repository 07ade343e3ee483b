"""gqe_attn_fwd_noalloc, the forward on the library's static device scratch,
against gqe_attn_fwd with a caller workspace, through the C ABI.

Calls run in a row on shrinking shapes (the 32K-token layer, then two small
layers), so each later call finds the scratch holding an earlier, larger
call's data. The same kernels run on the same inputs, so out, idx and w must
be bit-identical to the workspace form; the small layers are also held to the
oracle's bar (output within 1e-2*max|ref| + 1e-3 on rows whose routing agrees,
routing bit-exact away from near-ties)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.gqe_oracle as go
import sparse_moe_attention_amd as gq
from tests import harness as H
from workloads import CONFIGS, Shape, make_inputs

pytestmark = pytest.mark.gpu

CASES = [
    ("layer_32k", CONFIGS[3], 1003, False),
    ("multi_tile", Shape(B=2, T=1000, D=256, G=8, M=2, k=1, d=64), 5, True),
    ("ragged_bias_k2", Shape(B=3, T=200, D=128, G=3, M=3, k=2, d=32, router_bias=True, shared_kv_group=1), 6,
     True),
]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.load()
    torch.cuda.set_device(0)


def test_noalloc_matches_workspace_form():
    for name, s, seed, with_oracle in CASES:
        print(f"[noalloc {name}] {s}", flush=True)
        inp = make_inputs(s, seed=seed)
        dv = H.to_device(inp)
        ref = H.alloc_outputs(s)
        H.run_gqe(s, dv, ref)
        got = H.alloc_outputs(s)
        for t in got.values():
            t.fill_(7)
        gq.gqe_attn_fwd_noalloc(gq.shape_from(s), dv["x"], dv["Wr"], dv["br"], dv["Wq"], dv["Wk"], dv["Wv"],
                                dv["Wq_sh"], dv["Wo"], got["out"], got["idx"], got["w"])
        torch.cuda.synchronize()
        for key in ("out", "idx", "w"):
            assert torch.equal(got[key], ref[key]), (name, key)
        if with_oracle:
            f = H.f64_inputs(inp)
            o = go.gqe_forward(f, s.G, s.M, s.k, s.d, s.B, s.T, shared_kv_group=s.shared_kv_group)
            near = H.near_tie_rows(o["logits"], s)
            bad = (got["idx"].cpu().numpy() != o["idx"]).any(axis=(1, 2))
            assert not (bad & ~near).any(), (name, "routing")
            err, bound = H.out_error(H.np32(got["out"])[~bad], o["out"][~bad])
            assert err <= bound, (name, err, bound)
            print(f"[noalloc {name}] bit-identical to the workspace form; oracle err {err:.3e} <= {bound:.3e}",
                  flush=True)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    s = CONFIGS[5]
    assert gq.gqe_workspace_bytes(gq.shape_from(s)) > gq.GQE_NOALLOC_SCRATCH_BYTES
    x = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gq.GqeError) as e:
        gq.gqe_attn_fwd_noalloc(gq.shape_from(s), x, x, None, x, x, x, x, x, x)
    assert e.value.code == -7


def test_noalloc_graph_replays_match_eager():
    """The entry point's callers include HIP-graph capture: capture one
    gqe_attn_fwd_noalloc call, replay it three times with an eager call on
    another shape in between (which overwrites the shared scratch), and check
    every replay bit for bit against the workspace form."""
    s, seed = CASES[1][1], 5
    other, oseed = CASES[2][1], 6
    dv = H.to_device(make_inputs(s, seed=seed))
    dvo = H.to_device(make_inputs(other, seed=oseed))
    ref = H.alloc_outputs(s)
    H.run_gqe(s, dv, ref)
    got = H.alloc_outputs(s)
    oth = H.alloc_outputs(other)

    def call():
        gq.gqe_attn_fwd_noalloc(gq.shape_from(s), dv["x"], dv["Wr"], dv["br"], dv["Wq"], dv["Wk"], dv["Wv"],
                                dv["Wq_sh"], dv["Wo"], got["out"], got["idx"], got["w"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                       # first call on the device sets the scratch up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for r in range(3):
        for t in got.values():
            t.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in ("out", "idx", "w"):
            assert torch.equal(got[key], ref[key]), (r, key)
        gq.gqe_attn_fwd_noalloc(gq.shape_from(other), dvo["x"], dvo["Wr"], dvo["br"], dvo["Wq"], dvo["Wk"],
                                dvo["Wv"], dvo["Wq_sh"], dvo["Wo"], oth["out"], oth["idx"], oth["w"])
        torch.cuda.synchronize()
        print(f"[noalloc graph] replay {r} bit-identical to the workspace form", flush=True)
