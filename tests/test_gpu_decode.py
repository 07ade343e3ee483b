"""GPU parity of gqe_decode_step (one new token per sequence over a dense KV
cache) against the fp64 decode oracle, through the C ABI.

The caches hold seeded bf16 keys and values below each sequence's position
and NaN from there on (positions past the cache length must never be read as
data). Checked: the layer output on every sequence (the forward's bar,
max|err| <= 1e-2 max|ref| + 1e-3), the routing (bit-exact), the appended key
row and value column (bf16 of the oracle's projections, same bar), and that
nothing else in either cache changed (bit-exact). Shapes: an empty prefix, a
full cache, ragged positions, k = 2 with the shared head on group 1, and 17
heads on one group (two passes of 16).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.gqe_decode as gd
import sparse_moe_attention_amd as gq
from tests import harness as H
from workloads import Shape, make_inputs

pytestmark = pytest.mark.gpu

# (shape with T = cache capacity, positions)
CASES = {
    "ragged_k2_shared1": (Shape(B=3, T=256, D=128, G=3, M=3, k=2, d=32, router_bias=True, shared_kv_group=1),
                          [0, 100, 255]),
    "long_cache": (Shape(B=2, T=2048, D=256, G=8, M=2, k=1, d=64), [1500, 2047]),
    "short": (Shape(B=4, T=64, D=64, G=2, M=2, k=1, d=64), [5, 0, 63, 31]),
    "wide_pool": (Shape(B=2, T=1088, D=128, G=4, M=16, k=4, d=32, router_bias=True), [1087, 1024]),
    "seventeen_heads": (Shape(B=2, T=320, D=64, G=2, M=20, k=16, d=32), [300, 17]),
    "max_pool_256_experts": (Shape(B=2, T=192, D=64, G=4, M=64, k=3, d=32, router_bias=True, shared_kv_group=3),
                             [100, 191]),
    "many_sequences": (Shape(B=33, T=64, D=64, G=2, M=2, k=1, d=64), [(7 * b) % 64 for b in range(33)]),
    # T = 32 mod 64 at d = 64: a sequence's last 64-key step reaches past the cache end (those K rows
    # read as zeros, those V^T columns as the next row's first keys or zeros), in the last sequence too
    "tail_past_cache_end": (Shape(B=3, T=96, D=128, G=2, M=3, k=2, d=64, router_bias=True, shared_kv_group=1),
                            [95, 70, 64]),
    "two_chunks_tail": (Shape(B=2, T=2080, D=64, G=2, M=2, k=1, d=64), [2050, 2079]),
    # chunk lengths: the launch takes 512, 256, 128 or 64 keys per wave, the largest that still
    # gives 1024 workgroups (B * G * chunks); these take 128, 256 and 512 with ragged positions
    # (the shorter caches above take 64)
    "chunks_of_512_keys": (Shape(B=4, T=16384, D=128, G=8, M=2, k=1, d=64), [16383, 9000, 1025, 4096]),
    "chunks_of_1024_keys": (Shape(B=8, T=16384, D=64, G=8, M=2, k=1, d=64, router_bias=True),
                            [16383, 0, 2047, 2048, 12345, 8191, 100, 16000]),
    "chunks_of_2048_keys": (Shape(B=16, T=16384, D=64, G=8, M=2, k=1, d=64),
                            [16383, 0, 2047, 2048, 12345, 8191, 100, 16000, 1, 4095, 4096, 6000, 10000, 14000,
                             15000, 16382]),
    # more than 64 new tokens: the token projections take the tiled GEMM instead of the skinny one
    "seventy_sequences": (Shape(B=70, T=32, D=64, G=2, M=2, k=1, d=32, shared_kv_group=1),
                          [(5 * b) % 32 for b in range(70)]),
}


def make_caches(s: Shape, pos, seed: int):
    """bf16 caches in the library's layouts: keys [G][B][T][d], values
    transposed [G][d][B*T]; N(0, 1) below pos[b], NaN from pos[b] on."""
    gen = torch.Generator().manual_seed(seed)
    k = torch.randn(s.G, s.B, s.T, s.d, generator=gen).to(torch.bfloat16)
    v = torch.randn(s.G, s.B, s.T, s.d, generator=gen).to(torch.bfloat16)
    for b, p in enumerate(pos):
        k[:, b, p:] = float("nan")
        v[:, b, p:] = float("nan")
    vt = v.permute(0, 3, 1, 2).reshape(s.G, s.d, s.B * s.T).contiguous()
    return k, v, vt


@pytest.mark.parametrize("name", sorted(CASES))
def test_decode_parity(name):
    s, pos = CASES[name]
    print(f"[decode case {name}] {s} pos={pos}", flush=True)
    inp = make_inputs(Shape(B=s.B, T=1, D=s.D, G=s.G, M=s.M, k=s.k, d=s.d, router_bias=s.router_bias,
                            shared_kv_group=s.shared_kv_group), seed=500 + len(name))
    kc, vc, vtc = make_caches(s, pos, seed=600 + len(name))
    dv = H.to_device(inp)
    kd, vtd = kc.cuda(), vtc.cuda()
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    sh = gq.shape_from(s)
    ws = torch.empty(gq.gqe_decode_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    out = torch.empty(s.B, s.D, dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(s.B, s.G, s.k, dtype=torch.int32, device="cuda")
    w = torch.empty(s.B, s.G, s.k, dtype=torch.float32, device="cuda")
    gq.gqe_decode_step(sh, posd, dv["x"], dv["Wr"], dv["br"], dv["Wq"], dv["Wk"], dv["Wv"], dv["Wq_sh"], dv["Wo"],
                       kd, vtd, out, ws, idx, w)
    torch.cuda.synchronize()

    f = H.f64_inputs(inp)
    k64 = kc.float().numpy().astype(np.float64).transpose(1, 0, 2, 3)       # [B, G, T, d]
    v64 = vc.float().numpy().astype(np.float64).transpose(1, 0, 2, 3)
    ref = gd.gqe_decode(f, k64, v64, pos, s.G, s.M, s.k, s.d, shared_kv_group=s.shared_kv_group)
    assert (idx.cpu().numpy() == ref["idx"]).all(), (name, "routing")
    err, bound = H.out_error(H.np32(out), ref["out"])
    assert np.isfinite(H.np32(out)).all() and err <= bound, (name, "out", err, bound)

    # the appended row / column, and nothing else changed
    k_after = kd.cpu()
    v_after = vtd.cpu().reshape(s.G, s.d, s.B, s.T).permute(0, 2, 3, 1)    # [G, B, T, d]
    for b, p in enumerate(pos):
        err, bound = H.out_error(k_after[:, b, p].float().numpy(), ref["K_new"][b])
        assert err <= bound, (name, "appended key", b, err, bound)
        err, bound = H.out_error(v_after[:, b, p].float().numpy(), ref["V_new"][b])
        assert err <= bound, (name, "appended value", b, err, bound)
        k_after[:, b, p] = kc[:, b, p]
        v_after[:, b, p] = vc[:, b, p]
    assert torch.equal(k_after.view(torch.int16), kc.view(torch.int16)), (name, "key cache changed elsewhere")
    assert torch.equal(v_after.contiguous().view(torch.int16), vc.view(torch.int16)), (name, "value cache changed")


def test_decode_parity_at_bench_workload():
    """The launch the benchmark times: 16 sequences x 32767 cached positions
    of the 32K-token layer (B1 T32768 D1024 G8 M2 k1 d64 per sequence), new
    token at position 32767, the benchmark's seeded inputs. All 16 sequences
    run; three of them are checked against the oracle (the sequences are
    independent). Position 32767 holds NaN before the call: it is written,
    never read."""
    import dataclasses
    B, T = 16, 32768
    s = Shape(B=B, T=T, D=1024, G=8, M=2, k=1, d=64)
    print(f"[decode bench workload] {s}", flush=True)
    tok = make_inputs(dataclasses.replace(s, T=1), seed=4000)
    dv = H.to_device(tok)
    gen = torch.Generator(device="cuda").manual_seed(4001)
    kd = torch.randn(s.G, B, T, s.d, device="cuda", generator=gen).to(torch.bfloat16)
    vtd = torch.randn(s.G, s.d, B * T, device="cuda", generator=gen).to(torch.bfloat16)
    kd[:, :, T - 1] = float("nan")
    vtd.view(s.G, s.d, B, T)[:, :, :, T - 1] = float("nan")
    pos = [T - 1] * B
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    sh = gq.shape_from(s)
    ws = torch.empty(gq.gqe_decode_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, s.D, dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(B, s.G, s.k, dtype=torch.int32, device="cuda")
    w = torch.empty(B, s.G, s.k, dtype=torch.float32, device="cuda")
    gq.gqe_decode_step(sh, posd, dv["x"], dv["Wr"], dv["br"], dv["Wq"], dv["Wk"], dv["Wv"], dv["Wq_sh"], dv["Wo"],
                       kd, vtd, out, ws, idx, w)
    torch.cuda.synchronize()

    sel = [0, 9, 15]
    f = H.f64_inputs(tok)
    f_sel = dict(f, x=f["x"][sel])
    k64 = kd[:, sel].float().cpu().numpy().astype(np.float64).transpose(1, 0, 2, 3)   # [3, G, T, d]
    v64 = vtd.view(s.G, s.d, B, T)[:, :, sel].float().cpu().numpy().astype(np.float64).transpose(2, 0, 3, 1)
    ref = gd.gqe_decode(f_sel, k64, v64, [T - 1] * len(sel), s.G, s.M, s.k, s.d)
    assert (idx.cpu().numpy()[sel] == ref["idx"]).all(), "routing"
    got = H.np32(out)[sel]
    err, bound = H.out_error(got, ref["out"])
    assert np.isfinite(got).all() and err <= bound, ("out", err, bound)
    # the appended key row and value column of the checked sequences
    for i, b in enumerate(sel):
        err, bound = H.out_error(H.np32(kd[:, b, T - 1]), ref["K_new"][i])
        assert err <= bound, ("appended key", b, err, bound)
        err, bound = H.out_error(H.np32(vtd.view(s.G, s.d, B, T)[:, :, b, T - 1]), ref["V_new"][i])
        assert err <= bound, ("appended value", b, err, bound)
    assert torch.isfinite(out.float()).all()


def test_decode_positions_out_of_range():
    """Entries of pos outside [0, T) are documented to leave their sequence's
    cache untouched (no read, no write, outputs unspecified); the other
    sequences of the same call still match the oracle."""
    s = Shape(B=4, T=128, D=64, G=2, M=2, k=1, d=32, shared_kv_group=1)
    pos = [17, -1, 128, 127]
    valid = [0, 3]
    print(f"[decode out-of-range positions] {s} pos={pos}", flush=True)
    inp = make_inputs(Shape(B=s.B, T=1, D=s.D, G=s.G, M=s.M, k=s.k, d=s.d, shared_kv_group=s.shared_kv_group),
                      seed=901)
    kc, vc, vtc = make_caches(s, [p if 0 <= p < s.T else s.T for p in pos], seed=902)
    dv = H.to_device(inp)
    kd, vtd = kc.cuda(), vtc.cuda()
    posd = torch.tensor(pos, dtype=torch.int32, device="cuda")
    sh = gq.shape_from(s)
    ws = torch.empty(gq.gqe_decode_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    out = torch.empty(s.B, s.D, dtype=torch.bfloat16, device="cuda")
    gq.gqe_decode_step(sh, posd, dv["x"], dv["Wr"], dv["br"], dv["Wq"], dv["Wk"], dv["Wv"], dv["Wq_sh"], dv["Wo"],
                       kd, vtd, out, ws)
    torch.cuda.synchronize()
    f = H.f64_inputs(inp)
    f_sel = dict(f, x=f["x"][valid])
    k64 = kc[:, valid].float().numpy().astype(np.float64).transpose(1, 0, 2, 3)
    v64 = vc[:, valid].float().numpy().astype(np.float64).transpose(1, 0, 2, 3)
    ref = gd.gqe_decode(f_sel, k64, v64, [pos[b] for b in valid], s.G, s.M, s.k, s.d,
                        shared_kv_group=s.shared_kv_group)
    got = H.np32(out)[valid]
    err, bound = H.out_error(got, ref["out"])
    assert np.isfinite(got).all() and err <= bound, ("out", err, bound)
    # the caches of the out-of-range sequences are bit-identical
    k_after = kd.cpu()
    v_after = vtd.cpu().reshape(s.G, s.d, s.B, s.T)
    v_before = vtc.reshape(s.G, s.d, s.B, s.T)
    for b in (1, 2):
        assert torch.equal(k_after[:, b].view(torch.int16), kc[:, b].view(torch.int16)), ("key cache written", b)
        assert torch.equal(v_after[:, :, b].contiguous().view(torch.int16),
                           v_before[:, :, b].contiguous().view(torch.int16)), ("value cache written", b)
