"""The C ABI of libgqe.so on the CPU: it loads without a GPU, exports every
function include/gqe.h declares, and reports every validation status code
before any HIP call (host addresses below are never dereferenced)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import sparse_moe_attention_amd as gq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqe.h")

A = 0x10000          # a 16-byte aligned host address (never touched)
BAD = 0x10008        # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gq[ae]_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return gq.load()


def shape(**kw):
    base = dict(B=1, T=128, D=128, G=2, M=2, k=1, d_h=32, shared_kv_group=0, dtype=gq.GQE_BF16)
    base.update(kw)
    return gq.GqeShape(**base)


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) >= {"gqe_workspace_bytes", "gqe_route", "gqe_attn_fwd_routed", "gqe_attn_fwd",
                          "gqa_workspace_bytes", "gqa_attn_fwd", "gqe_status_str"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in gq.STATUS.items():
        assert gq.gqe_status_str(code).startswith(name)
    assert "unknown" in gq.gqe_status_str(-99)


@pytest.mark.parametrize("kw,code", [
    (dict(k=3), -2), (dict(k=0), -2), (dict(B=0), -2), (dict(T=0), -2), (dict(G=0), -2),
    (dict(shared_kv_group=2), -2), (dict(shared_kv_group=-1), -2),
    (dict(d_h=48), -3), (dict(D=100), -3), (dict(dtype=7), -3), (dict(M=65, k=1), -3),
    (dict(G=17, M=16), -3), (dict(B=1 << 20, T=1 << 20), -2), (dict(variant=4), -3), (dict(variant=-1), -3),
])
def test_shape_errors(lib, kw, code):
    s = shape(**kw)
    assert lib.gqe_workspace_bytes(ctypes.byref(s)) == 0
    rc = lib.gqe_attn_fwd(ctypes.byref(s), A, A, None, A, A, A, A, A, A, None, None, A, 1 << 40, None)
    assert rc == code
    rc = lib.gqe_route(ctypes.byref(s), A, A, None, A, A, None, None, A, 1 << 40, None)
    assert rc == code


def test_null_shape(lib):
    assert lib.gqe_workspace_bytes(None) == 0
    assert lib.gqe_attn_fwd(None, A, A, None, A, A, A, A, A, A, None, None, A, 1 << 40, None) == -1


def test_null_pointers(lib):
    s = shape()
    big = 1 << 40
    assert lib.gqe_attn_fwd(ctypes.byref(s), None, A, None, A, A, A, A, A, A, None, None, A, big, None) == -1
    assert lib.gqe_attn_fwd(ctypes.byref(s), A, A, None, A, A, A, A, A, None, None, None, A, big, None) == -1
    assert lib.gqe_route(ctypes.byref(s), A, A, None, None, A, None, None, A, big, None) == -1
    assert lib.gqe_attn_fwd_routed(ctypes.byref(s), A, A, A, A, A, A, None, A, A, None, A, big, None) == -1
    assert lib.gqa_attn_fwd(1, 128, 128, 4, 2, 32, 0, A, A, A, A, A, None, A, big, None) == -1


def test_alignment(lib):
    s = shape()
    big = 1 << 40
    assert lib.gqe_attn_fwd(ctypes.byref(s), BAD, A, None, A, A, A, A, A, A, None, None, A, big, None) == -5
    assert lib.gqe_attn_fwd(ctypes.byref(s), A, A, BAD, A, A, A, A, A, A, None, None, A, big, None) == -5
    assert lib.gqe_route(ctypes.byref(s), A, A, None, A, A, BAD, None, A, big, None) == -5
    assert lib.gqe_attn_fwd_routed(ctypes.byref(s), A, A, A, A, A, A, A, A, A, BAD, A, big, None) == -5
    assert lib.gqa_attn_fwd(1, 128, 128, 4, 2, 32, 0, A, A, A, A, A, A, BAD, big, None) == -5


def test_workspace_too_small(lib):
    s = shape()
    need = lib.gqe_workspace_bytes(ctypes.byref(s))
    assert need > 0
    assert lib.gqe_attn_fwd(ctypes.byref(s), A, A, None, A, A, A, A, A, A, None, None, A, need - 1, None) == -4
    assert lib.gqe_route(ctypes.byref(s), A, A, None, A, A, None, None, A, need - 1, None) == -4
    assert lib.gqe_attn_fwd_routed(ctypes.byref(s), A, A, A, A, A, A, A, A, A, None, A, need - 1, None) == -4
    g = lib.gqa_workspace_bytes(1, 128, 128, 4, 2, 32, 0)
    assert g > 0
    assert lib.gqa_attn_fwd(1, 128, 128, 4, 2, 32, 0, A, A, A, A, A, A, A, g - 1, None) == -4


def test_gqa_shape_errors(lib):
    assert lib.gqa_workspace_bytes(1, 128, 128, 5, 2, 32, 0) == 0          # Hq not a multiple of G
    assert lib.gqa_attn_fwd(1, 128, 128, 5, 2, 32, 0, A, A, A, A, A, A, A, 1 << 40, None) == -2
    assert lib.gqa_attn_fwd(1, 128, 128, 4, 2, 48, 0, A, A, A, A, A, A, A, 1 << 40, None) == -3
    assert lib.gqa_workspace_bytes(1, 128, 128, 512, 2, 32, 0) == 0        # Hq > 256


def test_workspace_monotone_in_tokens(lib):
    prev = 0
    for T in (1, 7, 64, 65, 128, 1000, 4096, 32768):
        s = shape(T=T, D=1024, G=8, M=2, d_h=64)
        n = lib.gqe_workspace_bytes(ctypes.byref(s))
        assert n > prev
        prev = n
    # the extreme-context layer fits comfortably in one MI355X's 288 GB
    s = shape(T=1 << 20, D=1024, G=8, M=2, d_h=64)
    assert lib.gqe_workspace_bytes(ctypes.byref(s)) < 8 << 30


def _bwd(lib, s, ws_bytes=1 << 40, coef=0.0, **over):
    """gqe_attn_bwd with every pointer A unless overridden by name."""
    names = ["x", "Wr", "Wq", "Wk", "Wv", "Wq_sh", "Wo", "dout", "dx", "dWr", "dbr", "dWq", "dWk", "dWv",
             "dWq_sh", "dWo", "aux_loss", "ws"]
    p = {n: A for n in names}
    p.update(over)
    return lib.gqe_attn_bwd(ctypes.byref(s), p["x"], p["Wr"], p["Wq"], p["Wk"], p["Wv"], p["Wq_sh"], p["Wo"],
                            p["dout"], ctypes.c_float(coef), p["dx"], p["dWr"], p["dbr"], p["dWq"], p["dWk"],
                            p["dWv"], p["dWq_sh"], p["dWo"], p["aux_loss"], p["ws"], ws_bytes, None)


def test_train_entry_points_validate(lib):
    s = shape()
    need = lib.gqe_train_workspace_bytes(ctypes.byref(s))
    assert need > lib.gqe_workspace_bytes(ctypes.byref(s)) > 0
    fwd = lambda sh, n: lib.gqe_attn_fwd_train(ctypes.byref(sh), A, A, None, A, A, A, A, A, A, None, None, A, n,
                                               None)
    assert fwd(s, need - 1) == -4
    assert _bwd(lib, s, need - 1) == -4
    # the training pair covers the full layer in bf16 only
    for kw in (dict(dtype=gq.GQE_F32), dict(variant=gq.GQE_HARD_CONCAT), dict(variant=gq.GQE_NO_SHARED),
               dict(variant=gq.GQE_WEIGHTED_CONCAT)):
        u = shape(**kw)
        assert lib.gqe_train_workspace_bytes(ctypes.byref(u)) == 0
        assert fwd(u, 1 << 40) == -3
        assert _bwd(lib, u) == -3
    assert _bwd(lib, shape(k=3)) == -2
    assert _bwd(lib, s, dx=None) == -1
    assert _bwd(lib, s, dout=None) == -1
    assert _bwd(lib, s, dWo=None) == -1
    assert _bwd(lib, s, dWq=BAD) == -5
    assert _bwd(lib, s, dbr=BAD) == -5
    assert _bwd(lib, s, coef=float("nan")) == -2
    assert _bwd(lib, s, coef=float("inf")) == -2


def test_train_workspace_sizes(lib):
    prev = 0
    for T in (1, 77, 256, 257, 4096, 32768):
        s = shape(T=T, D=1024, G=8, M=2, d_h=64)
        n = lib.gqe_train_workspace_bytes(ctypes.byref(s))
        assert n > prev
        prev = n
    s = shape(T=1 << 20, D=1024, G=8, M=2, d_h=64)
    assert lib.gqe_train_workspace_bytes(ctypes.byref(s)) < 64 << 30


def test_decode_entry_point_validates(lib):
    s = shape(T=256)
    need = lib.gqe_decode_workspace_bytes(ctypes.byref(s))
    assert need > 0
    call = lambda sh, n, **o: lib.gqe_decode_step(
        ctypes.byref(sh), o.get("pos", A), o.get("x", A), A, None, A, A, A, A, A, o.get("kc", A), A, o.get("out", A),
        None, None, A, n, None)
    assert call(s, need - 1) == -4
    assert call(s, need, pos=None) == -1
    assert call(s, need, kc=None) == -1
    assert call(s, need, out=BAD) == -5
    assert call(shape(T=250), 1 << 40) == -2                    # capacity not a multiple of 32
    assert lib.gqe_decode_workspace_bytes(ctypes.byref(shape(T=250))) == 0
    for kw in (dict(dtype=gq.GQE_F32), dict(variant=gq.GQE_NO_SHARED)):
        assert call(shape(T=256, **kw), 1 << 40) == -3


def test_decode_shape_errors(lib):
    """The decode step needs T a multiple of 32 and one group's values
    (d_h * B * T * 2 bytes) under 4 GiB; both are refused before any HIP call."""
    ok = shape(B=16, T=1 << 20, D=1024, G=8, M=2, d_h=64)          # 2 GiB of values per group
    assert lib.gqe_decode_workspace_bytes(ctypes.byref(ok)) > 0
    for bad in (shape(T=112), shape(B=32, T=1 << 20, D=1024, G=8, M=2, d_h=64)):
        assert lib.gqe_decode_workspace_bytes(ctypes.byref(bad)) == 0
        rc = lib.gqe_decode_step(ctypes.byref(bad), A, A, A, None, A, A, A, A, A, A, A, A, None, None, A,
                                 1 << 40, None)
        assert rc == -2


def test_noalloc_entry_point_validates(lib):
    """gqe_attn_fwd_noalloc: the checks of gqe_attn_fwd, plus the static
    scratch bound (GQE_ERR_SCRATCH), all before any HIP call."""
    s = shape()

    def call(sh, **o):
        return lib.gqe_attn_fwd_noalloc(ctypes.byref(sh) if sh is not None else None, o.get("x", A), A,
                                        o.get("br"), A, A, A, A, A, o.get("out", A), o.get("idx"), o.get("w"), None)

    assert call(None) == -1
    assert call(shape(k=3)) == -2
    assert call(shape(d_h=48)) == -3
    assert call(s, x=None) == -1
    assert call(s, out=None) == -1
    assert call(s, out=BAD) == -5
    assert call(s, br=BAD) == -5
    assert call(s, idx=BAD) == -5
    huge = shape(T=1 << 20, D=1024, G=8, M=2, d_h=64)
    assert lib.gqe_workspace_bytes(ctypes.byref(huge)) > gq.GQE_NOALLOC_SCRATCH_BYTES
    assert call(huge) == -7
    assert gq.gqe_status_str(-7).startswith("GQE_ERR_SCRATCH")
    # the 32K-token layer and the larger-pool layer fit the scratch
    for sh in (shape(T=32768, D=1024, G=8, M=2, d_h=64), shape(B=2, T=16384, D=2048, G=8, M=4, k=2, d_h=64)):
        assert 0 < lib.gqe_workspace_bytes(ctypes.byref(sh)) <= gq.GQE_NOALLOC_SCRATCH_BYTES


def test_train_routed_entry_point_validates(lib):
    s = shape()
    need = lib.gqe_train_workspace_bytes(ctypes.byref(s))

    def call(sh, n=need, **o):
        return lib.gqe_attn_fwd_train_routed(ctypes.byref(sh) if sh is not None else None, A, A, None, A, A, A, A,
                                             A, o.get("idx", A), o.get("out", A), o.get("w"), A, n, None)

    assert call(None) == -1
    assert call(s, idx=None) == -1
    assert call(s, out=None) == -1
    assert call(s, idx=BAD) == -5
    assert call(s, w=BAD) == -5
    assert call(s, n=need - 1) == -4
    assert call(shape(k=3)) == -2
    assert call(shape(dtype=gq.GQE_F32), n=1 << 40) == -3


def test_mfma_probe_validates(lib):
    """gqe_mfma_probe rejects a null or misaligned output and out-of-range
    sizes before it launches anything."""
    assert lib.gqe_mfma_probe(1024, 10, None, None) == -1
    assert lib.gqe_mfma_probe(0, 10, A, None) == -2
    assert lib.gqe_mfma_probe((1 << 20) + 1, 10, A, None) == -2
    assert lib.gqe_mfma_probe(1024, 0, A, None) == -2
    assert lib.gqe_mfma_probe(1024, 10, BAD, None) == -5
