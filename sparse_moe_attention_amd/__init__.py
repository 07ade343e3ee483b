"""Python binding of libgqe.so, the gfx950 GQE attention forward library.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. Torch supplies device memory and the current stream. If libgqe.so is
missing the import succeeds but every call raises; there is no fallback.

Entry points (same names as the C ABI in include/gqe.h):
    gqe_workspace_bytes(shape)
    gqe_route(shape, x, Wr, br, idx, w, logits=None, counts=None, ws=None)
    gqe_attn_fwd_routed(shape, x, Wq, Wk, Wv, Wq_sh, Wo, idx, w, out, slots_out=None, ws=None)
    gqe_attn_fwd(shape, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, out, idx_out=None, w_out=None, ws=None)
    gqe_attn_fwd_noalloc(shape, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, out, idx_out=None, w_out=None)
    gqa_workspace_bytes(B, T, D, Hq, G, d_h, dtype)
    gqa_attn_fwd(B, T, D, Hq, G, d_h, dtype, x, Wq, Wk, Wv, Wo, out, ws=None)
    gqe_train_workspace_bytes(shape)
    gqe_attn_fwd_train(shape, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, out, ws, idx_out=None, w_out=None)
    gqe_attn_fwd_train_routed(shape, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, idx, out, ws, w_out=None)
    gqe_attn_bwd(shape, x, Wr, Wq, Wk, Wv, Wq_sh, Wo, dout, aux_coef, grads, ws, dbr=None, aux_loss=None)
    gqe_decode_workspace_bytes(shape)
    gqe_decode_step(shape, pos, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, k_cache, vt_cache, out, ws, idx_out=None, w_out=None)
    gqe_mfma_probe(workgroups, iters, out)
    gqe_status_str(code)
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# GQE_LIB_PATH selects another build of the same library (the host-sanitizer
# build the ABI tests also run against); the default is the in-tree libgqe.so.
LIB_PATH = os.environ.get("GQE_LIB_PATH") or os.path.join(HERE, "libgqe.so")

GQE_BF16, GQE_F32 = 0, 1
# Merge variants (gqe_variant): the layer and the pages' three ablations.
GQE_FULL, GQE_WEIGHTED_CONCAT, GQE_HARD_CONCAT, GQE_NO_SHARED = 0, 1, 2, 3
VARIANT_CODES = {"full": GQE_FULL, "weighted_concat": GQE_WEIGHTED_CONCAT, "hard_concat": GQE_HARD_CONCAT,
                 "no_shared": GQE_NO_SHARED}
GQE_N_STAGES, GQA_N_STAGES = 8, 3
GQE_NOALLOC_SCRATCH_BYTES = 256 << 20     # static scratch of gqe_attn_fwd_noalloc (include/gqe.h)
GQE_STAGE_NAMES = ("proj_kv_qsh_router", "route", "scan", "scatter", "grouped_q", "attention",
                   "weighted_slot", "out_proj")
GQA_STAGE_NAMES = ("proj_qkv", "attention", "out_proj")
GQE_BWD_N_STAGES = 7
GQE_BWD_STAGE_NAMES = ("layouts", "slot_grads_dWo", "prep_router", "attn_dkdv", "attn_dq", "dx",
                       "dW")
GQE_DECODE_N_STAGES = 3
GQE_DECODE_STAGE_NAMES = ("token_side_and_append", "attention_over_cache", "merge_and_out_proj")
# Gradient outputs of gqe_attn_bwd, in argument order (fp32, shaped like the weights).
BWD_GRADS = ("dx", "dWr", "dWq", "dWk", "dWv", "dWq_sh", "dWo")

STATUS = {
    0: "GQE_OK", -1: "GQE_ERR_NULL", -2: "GQE_ERR_SHAPE", -3: "GQE_ERR_UNSUPPORTED",
    -4: "GQE_ERR_WORKSPACE", -5: "GQE_ERR_ALIGN", -6: "GQE_ERR_HIP", -7: "GQE_ERR_SCRATCH",
}


class GqeShape(ctypes.Structure):
    """Mirror of the C struct gqe_shape."""
    _fields_ = [
        ("B", ctypes.c_int64), ("T", ctypes.c_int64), ("D", ctypes.c_int64),
        ("G", ctypes.c_int32), ("M", ctypes.c_int32), ("k", ctypes.c_int32),
        ("d_h", ctypes.c_int32), ("shared_kv_group", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("variant", ctypes.c_int32),
    ]


class GqeError(RuntimeError):
    def __init__(self, code: int, text: str):
        super().__init__(text)
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    """Load libgqe.so (once) and declare its signatures. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m sparse_moe_attention_amd.build` "
            "(the library has no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, S, I32, I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    SH = ctypes.POINTER(GqeShape)
    lib.gqe_workspace_bytes.argtypes = [SH]
    lib.gqe_workspace_bytes.restype = S
    lib.gqe_route.argtypes = [SH, P, P, P, P, P, P, P, P, S, P]
    lib.gqe_route.restype = ctypes.c_int
    lib.gqe_attn_fwd_routed.argtypes = [SH, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.gqe_attn_fwd_routed.restype = ctypes.c_int
    lib.gqe_attn_fwd.argtypes = [SH, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.gqe_attn_fwd.restype = ctypes.c_int
    lib.gqe_attn_fwd_noalloc.argtypes = [SH, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.gqe_attn_fwd_noalloc.restype = ctypes.c_int
    lib.gqa_workspace_bytes.argtypes = [I64, I64, I64, I32, I32, I32, I32]
    lib.gqa_workspace_bytes.restype = S
    lib.gqa_attn_fwd.argtypes = [I64, I64, I64, I32, I32, I32, I32, P, P, P, P, P, P, P, S, P]
    lib.gqa_attn_fwd.restype = ctypes.c_int
    lib.gqe_attn_fwd_timed.argtypes = [SH, P, P, P, P, P, P, P, P, P, P, P, P, S, P, P]
    lib.gqe_attn_fwd_timed.restype = ctypes.c_int
    lib.gqa_attn_fwd_timed.argtypes = [I64, I64, I64, I32, I32, I32, I32, P, P, P, P, P, P, P, S, P, P]
    lib.gqa_attn_fwd_timed.restype = ctypes.c_int
    lib.gqe_train_workspace_bytes.argtypes = [SH]
    lib.gqe_train_workspace_bytes.restype = S
    lib.gqe_attn_fwd_train.argtypes = [SH, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.gqe_attn_fwd_train_routed.argtypes = [SH, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.gqe_attn_fwd_train_routed.restype = ctypes.c_int
    lib.gqe_attn_fwd_train.restype = ctypes.c_int
    bwd = [SH, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.gqe_attn_bwd.argtypes = bwd
    lib.gqe_attn_bwd.restype = ctypes.c_int
    lib.gqe_attn_bwd_timed.argtypes = bwd + [P]
    lib.gqe_attn_bwd_timed.restype = ctypes.c_int
    lib.gqe_decode_workspace_bytes.argtypes = [SH]
    lib.gqe_decode_workspace_bytes.restype = S
    dec = [SH, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.gqe_decode_step.argtypes = dec
    lib.gqe_decode_step.restype = ctypes.c_int
    lib.gqe_decode_step_timed.argtypes = dec + [P]
    lib.gqe_decode_step_timed.restype = ctypes.c_int
    lib.gqe_mfma_probe.argtypes = [I64, I32, P, P]
    lib.gqe_mfma_probe.restype = ctypes.c_int
    lib.gqe_status_str.argtypes = [ctypes.c_int]
    lib.gqe_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def gqe_status_str(code: int) -> str:
    return load().gqe_status_str(code).decode()


def _check(code: int) -> None:
    if code != 0:
        raise GqeError(code, gqe_status_str(code))


def make_shape(B, T, D, G, M, k, d_h, shared_kv_group=0, dtype=GQE_BF16, variant=GQE_FULL) -> GqeShape:
    return GqeShape(B, T, D, G, M, k, d_h, shared_kv_group, dtype, variant)


def shape_from(s) -> GqeShape:
    """GqeShape from any object with B, T, D, G, M, k, d (and optional dtype
    "bf16"/"f32", shared_kv_group) attributes."""
    dt = GQE_F32 if getattr(s, "dtype", "bf16") in ("f32", GQE_F32) else GQE_BF16
    v = getattr(s, "variant", GQE_FULL)
    v = VARIANT_CODES[v] if isinstance(v, str) else int(v)
    return make_shape(s.B, s.T, s.D, s.G, s.M, s.k, s.d, getattr(s, "shared_kv_group", 0), dt, v)


def _ptr(t):
    """Device address of a torch tensor (None -> NULL). Refuses host tensors
    and non-contiguous views; the library does the remaining checks."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libgqe takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libgqe takes contiguous tensors")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _workspace(nbytes: int, like):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=like.device)


def gqe_workspace_bytes(shape: GqeShape) -> int:
    return int(load().gqe_workspace_bytes(ctypes.byref(shape)))


def gqe_route(shape, x, Wr, br, idx, w, logits=None, counts=None, ws=None, stream=None):
    lib = load()
    if ws is None:
        ws = _workspace(gqe_workspace_bytes(shape), x)
    _check(lib.gqe_route(ctypes.byref(shape), _ptr(x), _ptr(Wr), _ptr(br), _ptr(idx), _ptr(w),
                         _ptr(logits), _ptr(counts), _ptr(ws), ws.numel(), _stream(stream)))


def gqe_attn_fwd_routed(shape, x, Wq, Wk, Wv, Wq_sh, Wo, idx, w, out, slots_out=None, ws=None, stream=None):
    lib = load()
    if ws is None:
        ws = _workspace(gqe_workspace_bytes(shape), x)
    _check(lib.gqe_attn_fwd_routed(ctypes.byref(shape), _ptr(x), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wq_sh),
                                   _ptr(Wo), _ptr(idx), _ptr(w), _ptr(out), _ptr(slots_out), _ptr(ws),
                                   ws.numel(), _stream(stream)))


def gqe_attn_fwd(shape, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, out, idx_out=None, w_out=None, ws=None, stream=None):
    lib = load()
    if ws is None:
        ws = _workspace(gqe_workspace_bytes(shape), x)
    _check(lib.gqe_attn_fwd(ctypes.byref(shape), _ptr(x), _ptr(Wr), _ptr(br), _ptr(Wq), _ptr(Wk), _ptr(Wv),
                            _ptr(Wq_sh), _ptr(Wo), _ptr(out), _ptr(idx_out), _ptr(w_out), _ptr(ws),
                            ws.numel(), _stream(stream)))


def gqe_attn_fwd_noalloc(shape, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, out, idx_out=None, w_out=None, stream=None):
    """gqe_attn_fwd on the library's static device scratch (no workspace, no
    allocation); shapes needing more than GQE_NOALLOC_SCRATCH_BYTES raise."""
    _check(load().gqe_attn_fwd_noalloc(ctypes.byref(shape), _ptr(x), _ptr(Wr), _ptr(br), _ptr(Wq), _ptr(Wk),
                                       _ptr(Wv), _ptr(Wq_sh), _ptr(Wo), _ptr(out), _ptr(idx_out), _ptr(w_out),
                                       _stream(stream)))


def gqa_workspace_bytes(B, T, D, Hq, G, d_h, dtype=GQE_BF16) -> int:
    return int(load().gqa_workspace_bytes(B, T, D, Hq, G, d_h, dtype))


def gqa_attn_fwd(B, T, D, Hq, G, d_h, dtype, x, Wq, Wk, Wv, Wo, out, ws=None, stream=None):
    lib = load()
    if ws is None:
        ws = _workspace(gqa_workspace_bytes(B, T, D, Hq, G, d_h, dtype), x)
    _check(lib.gqa_attn_fwd(B, T, D, Hq, G, d_h, dtype, _ptr(x), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wo),
                            _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))


def event_array(events):
    """ctypes array of raw hipEvent_t handles from torch.cuda.Event objects
    (None entries stay NULL). Each event must have been recorded once."""
    arr = (ctypes.c_void_p * len(events))()
    for i, e in enumerate(events):
        arr[i] = None if e is None else e.cuda_event
    return arr


def gqe_attn_fwd_timed(shape, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, out, events, idx_out=None, w_out=None,
                       ws=None, stream=None):
    """gqe_attn_fwd plus a hipEvent record before every stage (events: a
    ctypes array from event_array, GQE_N_STAGES + 1 entries)."""
    lib = load()
    if ws is None:
        ws = _workspace(gqe_workspace_bytes(shape), x)
    _check(lib.gqe_attn_fwd_timed(ctypes.byref(shape), _ptr(x), _ptr(Wr), _ptr(br), _ptr(Wq), _ptr(Wk),
                                  _ptr(Wv), _ptr(Wq_sh), _ptr(Wo), _ptr(out), _ptr(idx_out), _ptr(w_out),
                                  _ptr(ws), ws.numel(), _stream(stream), events))


def gqa_attn_fwd_timed(B, T, D, Hq, G, d_h, dtype, x, Wq, Wk, Wv, Wo, out, events, ws=None, stream=None):
    lib = load()
    if ws is None:
        ws = _workspace(gqa_workspace_bytes(B, T, D, Hq, G, d_h, dtype), x)
    _check(lib.gqa_attn_fwd_timed(B, T, D, Hq, G, d_h, dtype, _ptr(x), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wo),
                                  _ptr(out), _ptr(ws), ws.numel(), _stream(stream), events))


def gqe_train_workspace_bytes(shape: GqeShape) -> int:
    """Workspace of the training pair gqe_attn_fwd_train / gqe_attn_bwd (0: unsupported shape)."""
    return int(load().gqe_train_workspace_bytes(ctypes.byref(shape)))


def gqe_attn_fwd_train(shape, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, out, ws, idx_out=None, w_out=None, stream=None):
    """The forward of gqe_attn_fwd that also leaves in ws what gqe_attn_bwd reads."""
    _check(load().gqe_attn_fwd_train(ctypes.byref(shape), _ptr(x), _ptr(Wr), _ptr(br), _ptr(Wq), _ptr(Wk),
                                     _ptr(Wv), _ptr(Wq_sh), _ptr(Wo), _ptr(out), _ptr(idx_out), _ptr(w_out),
                                     _ptr(ws), ws.numel(), _stream(stream)))


def gqe_attn_fwd_train_routed(shape, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, idx, out, ws, w_out=None, stream=None):
    """gqe_attn_fwd_train with the caller's picks idx [N, G, k] instead of the router's."""
    _check(load().gqe_attn_fwd_train_routed(ctypes.byref(shape), _ptr(x), _ptr(Wr), _ptr(br), _ptr(Wq), _ptr(Wk),
                                            _ptr(Wv), _ptr(Wq_sh), _ptr(Wo), _ptr(idx), _ptr(out), _ptr(w_out),
                                            _ptr(ws), ws.numel(), _stream(stream)))


def gqe_attn_bwd(shape, x, Wr, Wq, Wk, Wv, Wq_sh, Wo, dout, aux_coef, grads, ws, dbr=None, aux_loss=None,
                 stream=None, events=None):
    """Gradients of <dout, out> + aux loss, after gqe_attn_fwd_train on the same
    ws. grads: dict of fp32 device tensors named as BWD_GRADS; events: optional
    ctypes array (GQE_BWD_N_STAGES + 1 entries) recorded around the stages."""
    lib = load()
    args = [ctypes.byref(shape), _ptr(x), _ptr(Wr), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wq_sh), _ptr(Wo),
            _ptr(dout), ctypes.c_float(aux_coef), _ptr(grads["dx"]), _ptr(grads["dWr"]), _ptr(dbr),
            _ptr(grads["dWq"]), _ptr(grads["dWk"]), _ptr(grads["dWv"]), _ptr(grads["dWq_sh"]),
            _ptr(grads["dWo"]), _ptr(aux_loss), _ptr(ws), ws.numel(), _stream(stream)]
    if events is None:
        _check(lib.gqe_attn_bwd(*args))
    else:
        _check(lib.gqe_attn_bwd_timed(*args, events))


def gqe_decode_workspace_bytes(shape: GqeShape) -> int:
    """Workspace of gqe_decode_step (shape.T = cache capacity; 0: unsupported)."""
    return int(load().gqe_decode_workspace_bytes(ctypes.byref(shape)))


def gqe_decode_step(shape, pos, x, Wr, br, Wq, Wk, Wv, Wq_sh, Wo, k_cache, vt_cache, out, ws, idx_out=None,
                    w_out=None, stream=None, events=None):
    """One new token per sequence over the dense KV cache (appends the token's
    key and value at pos[b]); events: optional ctypes array of
    GQE_DECODE_N_STAGES + 1 entries."""
    lib = load()
    args = [ctypes.byref(shape), _ptr(pos), _ptr(x), _ptr(Wr), _ptr(br), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wq_sh),
            _ptr(Wo), _ptr(k_cache), _ptr(vt_cache), _ptr(out), _ptr(idx_out), _ptr(w_out), _ptr(ws), ws.numel(),
            _stream(stream)]
    if events is None:
        _check(lib.gqe_decode_step(*args))
    else:
        _check(lib.gqe_decode_step_timed(*args, events))


def gqe_mfma_probe(workgroups, iters, out, stream=None):
    """Diagnostic matrix-core load: workgroups * 4 waves * iters * 8 bf16
    16x16x32 products (16384 flops each), no memory traffic; out: float32
    device tensor of `workgroups` entries (a checksum)."""
    _check(load().gqe_mfma_probe(int(workgroups), int(iters), _ptr(out), _stream(stream)))
