"""ctypes binding of libslr.so: argument marshalling only.

Every function here has the name of the C entry point it calls and does
nothing but build the argument structs, take device pointers from torch
tensors, allocate outputs / workspace with torch and check the status. All
arithmetic runs in the HIP kernels; if the library is missing the first call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SLR_LIB selects another build of the same library (the host-sanitized one in the CPU ABI tests)
LIB_PATH = os.environ.get("SLR_LIB") or os.path.join(_HERE, "libslr.so")

SLR_OK, SLR_EINVAL, SLR_EUNSUPPORTED, SLR_EWORKSPACE, SLR_EHIP, SLR_ESCRATCH = 0, -1, -2, -3, -4, -5
SLR_F32, SLR_BF16 = 0, 1
SLR_LR_ROPE_OUTSIDE, SLR_LR_ABS_PE = 0, 1
SLR_GATE_HEAD, SLR_GATE_TOKEN = 0, 1
SLR_FMAP_ELU1, SLR_FMAP_SILU, SLR_FMAP_FAVOR = 0, 1, 2
SLR_OP_ROPE3D, SLR_OP_SELECT, SLR_OP_LOWRANK_SUMMARY, SLR_OP_ATTENTION, SLR_OP_DENSE = 0, 1, 2, 3, 4
SLR_OP_ATTENTION_BWD = 5

EXPORTS = ("slr_workspace_bytes", "slr_rope3d", "slr_select_blocks", "slr_lowrank_summary",
           "slr_lowrank_summary_noalloc", "slr_attention_fwd", "slr_attention_fwd_staged", "slr_attention_fwd_train", "slr_dense_attention_fwd",
           "slr_attention_bwd", "slr_status_string")


class SlrShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32), ("T", ctypes.c_int32),
                ("Hg", ctypes.c_int32), ("Wg", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class SlrRopeCfg(ctypes.Structure):
    _fields_ = [("base", ctypes.c_double), ("pairs_t", ctypes.c_int32), ("pairs_h", ctypes.c_int32),
                ("pairs_w", ctypes.c_int32)]


class SlrSparseCfg(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int32), ("keep", ctypes.c_int32)]


class SlrLowrankCfg(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("mode", ctypes.c_int32), ("lr_pairs_t", ctypes.c_int32),
                ("lr_pairs_h", ctypes.c_int32), ("lr_pairs_w", ctypes.c_int32), ("eps", ctypes.c_float),
                ("Wq", ctypes.c_void_p), ("Wk", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("Et", ctypes.c_void_p), ("Eh", ctypes.c_void_p), ("Ew", ctypes.c_void_p),
                ("gate_mode", ctypes.c_int32), ("Wg", ctypes.c_void_p), ("bg", ctypes.c_void_p),
                ("feature_map", ctypes.c_int32), ("omega", ctypes.c_void_p)]


class SlrError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {status_string(code)} ({code})")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load libslr.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_rank_attention_rope3d_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.slr_workspace_bytes.argtypes = [ctypes.c_int, P(SlrShape), P(SlrRopeCfg), P(SlrSparseCfg),
                                          P(SlrLowrankCfg), P(sz)]
        L.slr_rope3d.argtypes = [P(SlrShape), P(SlrRopeCfg), vp, vp, vp, sz, vp]
        L.slr_select_blocks.argtypes = [P(SlrShape), P(SlrRopeCfg), P(SlrSparseCfg), vp, vp, vp, vp, vp, vp, sz, vp]
        L.slr_lowrank_summary.argtypes = [P(SlrShape), P(SlrRopeCfg), P(SlrLowrankCfg), vp, vp, vp, vp, vp, sz, vp]
        L.slr_lowrank_summary_noalloc.argtypes = [P(SlrShape), P(SlrRopeCfg), P(SlrLowrankCfg), vp, vp, vp, vp, vp]
        L.slr_attention_fwd.argtypes = [P(SlrShape), P(SlrRopeCfg), P(SlrSparseCfg), P(SlrLowrankCfg), vp, vp, vp,
                                        vp, vp, vp, vp, vp, sz, vp]
        L.slr_attention_fwd_staged.argtypes = [P(SlrShape), P(SlrRopeCfg), P(SlrSparseCfg), P(SlrLowrankCfg), vp,
                                               vp, vp, vp, vp, vp, vp, vp, sz, P(vp), vp]
        L.slr_dense_attention_fwd.argtypes = [P(SlrShape), P(SlrRopeCfg), vp, vp, vp, vp, vp, sz, vp]
        L.slr_attention_bwd.argtypes = [P(SlrShape), P(SlrRopeCfg), P(SlrSparseCfg), P(SlrLowrankCfg)] + [vp] * 21 + [sz, vp]
        L.slr_attention_fwd_train.argtypes = [P(SlrShape), P(SlrRopeCfg), P(SlrSparseCfg), P(SlrLowrankCfg)] + [vp] * 10 + [sz, vp]
        for f in EXPORTS[:-1]:
            getattr(L, f).restype = ctypes.c_int
        L.slr_status_string.argtypes = [ctypes.c_int]
        L.slr_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().slr_status_string(code).decode()


def _check(code: int, where: str) -> None:
    if code != SLR_OK:
        raise SlrError(code, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ---------------------------------------------------------------------------
# config structs from a layer description (any object with the fields of
# synth.Layer)

def shape_of(layer) -> SlrShape:
    return SlrShape(layer.B, layer.H, layer.D, layer.T, layer.Hg, layer.Wg,
                    SLR_BF16 if layer.dtype == "bf16" else SLR_F32)


def rope_of(layer) -> SlrRopeCfg:
    return SlrRopeCfg(float(layer.base), *layer.pairs)


def sparse_of(layer) -> SlrSparseCfg:
    return SlrSparseCfg(layer.block, layer.keep)


def lowrank_of(layer, params: Dict[str, torch.Tensor]) -> SlrLowrankCfg:
    abspe = layer.lr_mode == "abspe"
    lp = (0, 0, 0) if abspe else tuple(layer.lr_pairs)
    token = getattr(layer, "gate", "head") == "token"
    return SlrLowrankCfg(layer.rank, SLR_LR_ABS_PE if abspe else SLR_LR_ROPE_OUTSIDE, lp[0], lp[1], lp[2],
                         float(layer.eps), params["wq"].data_ptr(), params["wk"].data_ptr(),
                         None if token else params["gate"].data_ptr(),
                         params["et"].data_ptr() if abspe else None,
                         params["eh"].data_ptr() if abspe else None,
                         params["ew"].data_ptr() if abspe else None,
                         SLR_GATE_TOKEN if token else SLR_GATE_HEAD,
                         params["wg"].data_ptr() if token else None,
                         params["bg"].data_ptr() if token else None,
                         {"silu": SLR_FMAP_SILU, "favor": SLR_FMAP_FAVOR}.get(getattr(layer, "fmap", "elu1"),
                                                                              SLR_FMAP_ELU1),
                         params["omega"].data_ptr() if getattr(layer, "fmap", "elu1") == "favor" else None)


def slr_workspace_bytes(op: int, shape: SlrShape, rope: SlrRopeCfg, sparse: Optional[SlrSparseCfg] = None,
                        lowrank: Optional[SlrLowrankCfg] = None) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().slr_workspace_bytes(op, ctypes.byref(shape), ctypes.byref(rope),
                                     ctypes.byref(sparse) if sparse is not None else None,
                                     ctypes.byref(lowrank) if lowrank is not None else None, ctypes.byref(n)),
           "slr_workspace_bytes")
    return n.value


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _ws(op, shape, rope, sparse, lowrank, ws, device):
    need = slr_workspace_bytes(op, shape, rope, sparse, lowrank)
    if ws is None or ws.numel() < need:
        ws = workspace(need, device)
    return ws


def slr_rope3d(x: torch.Tensor, shape: SlrShape, rope: SlrRopeCfg, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    out = torch.empty_like(x)
    ws = _ws(SLR_OP_ROPE3D, shape, rope, None, None, ws, x.device)
    _check(lib().slr_rope3d(ctypes.byref(shape), ctypes.byref(rope), _ptr(x), _ptr(out), _ptr(ws),
                            ws.numel(), _stream()), "slr_rope3d")
    return out


def slr_select_blocks(q: torch.Tensor, k: torch.Tensor, shape: SlrShape, rope: SlrRopeCfg, sparse: SlrSparseCfg,
                      want_rot: bool = False, ws: Optional[torch.Tensor] = None):
    L = shape.T * shape.Hg * shape.Wg
    nblk = -(-L // sparse.block)
    idx = torch.empty((shape.B, shape.H, nblk, sparse.keep), dtype=torch.int32, device=q.device)
    q_rot = torch.empty_like(q) if want_rot else None
    k_rot = torch.empty_like(k) if want_rot else None
    ws = _ws(SLR_OP_SELECT, shape, rope, sparse, None, ws, q.device)
    _check(lib().slr_select_blocks(ctypes.byref(shape), ctypes.byref(rope), ctypes.byref(sparse), _ptr(q), _ptr(k),
                                   _ptr(idx), _ptr(q_rot), _ptr(k_rot), _ptr(ws), ws.numel(), _stream()),
           "slr_select_blocks")
    return (idx, q_rot, k_rot) if want_rot else idx


def slr_lowrank_summary(k: torch.Tensor, v: torch.Tensor, shape: SlrShape, rope: SlrRopeCfg,
                        lowrank: SlrLowrankCfg, ws: Optional[torch.Tensor] = None):
    S = torch.empty((shape.B, shape.H, lowrank.rank, shape.D), dtype=torch.float32, device=k.device)
    z = torch.empty((shape.B, shape.H, lowrank.rank), dtype=torch.float32, device=k.device)
    ws = _ws(SLR_OP_LOWRANK_SUMMARY, shape, rope, None, lowrank, ws, k.device)
    _check(lib().slr_lowrank_summary(ctypes.byref(shape), ctypes.byref(rope), ctypes.byref(lowrank), _ptr(k),
                                     _ptr(v), _ptr(S), _ptr(z), _ptr(ws), ws.numel(), _stream()),
           "slr_lowrank_summary")
    return S, z


def slr_lowrank_summary_noalloc(k: torch.Tensor, v: torch.Tensor, shape: SlrShape, rope: SlrRopeCfg,
                                lowrank: SlrLowrankCfg, S: Optional[torch.Tensor] = None,
                                z: Optional[torch.Tensor] = None):
    """slr_lowrank_summary with the library's fixed scratch instead of a
    workspace (S and z are still caller tensors)."""
    S = torch.empty((shape.B, shape.H, lowrank.rank, shape.D), dtype=torch.float32, device=k.device) if S is None else S
    z = torch.empty((shape.B, shape.H, lowrank.rank), dtype=torch.float32, device=k.device) if z is None else z
    _check(lib().slr_lowrank_summary_noalloc(ctypes.byref(shape), ctypes.byref(rope), ctypes.byref(lowrank),
                                             _ptr(k), _ptr(v), _ptr(S), _ptr(z), _stream()),
           "slr_lowrank_summary_noalloc")
    return S, z


def slr_attention_fwd(q, k, v, shape: SlrShape, rope: SlrRopeCfg, sparse: SlrSparseCfg, lowrank: SlrLowrankCfg,
                      out: Optional[torch.Tensor] = None, debug: bool = False, ws: Optional[torch.Tensor] = None):
    """Returns out, or (out, idx, o_sparse, o_lowrank) when debug."""
    out = torch.empty_like(q) if out is None else out
    idx = o_sp = o_lr = None
    if debug:
        L = shape.T * shape.Hg * shape.Wg
        nblk = -(-L // sparse.block)
        idx = torch.empty((shape.B, shape.H, nblk, sparse.keep), dtype=torch.int32, device=q.device)
        o_sp, o_lr = torch.empty_like(q), torch.empty_like(q)
    ws = _ws(SLR_OP_ATTENTION, shape, rope, sparse, lowrank, ws, q.device)
    _check(lib().slr_attention_fwd(ctypes.byref(shape), ctypes.byref(rope), ctypes.byref(sparse),
                                   ctypes.byref(lowrank), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(idx),
                                   _ptr(o_sp), _ptr(o_lr), _ptr(ws), ws.numel(), _stream()), "slr_attention_fwd")
    return (out, idx, o_sp, o_lr) if debug else out


def slr_attention_fwd_train(q, k, v, shape: SlrShape, rope: SlrRopeCfg, sparse: SlrSparseCfg,
                            lowrank: SlrLowrankCfg, ws: Optional[torch.Tensor] = None, outs=None, summary=None):
    """Training forward: returns (out, idx, o_sparse, lse [B, H, L] fp32);
    ``outs`` may supply those four tensors. ``summary`` = (S [B, H, r, D],
    z [B, H, r]) fp32 tensors receive the low-rank summary for
    slr_attention_bwd (None: not saved)."""
    if outs is None:
        L = shape.T * shape.Hg * shape.Wg
        nblk = -(-L // sparse.block)
        out, o_sp = torch.empty_like(q), torch.empty_like(q)
        idx = torch.empty((shape.B, shape.H, nblk, sparse.keep), dtype=torch.int32, device=q.device)
        lse = torch.empty((shape.B, shape.H, L), dtype=torch.float32, device=q.device)
    else:
        out, idx, o_sp, lse = outs
    ws = _ws(SLR_OP_ATTENTION, shape, rope, sparse, lowrank, ws, q.device)
    _check(lib().slr_attention_fwd_train(ctypes.byref(shape), ctypes.byref(rope), ctypes.byref(sparse),
                                         ctypes.byref(lowrank), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(idx),
                                         _ptr(o_sp), _ptr(lse), *(_ptr(t) for t in (summary or (None, None))),
                                         _ptr(ws), ws.numel(), _stream()),
           "slr_attention_fwd_train")
    return out, idx, o_sp, lse


def slr_attention_bwd(q, k, v, idx, o_sparse, lse, dout, shape: SlrShape, rope: SlrRopeCfg, sparse: SlrSparseCfg,
                      lowrank: SlrLowrankCfg, ws: Optional[torch.Tensor] = None, grads=None, summary=None):
    """Backward of the layer given dout (idx, o_sparse and lse saved by
    slr_attention_fwd_train). Returns (dq, dk, dv, dWq [H, D, r] fp32, dWk,
    dgate, dE): dgate is [H] fp32 for the per-head gate, (dWg [H, D], dbg [H])
    fp32 for the token gate; dE = (dEt [T, r], dEh [Hg, r], dEw [Wg, r]) fp32
    for the absolute-PE variant, else None; ``grads`` may supply those
    outputs; ``summary`` = the (S, z) slr_attention_fwd_train saved (None:
    recomputed)."""
    if grads is None:
        dev = q.device
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dWq = torch.empty((shape.H, shape.D, lowrank.rank), dtype=torch.float32, device=dev)
        dWk = torch.empty_like(dWq)
        dg = torch.empty((shape.H,), dtype=torch.float32, device=dev)
        if lowrank.gate_mode == SLR_GATE_TOKEN:
            dg = (torch.empty((shape.H, shape.D), dtype=torch.float32, device=dev), dg)
        dE = None
        if lowrank.mode == SLR_LR_ABS_PE:
            dE = tuple(torch.empty((n, lowrank.rank), dtype=torch.float32, device=dev)
                       for n in (shape.T, shape.Hg, shape.Wg))
    else:
        dq, dk, dv, dWq, dWk, dg, dE = grads
    ws = _ws(SLR_OP_ATTENTION_BWD, shape, rope, sparse, lowrank, ws, q.device)
    _check(lib().slr_attention_bwd(ctypes.byref(shape), ctypes.byref(rope), ctypes.byref(sparse),
                                   ctypes.byref(lowrank), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(o_sparse),
                                   _ptr(lse), *(_ptr(t) for t in (summary or (None, None))), _ptr(dout), _ptr(dq),
                                   _ptr(dk), _ptr(dv), _ptr(dWq), _ptr(dWk),
                                   *((None, _ptr(dg[0]), _ptr(dg[1])) if isinstance(dg, tuple) else (_ptr(dg), None, None)),
                                   *(_ptr(t) for t in (dE or (None, None, None))),
                                   _ptr(ws), ws.numel(), _stream()), "slr_attention_bwd")
    return dq, dk, dv, dWq, dWk, dg, dE


def slr_attention_fwd_staged(q, k, v, shape: SlrShape, rope: SlrRopeCfg, sparse: SlrSparseCfg,
                             lowrank: SlrLowrankCfg, out: torch.Tensor, ws: torch.Tensor, events) -> None:
    """slr_attention_fwd recording five caller-created hipEvent_t handles
    (integers) at the stage boundaries on the current stream."""
    ev = (ctypes.c_void_p * 5)(*events)
    _check(lib().slr_attention_fwd_staged(ctypes.byref(shape), ctypes.byref(rope), ctypes.byref(sparse),
                                          ctypes.byref(lowrank), _ptr(q), _ptr(k), _ptr(v), _ptr(out), None, None,
                                          None, _ptr(ws), ws.numel(), ev, _stream()), "slr_attention_fwd_staged")


def slr_dense_attention_fwd(q, k, v, shape: SlrShape, rope: SlrRopeCfg, out: Optional[torch.Tensor] = None,
                            ws: Optional[torch.Tensor] = None):
    out = torch.empty_like(q) if out is None else out
    ws = _ws(SLR_OP_DENSE, shape, rope, None, None, ws, q.device)
    _check(lib().slr_dense_attention_fwd(ctypes.byref(shape), ctypes.byref(rope), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(out), _ptr(ws), ws.numel(), _stream()), "slr_dense_attention_fwd")
    return out
