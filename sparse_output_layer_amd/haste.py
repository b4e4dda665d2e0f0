"""Thin Python binding of libhaste (include/haste.h), same names as the C ABI.

Argument marshalling only: shapes and dtypes are read from torch tensors,
device pointers and the current HIP stream are passed to the C entry points,
and a workspace tensor is allocated when the caller does not bring one.
Every step of the layer runs in the library's HIP kernels; if the library is
missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhaste.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "haste.h")

HASTE_OK, HASTE_ERR_INVALID, HASTE_ERR_UNSUPPORTED, HASTE_ERR_WORKSPACE, HASTE_ERR_HIP = range(5)
HASTE_F32, HASTE_BF16 = 0, 1
HASTE_TAIL_LEAN = 1   # tail flag: recompute dz in the dX pass instead of keeping it in ws
HASTE_TAIL_LAYOUT_READY = 2   # tail flag: ws already holds the feature order of idx


class HasteError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"haste status {status}: {msg}")
        self.status = status


class TailDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("D", ctypes.c_int32), ("L", ctypes.c_int64),
                ("G", ctypes.c_int32), ("F", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


class HeadDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("D", ctypes.c_int32), ("H", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class BceStruct(ctypes.Structure):
    _fields_ = [("row_ptr", ctypes.c_void_p), ("labels", ctypes.c_void_p),
                ("nnz", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("label_offset", ctypes.c_int64), ("grad_scale", ctypes.c_float),
                ("topk_buckets", ctypes.c_int32), ("loss", ctypes.c_void_p),
                ("topk", ctypes.c_int32), ("topk_kprime", ctypes.c_int32),
                ("topk_val", ctypes.c_void_p), ("topk_idx", ctypes.c_void_p)]


_lib = None
_vp, _sz, _i32, _i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
_PD = ctypes.POINTER(TailDesc)
_PH = ctypes.POINTER(HeadDesc)
_PB = ctypes.POINTER(BceStruct)

_SIGS = {
    "haste_abi_version": (ctypes.c_int, []),
    "haste_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "haste_last_error": (ctypes.c_char_p, []),
    "haste_tail_layout": (ctypes.c_int, [_PD, ctypes.POINTER(ctypes.c_int64)]),
    "haste_tail_workspace_bytes": (_sz, [_PD, _PB]),
    "haste_head_workspace_bytes": (_sz, [_PH, _PB]),
    "haste_tail_fwd_workspace_bytes": (_sz, [_PD, _PB]),
    "haste_tail_prepare_layout": (ctypes.c_int, [_PD, _vp, _vp, _sz, _vp]),
    "haste_tail_fwd": (ctypes.c_int, [_PD, _vp, _vp, _vp, _vp, _PB, _vp, _sz, _vp]),
    "haste_tail_bwd": (ctypes.c_int, [_PD, _vp, _vp, _vp, _vp, _PB, _vp, _vp, ctypes.c_int,
                                      _vp, _sz, _vp]),
    "haste_tail_step": (ctypes.c_int, [_PD, _vp, _vp, _vp, _PB, _vp, _vp, ctypes.c_int, _vp,
                                       _sz, _vp]),
    "haste_tail_step_sgd": (ctypes.c_int, [_PD, _vp, _vp, _vp, _PB, ctypes.c_float, _vp, _vp,
                                           ctypes.c_int, _vp, _sz, _vp]),
    "haste_sgd_update": (ctypes.c_int, [_i64, _i32, _vp, _vp, ctypes.c_float, _vp, _vp]),
    "haste_tail_prepare": (ctypes.c_int, [_PD, _vp, _PB, _vp, _sz, _vp]),
    "haste_tail_step_dw": (ctypes.c_int, [_PD, _vp, _vp, _vp, _PB, _vp, _vp, _sz, _vp]),
    "haste_tail_step_dx": (ctypes.c_int, [_PD, _vp, _vp, _vp, _PB, _vp, ctypes.c_int, _vp,
                                          _sz, _vp]),
    "haste_head_fwd": (ctypes.c_int, [_PH, _vp, _vp, _vp, _PB, _vp, _sz, _vp]),
    "haste_head_bwd": (ctypes.c_int, [_PH, _vp, _vp, _vp, _PB, _vp, _vp, ctypes.c_int, _vp,
                                      _sz, _vp]),
    "haste_head_step": (ctypes.c_int, [_PH, _vp, _vp, _PB, _vp, _vp, ctypes.c_int, _vp, _sz,
                                       _vp]),
    "haste_head_step_noalloc": (ctypes.c_int, [_PH, _vp, _vp, _PB, _vp, _vp, ctypes.c_int, _vp]),
    "haste_tail_group_positives": (ctypes.c_int, [_PD, _PB, _vp, _vp, _vp, _sz, _vp]),
    "haste_tail_validate": (ctypes.c_int, [_PD, _vp, _vp, _vp]),
    "haste_topk_merge": (ctypes.c_int, [_i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "haste_topk_expected_recall": (ctypes.c_double, [_i64, ctypes.c_int, ctypes.c_int, _i64]),
    "haste_topk_plan": (ctypes.c_int, [_i64, ctypes.c_int, ctypes.c_double, _i64, ctypes.POINTER(_i32)]),
    "haste_probe_mfma": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _vp, _vp]),
    "haste_tail_rewire": (ctypes.c_int, [_PD, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _vp]),
}


def lib():
    """Load libhaste.so (built in-tree by sparse_output_layer_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_output_layer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Entry-point names declared in include/haste.h."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(haste_[a-z_0-9]+)\s*\(", txt)))


def _check(status: int):
    if status != HASTE_OK:
        raise HasteError(status, lib().haste_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HASTE_BF16
    if t.dtype == torch.float32:
        return HASTE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


@dataclass
class Bce:
    """Positives (row-CSR, global label ids) and BCE options for one call."""
    row_ptr: torch.Tensor            # int32, B+1, device
    labels: torch.Tensor             # int32, nnz, device
    label_offset: int = 0
    grad_scale: float = 1.0
    loss: Optional[torch.Tensor] = None   # float32 scalar (1 element), device
    topk_val: Optional[torch.Tensor] = None   # float32 B x K, device: per-row top-K logits
    topk_idx: Optional[torch.Tensor] = None   # int32 B x K, device: their global label ids
    topk_kprime: int = 0             # 0: exact (K' = K); else K' per bucket, 1 <= K' <= K
    topk_buckets: int = 0            # 0: buckets of 32768 labels; else buckets per row

    def struct(self) -> BceStruct:
        _need(self.row_ptr, "row_ptr", torch.int32)
        _need(self.labels, "labels", torch.int32)
        if self.loss is not None:
            _need(self.loss, "loss", torch.float32)
        if (self.topk_val is None) != (self.topk_idx is None):
            raise ValueError("topk_val and topk_idx go together")
        if self.topk_val is not None:
            _need(self.topk_val, "topk_val", torch.float32)
            _need(self.topk_idx, "topk_idx", torch.int32)
            if self.topk_val.shape != self.topk_idx.shape or self.topk_val.dim() != 2:
                raise ValueError("topk_val / topk_idx must both be B x K")
        s = BceStruct()
        s.row_ptr = self.row_ptr.data_ptr()
        s.labels = self.labels.data_ptr() if self.labels.numel() else None
        s.nnz = int(self.labels.numel())
        s.label_offset = int(self.label_offset)
        s.grad_scale = float(self.grad_scale)
        s.loss = self.loss.data_ptr() if self.loss is not None else None
        s.topk = 0
        if self.topk_val is not None:
            s.topk = int(self.topk_val.shape[1])
            s.topk_val = self.topk_val.data_ptr()
            s.topk_idx = self.topk_idx.data_ptr()
            s.topk_kprime = int(self.topk_kprime)
            s.topk_buckets = int(self.topk_buckets)
        return s


def _bref(bce: Optional[Bce]):
    return None if bce is None else ctypes.pointer(bce.struct())


def tail_desc(X: torch.Tensor, idx: torch.Tensor, L: int, G: int, lean: bool = False,
              layout_ready: bool = False) -> TailDesc:
    B, D = X.shape
    return TailDesc(B=B, D=D, L=int(L), G=int(G), F=int(idx.shape[1]), dtype=_dtype_code(X),
                    flags=(HASTE_TAIL_LEAN if lean else 0) | (HASTE_TAIL_LAYOUT_READY if layout_ready else 0))


def head_desc(X: torch.Tensor, Wh: torch.Tensor) -> HeadDesc:
    B, D = X.shape
    return HeadDesc(B=B, D=D, H=int(Wh.shape[0]), dtype=_dtype_code(X))


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    if nbytes == 0:
        return None, 0
    if ws is not None and ws.numel() >= nbytes:
        return ws, ws.numel()
    t = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return t, nbytes


# ----------------------------------------------------------- entry points
def haste_abi_version() -> int:
    return lib().haste_abi_version()


def haste_tail_layout(L: int, G: int, F: int, B: int = 1, D: int = 1) -> dict:
    d = TailDesc(B=B, D=max(D, F), L=L, G=G, F=F, dtype=HASTE_BF16)
    out = (ctypes.c_int64 * 4)()
    _check(lib().haste_tail_layout(ctypes.byref(d), out))
    return {"n_groups": out[0], "index_count": out[1], "weight_rows": out[2],
            "last_group_live": out[3]}


def haste_tail_workspace_bytes(X, idx, L, G, bce: Optional[Bce] = None, lean=False) -> int:
    return lib().haste_tail_workspace_bytes(ctypes.byref(tail_desc(X, idx, L, G, lean)), _bref(bce))


def haste_tail_fwd_workspace_bytes(X, idx, L, G, bce: Optional[Bce] = None) -> int:
    return lib().haste_tail_fwd_workspace_bytes(ctypes.byref(tail_desc(X, idx, L, G)), _bref(bce))


def haste_tail_prepare_layout(X, idx, L, G, workspace: torch.Tensor, lean=False):
    """Forms idx's feature order in `workspace`; later calls on it pass
    layout_ready=True (tail flag HASTE_TAIL_LAYOUT_READY) to skip forming it."""
    _need(idx, "idx", torch.int32)
    d = tail_desc(X, idx, L, G, lean)
    _check(lib().haste_tail_prepare_layout(ctypes.byref(d), _ptr(idx), _ptr(workspace),
                                           workspace.numel(), _stream()))


def haste_head_workspace_bytes(X, Wh, bce: Optional[Bce] = None) -> int:
    return lib().haste_head_workspace_bytes(ctypes.byref(head_desc(X, Wh)), _bref(bce))


def _tail_in(X, idx, W):
    _need(X, "X")
    _need(idx, "idx", torch.int32)
    _need(W, "W", X.dtype)


def haste_tail_fwd(X, idx, W, L, G, Z=None, bce: Optional[Bce] = None, workspace=None, lean=False, layout_ready=False):
    _tail_in(X, idx, W)
    if Z is not None:
        _need(Z, "Z", X.dtype)
    d = tail_desc(X, idx, L, G, lean, layout_ready)
    b = _bref(bce)
    ws, nb = _workspace(lib().haste_tail_fwd_workspace_bytes(ctypes.byref(d), b), X.device, workspace)
    _check(lib().haste_tail_fwd(ctypes.byref(d), _ptr(X), _ptr(idx), _ptr(W), _ptr(Z), b,
                                _ptr(ws), nb, _stream()))
    return Z


def haste_tail_bwd(X, idx, W, L, G, dW, dX, dZ=None, bce: Optional[Bce] = None,
                   accumulate_dX=False, workspace=None, lean=False):
    _tail_in(X, idx, W)
    _need(dW, "dW", X.dtype)
    _need(dX, "dX", torch.float32)
    if dZ is not None:
        _need(dZ, "dZ", X.dtype)
    d = tail_desc(X, idx, L, G, lean)
    b = None if dZ is not None else _bref(bce)
    ws, nb = _workspace(lib().haste_tail_workspace_bytes(ctypes.byref(d), b), X.device, workspace)
    _check(lib().haste_tail_bwd(ctypes.byref(d), _ptr(X), _ptr(idx), _ptr(W), _ptr(dZ), b,
                                _ptr(dW), _ptr(dX), int(bool(accumulate_dX)), _ptr(ws), nb,
                                _stream()))


def haste_tail_step(X, idx, W, L, G, bce: Bce, dW, dX, accumulate_dX=False, workspace=None,
                    lean=False, layout_ready=False):
    _tail_in(X, idx, W)
    _need(dW, "dW", X.dtype)
    _need(dX, "dX", torch.float32)
    d = tail_desc(X, idx, L, G, lean, layout_ready)
    b = _bref(bce)
    ws, nb = _workspace(lib().haste_tail_workspace_bytes(ctypes.byref(d), b), X.device, workspace)
    _check(lib().haste_tail_step(ctypes.byref(d), _ptr(X), _ptr(idx), _ptr(W), b, _ptr(dW),
                                 _ptr(dX), int(bool(accumulate_dX)), _ptr(ws), nb, _stream()))


def haste_tail_step_sgd(X, idx, W, L, G, bce: Bce, lr, W_out, dX, accumulate_dX=False,
                        workspace=None, lean=False):
    """Training step with the SGD update fused into the dW pass: writes
    W_out = W - lr * dW (W_out must not overlap W) instead of dW."""
    _tail_in(X, idx, W)
    _need(W_out, "W_out", X.dtype)
    if W_out.shape != W.shape:
        raise ValueError("W_out must have W's shape")
    _need(dX, "dX", torch.float32)
    d = tail_desc(X, idx, L, G, lean)
    b = _bref(bce)
    ws, nb = _workspace(lib().haste_tail_workspace_bytes(ctypes.byref(d), b), X.device, workspace)
    _check(lib().haste_tail_step_sgd(ctypes.byref(d), _ptr(X), _ptr(idx), _ptr(W), b, float(lr),
                                     _ptr(W_out), _ptr(dX), int(bool(accumulate_dX)), _ptr(ws), nb,
                                     _stream()))


def haste_sgd_update(W, dW, lr, W_out=None):
    """W_out = W - lr * dW elementwise (W_out defaults to W: in place)."""
    W_out = W if W_out is None else W_out
    for t_, n in ((W, "W"), (dW, "dW"), (W_out, "W_out")):
        _need(t_, n, W.dtype)
    if dW.shape != W.shape or W_out.shape != W.shape:
        raise ValueError("W, dW and W_out must have one shape")
    dt = HASTE_BF16 if W.dtype == torch.bfloat16 else HASTE_F32
    _check(lib().haste_sgd_update(W.numel(), dt, _ptr(W), _ptr(dW), float(lr), _ptr(W_out), _stream()))


def haste_tail_prepare(X, idx, L, G, bce: Bce, workspace: torch.Tensor, lean=False):
    """Split step, part 1: transposed X and group-major positives into
    `workspace` (keep it for haste_tail_step_dw / haste_tail_step_dx)."""
    _need(X, "X")
    d = tail_desc(X, idx, L, G, lean)
    _check(lib().haste_tail_prepare(ctypes.byref(d), _ptr(X), _bref(bce), _ptr(workspace),
                                    workspace.numel(), _stream()))


def haste_tail_step_dw(X, idx, W, L, G, bce: Bce, dW, workspace: torch.Tensor, lean=False, layout_ready=False):
    """Split step, part 2: loss and dW (one kernel)."""
    _tail_in(X, idx, W)
    _need(dW, "dW", X.dtype)
    d = tail_desc(X, idx, L, G, lean, layout_ready)
    b = _bref(bce)
    _check(lib().haste_tail_step_dw(ctypes.byref(d), _ptr(X), _ptr(idx), _ptr(W), b, _ptr(dW),
                                    _ptr(workspace), workspace.numel(), _stream()))


def haste_tail_step_dx(X, idx, W, L, G, bce: Bce, dX, workspace: torch.Tensor,
                       accumulate_dX=False, lean=False):
    """Second half of haste_tail_step (dX), using what _dw left in `workspace`."""
    _tail_in(X, idx, W)
    _need(dX, "dX", torch.float32)
    d = tail_desc(X, idx, L, G, lean)
    b = _bref(bce)
    _check(lib().haste_tail_step_dx(ctypes.byref(d), _ptr(X), _ptr(idx), _ptr(W), b, _ptr(dX),
                                    int(bool(accumulate_dX)), _ptr(workspace), workspace.numel(),
                                    _stream()))


def haste_head_fwd(X, Wh, Zh=None, bce: Optional[Bce] = None, workspace=None):
    _need(X, "X")
    _need(Wh, "Wh", X.dtype)
    if Zh is not None:
        _need(Zh, "Zh", X.dtype)
    d = head_desc(X, Wh)
    b = _bref(bce)
    ws, nb = _workspace(lib().haste_head_workspace_bytes(ctypes.byref(d), b), X.device, workspace)
    _check(lib().haste_head_fwd(ctypes.byref(d), _ptr(X), _ptr(Wh), _ptr(Zh), b, _ptr(ws), nb,
                                _stream()))
    return Zh


def haste_head_bwd(X, Wh, dWh, dX, dZh=None, bce: Optional[Bce] = None, accumulate_dX=False,
                   workspace=None):
    _need(X, "X")
    _need(Wh, "Wh", X.dtype)
    _need(dWh, "dWh", X.dtype)
    _need(dX, "dX", torch.float32)
    if dZh is not None:
        _need(dZh, "dZh", X.dtype)
    d = head_desc(X, Wh)
    b = None if dZh is not None else _bref(bce)
    ws, nb = _workspace(lib().haste_head_workspace_bytes(ctypes.byref(d), b), X.device, workspace)
    _check(lib().haste_head_bwd(ctypes.byref(d), _ptr(X), _ptr(Wh), _ptr(dZh), b, _ptr(dWh),
                                _ptr(dX), int(bool(accumulate_dX)), _ptr(ws), nb, _stream()))


def haste_head_step(X, Wh, bce: Bce, dWh, dX, accumulate_dX=False, workspace=None):
    _need(X, "X")
    _need(Wh, "Wh", X.dtype)
    _need(dWh, "dWh", X.dtype)
    _need(dX, "dX", torch.float32)
    d = head_desc(X, Wh)
    b = _bref(bce)
    ws, nb = _workspace(lib().haste_head_workspace_bytes(ctypes.byref(d), b), X.device, workspace)
    _check(lib().haste_head_step(ctypes.byref(d), _ptr(X), _ptr(Wh), b, _ptr(dWh), _ptr(dX),
                                 int(bool(accumulate_dX)), _ptr(ws), nb, _stream()))


def haste_head_step_noalloc(X, Wh, bce: Bce, dWh, dX, accumulate_dX=False):
    """haste_head_step with the library's static device scratch as workspace
    (no allocation by the call or the binding); calls overlapping on one GPU race."""
    _need(X, "X")
    _need(Wh, "Wh", X.dtype)
    _need(dWh, "dWh", X.dtype)
    _need(dX, "dX", torch.float32)
    d = head_desc(X, Wh)
    _check(lib().haste_head_step_noalloc(ctypes.byref(d), _ptr(X), _ptr(Wh), _bref(bce), _ptr(dWh),
                                         _ptr(dX), int(bool(accumulate_dX)), _stream()))


def haste_tail_group_positives(B, D, L, G, F, bce: Bce, dtype=torch.bfloat16, workspace=None):
    d = TailDesc(B=B, D=D, L=L, G=G, F=F,
                 dtype=HASTE_BF16 if dtype == torch.bfloat16 else HASTE_F32)
    b = _bref(bce)
    dev = bce.row_ptr.device
    ng = (L + G - 1) // G
    grp_ptr = torch.empty(ng + 1, dtype=torch.int32, device=dev)
    ent = torch.empty(max(1, bce.labels.numel()), dtype=torch.int32, device=dev)
    ws, nb = _workspace(lib().haste_tail_workspace_bytes(ctypes.byref(d), b), dev, workspace)
    _check(lib().haste_tail_group_positives(ctypes.byref(d), b, _ptr(grp_ptr), _ptr(ent),
                                            _ptr(ws), nb, _stream()))
    return grp_ptr, ent


def haste_probe_mfma(blocks: int, iters: int, sink=None):
    """Measurement utility: blocks x 4 waves x iters x 16 bf16 MFMAs (16x16x32)
    with no memory traffic, on the current stream; returns the flop count."""
    if sink is None:
        sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    _check(lib().haste_probe_mfma(int(blocks), int(iters), _ptr(sink), _stream()))
    return blocks * 4 * iters * 16 * (16 * 16 * 32 * 2)


def haste_tail_validate(idx, D, L, G) -> torch.Tensor:
    _need(idx, "idx", torch.int32)
    d = TailDesc(B=1, D=D, L=L, G=G, F=int(idx.shape[1]), dtype=HASTE_BF16)
    out = torch.empty(1, dtype=torch.int32, device=idx.device)
    _check(lib().haste_tail_validate(ctypes.byref(d), _ptr(idx), _ptr(out), _stream()))
    return out


def haste_tail_rewire(idx, W, D, L, G, k_prune, cand=None, idx_out=None, W_out=None):
    """One prune-and-regrow step of every group's fan-in set; returns
    (idx_out, W_out).  cand: N_g x n_cand int32 regrowth candidates (or None);
    idx_out / W_out default to new tensors and may be idx / W (in place)."""
    _need(idx, "idx", torch.int32)
    _need(W, "W")
    F = int(idx.shape[1])
    dt = HASTE_BF16 if W.dtype == torch.bfloat16 else HASTE_F32
    d = TailDesc(B=1, D=D, L=L, G=G, F=F, dtype=dt)
    idx_out = torch.empty_like(idx) if idx_out is None else idx_out
    W_out = torch.empty_like(W) if W_out is None else W_out
    n_cand = 0
    if cand is not None:
        _need(cand, "cand", torch.int32)
        n_cand = int(cand.shape[1]) if cand.dim() == 2 else 0
    _check(lib().haste_tail_rewire(ctypes.byref(d), _ptr(idx), _ptr(W), int(k_prune),
                                   _ptr(cand) if cand is not None else None, n_cand,
                                   _ptr(idx_out), _ptr(W_out), _stream()))
    return idx_out, W_out


def haste_topk_expected_recall(n: int, K: int, kprime: int, buckets: int = 0) -> float:
    """Expected recall of the two-stage top-K for rows of n logits (host)."""
    r = lib().haste_topk_expected_recall(int(n), int(K), int(kprime), int(buckets))
    if r < 0:
        raise ValueError(f"invalid top-K parameters n={n} K={K} K'={kprime} buckets={buckets}")
    return r


def haste_topk_plan(n: int, K: int, target: float, min_buckets: int = 1):
    """(K', buckets >= min_buckets) with expected recall >= target and the
    fewest stage-2 candidates."""
    out = (_i32 * 2)()
    _check(lib().haste_topk_plan(int(n), int(K), float(target), int(min_buckets), out))
    return int(out[0]), int(out[1])


def haste_topk_merge(a_val, a_idx, b_val, b_idx):
    B, K = a_val.shape
    for t, n in ((a_val, "a_val"), (b_val, "b_val")):
        _need(t, n, torch.float32)
    for t, n in ((a_idx, "a_idx"), (b_idx, "b_idx")):
        _need(t, n, torch.int32)
    ov = torch.empty_like(a_val)
    oi = torch.empty_like(a_idx)
    _check(lib().haste_topk_merge(B, K, _ptr(a_val), _ptr(a_idx), _ptr(b_val), _ptr(b_idx),
                                  _ptr(ov), _ptr(oi), _stream()))
    return ov, oi
