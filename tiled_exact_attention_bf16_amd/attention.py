"""Thin torch binding of the C ABI (argument marshalling only).

torch supplies device memory and the current HIP stream; every step of the
attention computation runs in the library's gfx950 kernels.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import _lib as L


@dataclass
class Tuning:
    """Forward variant: FMA-exp2 share (of 16), lazy threshold (log2 units), query tiles per
    workgroup, key splits (1 = none).  -1 keeps the library default."""
    exp2_poly_per16: int = -1
    rescale_threshold_log2: int = -1
    q_tiles_per_workgroup: int = -1
    key_splits: int = -1

    def c(self):
        return L.FwdTuning(self.exp2_poly_per16, self.rescale_threshold_log2, self.q_tiles_per_workgroup,
                           self.key_splits)


# ---- argument checks: the C library sees only pointers and sizes, so the tensors'
# dtype, shape and device are checked here before any pointer is handed over (all
# dtype and shape checks first, then the devices) ----

def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check_tensor(name: str, t, dtype: torch.dtype, shape: tuple) -> None:
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
    _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_devices(**tensors) -> None:
    """Every tensor on the GPU, and all on the device of the first one."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        _need(t.device.type == "cuda", f"{name} must be a GPU tensor, got device {t.device}")
        dev = t.device if dev is None else dev
        _need(t.device == dev, f"{name} is on {t.device}, expected {dev} (all tensors on one device)")


def _check_lengths(name: str, cu) -> None:
    _need(isinstance(cu, torch.Tensor) and cu.dtype == torch.int32 and cu.dim() == 1 and cu.numel() >= 1,
          f"{name} must be a 1-D int32 tensor of batch+1 prefix sums")
    _need(cu.is_contiguous(), f"{name} must be contiguous")


def _check_qkv(q, k, v, cu_seqlens_q, cu_seqlens_k) -> None:
    """Dtypes and shapes of the inputs: [B, S, H, D] (fixed length) or [T, H, D] (packed)."""
    varlen = cu_seqlens_q is not None
    rank = 3 if varlen else 4
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
        _need(t.dtype == torch.bfloat16, f"{name} must be torch.bfloat16, got {t.dtype}")
        _need(t.dim() == rank, f"{name} must be {'[T, H, D]' if varlen else '[B, S, H, D]'}, got {tuple(t.shape)}")
    _need(tuple(v.shape) == tuple(k.shape), f"v must have the shape of k {tuple(k.shape)}, got {tuple(v.shape)}")
    _need(q.shape[-1] == k.shape[-1], f"q and k must share the head dimension ({q.shape[-1]} vs {k.shape[-1]})")
    _need(q.shape[-2] == k.shape[-2], f"q and k must have the same number of heads ({q.shape[-2]} vs {k.shape[-2]})")
    if varlen:
        _check_lengths("cu_seqlens_q", cu_seqlens_q)
        if cu_seqlens_k is not None:
            _check_lengths("cu_seqlens_k", cu_seqlens_k)
            _need(cu_seqlens_k.numel() == cu_seqlens_q.numel(), "cu_seqlens_k must have as many entries as cu_seqlens_q")
    else:
        _need(q.shape[0] == k.shape[0], f"q and k must have the same batch ({q.shape[0]} vs {k.shape[0]})")
        _need(cu_seqlens_k is None, "cu_seqlens_k without cu_seqlens_q")


def _lse_shape(q, varlen: bool) -> tuple:
    return (q.shape[1], q.shape[0]) if varlen else (q.shape[0], q.shape[2], q.shape[1])


def _check_lse(lse, q, varlen: bool) -> None:
    _check_tensor("lse", lse, torch.float32, _lse_shape(q, varlen))
    # the library writes LSE as a dense [B, H, S_q] / [H, T_q] array
    _need(lse.is_contiguous(), "lse must be contiguous")


def _check_workspace(ws) -> None:
    if ws is not None:
        _need(isinstance(ws, torch.Tensor) and ws.dtype == torch.uint8 and ws.is_contiguous(),
              "workspace must be a contiguous uint8 tensor")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides(t: torch.Tensor, varlen: bool):
    if t.stride(-1) != 1:
        raise ValueError("the head dimension must be contiguous")
    if varlen:
        if t.dim() != 3:
            raise ValueError("packed variable-length tensors are [T, H, D]")
        return L.Strides(0, t.stride(0), t.stride(1))
    if t.dim() != 4:
        raise ValueError("fixed-length tensors are [B, S, H, D]")
    return L.Strides(t.stride(0), t.stride(1), t.stride(2))


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _max_len(cu: torch.Tensor) -> int:
    # host copy of the lengths (a synchronisation); pass max_seqlen to avoid it
    return int((cu[1:] - cu[:-1]).max().item()) if cu.numel() > 1 else 0


def fwd_args(q, k, v, o, lse, softmax_scale, causal, cu_seqlens_q=None, cu_seqlens_k=None,
             max_seqlen_q=None, max_seqlen_k=None) -> L.FwdArgs:
    varlen = cu_seqlens_q is not None
    a = L.FwdArgs()
    a.q, a.k, a.v, a.o, a.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse)
    a.q_stride, a.k_stride = _strides(q, varlen), _strides(k, varlen)
    a.v_stride, a.o_stride = _strides(v, varlen), _strides(o, varlen)
    a.num_heads, a.head_dim = q.shape[-2], q.shape[-1]
    a.softmax_scale = softmax_scale
    a.causal = int(bool(causal))
    a.o_dtype = L.FA_DTYPE_F32 if o.dtype == torch.float32 else L.FA_DTYPE_BF16
    if varlen:
        a.batch = cu_seqlens_q.numel() - 1
        a.cu_seqlens_q = _ptr(cu_seqlens_q)
        a.cu_seqlens_k = _ptr(cu_seqlens_k) if cu_seqlens_k is not None else None
        a.total_q, a.total_k = q.shape[0], k.shape[0]
        a.max_seqlen_q = _max_len(cu_seqlens_q) if max_seqlen_q is None else max_seqlen_q
        if cu_seqlens_k is None:
            a.max_seqlen_k = a.max_seqlen_q
        else:
            a.max_seqlen_k = _max_len(cu_seqlens_k) if max_seqlen_k is None else max_seqlen_k
    else:
        a.batch, a.seqlen_q, a.seqlen_k = q.shape[0], q.shape[1], k.shape[1]
    return a


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, softmax_scale: Optional[float] = None,
        causal: bool = False, cu_seqlens_q: Optional[torch.Tensor] = None,
        cu_seqlens_k: Optional[torch.Tensor] = None, max_seqlen_q: Optional[int] = None,
        max_seqlen_k: Optional[int] = None, tuning: Optional[Tuning] = None,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Exact attention forward.  Returns (O bf16 like q, LSE fp32 [B,H,S] or [H,T]).  An
    fp32 `out` receives the normalised output before its bf16 rounding (a diagnostic)."""
    _check_qkv(q, k, v, cu_seqlens_q, cu_seqlens_k)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.shape[-1])
    varlen = cu_seqlens_q is not None
    if out is not None:
        _check_tensor("out", out, torch.float32 if out.dtype == torch.float32 else torch.bfloat16, q.shape)
    if lse is not None:
        _check_lse(lse, q, varlen)
    _check_workspace(workspace)
    _check_devices(q=q, k=k, v=v, out=out, lse=lse, workspace=workspace, cu_seqlens_q=cu_seqlens_q,
                   cu_seqlens_k=cu_seqlens_k)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(_lse_shape(q, varlen), dtype=torch.float32, device=q.device)
    a = fwd_args(q, k, v, out, lse, softmax_scale, causal, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    lib = L.lib()
    t = (tuning or Tuning()).c()
    need = ctypes.c_size_t(0)
    L.check(lib.fa_fwd_workspace_size(ctypes.byref(a), ctypes.byref(t), ctypes.byref(need)), "fa_fwd_workspace_size")
    if need.value > 0 and (workspace is None or workspace.numel() < need.value):
        workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
    L.check(lib.fa_fwd(ctypes.byref(a), ctypes.byref(t), _ptr(workspace) if need.value else None,
                       need.value, _stream(stream)), "fa_fwd")
    return out, lse


def fwd_workspace(q, k, v, softmax_scale=None, causal=False, cu_seqlens_q=None, cu_seqlens_k=None,
                  max_seqlen_q=None, max_seqlen_k=None, tuning: Optional[Tuning] = None) -> Optional[torch.Tensor]:
    """A device workspace of the size fa_fwd needs for these arguments (None if 0 bytes),
    for callers that reuse one across calls."""
    _check_qkv(q, k, v, cu_seqlens_q, cu_seqlens_k)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.shape[-1])
    varlen = cu_seqlens_q is not None
    a = fwd_args(q, k, v, q, q, softmax_scale, causal, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    t = (tuning or Tuning()).c()
    need = ctypes.c_size_t(0)
    L.check(L.lib().fa_fwd_workspace_size(ctypes.byref(a), ctypes.byref(t), ctypes.byref(need)),
            "fa_fwd_workspace_size")
    return torch.empty(need.value, dtype=torch.uint8, device=q.device) if need.value else None


def build_schedule(q, k, cu_seqlens, causal, max_seqlen=None, tuning: Optional[Tuning] = None, stream=None):
    """Runs only the variable-length longest-first list builder; returns (tile_rows, [(seq, tile), ...])."""
    _check_qkv(q, k, k, cu_seqlens, None)
    _check_devices(q=q, k=k, cu_seqlens=cu_seqlens)
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    a = fwd_args(q, k, k, o, lse, 1.0, causal, cu_seqlens, None, max_seqlen, None)
    lib = L.lib()
    t = (tuning or Tuning()).c()
    need = ctypes.c_size_t(0)
    L.check(lib.fa_fwd_workspace_size(ctypes.byref(a), ctypes.byref(t), ctypes.byref(need)), "fa_fwd_workspace_size")
    ws = torch.zeros(max(need.value, 256), dtype=torch.uint8, device=q.device)
    L.check(lib.fa_fwd_build_schedule(ctypes.byref(a), ctypes.byref(t), _ptr(ws), ws.numel(), _stream(stream)),
            "fa_fwd_build_schedule")
    words = ws.view(torch.int32).cpu()
    n = int(words[0])
    items = [(int(words[1 + 2 * i]), int(words[2 + 2 * i])) for i in range(n)]
    return int(lib.fa_fwd_tile_rows(ctypes.byref(t))), items


def exp2_probe(x: torch.Tensor, stream=None):
    """(software 2^x, hardware v_exp_f32) of a contiguous fp32 device tensor, as the
    forward kernel evaluates them (fa_exp2_probe)."""
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous fp32 device tensor")
    y_poly, y_hw = torch.empty_like(x), torch.empty_like(x)
    L.check(L.lib().fa_exp2_probe(_ptr(x), _ptr(y_poly), _ptr(y_hw), x.numel(), _stream(stream)), "fa_exp2_probe")
    return y_poly, y_hw


def bwd_args(dout, q, k, v, o, lse, dq, dk, dv, softmax_scale, causal, deterministic, grad_dtype,
             cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None) -> L.BwdArgs:
    varlen = cu_seqlens_q is not None
    a = L.BwdArgs()
    a.q, a.k, a.v, a.o, a.dout, a.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse)
    a.dq, a.dk, a.dv = _ptr(dq), _ptr(dk), _ptr(dv)
    a.q_stride, a.k_stride, a.v_stride = _strides(q, varlen), _strides(k, varlen), _strides(v, varlen)
    a.o_stride, a.do_stride = _strides(o, varlen), _strides(dout, varlen)
    a.dq_stride, a.dk_stride, a.dv_stride = _strides(dq, varlen), _strides(dk, varlen), _strides(dv, varlen)
    a.num_heads, a.head_dim = q.shape[-2], q.shape[-1]
    a.softmax_scale = softmax_scale
    a.causal = int(bool(causal))
    a.deterministic = int(bool(deterministic))
    a.grad_dtype = L.FA_DTYPE_F32 if grad_dtype == torch.float32 else L.FA_DTYPE_BF16
    if varlen:
        a.batch = cu_seqlens_q.numel() - 1
        a.cu_seqlens_q = _ptr(cu_seqlens_q)
        a.cu_seqlens_k = _ptr(cu_seqlens_k) if cu_seqlens_k is not None else None
        a.total_q, a.total_k = q.shape[0], k.shape[0]
        a.max_seqlen_q = _max_len(cu_seqlens_q) if max_seqlen_q is None else max_seqlen_q
        if cu_seqlens_k is None:
            a.max_seqlen_k = a.max_seqlen_q
        else:
            a.max_seqlen_k = _max_len(cu_seqlens_k) if max_seqlen_k is None else max_seqlen_k
    else:
        a.batch, a.seqlen_q, a.seqlen_k = q.shape[0], q.shape[1], k.shape[1]
    return a


def bwd_noalloc(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                lse: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor,
                softmax_scale: Optional[float] = None, causal: bool = False, deterministic: bool = False,
                cu_seqlens_q: Optional[torch.Tensor] = None, cu_seqlens_k: Optional[torch.Tensor] = None,
                max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None, stream=None):
    """The backward through fa_bwd_noalloc: the library's static workspace, no device
    allocation anywhere in the call (the caller passes dq, dk, dv; their dtype is the
    gradient dtype)."""
    grad_dtype = dq.dtype
    if grad_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dq must be float32 or bfloat16")
    _check_qkv(q, k, v, cu_seqlens_q, cu_seqlens_k)
    _check_tensor("o", o, torch.bfloat16, q.shape)
    _check_tensor("dout", dout, torch.bfloat16, q.shape)
    _check_lse(lse, q, cu_seqlens_q is not None)
    for name, g, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor(name, g, grad_dtype, ref.shape)
    _check_devices(q=q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, cu_seqlens_q=cu_seqlens_q,
                   cu_seqlens_k=cu_seqlens_k)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.shape[-1])
    a = bwd_args(dout, q, k, v, o, lse, dq, dk, dv, softmax_scale, causal, deterministic, grad_dtype,
                 cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    L.check(L.lib().fa_bwd_noalloc(ctypes.byref(a), _stream(stream)), "fa_bwd_noalloc")
    return dq, dk, dv


def bwd(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
        lse: torch.Tensor, softmax_scale: Optional[float] = None, causal: bool = False,
        deterministic: bool = False, grad_dtype: torch.dtype = torch.float32,
        cu_seqlens_q: Optional[torch.Tensor] = None, cu_seqlens_k: Optional[torch.Tensor] = None,
        max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
        dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, stream=None, phases: int = L.FA_BWD_PHASE_ALL):
    """Exact attention backward from the saved LSE.  Returns (dQ, dK, dV) in grad_dtype.

    ``phases`` selects a subset of the backward's kernels (fa_bwd_phases); the
    default runs all of them."""
    if grad_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("grad_dtype must be float32 or bfloat16")
    _check_qkv(q, k, v, cu_seqlens_q, cu_seqlens_k)
    varlen = cu_seqlens_q is not None
    _check_tensor("o", o, torch.bfloat16, q.shape)
    _check_tensor("dout", dout, torch.bfloat16, q.shape)
    _check_lse(lse, q, varlen)
    for name, g, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if g is not None:
            _check_tensor(name, g, grad_dtype, ref.shape)
    _check_workspace(workspace)
    _check_devices(q=q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, workspace=workspace,
                   cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.shape[-1])
    dq = torch.empty(q.shape, dtype=grad_dtype, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=grad_dtype, device=q.device) if dk is None else dk
    dv = torch.empty(v.shape, dtype=grad_dtype, device=q.device) if dv is None else dv
    a = bwd_args(dout, q, k, v, o, lse, dq, dk, dv, softmax_scale, causal, deterministic, grad_dtype,
                 cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    lib = L.lib()
    need = ctypes.c_size_t(0)
    L.check(lib.fa_bwd_workspace_size(ctypes.byref(a), ctypes.byref(need)), "fa_bwd_workspace_size")
    if need.value > 0 and (workspace is None or workspace.numel() < need.value):
        workspace = torch.empty(need.value, dtype=torch.uint8, device=q.device)
    if phases == L.FA_BWD_PHASE_ALL:
        L.check(lib.fa_bwd(ctypes.byref(a), _ptr(workspace) if need.value else None, need.value, _stream(stream)),
                "fa_bwd")
    else:
        L.check(lib.fa_bwd_phases(ctypes.byref(a), phases, _ptr(workspace) if need.value else None, need.value,
                                  _stream(stream)), "fa_bwd_phases")
    return dq, dk, dv
