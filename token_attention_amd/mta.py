"""ctypes binding of libmta (argument marshalling only).

Every function forwards torch device tensors to the C ABI declared in
``include/mta.h``; all arithmetic runs in the library's HIP kernels. There is no
CPU fallback: a missing library or a CPU tensor raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmta.so")

# flag bits, identical to include/mta.h
KQ_PRE = 0x1
KQ_POST = 0x2
MIX_PRE = 0x4
MIX_POST = 0x8
GN = 0x10
FP32 = 0x20

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE = 0, 1, 2, 3, 4

EXPORTED = [
    "mta_forward", "mta_forward_rows", "mta_forward_materialized", "mta_materialized_workspace_bytes",
    "mta_attention_plain", "mta_check_args", "mta_status_string", "mta_last_error", "mta_version",
    "mta_backward_materialized", "mta_backward_workspace_bytes", "mta_forward_rows_split",
    "mta_forward_rows_split_workspace_bytes", "mta_forward_rows_split_plan", "mta_forward_rows_split_noalloc",
    "mta_forward_train", "mta_backward_fused", "mta_backward_fused_workspace_bytes",
]

NOALLOC_SCRATCH_BYTES = 32 << 20  # MTA_NOALLOC_SCRATCH_BYTES

_lib = None


class MTAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libmta status {status}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libmta.so (built by ``token_attention_amd.build``); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing; run `python -m token_attention_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, fp, i, u = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_uint
        L.mta_forward.argtypes = [vp, vp, vp, fp, fp, fp, fp, ctypes.c_float, vp] + [i] * 7 + [u, vp]
        L.mta_forward.restype = i
        L.mta_forward_rows.argtypes = [vp, vp, vp, fp, fp, fp, fp, ctypes.c_float, vp] + [i] * 8 + [u, vp]
        L.mta_forward_rows.restype = i
        L.mta_forward_rows_split.argtypes = [vp, vp, vp, fp, fp, fp, fp, ctypes.c_float, vp] + [i] * 8 + \
            [u, vp, ctypes.c_size_t, vp]
        L.mta_forward_rows_split.restype = i
        L.mta_forward_rows_split_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, fp, ctypes.c_float, vp] + [i] * 8 + \
            [u, vp]
        L.mta_forward_rows_split_noalloc.restype = i
        L.mta_forward_rows_split_plan.argtypes = [i] * 8 + [u, i, ctypes.POINTER(i), ctypes.POINTER(i)]
        L.mta_forward_rows_split_plan.restype = i
        L.mta_forward_rows_split_workspace_bytes.argtypes = [i] * 8 + [u]
        L.mta_forward_rows_split_workspace_bytes.restype = ctypes.c_size_t
        L.mta_forward_materialized.argtypes = [vp, vp, vp, fp, fp, fp, fp, ctypes.c_float, vp] + [i] * 7 + \
            [u, vp, ctypes.c_size_t, vp]
        L.mta_forward_materialized.restype = i
        L.mta_materialized_workspace_bytes.argtypes = [i, i, i, u]
        L.mta_materialized_workspace_bytes.restype = ctypes.c_size_t
        L.mta_backward_materialized.argtypes = [vp, vp, vp, fp, fp, fp, fp, ctypes.c_float, vp, vp, vp, vp, fp, fp,
                                                fp, fp, fp] + [i] * 7 + [u, vp, ctypes.c_size_t, vp]
        L.mta_backward_materialized.restype = i
        L.mta_backward_workspace_bytes.argtypes = [i] * 7 + [u]
        L.mta_backward_workspace_bytes.restype = ctypes.c_size_t
        L.mta_forward_train.argtypes = [vp, vp, vp, fp, fp, fp, fp, ctypes.c_float, vp, vp, vp] + [i] * 7 + [u, vp]
        L.mta_forward_train.restype = i
        L.mta_backward_fused.argtypes = [vp, vp, vp, fp, fp, fp, fp, ctypes.c_float, vp, vp, vp, vp, vp, vp, fp, fp,
                                         fp, fp, fp] + [i] * 7 + [u, vp, ctypes.c_size_t, vp]
        L.mta_backward_fused.restype = i
        L.mta_backward_fused_workspace_bytes.argtypes = [i] * 7 + [u]
        L.mta_backward_fused_workspace_bytes.restype = ctypes.c_size_t
        L.mta_attention_plain.argtypes = [vp, vp, vp, vp, i, i, i, i, u, vp]
        L.mta_attention_plain.restype = i
        L.mta_check_args.argtypes = [vp, vp, vp, fp, fp, fp, fp, vp] + [i] * 7 + [u]
        L.mta_check_args.restype = i
        L.mta_status_string.argtypes = [i]
        L.mta_status_string.restype = ctypes.c_char_p
        L.mta_last_error.argtypes = []
        L.mta_last_error.restype = ctypes.c_char_p
        L.mta_version.argtypes = []
        L.mta_version.restype = i
        _lib = L
    return _lib


def _check(status: int):
    if status != OK:
        msg = lib().mta_last_error().decode() or lib().mta_status_string(status).decode()
        raise MTAError(status, msg)


def placement_flags(kq: Optional[str], mix: Optional[str], gn: bool, fp32: bool) -> int:
    """Flag bits of a placement: kq / mix are None, "pre", "post" or "both" (with "both"
    theta holds [2, M, c_q, c_k] and w [2, M/c_h, c_h, c_h], the side before softmax first)."""
    f = {None: 0, "pre": KQ_PRE, "post": KQ_POST, "both": KQ_PRE | KQ_POST}[kq]
    f |= {None: 0, "pre": MIX_PRE, "post": MIX_POST, "both": MIX_PRE | MIX_POST}[mix]
    if gn:
        f |= GN
    if fp32:
        f |= FP32
    return f


def _dev(t: Optional[torch.Tensor], name: str, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


_SIDES = {None: 0, "pre": 1, "post": 1, "both": 2}


def _params(q, theta, w, gamma, beta, c_q, c_k, c_h, kq, mix, gn):
    """Check the parameter tensors against the sizes the library reads through their pointers
    (the C ABI receives bare pointers and cannot see their extents): theta [sides, M, c_q, c_k],
    w [sides, M/c_h, c_h, c_h] (sides = 2 for "both", the leading axis dropped for one side),
    gamma and beta [M*d], all on the device of q."""
    B, T, M, d = q.shape
    want = {
        "theta": (theta, _SIDES[kq] * M * c_q * c_k if kq else None),
        "w": (w, _SIDES[mix] * M * c_h if mix else None),
        "gamma": (gamma, M * d if gn else None),
        "beta": (beta, M * d if gn else None),
    }
    for name, (t, n) in want.items():
        if n is None or t is None:
            continue
        if t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}, got {t.device}")
        if t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements; this placement reads {n}")


def _common(q, k, v, out):
    if q.dim() != 4:
        raise ValueError("q must be [B, T, M, d]")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("tensors must be bfloat16 or float32")
    if out is None:
        out = torch.empty_like(q)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    return out


def forward(q, k, v, theta=None, w=None, gamma=None, beta=None, lam: float = 1.0, *, c_q: int = 1,
            c_k: int = 1, c_h: int = 1, kq: Optional[str] = None, mix: Optional[str] = None,
            gn: bool = False, out=None, stream=None) -> torch.Tensor:
    """Fused forward (``mta_forward``). q, k, v: [B, T, M, d] bf16 or fp32 on the GPU."""
    out = _common(q, k, v, out)
    B, T, M, d = q.shape
    _params(q, theta, w, gamma, beta, c_q, c_k, c_h, kq, mix, gn)
    fl = placement_flags(kq, mix, gn, q.dtype == torch.float32)
    _check(lib().mta_forward(
        _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dev(theta, "theta", torch.float32),
        _dev(w, "w", torch.float32), _dev(gamma, "gamma", torch.float32), _dev(beta, "beta", torch.float32),
        float(lam), _dev(out, "out"), B, T, M, d, c_q, c_k, c_h, fl, _stream(stream)))
    return out


def forward_rows(q, k, v, theta=None, w=None, gamma=None, beta=None, lam: float = 1.0, *, row_begin: int,
                 c_q: int = 1, c_k: int = 1, c_h: int = 1, kq: Optional[str] = None, mix: Optional[str] = None,
                 gn: bool = False, out=None, stream=None) -> torch.Tensor:
    """``mta_forward_rows``: output rows row_begin .. T-1 only (decode step, prefill chunk);
    rows of ``out`` before row_begin are left as they are."""
    out = _common(q, k, v, out)
    B, T, M, d = q.shape
    _params(q, theta, w, gamma, beta, c_q, c_k, c_h, kq, mix, gn)
    fl = placement_flags(kq, mix, gn, q.dtype == torch.float32)
    _check(lib().mta_forward_rows(
        _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dev(theta, "theta", torch.float32),
        _dev(w, "w", torch.float32), _dev(gamma, "gamma", torch.float32), _dev(beta, "beta", torch.float32),
        float(lam), _dev(out, "out"), B, T, M, d, c_q, c_k, c_h, int(row_begin), fl, _stream(stream)))
    return out


def rows_split_workspace_bytes(B: int, T: int, M: int, d: int, *, row_begin: int, c_q: int = 1, c_k: int = 1,
                               c_h: int = 1, kq: Optional[str] = None, mix: Optional[str] = None, gn: bool = False,
                               fp32: bool = False) -> int:
    return int(lib().mta_forward_rows_split_workspace_bytes(B, T, M, d, c_q, c_k, c_h, int(row_begin),
                                                            placement_flags(kq, mix, gn, fp32)))


def rows_split_plan(B: int, T: int, M: int, d: int, *, row_begin: int, c_q: int = 1, c_k: int = 1, c_h: int = 1,
                    kq: Optional[str] = None, mix: Optional[str] = None, gn: bool = False, fp32: bool = False,
                    compute_units: int = 0):
    """``mta_forward_rows_split_plan``: (number of key chunks, keys per chunk) of the split on a
    device with ``compute_units`` compute units (0: the current device)."""
    n, keys = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().mta_forward_rows_split_plan(B, T, M, d, c_q, c_k, c_h, int(row_begin),
                                             placement_flags(kq, mix, gn, fp32), int(compute_units),
                                             ctypes.byref(n), ctypes.byref(keys)))
    return n.value, keys.value


def forward_rows_split(q, k, v, theta=None, w=None, gamma=None, beta=None, lam: float = 1.0, *, row_begin: int,
                       c_q: int = 1, c_k: int = 1, c_h: int = 1, kq: Optional[str] = None, mix: Optional[str] = None,
                       gn: bool = False, out=None, workspace=None, stream=None) -> torch.Tensor:
    """``mta_forward_rows_split``: rows row_begin .. T-1 with the key range split over workgroups
    (decode steps, short chunks); rows of ``out`` before row_begin are left as they are."""
    out = _common(q, k, v, out)
    B, T, M, d = q.shape
    _params(q, theta, w, gamma, beta, c_q, c_k, c_h, kq, mix, gn)
    fp32 = q.dtype == torch.float32
    fl = placement_flags(kq, mix, gn, fp32)
    need = rows_split_workspace_bytes(B, T, M, d, row_begin=row_begin, c_q=c_q, c_k=c_k, c_h=c_h, kq=kq, mix=mix,
                                      gn=gn, fp32=fp32)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().mta_forward_rows_split(
        _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dev(theta, "theta", torch.float32),
        _dev(w, "w", torch.float32), _dev(gamma, "gamma", torch.float32), _dev(beta, "beta", torch.float32),
        float(lam), _dev(out, "out"), B, T, M, d, c_q, c_k, c_h, int(row_begin), fl, ws_ptr, ws_bytes,
        _stream(stream)))
    return out


def forward_rows_split_noalloc(q, k, v, theta=None, w=None, gamma=None, beta=None, lam: float = 1.0, *,
                               row_begin: int, out, c_q: int = 1, c_k: int = 1, c_h: int = 1,
                               kq: Optional[str] = None, mix: Optional[str] = None, gn: bool = False,
                               stream=None) -> torch.Tensor:
    """``mta_forward_rows_split_noalloc``: ``forward_rows_split`` with the partial results in the
    library's own device scratch (no workspace, no allocation; ``out`` must be given). Calls that
    overlap on one GPU share that scratch and race."""
    if out is None:
        raise ValueError("out is required (this entry point allocates nothing)")
    out = _common(q, k, v, out)
    B, T, M, d = q.shape
    _params(q, theta, w, gamma, beta, c_q, c_k, c_h, kq, mix, gn)
    fl = placement_flags(kq, mix, gn, q.dtype == torch.float32)
    _check(lib().mta_forward_rows_split_noalloc(
        _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dev(theta, "theta", torch.float32),
        _dev(w, "w", torch.float32), _dev(gamma, "gamma", torch.float32), _dev(beta, "beta", torch.float32),
        float(lam), _dev(out, "out"), B, T, M, d, c_q, c_k, c_h, int(row_begin), fl, _stream(stream)))
    return out


def materialized_workspace_bytes(B: int, T: int, M: int) -> int:
    return int(lib().mta_materialized_workspace_bytes(B, T, M, 0))


def forward_materialized(q, k, v, theta=None, w=None, gamma=None, beta=None, lam: float = 1.0, *,
                         c_q: int = 1, c_k: int = 1, c_h: int = 1, kq: Optional[str] = None,
                         mix: Optional[str] = None, gn: bool = False, out=None, workspace=None,
                         stream=None) -> torch.Tensor:
    """Unfused forward (``mta_forward_materialized``) with fp32 T x T maps in ``workspace``."""
    out = _common(q, k, v, out)
    B, T, M, d = q.shape
    _params(q, theta, w, gamma, beta, c_q, c_k, c_h, kq, mix, gn)
    need = materialized_workspace_bytes(B, T, M)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    fl = placement_flags(kq, mix, gn, q.dtype == torch.float32)
    _check(lib().mta_forward_materialized(
        _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dev(theta, "theta", torch.float32),
        _dev(w, "w", torch.float32), _dev(gamma, "gamma", torch.float32), _dev(beta, "beta", torch.float32),
        float(lam), _dev(out, "out"), B, T, M, d, c_q, c_k, c_h, fl, _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def backward_workspace_bytes(B: int, T: int, M: int, d: int, *, c_q: int = 1, c_k: int = 1, c_h: int = 1,
                             kq: Optional[str] = None, mix: Optional[str] = None, gn: bool = False,
                             fp32: bool = False) -> int:
    return int(lib().mta_backward_workspace_bytes(B, T, M, d, c_q, c_k, c_h, placement_flags(kq, mix, gn, fp32)))


def backward_materialized(q, k, v, theta=None, w=None, gamma=None, beta=None, lam: float = 1.0, *, dout,
                          c_q: int = 1, c_k: int = 1, c_h: int = 1, kq: Optional[str] = None,
                          mix: Optional[str] = None, gn: bool = False, workspace=None, stream=None) -> dict:
    """Gradients (``mta_backward_materialized``) of sum(out * dout). Returns a dict with
    dq, dk, dv (input dtype) and, where the placement has them, dtheta, dw, dgamma, dbeta
    (fp32, parameter shapes) and dlambda (fp32 tensor of one element)."""
    _common(q, k, v, None)
    if dout.shape != q.shape or dout.dtype != q.dtype:
        raise ValueError("dout must match q in shape and dtype")
    B, T, M, d = q.shape
    _params(q, theta, w, gamma, beta, c_q, c_k, c_h, kq, mix, gn)
    fp32 = q.dtype == torch.float32
    fl = placement_flags(kq, mix, gn, fp32)
    g = {"dq": torch.empty_like(q), "dk": torch.empty_like(q), "dv": torch.empty_like(q)}
    g["dtheta"] = torch.empty_like(theta) if kq else None
    g["dw"] = torch.empty_like(w) if mix else None
    g["dgamma"] = torch.empty_like(gamma) if gn else None
    g["dbeta"] = torch.empty_like(beta) if gn else None
    g["dlambda"] = torch.empty(1, dtype=torch.float32, device=q.device) if gn else None
    need = backward_workspace_bytes(B, T, M, d, c_q=c_q, c_k=c_k, c_h=c_h, kq=kq, mix=mix, gn=gn, fp32=fp32)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib().mta_backward_materialized(
        _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dev(theta, "theta", torch.float32),
        _dev(w, "w", torch.float32), _dev(gamma, "gamma", torch.float32), _dev(beta, "beta", torch.float32),
        float(lam), _dev(dout, "dout"), _dev(g["dq"], "dq"), _dev(g["dk"], "dk"), _dev(g["dv"], "dv"),
        _dev(g["dtheta"], "dtheta"), _dev(g["dw"], "dw"), _dev(g["dgamma"], "dgamma"), _dev(g["dbeta"], "dbeta"),
        _dev(g["dlambda"], "dlambda"), B, T, M, d, c_q, c_k, c_h, fl, _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return g


def forward_train(q, k, v, theta=None, w=None, gamma=None, beta=None, lam: float = 1.0, *, c_q: int = 1,
                  c_k: int = 1, c_h: int = 1, kq: Optional[str] = None, mix: Optional[str] = None,
                  gn: bool = False, out=None, lse=None, out_pre_gn=None, stream=None):
    """``mta_forward_train``: the fused forward (bf16) that also keeps what ``backward_fused``
    needs. Returns (out, lse [B, T, M] fp32, out_pre_gn [B, T, M, d] fp32 or None without
    GroupNorm)."""
    out = _common(q, k, v, out)
    B, T, M, d = q.shape
    _params(q, theta, w, gamma, beta, c_q, c_k, c_h, kq, mix, gn)
    if lse is None:
        lse = torch.empty((B, T, M), dtype=torch.float32, device=q.device)
    if out_pre_gn is None and gn:
        out_pre_gn = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if lse.shape != (B, T, M) or (out_pre_gn is not None and out_pre_gn.shape != q.shape):
        raise ValueError("lse must be [B, T, M] and out_pre_gn [B, T, M, d]")
    fl = placement_flags(kq, mix, gn, q.dtype == torch.float32)
    _check(lib().mta_forward_train(
        _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dev(theta, "theta", torch.float32),
        _dev(w, "w", torch.float32), _dev(gamma, "gamma", torch.float32), _dev(beta, "beta", torch.float32),
        float(lam), _dev(out, "out"), _dev(lse, "lse", torch.float32), _dev(out_pre_gn, "out_pre_gn", torch.float32),
        B, T, M, d, c_q, c_k, c_h, fl, _stream(stream)))
    return out, lse, out_pre_gn


def backward_fused_workspace_bytes(B: int, T: int, M: int, d: int, *, c_q: int = 1, c_k: int = 1, c_h: int = 1,
                                   kq: Optional[str] = None, mix: Optional[str] = None, gn: bool = False) -> int:
    return int(lib().mta_backward_fused_workspace_bytes(B, T, M, d, c_q, c_k, c_h, placement_flags(kq, mix, gn, False)))


def backward_fused(q, k, v, theta=None, w=None, gamma=None, beta=None, lam: float = 1.0, *, dout, lse,
                   out_pre_gn=None, c_q: int = 1, c_k: int = 1, c_h: int = 1, kq: Optional[str] = None,
                   mix: Optional[str] = None, gn: bool = False, workspace=None, stream=None) -> dict:
    """Gradients of sum(out * dout) by the fused backward (``mta_backward_fused``), from the
    ``lse`` and ``out_pre_gn`` of ``forward_train``. Returns the same dict as
    ``backward_materialized``."""
    _common(q, k, v, None)
    if dout.shape != q.shape or dout.dtype != q.dtype:
        raise ValueError("dout must match q in shape and dtype")
    B, T, M, d = q.shape
    _params(q, theta, w, gamma, beta, c_q, c_k, c_h, kq, mix, gn)
    fl = placement_flags(kq, mix, gn, q.dtype == torch.float32)
    g = {"dq": torch.empty_like(q), "dk": torch.empty_like(q), "dv": torch.empty_like(q)}
    g["dtheta"] = torch.empty_like(theta) if kq else None
    g["dw"] = torch.empty_like(w) if mix else None
    g["dgamma"] = torch.empty_like(gamma) if gn else None
    g["dbeta"] = torch.empty_like(beta) if gn else None
    g["dlambda"] = torch.empty(1, dtype=torch.float32, device=q.device) if gn else None
    need = backward_fused_workspace_bytes(B, T, M, d, c_q=c_q, c_k=c_k, c_h=c_h, kq=kq, mix=mix, gn=gn)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().mta_backward_fused(
        _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dev(theta, "theta", torch.float32),
        _dev(w, "w", torch.float32), _dev(gamma, "gamma", torch.float32), _dev(beta, "beta", torch.float32),
        float(lam), _dev(lse, "lse", torch.float32), _dev(out_pre_gn, "out_pre_gn", torch.float32),
        _dev(dout, "dout"), _dev(g["dq"], "dq"), _dev(g["dk"], "dk"), _dev(g["dv"], "dv"),
        _dev(g["dtheta"], "dtheta"), _dev(g["dw"], "dw"), _dev(g["dgamma"], "dgamma"), _dev(g["dbeta"], "dbeta"),
        _dev(g["dlambda"], "dlambda"), B, T, M, d, c_q, c_k, c_h, fl, _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return g


def attention_plain(q, k, v, *, out=None, stream=None) -> torch.Tensor:
    """Plain causal attention (``mta_attention_plain``)."""
    out = _common(q, k, v, out)
    B, T, M, d = q.shape
    fl = FP32 if q.dtype == torch.float32 else 0
    _check(lib().mta_attention_plain(_dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
                                     _dev(out, "out"), B, T, M, d, fl, _stream(stream)))
    return out


def check_args(q_ptr, k_ptr, v_ptr, theta_ptr, w_ptr, gamma_ptr, beta_ptr, out_ptr, B, T, M, d, c_q, c_k,
               c_h, flags) -> int:
    """Host-only validation (``mta_check_args``) on raw pointer values; returns the status."""
    return int(lib().mta_check_args(q_ptr, k_ptr, v_ptr, theta_ptr, w_ptr, gamma_ptr, beta_ptr, out_ptr,
                                    B, T, M, d, c_q, c_k, c_h, flags))


def last_error() -> str:
    return lib().mta_last_error().decode()


class _MTATrainFn(torch.autograd.Function):
    """Autograd node of the layer. bf16: ``forward_train`` in the forward and ``backward_fused``
    in the backward, or ``backward_materialized`` for the placements whose fused tiles do not fit
    the LDS (the library reports them unsupported); fp32: ``forward`` and
    ``backward_materialized``. The gate value enters as a float; its gradient is returned for a
    ``lam`` tensor only."""

    @staticmethod
    def forward(ctx, q, k, v, theta, w, gamma, beta, lam_t, lam, cfg):
        c_q, c_k, c_h, kq, mix, gn = cfg
        kw = dict(c_q=c_q, c_k=c_k, c_h=c_h, kq=kq, mix=mix, gn=gn)
        if q.dtype == torch.float32:
            out, lse, o32 = forward(q, k, v, theta, w, gamma, beta, lam, **kw), None, None
        else:
            out, lse, o32 = forward_train(q, k, v, theta, w, gamma, beta, lam, **kw)
        ctx.save_for_backward(q, k, v, theta, w, gamma, beta, lse, o32)
        ctx.lam, ctx.cfg = lam, cfg
        ctx.lam_shape = lam_t.shape if lam_t is not None else None
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, theta, w, gamma, beta, lse, o32 = ctx.saved_tensors
        c_q, c_k, c_h, kq, mix, gn = ctx.cfg
        kw = dict(c_q=c_q, c_k=c_k, c_h=c_h, kq=kq, mix=mix, gn=gn)
        dout = dout.contiguous()
        g = None
        if lse is not None:
            try:
                g = backward_fused(q, k, v, theta, w, gamma, beta, ctx.lam, dout=dout, lse=lse, out_pre_gn=o32, **kw)
            except MTAError as e:
                if e.status != ERR_UNSUPPORTED:
                    raise
        if g is None:
            g = backward_materialized(q, k, v, theta, w, gamma, beta, ctx.lam, dout=dout, **kw)
        dlam = None
        if ctx.lam_shape is not None:
            dlam = g["dlambda"].reshape(ctx.lam_shape) if gn else torch.zeros(ctx.lam_shape, device=q.device)
        return (g["dq"], g["dk"], g["dv"], g["dtheta"], g["dw"], g["dgamma"], g["dbeta"], dlam, None, None)


def mta_layer(q, k, v, theta=None, w=None, gamma=None, beta=None, lam=1.0, *, c_q: int = 1, c_k: int = 1,
              c_h: int = 1, kq: Optional[str] = None, mix: Optional[str] = None,
              gn: bool = False) -> torch.Tensor:
    """The layer as a differentiable torch operation (bf16 or fp32 q, k, v on the GPU): the
    fused forward, and on ``loss.backward()`` the gradients of q, k, v, theta, w, gamma, beta
    and, if ``lam`` is a tensor, of the gate value (read once with ``.item()``, which waits for
    the device). bf16 takes the fused backward (the unfused one where the fused tiles do not
    fit), fp32 the unfused backward. Parameters are fp32 tensors in the shapes ``forward``
    takes."""
    lam_t = lam if isinstance(lam, torch.Tensor) else None
    lam_f = float(lam_t.detach().item()) if lam_t is not None else float(lam)
    cfg = (c_q, c_k, c_h, kq, mix, gn)
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    return _MTATrainFn.apply(q, k, v, theta, w, gamma, beta, lam_t, lam_f, cfg)
