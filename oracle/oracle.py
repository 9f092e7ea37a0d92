"""ctypes front end of the C++ fp64 oracle (test infrastructure only)."""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mta_oracle.cpp")
_LIB = os.path.join(_HERE, "libmta_oracle.so")
_lib = None

# placement bits: 1 before softmax, 2 after softmax, 3 both sides
_SIDES = {None: 0, "pre": 1, "post": 2, "both": 3}


def library_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (-O3, OpenMP) into ``oracle/libmta_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["g++", "-O3", "-march=x86-64-v3", "-fopenmp", "-std=c++17", "-shared", "-fPIC",
               "-Wall", "-Wextra", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.mta_oracle_forward.argtypes = [dp, dp, dp, dp, dp, dp, dp, ctypes.c_double, dp] + \
            [ctypes.c_int] * 10 + [ctypes.POINTER(ctypes.c_int), ctypes.c_int, dp, ctypes.c_int]
        lib.mta_oracle_forward.restype = ctypes.c_int
        lib.mta_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().mta_oracle_max_threads())


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def forward(q, k, v, theta=None, w=None, gamma=None, beta=None, lam: float = 1.0, *,
            c_q: int = 1, c_k: int = 1, c_h: int = 1, kq: Optional[str] = None,
            mix: Optional[str] = None, gn: bool = False, rows=None, return_maps: bool = False,
            n_threads: int = 0):
    """Evaluate the layer in fp64.

    q, k, v: ``[B, T, M, d]``. ``kq`` and ``mix`` are ``None``, ``"pre"``, ``"post"`` or
    ``"both"`` (before and after softmax, each side with its own parameters). theta
    ``[M, c_q, c_k]`` (``[2, M, c_q, c_k]`` for ``"both"``: the kernels before softmax,
    then those after); w ``[M/c_h, c_h, c_h]`` (``[2, M/c_h, c_h, c_h]`` for ``"both"``);
    gamma, beta ``[M*d]``. ``rows``: optional list of query rows to compute (all
    otherwise). Returns ``out`` (``[B, T, M, d]`` float64; rows not requested are
    NaN) and, with ``return_maps``, the attention rows applied to V
    (``[B, M, n_rows, T]``).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, M, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    if kq is None:
        c_q = c_k = 1
    n_kq = 2 if kq == "both" else 1
    n_mix = 2 if mix == "both" else 1
    th = _f64(theta) if kq is not None else np.zeros((M, c_q, c_k))
    ww = _f64(w) if mix is not None else np.zeros((M // c_h, c_h, c_h))
    ga = _f64(gamma) if gn else np.ones(M * d)
    be = _f64(beta) if gn else np.zeros(M * d)
    assert th.shape == ((n_kq,) if n_kq > 1 else ()) + (M, c_q, c_k), th.shape
    assert ww.shape == ((n_mix,) if n_mix > 1 else ()) + (M // c_h, c_h, c_h), ww.shape
    out = np.full((B, T, M, d), np.nan)
    if rows is None:
        rows_arr, n_rows, rows_ptr = None, T, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
        n_rows = int(rows_arr.size)
        rows_ptr = rows_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int))
    maps = np.zeros((B, M, n_rows, T)) if return_maps else None
    rc = _load().mta_oracle_forward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(th), _ptr(ww), _ptr(ga), _ptr(be), float(lam), _ptr(out),
        B, T, M, d, c_q, c_k, c_h, _SIDES[kq], _SIDES[mix], int(bool(gn)), rows_ptr,
        n_rows if rows_arr is not None else 0, _ptr(maps), int(n_threads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return (out, maps) if return_maps else out


def forward_cfg(cfg, inputs: dict, rows=None, return_maps: bool = False, n_threads: int = 0):
    """``forward`` with the sizes and placement of an ``mta_inputs.MTAConfig``."""
    return forward(inputs["q"], inputs["k"], inputs["v"], inputs["theta"], inputs["w"],
                   inputs["gamma"], inputs["beta"], inputs["lam"], c_q=cfg.c_q, c_k=cfg.c_k,
                   c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn, rows=rows,
                   return_maps=return_maps, n_threads=n_threads)
