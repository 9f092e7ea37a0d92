"""fp64 CPU oracle of the layer's gradients (test infrastructure only).

The forward pass of the page "Multi-Token Attention | Summary" (greeksharifa.github.io)
written once more, as plain PyTorch CPU operations on whole T x T maps in float64, so
that autograd yields the exact gradients of every input and parameter: §2 (logits
QK^T/sqrt(d), causal softmax, AV), §3.1 (key-query convolution: Mask_0 before it and
Mask_-inf after it before softmax; Mask_0 after it after softmax), §3.2 (head mixing
in groups of c_h heads), §3.3 (per-head GroupNorm and scalar gate); each convolution
or mixing may act before softmax, after it, or on both sides (§4), with the same
composition order as ``mta_oracle.cpp``.

It shares no code with the C++ oracle or the GPU library. Its forward is pinned to
the C++ oracle and its gradients to central finite differences of the C++ oracle.
"""
from __future__ import annotations

import math

import numpy as np
import torch

_DT = torch.float64


def _sides(placement, params):
    """(before-softmax, after-softmax) parameters of a placement; None where absent."""
    if placement == "both":
        return params[0], params[1]
    return (params if placement == "pre" else None), (params if placement == "post" else None)


def _conv(Z, th):
    """Y[b,m,i,j] = sum_{a,e} th[m,a,e] * Z[b,m,i-a,j-e+h0], zero outside the map (§3.1)."""
    T = Z.shape[-1]
    c_q, c_k = th.shape[-2], th.shape[-1]
    h0 = (c_k - 1) // 2
    # pad[i + c_q - 1][j + h0] = Z[i][j]
    pad = torch.nn.functional.pad(Z, (h0, h0, c_q - 1, 0))
    Y = torch.zeros_like(Z)
    for a in range(c_q):
        for e in range(c_k):
            # Z[i-a][j-e+h0] = pad[i-a+c_q-1][j-e+2h0]
            shifted = pad[..., c_q - 1 - a:c_q - 1 - a + T, 2 * h0 - e:2 * h0 - e + T]
            Y = Y + th[:, a, e].reshape(1, -1, 1, 1) * shifted
    return Y


def _mix(X, w, c_h):
    """X_u <- sum_u' w[g][u][u'] X_u' within each group of c_h heads (§3.2)."""
    B, M, T, _ = X.shape
    Xg = X.reshape(B, M // c_h, c_h, T, T)
    return torch.einsum("guv,bgvij->bguij", w, Xg).reshape(B, M, T, T)


def _softmax_input(q, k, theta, w, *, c_h, kq, mix):
    """The logits that enter the softmax, [B,M,T,T] with -inf above the diagonal (§2, §3.1, §3.2)."""
    T, d = q.shape[1], q.shape[3]
    th_pre, _ = _sides(kq, theta)
    w_pre, _ = _sides(mix, w)
    qh, kh = (x.permute(0, 2, 1, 3) for x in (q, k))  # [B,M,T,d]
    future = torch.triu(torch.ones(T, T, dtype=torch.bool), 1)
    L = qh @ kh.transpose(-1, -2) / math.sqrt(d)
    if w_pre is not None:
        L = _mix(L, w_pre, c_h)
    if th_pre is not None:
        L = _conv(L.masked_fill(future, 0.0), th_pre)
    return L.masked_fill(future, -math.inf)


def forward_torch(q, k, v, theta, w, gamma, beta, lam, *, c_q, c_k, c_h, kq, mix, gn):
    """The layer on float64 torch tensors (q, k, v [B,T,M,d]); returns out [B,T,M,d]."""
    B, T, M, d = q.shape
    th_post = _sides(kq, theta)[1]
    w_post = _sides(mix, w)[1]
    vh = v.permute(0, 2, 1, 3)  # [B,M,T,d]
    future = torch.triu(torch.ones(T, T, dtype=torch.bool), 1)
    A = torch.softmax(_softmax_input(q, k, theta, w, c_h=c_h, kq=kq, mix=mix), dim=-1)
    if th_post is not None:
        A = _conv(A, th_post).masked_fill(future, 0.0)
    if w_post is not None:
        A = _mix(A, w_post, c_h)
    O = (A @ vh).permute(0, 2, 1, 3)  # [B,T,M,d]
    if gn:
        mu = O.mean(dim=-1, keepdim=True)
        var = ((O - mu) ** 2).mean(dim=-1, keepdim=True)
        O = lam * (gamma.reshape(M, d) * (O - mu) / torch.sqrt(var + 1e-5) + beta.reshape(M, d))
    return O


def row_logsumexp(q, k, theta=None, w=None, *, c_q=1, c_k=1, c_h=1, kq=None, mix=None):
    """Natural log-sum-exp of every softmax row, [B,T,M] float64: log sum_{j<=i} exp(C[i][j])
    over the logits C that enter the softmax (after the convolution and mixing before it)."""
    del c_q, c_k  # the shapes of theta carry them

    def t(x):
        return None if x is None else torch.tensor(np.asarray(x, dtype=np.float64), dtype=_DT)

    C = _softmax_input(t(q), t(k), t(theta) if kq else None, t(w) if mix else None, c_h=c_h, kq=kq, mix=mix)
    return torch.logsumexp(C, dim=-1).permute(0, 2, 1).numpy().copy()


def backward(q, k, v, theta, w, gamma, beta, lam, dout, *, c_q=1, c_k=1, c_h=1, kq=None, mix=None, gn=False):
    """Gradients of sum(out * dout) with respect to every input, in float64.

    Array arguments are numpy arrays (or None where the placement does not use them);
    returns a dict with ``out`` and ``dq``, ``dk``, ``dv``, ``dtheta`` (shape of theta),
    ``dw`` (shape of w), ``dgamma``, ``dbeta``, ``dlambda`` (None where unused).
    """
    def leaf(x):
        return None if x is None else torch.tensor(np.asarray(x, dtype=np.float64), dtype=_DT, requires_grad=True)

    tq, tk, tv = leaf(q), leaf(k), leaf(v)
    tth = leaf(theta) if kq is not None else None
    tw = leaf(w) if mix is not None else None
    tg = leaf(gamma) if gn else None
    tb = leaf(beta) if gn else None
    tl = leaf(np.float64(lam)) if gn else None
    out = forward_torch(tq, tk, tv, tth, tw, tg, tb, tl, c_q=c_q, c_k=c_k, c_h=c_h, kq=kq, mix=mix, gn=gn)
    out.backward(torch.tensor(np.asarray(dout, dtype=np.float64), dtype=_DT))

    def grad(x):
        return None if x is None else x.grad.detach().numpy().copy()

    return {"out": out.detach().numpy(), "dq": grad(tq), "dk": grad(tk), "dv": grad(tv), "dtheta": grad(tth),
            "dw": grad(tw), "dgamma": grad(tg), "dbeta": grad(tb),
            "dlambda": None if tl is None else float(tl.grad)}
