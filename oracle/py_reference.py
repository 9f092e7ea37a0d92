"""Second, pure-Python fp64 transcription of the layer (test infrastructure only).

Written independently of ``mta_oracle.cpp`` (whole maps with explicit padding
instead of per-row lookups) so that an indexing slip in either shows up as a
disagreement on tiny inputs. It follows the same page, "Multi-Token Attention |
Summary": §2 (logits, causal softmax, AV), §3.1 (key-query convolution with the
two masks), §3.2 (head mixing), §3.3 (GroupNorm and scalar gate).
"""
from __future__ import annotations

import math

import numpy as np


def _conv_full(Z: np.ndarray, th: np.ndarray) -> np.ndarray:
    """Y[i][j] = sum_{a,e} th[a][e] * Z[i-a][j-e+h0] with zero padding (T x T map)."""
    T = Z.shape[0]
    c_q, c_k = th.shape
    h0 = (c_k - 1) // 2
    pad = np.zeros((T + c_q - 1, T + 2 * h0))
    pad[c_q - 1:, h0:h0 + T] = Z  # pad[r + c_q - 1][s + h0] = Z[r][s]
    Y = np.zeros((T, T))
    for i in range(T):
        for j in range(T):
            acc = 0.0
            for a in range(c_q):
                for e in range(c_k):
                    # Z[i-a][j-e+h0] lives at pad[i-a+c_q-1][j-e+2*h0]
                    acc += th[a, e] * pad[i - a + c_q - 1, j - e + 2 * h0]
            Y[i, j] = acc
    return Y


def _sides(placement, params):
    """(before-softmax, after-softmax) parameters of a placement; None where absent."""
    if placement == "both":
        return params[0], params[1]
    return (params if placement == "pre" else None), (params if placement == "post" else None)


def forward(q, k, v, theta, w, gamma, beta, lam, *, c_q, c_k, c_h, kq, mix, gn):
    """kq / mix: None, "pre", "post" or "both"; with "both" theta / w hold the
    before-softmax parameters at index 0 and the after-softmax ones at index 1."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, M, d = q.shape
    th_pre, th_post = _sides(kq, theta)
    w_pre, w_post = _sides(mix, w)
    out = np.zeros((B, T, M, d))
    future = np.triu(np.ones((T, T), dtype=bool), 1)  # j > i
    for b in range(B):
        for g in range(M // c_h):
            heads = [g * c_h + u for u in range(c_h)]
            logit = [q[b, :, m, :] @ k[b, :, m, :].T / math.sqrt(d) for m in heads]
            if w_pre is not None:
                logit = [sum(w_pre[g, u, x] * logit[x] for x in range(c_h)) for u in range(c_h)]
            A = []
            for u, m in enumerate(heads):
                L = logit[u]
                if th_pre is not None:
                    L = _conv_full(np.where(future, 0.0, L), np.asarray(th_pre[m], np.float64))
                L = np.where(future, -np.inf, L)
                P = np.exp(L - L.max(axis=1, keepdims=True))
                P = P / P.sum(axis=1, keepdims=True)
                if th_post is not None:
                    P = np.where(future, 0.0, _conv_full(P, np.asarray(th_post[m], np.float64)))
                A.append(P)
            if w_post is not None:
                A = [sum(w_post[g, u, x] * A[x] for x in range(c_h)) for u in range(c_h)]
            for u, m in enumerate(heads):
                O = A[u] @ v[b, :, m, :]
                if gn:
                    mu = O.mean(axis=1, keepdims=True)
                    var = ((O - mu) ** 2).mean(axis=1, keepdims=True)
                    O = lam * (np.asarray(gamma[m * d:(m + 1) * d]) * (O - mu) / np.sqrt(var + 1e-5)
                               + np.asarray(beta[m * d:(m + 1) * d]))
                out[b, :, m, :] = O
    return out
