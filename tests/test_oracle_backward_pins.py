"""Pins of the fp64 gradient oracle (``oracle/backward.py``).

Page: "Multi-Token Attention | Summary" (greeksharifa.github.io). The gradient oracle
differentiates its own plain PyTorch forward; these tests tie that forward to the C++
oracle, its gradients to central finite differences of the C++ oracle (an independent
implementation), and special cases to library routines (torch SDPA and layer_norm
under autograd).
"""
import math

import numpy as np
import pytest
import torch

from oracle import backward as bw
from oracle import oracle

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")

PLACEMENTS = [("pre", "post", True), ("post", "pre", True), ("both", "both", True), (None, None, False),
              ("pre", "pre", False), ("post", "post", True), ("both", None, False), (None, "both", True)]


def _problem(kq, mix, gn, seed, B=1, T=11, M=4, d=4, c_q=3, c_k=5, c_h=2):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, T, M, d)) for _ in range(3))
    th = rng.standard_normal(((2,) if kq == "both" else ()) + (M, c_q, c_k)) * 0.4
    w = rng.standard_normal(((2,) if mix == "both" else ()) + (M // c_h, c_h, c_h)) * 0.6
    gamma, beta = rng.standard_normal(M * d), rng.standard_normal(M * d)
    dout = rng.standard_normal((B, T, M, d))
    kw = dict(c_q=c_q, c_k=c_k, c_h=c_h, kq=kq, mix=mix, gn=gn)
    return dict(q=q, k=k, v=v, theta=th, w=w, gamma=gamma, beta=beta, lam=0.7), dout, kw


@pytest.mark.parametrize("kq,mix,gn", PLACEMENTS)
def test_torch_forward_matches_cpp_oracle(kq, mix, gn):
    x, dout, kw = _problem(kq, mix, gn, 1, B=2, T=13)
    g = bw.backward(x["q"], x["k"], x["v"], x["theta"], x["w"], x["gamma"], x["beta"], x["lam"], dout, **kw)
    ref = oracle.forward(x["q"], x["k"], x["v"], x["theta"], x["w"], x["gamma"], x["beta"], x["lam"], **kw)
    np.testing.assert_allclose(g["out"], ref, atol=1e-12)


@pytest.mark.parametrize("kq,mix,gn", PLACEMENTS)
def test_gradients_match_finite_differences_of_cpp_oracle(kq, mix, gn):
    # F(x) = <out(x), dout>; for each input a random direction U: <dF/dx, U> against
    # (F(x + hU) - F(x - hU)) / 2h evaluated with the C++ oracle.
    x, dout, kw = _problem(kq, mix, gn, 2)
    g = bw.backward(x["q"], x["k"], x["v"], x["theta"], x["w"], x["gamma"], x["beta"], x["lam"], dout, **kw)

    def F(xx):
        out = oracle.forward(xx["q"], xx["k"], xx["v"], xx["theta"], xx["w"], xx["gamma"], xx["beta"], xx["lam"],
                             **kw)
        return float((out * dout).sum())

    names = ["q", "k", "v"] + (["theta"] if kq else []) + (["w"] if mix else []) + \
        (["gamma", "beta", "lam"] if gn else [])
    grad_of = {"q": "dq", "k": "dk", "v": "dv", "theta": "dtheta", "w": "dw", "gamma": "dgamma", "beta": "dbeta",
               "lam": "dlambda"}
    rng = np.random.default_rng(3)
    h = 1e-5
    for n in names:
        U = rng.standard_normal(np.shape(x[n]))
        plus, minus = dict(x), dict(x)
        plus[n] = x[n] + h * U
        minus[n] = x[n] - h * U
        fd = (F(plus) - F(minus)) / (2 * h)
        an = float(np.sum(np.asarray(g[grad_of[n]]) * U))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (n, fd, an)


def test_identity_kernels_give_sdpa_gradients():
    # theta = delta, w = I, no GroupNorm: the layer is plain causal attention, so its
    # gradients are those of torch's scaled_dot_product_attention (fp64 autograd).
    x, dout, kw = _problem("both", "both", False, 4, B=2, T=17, M=4, d=8)
    c_q, c_k, c_h, M = kw["c_q"], kw["c_k"], kw["c_h"], 4
    th = np.zeros((2, M, c_q, c_k))
    th[:, :, 0, (c_k - 1) // 2] = 1.0
    w = np.stack([np.tile(np.eye(c_h), (M // c_h, 1, 1))] * 2)
    g = bw.backward(x["q"], x["k"], x["v"], th, w, None, None, 1.0, dout, **kw)
    tq, tk, tv = (torch.tensor(x[n], requires_grad=True) for n in ("q", "k", "v"))
    o = torch.nn.functional.scaled_dot_product_attention(tq.permute(0, 2, 1, 3), tk.permute(0, 2, 1, 3),
                                                         tv.permute(0, 2, 1, 3), is_causal=True)
    o.permute(0, 2, 1, 3).backward(torch.tensor(dout))
    for n, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(g[n], t.grad.numpy(), atol=1e-12, err_msg=n)


def test_groupnorm_gate_gradients_match_layer_norm():
    # No convolution or mixing: out = lambda * layer_norm(SDPA(q, k, v)) per head.
    B, T, M, d = 2, 9, 2, 8
    x, dout, kw = _problem(None, None, True, 5, B=B, T=T, M=M, d=d)
    g = bw.backward(x["q"], x["k"], x["v"], None, None, x["gamma"], x["beta"], x["lam"], dout, **kw)
    tq, tk, tv = (torch.tensor(x[n], requires_grad=True) for n in ("q", "k", "v"))
    tg, tb = torch.tensor(x["gamma"], requires_grad=True), torch.tensor(x["beta"], requires_grad=True)
    tl = torch.tensor(x["lam"], dtype=torch.float64, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(tq.permute(0, 2, 1, 3), tk.permute(0, 2, 1, 3),
                                                         tv.permute(0, 2, 1, 3), is_causal=True).permute(0, 2, 1, 3)
    y = torch.stack([tl * torch.nn.functional.layer_norm(o[:, :, m], (d,), tg[m * d:(m + 1) * d],
                                                         tb[m * d:(m + 1) * d], eps=1e-5) for m in range(M)], dim=2)
    y.backward(torch.tensor(dout))
    for n, t in (("dq", tq), ("dk", tk), ("dv", tv), ("dgamma", tg), ("dbeta", tb)):
        np.testing.assert_allclose(g[n], t.grad.numpy(), atol=1e-12, err_msg=n)
    assert math.isclose(g["dlambda"], float(tl.grad), rel_tol=1e-12, abs_tol=1e-12)


# ---- the per-row log-sum-exp that the training forward reports and the fused backward uses
def _brute_lse(S, i):
    """log sum_{j <= i} exp(S[j]) by a plain loop."""
    return math.log(math.fsum(math.exp(S[j]) for j in range(i + 1)))


def _dots(x, b, i, m):
    """q_i . k_j / sqrt(d) for every j, by plain loops."""
    d = x["q"].shape[3]
    return [sum(x["q"][b, i, m, t] * x["k"][b, j, m, t] for t in range(d)) / math.sqrt(d)
            for j in range(x["q"].shape[1])]


def test_row_logsumexp_plain_attention_by_brute_force():
    x, _, _ = _problem(None, None, False, 6, B=2, T=7, M=2, d=4)
    got = bw.row_logsumexp(x["q"], x["k"])
    for b in range(2):
        for m in range(2):
            for i in range(7):
                assert math.isclose(got[b, i, m], _brute_lse(_dots(x, b, i, m), i), rel_tol=0, abs_tol=1e-12)


def test_row_logsumexp_closed_forms_of_the_convolution():
    # theta = alpha delta(0, h0): the logits scaled by alpha. theta = delta(1, h0): row i sees the
    # previous row's logits at keys j < i and a zero-padded logit at j = i; row 0 sees one zero.
    B, T, M, d, c_q, c_k = 1, 6, 2, 4, 2, 3
    x, _, _ = _problem(None, None, False, 7, B=B, T=T, M=M, d=d)
    h0 = (c_k - 1) // 2
    th = np.zeros((M, c_q, c_k))
    th[:, 0, h0] = 1.7
    got = bw.row_logsumexp(x["q"], x["k"], th, c_q=c_q, c_k=c_k, kq="pre")
    lag = np.zeros((M, c_q, c_k))
    lag[:, 1, h0] = 1.0
    got_lag = bw.row_logsumexp(x["q"], x["k"], lag, c_q=c_q, c_k=c_k, kq="pre")
    for m in range(M):
        for i in range(T):
            S = _dots(x, 0, i, m)
            assert math.isclose(got[0, i, m], _brute_lse([1.7 * s for s in S], i), abs_tol=1e-12)
            row = (_dots(x, 0, i - 1, m)[:i] if i > 0 else []) + [0.0]
            assert math.isclose(got_lag[0, i, m], _brute_lse(row, i), abs_tol=1e-12)


def test_row_logsumexp_permutation_mixing_and_post_steps():
    # Mixing before softmax by a permutation renames the heads' logits; the steps after softmax
    # do not change the softmax input at all.
    x, _, _ = _problem(None, None, False, 8, B=1, T=9, M=4, d=4)
    perm = [2, 0, 3, 1]
    w = np.zeros((1, 4, 4))
    for u, v in enumerate(perm):
        w[0, u, v] = 1.0
    plain = bw.row_logsumexp(x["q"], x["k"])
    mixed = bw.row_logsumexp(x["q"], x["k"], None, w, c_h=4, mix="pre")
    np.testing.assert_allclose(mixed, plain[:, :, perm], atol=1e-12)
    th = np.random.default_rng(9).standard_normal((4, 3, 5))
    post = bw.row_logsumexp(x["q"], x["k"], th, w, c_q=3, c_k=5, c_h=4, kq="post", mix="post")
    np.testing.assert_allclose(post, plain, atol=1e-12)
