"""Pins of the fp64 oracle to facts fixed by the page and by mathematics.

Page: "Multi-Token Attention | Summary" (greeksharifa.github.io). Each test names
the passage it relies on. None of these tests compares the oracle with itself:
the expected values come from library routines (torch SDPA / layer_norm in
float64), closed forms of special kernels, invariants, a hand-worked example and
an independent pure-Python transcription.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import mta_inputs
from oracle import oracle
from oracle import py_reference

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(B, T, M, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((B, T, M, d)) for _ in range(3)]


def _delta(M, c_q, c_k, a=0, e=None, scale=1.0):
    th = np.zeros((M, c_q, c_k))
    th[:, a, (c_k - 1) // 2 if e is None else e] = scale
    return th


def _eye(M, c_h):
    return np.tile(np.eye(c_h), (M // c_h, 1, 1))


def _sdpa(q, k, v, scale=None):
    """torch SDPA (causal) in float64 on [B, T, M, d] arrays."""
    tq = torch.from_numpy(np.ascontiguousarray(q)).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.ascontiguousarray(k)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(np.ascontiguousarray(v)).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def _softmax_rows(L):
    L = L - L.max(axis=-1, keepdims=True)
    P = np.exp(L)
    return P / P.sum(axis=-1, keepdims=True)


# --- (a) identity kernels reduce to plain causal attention ------------------------
# Identity initialisation of both convolutions leaves standard attention unchanged
# (§4.6 ablation on initialisation; Appendix I inserts identity-initialised MTA into
# pretrained models).
@pytest.mark.parametrize("kq,mix,c_q,c_k,c_h", [("pre", "post", 3, 5, 2), ("post", "pre", 4, 9, 4),
                                                ("pre", "post", 6, 11, 4), (None, None, 1, 1, 1),
                                                ("both", "both", 3, 5, 2)])
def test_identity_kernels_equal_sdpa(kq, mix, c_q, c_k, c_h):
    B, T, M, d = 2, 37, 4, 8
    q, k, v = _rand(B, T, M, d, 1)
    th, w = _delta(M, c_q, c_k), _eye(M, c_h)
    if kq == "both":
        th = np.stack([th, th])
    if mix == "both":
        w = np.stack([w, w])
    out = oracle.forward(q, k, v, th, w, c_q=c_q, c_k=c_k, c_h=c_h, kq=kq, mix=mix, gn=False)
    np.testing.assert_allclose(out, _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_scaled_delta_changes_temperature():
    # theta = alpha * delta(0, centre): conv(Mask_0(S)) = alpha*S on j <= i, so the
    # pre-softmax equation (§3.1) gives softmax(alpha * QK^T / sqrt(d)).
    B, T, M, d, c_q, c_k = 1, 29, 2, 8, 3, 5
    q, k, v = _rand(B, T, M, d, 2)
    alpha = 1.7
    out = oracle.forward(q, k, v, _delta(M, c_q, c_k, scale=alpha), None, c_q=c_q, c_k=c_k, c_h=1,
                         kq="pre")
    np.testing.assert_allclose(out, _sdpa(q, k, v, scale=alpha / math.sqrt(d)), atol=1e-12)


def _plain_logits(q, k):
    d = q.shape[-1]
    return np.einsum("bimc,bjmc->bmij", q, k) / math.sqrt(d)


def test_pre_query_lag_kernel():
    # theta = delta(1, centre): row i reads the logits of row i-1 (query axis only
    # looks at current and past rows, §3.1). Mask_0 removes S[i-1][i], so row i's
    # logits are [S[i-1][0..i-1], 0]; row 0 reads a padded row and gets [0].
    B, T, M, d, c_q, c_k = 1, 23, 2, 8, 2, 3
    q, k, v = _rand(B, T, M, d, 3)
    out = oracle.forward(q, k, v, _delta(M, c_q, c_k, a=1), None, c_q=c_q, c_k=c_k, c_h=1, kq="pre")
    S = _plain_logits(q, k)
    exp = np.zeros_like(out)
    for m in range(M):
        for i in range(T):
            row = np.array([S[0, m, i - 1, j] if j < i else 0.0 for j in range(i + 1)])
            exp[0, i, m] = _softmax_rows(row) @ v[0, :i + 1, m]
    np.testing.assert_allclose(out, exp, atol=1e-12)


@pytest.mark.parametrize("shift", [+1, -1, +2])
def test_pre_key_shift_kernel(shift):
    # theta = delta(0, centre+shift) pins the key-axis direction of the kernel:
    # logit[i][j] = Z[i][j-shift] (zero outside the map and where j-shift > i).
    B, T, M, d, c_q, c_k = 1, 21, 2, 8, 1, 5
    q, k, v = _rand(B, T, M, d, 4)
    h0 = (c_k - 1) // 2
    out = oracle.forward(q, k, v, _delta(M, c_q, c_k, e=h0 + shift), None, c_q=c_q, c_k=c_k, c_h=1,
                         kq="pre")
    S = _plain_logits(q, k)
    exp = np.zeros_like(out)
    for m in range(M):
        for i in range(T):
            row = np.array([S[0, m, i, j - shift] if 0 <= j - shift <= i else 0.0 for j in range(i + 1)])
            exp[0, i, m] = _softmax_rows(row) @ v[0, :i + 1, m]
    np.testing.assert_allclose(out, exp, atol=1e-12)


def test_post_query_lag_kernel():
    # After softmax (§3.1, weights combined additively) a delta(1, centre) kernel
    # hands row i the weights of row i-1: O_i = O^plain_{i-1}, O_0 = 0.
    B, T, M, d, c_q, c_k = 2, 19, 2, 8, 3, 3
    q, k, v = _rand(B, T, M, d, 5)
    out = oracle.forward(q, k, v, _delta(M, c_q, c_k, a=1), None, c_q=c_q, c_k=c_k, c_h=1, kq="post")
    plain = _sdpa(q, k, v)
    np.testing.assert_allclose(out[:, 1:], plain[:, :-1], atol=1e-12)
    np.testing.assert_allclose(out[:, 0], 0.0, atol=0)


def test_post_key_shift_kernel():
    # delta(0, centre+1) after softmax: C[i][j] = A[i][j-1] for 1 <= j <= i, so
    # O_i = sum_{s < i} A[i][s] v_{s+1}; the weight A[i][i] is pushed past the
    # diagonal and removed by Mask_0.
    B, T, M, d, c_q, c_k = 1, 17, 2, 8, 1, 3
    q, k, v = _rand(B, T, M, d, 6)
    out = oracle.forward(q, k, v, _delta(M, c_q, c_k, e=2), None, c_q=c_q, c_k=c_k, c_h=1, kq="post")
    S = _plain_logits(q, k)
    exp = np.zeros_like(out)
    for m in range(M):
        for i in range(T):
            A = _softmax_rows(S[0, m, i, :i + 1])
            exp[0, i, m] = sum(A[s] * v[0, s + 1, m] for s in range(i))
    np.testing.assert_allclose(out, exp, atol=1e-12)


def test_post_conv_is_linear_in_theta():
    B, T, M, d, c_q, c_k = 1, 15, 2, 4, 3, 5
    q, k, v = _rand(B, T, M, d, 7)
    rng = np.random.default_rng(8)
    t1, t2 = rng.standard_normal((M, c_q, c_k)), rng.standard_normal((M, c_q, c_k))
    f = lambda th: oracle.forward(q, k, v, th, None, c_q=c_q, c_k=c_k, c_h=1, kq="post")
    np.testing.assert_allclose(f(t1 + 2.5 * t2), f(t1) + 2.5 * f(t2), atol=1e-12)


# --- head mixing (§3.2) and the doubled-rank view (Appendix B) --------------------
def test_post_mix_equals_mixed_value_heads():
    # Mixing weights after softmax: O^u = sum_u' w[u][u'] A^{u'} V^u, i.e. plain
    # attention of head u' applied to the values of head u (Appendix B value view).
    B, T, M, d, c_h = 1, 21, 4, 8, 2
    q, k, v = _rand(B, T, M, d, 9)
    w = np.random.default_rng(10).standard_normal((M // c_h, c_h, c_h))
    out = oracle.forward(q, k, v, None, w, c_h=c_h, mix="post")
    exp = np.zeros_like(out)
    for g in range(M // c_h):
        for u in range(c_h):
            m = g * c_h + u
            for x in range(c_h):
                mx = g * c_h + x
                exp[:, :, m] += w[g, u, x] * _sdpa(q[:, :, mx:mx + 1], k[:, :, mx:mx + 1],
                                                   v[:, :, m:m + 1])[:, :, 0]
    np.testing.assert_allclose(out, exp, atol=1e-12)


def test_pre_mix_equals_wide_query_key_heads():
    # Mixing logits before softmax equals one attention head of width c_h*d over
    # q~ = [w[u][0] q^0, ..., w[u][c_h-1] q^{c_h-1}], k~ = [k^0, ..., k^{c_h-1}], with
    # the per-head 1/sqrt(d) scale (Appendix B query/key view).
    B, T, M, d, c_h = 1, 19, 4, 8, 4
    q, k, v = _rand(B, T, M, d, 11)
    w = np.random.default_rng(12).standard_normal((M // c_h, c_h, c_h))
    out = oracle.forward(q, k, v, None, w, c_h=c_h, mix="pre")
    exp = np.zeros_like(out)
    for g in range(M // c_h):
        heads = list(range(g * c_h, (g + 1) * c_h))
        kk = np.concatenate([k[:, :, h:h + 1] for h in heads], axis=-1)
        for u in range(c_h):
            qq = np.concatenate([w[g, u, x] * q[:, :, heads[x]:heads[x] + 1] for x in range(c_h)], axis=-1)
            m = heads[u]
            exp[:, :, m] = _sdpa(qq, kk, v[:, :, m:m + 1], scale=1.0 / math.sqrt(d))[:, :, 0]
    np.testing.assert_allclose(out, exp, atol=1e-12)


def test_mix_permutation_permutes_maps():
    B, T, M, d, c_q, c_k, c_h = 1, 13, 4, 4, 2, 3, 4
    q, k, v = _rand(B, T, M, d, 13)
    th = np.random.default_rng(14).standard_normal((M, c_q, c_k)) * 0.3
    perm = np.eye(c_h)[[2, 0, 3, 1]][None]
    _, maps = oracle.forward(q, k, v, th, perm, c_q=c_q, c_k=c_k, c_h=c_h, kq="pre", mix="post",
                             return_maps=True)
    _, base = oracle.forward(q, k, v, th, _eye(M, c_h), c_q=c_q, c_k=c_k, c_h=c_h, kq="pre",
                             mix="post", return_maps=True)
    np.testing.assert_array_equal(maps[:, [0, 1, 2, 3]], base[:, [2, 0, 3, 1]])


# --- each head its own kernels, each group its own mixing weights ---------------------
# The convolution kernels are per head and the mixing weights per group of c_h heads (§3.1,
# §3.2). Closed forms that differ from head to head and from group to group fail when an index
# lands on another head's kernel or another group's weights.
@pytest.mark.parametrize("kq", ["pre", "post"])
def test_each_head_uses_its_own_kernel(kq):
    # head m's kernel alpha_m * delta(0, centre). Before softmax it scales head m's logits:
    # softmax(alpha_m QK^T / sqrt(d)). After softmax it scales head m's weights: alpha_m times
    # plain attention.
    B, T, M, d, c_q, c_k, c_h = 2, 23, 4, 8, 3, 5, 2
    q, k, v = _rand(B, T, M, d, 40)
    alpha = np.array([0.5, 1.0, 1.7, 2.3])
    th = _delta(M, c_q, c_k) * alpha[:, None, None]
    out = oracle.forward(q, k, v, th, None, c_q=c_q, c_k=c_k, c_h=c_h, kq=kq)
    for m in range(M):
        hq, hk, hv = q[:, :, m:m + 1], k[:, :, m:m + 1], v[:, :, m:m + 1]
        if kq == "pre":
            exp = _sdpa(hq, hk, hv, scale=alpha[m] / math.sqrt(d))
        else:
            exp = alpha[m] * _sdpa(hq, hk, hv)
        np.testing.assert_allclose(out[:, :, m:m + 1], exp, atol=1e-12)


@pytest.mark.parametrize("mix", ["pre", "post"])
def test_each_group_uses_its_own_mixing_weights(mix):
    # group 0 swaps its two heads, group 1 keeps them: w[g][u][u'] = 1 where u' = pi_g(u).
    # Mixed logits (before softmax) or mixed weights (after it) of head u are those of head
    # pi_g(u), so either way head u attends with the queries and keys of head pi_g(u) and its
    # own values.
    B, T, M, d, c_h = 2, 19, 4, 8, 2
    q, k, v = _rand(B, T, M, d, 41)
    w = np.stack([np.eye(2)[[1, 0]], np.eye(2)])
    src = [1, 0, 2, 3]
    out = oracle.forward(q, k, v, None, w, c_h=c_h, mix=mix)
    np.testing.assert_allclose(out, _sdpa(q[:, :, src], k[:, :, src], v), atol=1e-12)


# --- (b) row sums and (c) causality ------------------------------------------------
def test_rows_sum_to_one_after_pre_conv():
    B, T, M, d, c_q, c_k, c_h = 1, 31, 4, 8, 4, 7, 2
    q, k, v = _rand(B, T, M, d, 15)
    rng = np.random.default_rng(16)
    th = rng.standard_normal((M, c_q, c_k))
    w = rng.standard_normal((M // c_h, c_h, c_h))
    _, maps = oracle.forward(q, k, v, th, None, c_q=c_q, c_k=c_k, c_h=c_h, kq="pre", return_maps=True)
    np.testing.assert_allclose(maps.sum(-1), 1.0, atol=1e-13)
    assert (maps >= 0).all()
    # With mixing after softmax the rows of head u sum to sum_u' w[u][u'].
    _, maps = oracle.forward(q, k, v, th, w, c_q=c_q, c_k=c_k, c_h=c_h, kq="pre", mix="post",
                             return_maps=True)
    for g in range(M // c_h):
        for u in range(c_h):
            np.testing.assert_allclose(maps[0, g * c_h + u].sum(-1), w[g, u].sum(), atol=1e-12)


@pytest.mark.parametrize("kq,mix", [("pre", "post"), ("post", "pre"), ("pre", "pre"), ("post", "post"),
                                    ("both", "both")])
def test_causality_under_future_perturbation(kq, mix):
    B, T, M, d, c_q, c_k, c_h = 1, 24, 4, 8, 3, 5, 2
    q, k, v = _rand(B, T, M, d, 17)
    rng = np.random.default_rng(18)
    th = rng.standard_normal(((2,) if kq == "both" else ()) + (M, c_q, c_k))
    w = rng.standard_normal(((2,) if mix == "both" else ()) + (M // c_h, c_h, c_h))
    gamma, beta = rng.standard_normal(M * d), rng.standard_normal(M * d)
    kw = dict(c_q=c_q, c_k=c_k, c_h=c_h, kq=kq, mix=mix, gn=True)
    base = oracle.forward(q, k, v, th, w, gamma, beta, 0.7, **kw)
    for i in (0, 5, 11, 22):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        for a in (q2, k2, v2):
            a[:, i + 1:] += 3.0 * rng.standard_normal(a[:, i + 1:].shape)
        pert = oracle.forward(q2, k2, v2, th, w, gamma, beta, 0.7, **kw)
        np.testing.assert_allclose(pert[:, :i + 1], base[:, :i + 1], atol=1e-13)
        assert np.abs(pert[:, i + 1:] - base[:, i + 1:]).max() > 1e-6


# --- both sides of softmax (§4: the default placement of the experiments) ----------
def test_both_sides_kernel_order():
    # Before softmax alpha*delta(0, centre) sharpens the logits (temperature alpha);
    # after softmax delta(1, centre) hands row i the weights of row i-1. So
    # O_i = SDPA_alpha(i-1) and O_0 = 0. With the two kernels swapped the result is a
    # different function (row i would see the lagged logits [S[i-1][0..i-1], 0]).
    B, T, M, d, c_q, c_k = 2, 23, 2, 8, 3, 5
    q, k, v = _rand(B, T, M, d, 31)
    alpha = 1.6
    th = np.stack([_delta(M, c_q, c_k, scale=alpha), _delta(M, c_q, c_k, a=1)])
    out = oracle.forward(q, k, v, th, None, c_q=c_q, c_k=c_k, c_h=1, kq="both")
    exp = _sdpa(q, k, v, scale=alpha / math.sqrt(d))
    np.testing.assert_allclose(out[:, 1:], exp[:, :-1], atol=1e-12)
    np.testing.assert_allclose(out[:, 0], 0.0, atol=0)


def test_both_sides_lag_kernels_compose():
    # delta(1, centre) on both sides: before softmax row r gets [S[r-1][0..r-1], 0]
    # (row 0: [1]); after softmax row i takes row i-1 of that. So O_i is the lagged
    # softmax of row i-1 applied to V, and O_0 = 0.
    B, T, M, d, c_q, c_k = 1, 19, 2, 8, 2, 3
    q, k, v = _rand(B, T, M, d, 32)
    lag = _delta(M, c_q, c_k, a=1)
    out = oracle.forward(q, k, v, np.stack([lag, lag]), None, c_q=c_q, c_k=c_k, c_h=1, kq="both")
    S = _plain_logits(q, k)
    exp = np.zeros_like(out)
    for m in range(M):
        for i in range(1, T):
            r = i - 1
            row = np.array([S[0, m, r - 1, j] if j < r else 0.0 for j in range(r + 1)])
            exp[0, i, m] = _softmax_rows(row) @ v[0, :r + 1, m]
    np.testing.assert_allclose(out, exp, atol=1e-12)


def test_both_sides_reduce_to_one_side():
    # An identity kernel on one side leaves the other side's placement.
    B, T, M, d, c_q, c_k, c_h = 1, 21, 4, 8, 3, 5, 2
    q, k, v = _rand(B, T, M, d, 33)
    rng = np.random.default_rng(34)
    th = rng.standard_normal((M, c_q, c_k)) * 0.5
    w = rng.standard_normal((M // c_h, c_h, c_h))
    dl, ey = _delta(M, c_q, c_k), _eye(M, c_h)
    kw = dict(c_q=c_q, c_k=c_k, c_h=c_h)
    f = lambda th_, w_, kq, mix: oracle.forward(q, k, v, th_, w_, kq=kq, mix=mix, **kw)
    np.testing.assert_allclose(f(np.stack([dl, th]), None, "both", None), f(th, None, "post", None), atol=1e-12)
    np.testing.assert_allclose(f(np.stack([th, dl]), None, "both", None), f(th, None, "pre", None), atol=1e-12)
    np.testing.assert_allclose(f(None, np.stack([ey, w]), None, "both"), f(None, w, None, "post"), atol=1e-12)
    np.testing.assert_allclose(f(None, np.stack([w, ey]), None, "both"), f(None, w, None, "pre"), atol=1e-12)


def test_both_sides_mix_permutations_compose():
    # Permutation mixing: before softmax head u takes the logits of head pi(u), after
    # softmax the weights of head sigma(u); so head u attends with the plain map of
    # head pi(sigma(u)) over its own values. pi and sigma do not commute, so swapping
    # the two sides' parameters gives another result.
    B, T, M, d, c_h = 1, 17, 4, 8, 4
    q, k, v = _rand(B, T, M, d, 35)
    pi, sigma = [1, 2, 3, 0], [1, 0, 2, 3]
    w = np.stack([np.eye(c_h)[pi][None], np.eye(c_h)[sigma][None]])
    out = oracle.forward(q, k, v, None, w, c_h=c_h, mix="both")
    exp = np.zeros_like(out)
    for u in range(c_h):
        src = pi[sigma[u]]
        exp[:, :, u] = _sdpa(q[:, :, src:src + 1], k[:, :, src:src + 1], v[:, :, u:u + 1])[:, :, 0]
    np.testing.assert_allclose(out, exp, atol=1e-12)
    assert pi[sigma[0]] != sigma[pi[0]]


# --- GroupNorm and gate (§3.3) ------------------------------------------------------
def test_groupnorm_gate_matches_layer_norm():
    B, T, M, d, c_q, c_k, c_h = 2, 17, 4, 16, 3, 5, 2
    q, k, v = _rand(B, T, M, d, 19)
    rng = np.random.default_rng(20)
    th = rng.standard_normal((M, c_q, c_k)) * 0.3
    w = rng.standard_normal((M // c_h, c_h, c_h))
    gamma, beta, lam = rng.standard_normal(M * d), rng.standard_normal(M * d), 0.37
    kw = dict(c_q=c_q, c_k=c_k, c_h=c_h, kq="pre", mix="post")
    raw = oracle.forward(q, k, v, th, w, **kw)
    out = oracle.forward(q, k, v, th, w, gamma, beta, lam, gn=True, **kw)
    exp = np.zeros_like(out)
    for m in range(M):
        exp[:, :, m] = lam * torch.nn.functional.layer_norm(
            torch.from_numpy(raw[:, :, m]), (d,), torch.from_numpy(gamma[m * d:(m + 1) * d]),
            torch.from_numpy(beta[m * d:(m + 1) * d]), eps=1e-5).numpy()
    np.testing.assert_allclose(out, exp, atol=1e-12)


def test_zero_logits_give_running_mean():
    # q = 0 makes every logit 0, and any convolution of zeros is zero, so each row
    # attends uniformly to keys 0..i: O_i = mean(v_0..v_i).
    B, T, M, d, c_q, c_k = 1, 20, 2, 4, 3, 5
    _, k, v = _rand(B, T, M, d, 21)
    q = np.zeros_like(k)
    th = np.random.default_rng(22).standard_normal((M, c_q, c_k))
    out = oracle.forward(q, k, v, th, None, c_q=c_q, c_k=c_k, c_h=1, kq="pre")
    exp = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None, None]
    np.testing.assert_allclose(out, exp, atol=1e-13)


# --- hand-worked two-token examples -------------------------------------------------
def test_hand_examples():
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        spec = json.load(f)
    for ex in spec["examples"]:
        T = ex["T"]
        shape = (1, T, 1, 1)
        q, k, v = (np.array(ex[n], dtype=np.float64).reshape(shape) for n in ("q", "k", "v"))
        th = np.array(ex["theta"], dtype=np.float64)
        th = th[:, None] if ex["placement"]["kq"] == "both" else th[None]
        out = oracle.forward(q, k, v, th, None, c_q=ex["c_q"], c_k=ex["c_k"], c_h=1,
                             kq=ex["placement"]["kq"])
        np.testing.assert_allclose(out.reshape(-1), ex["expected_out"], atol=1e-14, err_msg=ex["name"])


# --- agreement with the independent transcription, and row sampling ---------------
@pytest.mark.parametrize("kq,mix,gn", [("pre", "post", True), ("post", "pre", True), ("pre", None, False),
                                       (None, "post", False), ("post", "post", True), ("pre", "pre", True),
                                       (None, None, False), ("both", None, False), ("both", "both", True),
                                       ("both", "post", True), ("both", "pre", False), ("pre", "both", True),
                                       ("post", "both", False), (None, "both", True)])
def test_cpp_oracle_matches_python_transcription(kq, mix, gn):
    B, T, M, d, c_q, c_k, c_h = 2, 14, 4, 4, 3, 5, 2
    q, k, v = _rand(B, T, M, d, 23)
    rng = np.random.default_rng(24)
    th = rng.standard_normal(((2,) if kq == "both" else ()) + (M, c_q, c_k))
    w = rng.standard_normal(((2,) if mix == "both" else ()) + (M // c_h, c_h, c_h))
    gamma, beta = rng.standard_normal(M * d), rng.standard_normal(M * d)
    kw = dict(c_q=c_q, c_k=c_k, c_h=c_h, kq=kq, mix=mix, gn=gn)
    a = oracle.forward(q, k, v, th, w, gamma, beta, 0.6, **kw)
    if kq is None:
        th = np.zeros((M, 1, 1))
        kw.update(c_q=1, c_k=1)
    b = py_reference.forward(q, k, v, th, w, gamma, beta, 0.6, **kw)
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_row_subset_matches_full():
    cfg = mta_inputs.config(0)
    inp = mta_inputs.make_inputs(cfg)
    full = oracle.forward_cfg(cfg, inp)
    rows = [0, 1, 2, 30, 31, 63]
    part = oracle.forward_cfg(cfg, inp, rows=rows)
    np.testing.assert_array_equal(part[:, rows], full[:, rows])
    assert np.isnan(part[:, 5]).all()


def test_input_generator_is_seeded_and_bf16_exact():
    cfg = mta_inputs.config(1).replace(T=64, B=1)
    a, b = mta_inputs.make_inputs(cfg), mta_inputs.make_inputs(cfg)
    for n in ("q", "k", "v", "theta", "w"):
        np.testing.assert_array_equal(a[n], b[n])
    for n in ("q", "k", "v"):
        np.testing.assert_array_equal(mta_inputs.round_bf16(a[n]), a[n])
        np.testing.assert_array_equal(mta_inputs.bits_to_float(mta_inputs.bf16_bits(a[n])), a[n])
    # round-to-nearest-even on ties: 1 + 2^-8 lies halfway between two bf16 values
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5], dtype=np.float32)
    np.testing.assert_array_equal(mta_inputs.round_bf16(x), [1.0, 1.0 + 2.0 ** -6, -2.5])


def test_planted_pairs_are_correlated():
    cfg = mta_inputs.config(3).replace(T=2048, M=2, d=64)
    inp = mta_inputs.make_inputs(cfg)
    k = inp["k"][0]
    best = []
    for n in range(cfg.T // 512):
        blk = k[n * 512:(n + 1) * 512, 0]
        c = [np.dot(blk[p], blk[p + 5]) / (np.linalg.norm(blk[p]) * np.linalg.norm(blk[p + 5]))
             for p in range(512 - 5)]
        best.append(max(c))
    assert min(best) > 0.8
