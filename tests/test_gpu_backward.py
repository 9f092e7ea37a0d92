"""GPU parity of the backward pass (mta_backward_materialized) against the fp64 gradient oracle.

Bar (per gradient tensor G, relative to its scale s): bf16 tensors max|err| <= 2e-2 s and
mean|err| <= 2e-3 s, the forward's bars carried over to unit scale; fp32 tensors max|err| <= 1e-4 s
and mean |err| <= 1e-5 s (a single value has only the max bar). The scale is max|G_ref|, except for the gate gradient, a single sum
over all B*T*M*d output elements of dout * (gamma xhat + beta) with heavy cancellation: its scale
is the root-sum-square of those terms (a rounding error eps per term gives about eps times that).
Both sides get the identical (bf16-rounded) inputs and output gradient.

GroupNorm makes each (token, head) output invariant to a positive rescaling of that head's
weights, so where a parameter only rescales a whole row (mixing weight of a one-head group after
softmax; every kernel and weight when T <= 2) its exact gradient nearly cancels to zero and says
nothing about the kernels' precision; those cases run without GroupNorm.
"""
import sys

import numpy as np
import pytest
import torch

import mta_inputs
import token_attention_amd as ta
from oracle import backward as obw

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 2e-3), "fp32": (1e-4, 1e-5)}
NAMES = ("dq", "dk", "dv", "dtheta", "dw", "dgamma", "dbeta", "dlambda")


def log(msg):
    sys.__stdout__.write(msg + "\n")
    sys.__stdout__.flush()


def grads_case(cfg, seed=101):
    inp = mta_inputs.make_inputs(cfg)
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal((cfg.B, cfg.T, cfg.M, cfg.d)).astype(np.float32)
    if cfg.dtype == "bf16":
        dout = mta_inputs.round_bf16(dout)
    inp["gamma"] = (1.0 + 0.3 * rng.standard_normal(cfg.M * cfg.d)).astype(np.float32)
    inp["beta"] = (0.2 * rng.standard_normal(cfg.M * cfg.d)).astype(np.float32)
    return inp, dout


def gpu_grads(cfg, inp, dout):
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    d = {n: torch.from_numpy(inp[n]).cuda().to(dt).contiguous() for n in ("q", "k", "v")}
    p = {n: torch.from_numpy(np.ascontiguousarray(inp[n], np.float32)).cuda() for n in ("theta", "w", "gamma", "beta")}
    g = ta.backward_materialized(d["q"], d["k"], d["v"], p["theta"], p["w"], p["gamma"], p["beta"], inp["lam"],
                                 dout=torch.from_numpy(dout).cuda().to(dt), c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h,
                                 kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
    torch.cuda.synchronize()
    return {n: (None if t is None else t.float().cpu().numpy().astype(np.float64)) for n, t in g.items()}


def oracle_grads(cfg, inp, dout):
    return obw.backward(inp["q"], inp["k"], inp["v"], inp["theta"] if cfg.kq else None,
                        inp["w"] if cfg.mix else None, inp["gamma"], inp["beta"], inp["lam"], dout,
                        c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)


def check(cfg, got, want, what, dout, lam):
    tmax, tmean = TOL[cfg.dtype]
    for n in NAMES:
        w = want[n]
        if w is None:
            assert got.get(n) is None, f"{what}: {n} should be absent"
            continue
        gv = np.asarray(got[n], dtype=np.float64).reshape(np.shape(w))
        assert np.isfinite(gv).all(), f"{what}: {n} not finite"
        err = np.abs(gv - w)
        if n == "dlambda":
            scale = float(np.sqrt(np.sum((dout.astype(np.float64) * want["out"] / lam) ** 2)))
        else:
            scale = max(float(np.max(np.abs(w))), 1e-30)
        log(f"  {what} {n}: scale {scale:.3e} max|err|/scale {err.max() / scale:.2e} mean|err|/scale "
            f"{err.mean() / scale:.2e}")
        assert err.max() <= tmax * scale, f"{what}: {n} max error {err.max()} > {tmax} x {scale}"
        if err.size > 1:  # a single value (the gate gradient) has only the max bar
            assert err.mean() <= tmean * scale, f"{what}: {n} mean error {err.mean()} > {tmean} x {scale}"


PLACEMENTS = [("pre", "post"), ("post", "pre"), ("pre", None), ("post", None), (None, "post"), (None, "pre"),
              ("pre", "pre"), ("post", "post"), (None, None), ("both", "both"), ("both", None), (None, "both")]


@pytest.mark.parametrize("kq,mix", PLACEMENTS)
def test_backward_every_placement(kq, mix):
    cfg = mta_inputs.MTAConfig("bwd", 2, 97, 8, 64, 3, 7, 4, kq, mix, True, "bf16", 0.2, 0.3, 1.0, 0.0, 0.9, seed=31)
    inp, dout = grads_case(cfg)
    check(cfg, gpu_grads(cfg, inp, dout), oracle_grads(cfg, inp, dout), dout=dout, lam=inp["lam"], what=f"{kq}/{mix}")


@pytest.mark.parametrize("d,dtype,c_q,c_k,c_h", [(32, "bf16", 4, 9, 2), (96, "bf16", 6, 11, 2), (128, "bf16", 8, 17, 4),
                                                 (128, "bf16", 1, 1, 1), (16, "fp32", 3, 5, 2), (64, "fp32", 2, 3, 4)])
@pytest.mark.parametrize("gn", [True, False])
def test_backward_shapes_and_sizes(d, dtype, c_q, c_k, c_h, gn):
    mix = "pre" if c_h == 1 else "post"  # a one-head group mixed after softmax only rescales rows
    cfg = mta_inputs.MTAConfig("bwd_shape", 1, 150, 4, d, c_q, c_k, c_h, "pre", mix, gn, dtype, 0.2, 0.3, 1.0, 0.0,
                               0.8, seed=32)
    inp, dout = grads_case(cfg)
    check(cfg, gpu_grads(cfg, inp, dout), oracle_grads(cfg, inp, dout), dout=dout, lam=inp["lam"],
          what=f"d={d} {dtype} {c_q}x{c_k} c_h={c_h} gn={gn}")


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 200])
def test_backward_ragged_lengths(T):
    cfg = mta_inputs.MTAConfig("bwd_T", 2, T, 4, 32, 4, 9, 2, "both", "both", T > 2, "bf16", 0.2, 0.2, 1.0, 0.0,
                               0.8, seed=33)
    inp, dout = grads_case(cfg)
    check(cfg, gpu_grads(cfg, inp, dout), oracle_grads(cfg, inp, dout), dout=dout, lam=inp["lam"], what=f"T={T}")


def test_backward_medium_size():
    """Several 64-tiles and 128-tiles in both directions, every operation on both sides."""
    cfg = mta_inputs.MTAConfig("bwd_mid", 1, 600, 8, 128, 4, 9, 4, "both", "both", True, "bf16", 0.05, 0.05, 1.0, 0.0,
                               1.0 / 12 ** 0.5, seed=36)
    inp, dout = grads_case(cfg)
    check(cfg, gpu_grads(cfg, inp, dout), oracle_grads(cfg, inp, dout), dout=dout, lam=inp["lam"], what="T=600")


def test_backward_tiny_fp32_workload():
    cfg = mta_inputs.config(0)
    inp, dout = grads_case(cfg)
    check(cfg, gpu_grads(cfg, inp, dout), oracle_grads(cfg, inp, dout), dout=dout, lam=inp["lam"], what="tiny fp32")


def test_backward_is_deterministic():
    cfg = mta_inputs.MTAConfig("bwd_det", 2, 130, 8, 64, 4, 9, 4, "post", "pre", True, "bf16", 0.1, 0.1, seed=34)
    inp, dout = grads_case(cfg)
    a, b = gpu_grads(cfg, inp, dout), gpu_grads(cfg, inp, dout)
    for n in NAMES:
        if a[n] is not None:
            assert np.array_equal(a[n], b[n]), n


def test_backward_workspace_too_small_is_reported():
    cfg = mta_inputs.MTAConfig("bwd_ws", 1, 64, 4, 64, 3, 5, 2, "pre", "post", True, "bf16", 0.1, 0.1, seed=35)
    inp, dout = grads_case(cfg)
    q = torch.from_numpy(inp["q"]).cuda().to(torch.bfloat16)
    p = {n: torch.from_numpy(np.ascontiguousarray(inp[n], np.float32)).cuda() for n in ("theta", "w", "gamma", "beta")}
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(ta.MTAError) as e:
        ta.backward_materialized(q, q.clone(), q.clone(), p["theta"], p["w"], p["gamma"], p["beta"], 0.8,
                                 dout=q.clone(), c_q=3, c_k=5, c_h=2, kq="pre", mix="post", gn=True, workspace=ws)
    assert e.value.status == ta.mta.ERR_WORKSPACE
