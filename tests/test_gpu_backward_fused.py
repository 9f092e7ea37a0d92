"""GPU parity of the training forward (mta_forward_train) and the fused backward
(mta_backward_fused) against the fp64 oracles.

The fused backward gets the lse and out_pre_gn that mta_forward_train wrote on the GPU, so
its error includes theirs. Gradients are held to the materialized backward's bar (per tensor,
relative to its scale: max |err| <= 2e-2 s, mean |err| <= 2e-3 s; the gate gradient's scale is
the root-sum-square of its terms), see test_gpu_backward.py.

The log-sum-exp bar: the fused forward rounds the logits that its convolutions and mixing
read to fp16 (relative error 2^-11) and sums the softmax in fp32, so at logits of unit scale
the log-sum-exp of a row is off by a few 1e-4; max |err| <= 5e-3 and mean |err| <= 5e-4 leave
a margin of about ten. out_pre_gn is the layer output before GroupNorm: the bf16 output bar
(2e-2 / 2e-3 on values of unit scale).
"""
import numpy as np
import pytest
import torch

import mta_inputs
import token_attention_amd as ta
from oracle import backward as obw
from oracle import oracle
from test_gpu_backward import NAMES, check, grads_case, log, oracle_grads

pytestmark = pytest.mark.gpu

LSE_TOL = (5e-3, 5e-4)


def to_gpu(cfg, inp):
    d = {n: torch.from_numpy(inp[n]).cuda().to(torch.bfloat16).contiguous() for n in ("q", "k", "v")}
    p = {n: torch.from_numpy(np.ascontiguousarray(inp[n], np.float32)).cuda() for n in ("theta", "w", "gamma", "beta")}
    return d, p


def train_forward(cfg, d, p, lam):
    return ta.forward_train(d["q"], d["k"], d["v"], p["theta"], p["w"], p["gamma"], p["beta"], lam, c_q=cfg.c_q,
                            c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)


def fused_grads(cfg, inp, dout):
    d, p = to_gpu(cfg, inp)
    _, lse, opre = train_forward(cfg, d, p, inp["lam"])
    g = ta.backward_fused(d["q"], d["k"], d["v"], p["theta"], p["w"], p["gamma"], p["beta"], inp["lam"],
                          dout=torch.from_numpy(dout).cuda().to(torch.bfloat16), lse=lse, out_pre_gn=opre,
                          c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
    torch.cuda.synchronize()
    return {n: (None if t is None else t.float().cpu().numpy().astype(np.float64)) for n, t in g.items()}


PLACEMENTS = [("pre", "post"), ("post", "pre"), ("pre", None), ("post", None), (None, "post"), (None, "pre"),
              ("pre", "pre"), ("post", "post"), (None, None), ("both", "both"), ("both", None), (None, "both")]


@pytest.mark.parametrize("kq,mix", PLACEMENTS)
def test_forward_train_outputs(kq, mix):
    """out equals mta_forward bit for bit; lse and out_pre_gn against the oracle."""
    cfg = mta_inputs.MTAConfig("train_fwd", 2, 97, 8, 64, 3, 7, 4, kq, mix, True, "bf16", 0.2, 0.3, 1.0, 0.0, 0.9,
                               seed=41)
    inp, _ = grads_case(cfg)
    d, p = to_gpu(cfg, inp)
    out, lse, opre = train_forward(cfg, d, p, inp["lam"])
    ref_out = ta.forward(d["q"], d["k"], d["v"], p["theta"], p["w"], p["gamma"], p["beta"], inp["lam"], c_q=cfg.c_q,
                         c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    want = obw.row_logsumexp(inp["q"], inp["k"], inp["theta"] if kq else None, inp["w"] if mix else None,
                             c_h=cfg.c_h, kq=kq, mix=mix)
    err = np.abs(lse.cpu().numpy().astype(np.float64) - want)
    log(f"  {kq}/{mix} lse max {err.max():.2e} mean {err.mean():.2e}")
    assert err.max() <= LSE_TOL[0] and err.mean() <= LSE_TOL[1]
    o_want = oracle.forward(inp["q"], inp["k"], inp["v"], inp["theta"], inp["w"], kq=kq, mix=mix, c_q=cfg.c_q,
                            c_k=cfg.c_k, c_h=cfg.c_h, gn=False)
    oerr = np.abs(opre.cpu().numpy().astype(np.float64) - o_want)
    log(f"  {kq}/{mix} out_pre_gn max {oerr.max():.2e} mean {oerr.mean():.2e}")
    assert oerr.max() <= 2e-2 and oerr.mean() <= 2e-3


def test_forward_train_lse_on_the_headline_shape():
    """The log-sum-exp of the T=4096 variant (two-phase schedule) on sampled rows."""
    cfg = mta_inputs.config("variant_bf16")
    inp = mta_inputs.make_inputs(cfg)
    d, p = to_gpu(cfg, inp)
    _, lse, _ = train_forward(cfg, d, p, inp["lam"])
    torch.cuda.synchronize()
    rows = mta_inputs.sample_rows(cfg.T, row_tile=61, n_random=8)
    # the oracle's log-sum-exp over the needed leading block of rows of one head group
    T1 = int(rows.max()) + 1
    sl = slice(0, cfg.c_h)
    # pre-softmax mixing only (the convolution acts after softmax): rows of group 0, batch 0
    want = obw.row_logsumexp(inp["q"][:1, :T1, sl], inp["k"][:1, :T1, sl], None, inp["w"][:1], c_h=cfg.c_h,
                             kq=None, mix="pre")
    got = lse[0, :T1, sl].cpu().numpy().astype(np.float64)
    err = np.abs(got[rows] - want[0][rows])
    log(f"  variant lse on {len(rows)} rows: max {err.max():.2e} mean {err.mean():.2e}")
    assert err.max() <= LSE_TOL[0] and err.mean() <= LSE_TOL[1]


@pytest.mark.parametrize("kq,mix", PLACEMENTS)
def test_backward_fused_every_placement(kq, mix):
    cfg = mta_inputs.MTAConfig("bwd", 2, 97, 8, 64, 3, 7, 4, kq, mix, True, "bf16", 0.2, 0.3, 1.0, 0.0, 0.9, seed=31)
    inp, dout = grads_case(cfg)
    check(cfg, fused_grads(cfg, inp, dout), oracle_grads(cfg, inp, dout), dout=dout, lam=inp["lam"],
          what=f"fused {kq}/{mix}")


@pytest.mark.parametrize("d,c_q,c_k,c_h", [(32, 4, 9, 2), (96, 6, 11, 2), (128, 8, 17, 4), (128, 1, 1, 1),
                                           (64, 2, 3, 4)])
@pytest.mark.parametrize("gn", [True, False])
def test_backward_fused_shapes_and_sizes(d, c_q, c_k, c_h, gn):
    mix = "pre" if c_h == 1 else "post"  # a one-head group mixed after softmax only rescales rows
    cfg = mta_inputs.MTAConfig("bwd_shape", 1, 150, 4, d, c_q, c_k, c_h, "pre", mix, gn, "bf16", 0.2, 0.3, 1.0, 0.0,
                               0.8, seed=32)
    inp, dout = grads_case(cfg)
    check(cfg, fused_grads(cfg, inp, dout), oracle_grads(cfg, inp, dout), dout=dout, lam=inp["lam"],
          what=f"fused d={d} {c_q}x{c_k} c_h={c_h} gn={gn}")


@pytest.mark.parametrize("kq,mix,c_q,c_k,c_h,d", [("post", "pre", 4, 9, 4, 128), ("pre", "post", 4, 9, 4, 128),
                                                  ("both", "both", 4, 9, 4, 128), ("pre", "post", 6, 11, 2, 96),
                                                  ("pre", "post", 6, 11, 4, 128)])
def test_backward_fused_specialised_kernels(kq, mix, c_q, c_k, c_h, d):
    """Each kernel shape compiled with its plan as constants (the benchmark workloads' placements
    and kernel sizes), over several tiles and a ragged tail."""
    cfg = mta_inputs.MTAConfig("bwd_spec", 1, 130, 8, d, c_q, c_k, c_h, kq, mix, True, "bf16", 0.1, 0.1, 1.0, 0.0,
                               1.0 / 12 ** 0.5, seed=38)
    inp, dout = grads_case(cfg)
    check(cfg, fused_grads(cfg, inp, dout), oracle_grads(cfg, inp, dout), dout=dout, lam=inp["lam"],
          what=f"fused {kq}/{mix} {c_q}x{c_k} c_h={c_h} d={d}")


@pytest.mark.parametrize("T", [1, 2, 12, 13, 14, 16, 17, 26, 27, 40])
def test_backward_fused_variant_kernel_ragged_lengths(T):
    """The specialised kernel of the convolution after softmax with mixing before (its key-major
    pass steps 13 query rows at a time): lengths around one and two steps and one 16-key tile."""
    cfg = mta_inputs.MTAConfig("bwd_var_T", 1, T, 4, 128, 4, 9, 4, "post", "pre", T > 2, "bf16", 0.2, 0.2, 1.0,
                               0.0, 0.8, seed=39)
    inp, dout = grads_case(cfg)
    check(cfg, fused_grads(cfg, inp, dout), oracle_grads(cfg, inp, dout), dout=dout, lam=inp["lam"],
          what=f"fused variant kernel T={T}")


@pytest.mark.parametrize("sigma", [2.0, 3.0])
@pytest.mark.parametrize("base", ["slice880m_bf16", "longctx_bf16", "variant_bf16", "both_sides_bf16"])
def test_backward_fused_large_logits(base, sigma):
    """q and k scaled by sigma (logit standard deviation sigma^2: rows with several competing large
    logits), on each benchmark placement and kernel size: the forward's log-sum-exp comes from
    fp16-held logits whose error grows with their magnitude, and the backward renormalises its
    recomputed softmax against it."""
    c = mta_inputs.config(base)
    over = dict(plant_block=0) if base == "longctx_bf16" else {}
    cfg = c.replace(B=1, T=256, M=2 * c.c_h, **over)
    inp, dout = grads_case(cfg)
    for n in ("q", "k"):
        inp[n] = mta_inputs.round_bf16(inp[n] * sigma)
    check(cfg, fused_grads(cfg, inp, dout), oracle_grads(cfg, inp, dout), dout=dout, lam=inp["lam"],
          what=f"fused {base} sigma={sigma}")


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 63, 200])
def test_backward_fused_ragged_lengths(T):
    cfg = mta_inputs.MTAConfig("bwd_T", 2, T, 4, 32, 4, 9, 2, "both", "both", T > 2, "bf16", 0.2, 0.2, 1.0, 0.0,
                               0.8, seed=33)
    inp, dout = grads_case(cfg)
    check(cfg, fused_grads(cfg, inp, dout), oracle_grads(cfg, inp, dout), dout=dout, lam=inp["lam"],
          what=f"fused T={T}")


def test_backward_fused_medium_size():
    """Many 16-tiles in both directions, every operation on both sides, four-head groups."""
    cfg = mta_inputs.MTAConfig("bwd_mid", 1, 600, 8, 128, 4, 9, 4, "both", "both", True, "bf16", 0.05, 0.05, 1.0,
                               0.0, 1.0 / 12 ** 0.5, seed=36)
    inp, dout = grads_case(cfg)
    check(cfg, fused_grads(cfg, inp, dout), oracle_grads(cfg, inp, dout), dout=dout, lam=inp["lam"],
          what="fused T=600")


def test_backward_fused_matches_materialized_at_t1024():
    """The headline placement at T=1024 against the materialized backward (itself oracle-checked)."""
    from test_gpu_backward import gpu_grads
    cfg = mta_inputs.MTAConfig("bwd_1k", 1, 1024, 8, 128, 4, 9, 4, "post", "pre", True, "bf16", 0.05, 0.05, 1.0, 0.0,
                               1.0 / 12 ** 0.5, seed=37)
    inp, dout = grads_case(cfg)
    got, want = fused_grads(cfg, inp, dout), gpu_grads(cfg, inp, dout)
    for n in NAMES:
        if want[n] is None:
            continue
        w = np.asarray(want[n]).reshape(np.shape(got[n]))
        err = np.abs(got[n] - w)
        scale = max(float(np.max(np.abs(w))), 1e-30)
        log(f"  T=1024 {n}: max|err|/scale {err.max() / scale:.2e} mean {err.mean() / scale:.2e}")
        assert err.max() <= 2e-2 * scale
        if err.size > 1:
            assert err.mean() <= 2e-3 * scale


@pytest.mark.parametrize("workload", [4, 1])
def test_backward_fused_full_size_matches_materialized(workload):
    """The benchmark workloads at full size (T=4096 variant; 880M slice), in the launch
    configuration the benchmark times: the fused backward against the materialized backward
    (which the oracle checks at small sizes) at the same bar, compared on the GPU; then a second
    fused call, whose fixed-order gradients must repeat bit for bit."""
    cfg = mta_inputs.config(workload)
    inp, dout_np = grads_case(cfg)
    d, p = to_gpu(cfg, inp)
    dout = torch.from_numpy(dout_np).cuda().to(torch.bfloat16)
    kw = dict(c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
    _, lse, opre = train_forward(cfg, d, p, inp["lam"])

    def fused():
        return ta.backward_fused(d["q"], d["k"], d["v"], p["theta"], p["w"], p["gamma"], p["beta"], inp["lam"],
                                 dout=dout, lse=lse, out_pre_gn=opre, **kw)

    got = fused()
    want = ta.backward_materialized(d["q"], d["k"], d["v"], p["theta"], p["w"], p["gamma"], p["beta"], inp["lam"],
                                    dout=dout, **kw)
    torch.cuda.synchronize()
    for n in NAMES:
        if want[n] is None:
            assert got[n] is None
            continue
        g, w = got[n].float().reshape(-1), want[n].float().reshape(-1)
        assert torch.isfinite(g).all(), f"{cfg.name} {n} not finite"
        err = (g - w).abs()
        scale = max(float(w.abs().max()), 1e-30)
        emax, emean = float(err.max()) / scale, float(err.mean()) / scale
        log(f"  {cfg.name} full size {n}: max|err|/scale {emax:.2e} mean {emean:.2e}")
        assert emax <= 2e-2
        if err.numel() > 1:
            assert emean <= 2e-3
    again = fused()
    torch.cuda.synchronize()
    for n in ("dk", "dv", "dtheta", "dw", "dgamma", "dbeta", "dlambda"):
        if got[n] is not None:
            assert torch.equal(got[n], again[n]), f"{cfg.name} {n} differs between two calls"


def test_backward_fused_parameter_gradients_are_deterministic():
    cfg = mta_inputs.MTAConfig("bwd_det", 2, 130, 8, 64, 4, 9, 4, "post", "pre", True, "bf16", 0.1, 0.1, seed=34)
    inp, dout = grads_case(cfg)
    a, b = fused_grads(cfg, inp, dout), fused_grads(cfg, inp, dout)
    for n in ("dk", "dv", "dtheta", "dw", "dgamma", "dbeta", "dlambda"):
        if a[n] is not None:
            assert np.array_equal(a[n], b[n]), n


def test_backward_fused_rejections():
    cfg = mta_inputs.MTAConfig("bwd_ws", 1, 64, 4, 64, 3, 5, 2, "pre", "post", True, "bf16", 0.1, 0.1, seed=35)
    inp, dout = grads_case(cfg)
    d, p = to_gpu(cfg, inp)
    _, lse, opre = train_forward(cfg, d, p, inp["lam"])
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    kw = dict(c_q=3, c_k=5, c_h=2, kq="pre", mix="post", gn=True)
    with pytest.raises(ta.MTAError) as e:
        ta.backward_fused(d["q"], d["k"], d["v"], p["theta"], p["w"], p["gamma"], p["beta"], 0.8, dout=d["q"].clone(),
                          lse=lse, out_pre_gn=opre, workspace=ws, **kw)
    assert e.value.status == ta.mta.ERR_WORKSPACE
    with pytest.raises(ta.MTAError) as e:  # GroupNorm needs the output before it
        ta.backward_fused(d["q"], d["k"], d["v"], p["theta"], p["w"], p["gamma"], p["beta"], 0.8, dout=d["q"].clone(),
                          lse=lse, out_pre_gn=None, **kw)
    assert e.value.status == ta.mta.ERR_INVALID_ARG


def test_backward_fused_largest_kernels_on_both_sides():
    """8 x 17 kernels before and after softmax with four-head groups mixed on both sides: the
    largest tile regions, which still fit the LDS of one workgroup."""
    cfg = mta_inputs.MTAConfig("bwd_big", 1, 70, 4, 128, 8, 17, 4, "both", "both", True, "bf16", 0.1, 0.1, 1.0, 0.0,
                               0.8, seed=38)
    inp, dout = grads_case(cfg)
    check(cfg, fused_grads(cfg, inp, dout), oracle_grads(cfg, inp, dout), dout=dout, lam=inp["lam"],
          what="fused 8x17 both sides")


@pytest.mark.parametrize("kq,mix,gn", [("post", "pre", True), ("pre", "post", True), ("both", "both", True),
                                       (None, None, False)])
def test_autograd_layer_gradients(kq, mix, gn):
    """mta_layer under torch autograd: out equals forward_train's, the gradients that
    loss.backward() leaves on q, k, v, theta, w, gamma, beta and a gate tensor equal those of
    backward_fused called directly (fixed-order reductions bit for bit; dq, summed with atomics,
    within fp32 reordering), and they match the oracle at the backward bar."""
    cfg = mta_inputs.MTAConfig("autograd", 2, 70, 8, 64, 4, 9, 4, kq, mix, gn, "bf16", 0.2, 0.3, 1.0, 0.0, 0.9,
                               seed=43)
    inp, dout = grads_case(cfg)
    d, p = to_gpu(cfg, inp)
    leaves = {n: t.clone().requires_grad_(True) for n, t in {**d, **p}.items()}
    lam_t = torch.tensor(float(inp["lam"]), device="cuda", requires_grad=True)
    out = ta.mta_layer(leaves["q"], leaves["k"], leaves["v"], leaves["theta"] if kq else None,
                       leaves["w"] if mix else None, leaves["gamma"] if gn else None, leaves["beta"] if gn else None,
                       lam_t, c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=kq, mix=mix, gn=gn)
    dout_t = torch.from_numpy(dout).cuda().to(torch.bfloat16)
    (out.float() * dout_t.float()).sum().backward()
    ref_out, lse, opre = train_forward(cfg, d, p, inp["lam"])
    ref = ta.backward_fused(d["q"], d["k"], d["v"], p["theta"], p["w"], p["gamma"], p["beta"], inp["lam"],
                            dout=dout_t, lse=lse, out_pre_gn=opre, c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=kq,
                            mix=mix, gn=gn)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), ref_out)
    got = {"dq": leaves["q"].grad, "dk": leaves["k"].grad, "dv": leaves["v"].grad,
           "dtheta": leaves["theta"].grad if kq else None, "dw": leaves["w"].grad if mix else None,
           "dgamma": leaves["gamma"].grad if gn else None, "dbeta": leaves["beta"].grad if gn else None,
           "dlambda": lam_t.grad.reshape(1) if gn else None}
    for n, want in ref.items():
        if want is None:
            assert got[n] is None, n
            continue
        if n == "dq":
            assert torch.allclose(got[n].float(), want.float(), rtol=2e-2, atol=1e-3 * float(want.float().abs().max()))
        else:
            assert torch.equal(got[n], want), n
    if not gn:
        assert float(lam_t.grad) == 0.0
    check(cfg, {n: (None if t is None else t.float().cpu().numpy().astype(np.float64)) for n, t in got.items()},
          oracle_grads(cfg, inp, dout), dout=dout, lam=inp["lam"], what=f"autograd {kq}/{mix}")


@pytest.mark.parametrize("kq,mix,c_h", [("pre", "post", 2), ("both", "both", 4)])
def test_autograd_layer_fp32(kq, mix, c_h):
    """mta_layer with fp32 tensors: the fused fp32 forward and the unfused backward; the
    gradients equal a direct backward_materialized call and match the gradient oracle."""
    cfg = mta_inputs.MTAConfig("autograd32", 1, 40, 4, 32, 3, 5, c_h, kq, mix, True, "fp32", 0.2, 0.3, 1.0, 0.0, 0.9,
                               seed=44)
    inp, dout = grads_case(cfg)
    d = {n: torch.from_numpy(np.ascontiguousarray(inp[n], np.float32)).cuda() for n in ("q", "k", "v")}
    p = {n: torch.from_numpy(np.ascontiguousarray(inp[n], np.float32)).cuda() for n in ("theta", "w", "gamma", "beta")}
    leaves = {n: t.clone().requires_grad_(True) for n, t in {**d, **p}.items()}
    lam_t = torch.tensor(float(inp["lam"]), device="cuda", requires_grad=True)
    out = ta.mta_layer(leaves["q"], leaves["k"], leaves["v"], leaves["theta"], leaves["w"], leaves["gamma"],
                       leaves["beta"], lam_t, c_q=cfg.c_q, c_k=cfg.c_k, c_h=c_h, kq=kq, mix=mix, gn=True)
    dout_t = torch.from_numpy(dout).cuda()
    (out * dout_t).sum().backward()
    ref = ta.backward_materialized(d["q"], d["k"], d["v"], p["theta"], p["w"], p["gamma"], p["beta"], inp["lam"],
                                   dout=dout_t, c_q=cfg.c_q, c_k=cfg.c_k, c_h=c_h, kq=kq, mix=mix, gn=True)
    torch.cuda.synchronize()
    got = {"dq": leaves["q"].grad, "dk": leaves["k"].grad, "dv": leaves["v"].grad, "dtheta": leaves["theta"].grad,
           "dw": leaves["w"].grad, "dgamma": leaves["gamma"].grad, "dbeta": leaves["beta"].grad,
           "dlambda": lam_t.grad.reshape(1)}
    for n, want in ref.items():
        assert torch.allclose(got[n], want, rtol=1e-5, atol=1e-6 * float(want.abs().max())), n
    check(cfg, {n: t.double().cpu().numpy() for n, t in got.items()}, oracle_grads(cfg, inp, dout), dout=dout,
          lam=inp["lam"], what=f"autograd fp32 {kq}/{mix}")
