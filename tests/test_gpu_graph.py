"""The fused forward, the split decode step and a training step (forward_train + the fused
backward) captured in a HIP graph (torch.cuda.CUDAGraph).

The library only launches kernels on the caller's stream (no memset, allocation or
synchronisation), so a serving loop can capture a step once and replay it. Between replays the
test changes the last query and key rows in place with eager work and synchronises. Every replay
must equal the eager call on the same inputs bit for bit (the same kernels in the same order),
and the last one is also checked against the oracle.
"""
import numpy as np
import pytest
import torch

import mta_inputs
import token_attention_amd as ta
from oracle import oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("split", [False, True])
def test_step_replays_in_a_graph(split):
    cfg = mta_inputs.MTAConfig("graph", 2, 1000, 8, 128, 4, 9, 4, "post", "pre", True, "bf16", 0.1, 0.1, 1.0, 0.0,
                               0.8, seed=46)
    inp = mta_inputs.make_inputs(cfg)
    d = {n: torch.from_numpy(inp[n]).cuda().to(torch.bfloat16).contiguous() for n in ("q", "k", "v")}
    p = {n: torch.from_numpy(np.ascontiguousarray(inp[n], np.float32)).cuda() for n in ("theta", "w", "gamma", "beta")}
    kw = dict(c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
    rb = cfg.T - 1 if split else 0
    need = ta.rows_split_workspace_bytes(cfg.B, cfg.T, cfg.M, cfg.d, row_begin=rb, **kw) if split else 0
    assert not split or need > 0
    ws_g = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    ws_e = torch.empty_like(ws_g)
    out_g, out_e = torch.zeros_like(d["q"]), torch.zeros_like(d["q"])

    def step(out, ws):
        args = (d["q"], d["k"], d["v"], p["theta"], p["w"], p["gamma"], p["beta"], inp["lam"])
        if split:
            ta.forward_rows_split(*args, row_begin=rb, out=out, workspace=ws, **kw)
        else:
            ta.forward(*args, out=out, **kw)

    side = torch.cuda.Stream()  # warm-up off the default stream before capture
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out_g, ws_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(out_g, ws_g)
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda").manual_seed(7)
    shape = (cfg.B, 8, cfg.M, cfg.d)
    for rep in range(3):
        d["q"][:, -8:] = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
        d["k"][:, -8:] = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(out_e, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g[:, rb:], out_e[:, rb:]), f"replay {rep} differs from the eager call"

    rows = np.unique(np.array([rb, (rb + cfg.T) // 2, cfg.T - 9, cfg.T - 1], dtype=np.int32))
    rows = rows[rows >= rb]
    now = dict(inp, q=d["q"].float().cpu().numpy(), k=d["k"].float().cpu().numpy())
    want = oracle.forward_cfg(cfg, now, rows=rows)
    got = out_g.float().cpu().numpy().astype(np.float64)
    err = np.abs(got[:, rows] - want[:, rows])
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())


@pytest.mark.parametrize("kq,mix", [("post", "pre"), ("both", "both")])
def test_training_step_replays_in_a_graph(kq, mix):
    """mta_forward_train and mta_backward_fused captured together (a layer's training step) and
    replayed with new inputs written in place between replays: every replay equals the eager
    step; the fixed-order gradients bit for bit, dQ (summed with atomics in no fixed order) to
    rounding."""
    cfg = mta_inputs.MTAConfig("graph_train", 2, 600, 8, 128, 4, 9, 4, kq, mix, True, "bf16", 0.1, 0.1, 1.0, 0.0,
                               0.8, seed=47)
    inp = mta_inputs.make_inputs(cfg)
    d = {n: torch.from_numpy(inp[n]).cuda().to(torch.bfloat16).contiguous() for n in ("q", "k", "v")}
    p = {n: torch.from_numpy(np.ascontiguousarray(inp[n], np.float32)).cuda() for n in ("theta", "w", "gamma", "beta")}
    kw = dict(c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
    gen = torch.Generator(device="cuda").manual_seed(8)
    dout = torch.randn(d["q"].shape, generator=gen, device="cuda").to(torch.bfloat16)
    need = ta.backward_fused_workspace_bytes(cfg.B, cfg.T, cfg.M, cfg.d, **kw)

    def buffers():
        return {"out": torch.empty_like(d["q"]),
                "lse": torch.empty((cfg.B, cfg.T, cfg.M), dtype=torch.float32, device="cuda"),
                "opre": torch.empty(d["q"].shape, dtype=torch.float32, device="cuda"),
                "ws": torch.empty(need, dtype=torch.uint8, device="cuda")}

    def step(bf):
        args = (d["q"], d["k"], d["v"], p["theta"], p["w"], p["gamma"], p["beta"], inp["lam"])
        ta.forward_train(*args, out=bf["out"], lse=bf["lse"], out_pre_gn=bf["opre"], **kw)
        return ta.backward_fused(*args, dout=dout, lse=bf["lse"], out_pre_gn=bf["opre"], workspace=bf["ws"], **kw)

    bg, be = buffers(), buffers()
    side = torch.cuda.Stream()  # warm-up off the default stream before capture
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(bg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        got = step(bg)
    torch.cuda.synchronize()

    shape = (cfg.B, 16, cfg.M, cfg.d)
    for rep in range(3):
        for n in ("q", "k", "v"):
            d[n][:, 100 * rep:100 * rep + 16] = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
        dout[:, -16:] = torch.randn(shape, generator=gen, device="cuda").to(torch.bfloat16)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = step(be)
        torch.cuda.synchronize()
        for n in ("out", "lse", "opre"):
            assert torch.equal(bg[n], be[n]), f"replay {rep}: {n} differs from the eager step"
        for n in ("dk", "dv", "dtheta", "dw", "dgamma", "dbeta", "dlambda"):
            assert torch.equal(got[n], want[n]), f"replay {rep}: {n} differs from the eager step"
        err = (got["dq"].float() - want["dq"].float()).abs().max()
        assert float(err) <= 1e-2 * float(want["dq"].float().abs().max()), f"replay {rep}: dq {float(err)}"
