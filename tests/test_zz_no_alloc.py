"""The entry point that allocates nothing (mta_forward_rows_split_noalloc, partial results in
the library's device scratch) against the one that takes a caller workspace
(mta_forward_rows_split), through the C ABI on the GPU. Both launch the same kernels with the
same key split, so their outputs agree bit for bit. Two calls in a row share the scratch: the
second, smaller one must not see the first one's partial results."""
import sys

import numpy as np
import pytest
import torch

import mta_inputs
import token_attention_amd as ta
from oracle import oracle

pytestmark = pytest.mark.gpu


def log(msg):
    sys.__stdout__.write(msg + "\n")
    sys.__stdout__.flush()


def _dev(cfg, inp):
    d = {n: torch.from_numpy(inp[n]).to("cuda").to(torch.bfloat16).contiguous() for n in ("q", "k", "v")}
    for n in ("theta", "w", "gamma", "beta"):
        d[n] = torch.from_numpy(np.ascontiguousarray(inp[n], dtype=np.float32)).to("cuda")
    return d


def _both(cfg, row_begin):
    inp = mta_inputs.make_inputs(cfg)
    d = _dev(cfg, inp)
    kw = dict(c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn, row_begin=row_begin)
    args = (d["q"], d["k"], d["v"], d["theta"], d["w"], d["gamma"], d["beta"], inp["lam"])
    n, keys = ta.rows_split_plan(cfg.B, cfg.T, cfg.M, cfg.d, c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq,
                                 mix=cfg.mix, gn=cfg.gn, row_begin=row_begin)
    log(f"  {cfg.name} B={cfg.B} T={cfg.T} M={cfg.M} rows {row_begin}..{cfg.T - 1}: {n} key chunks of {keys}")
    assert n > 1, "the case must exercise the scratch"
    out_ws = ta.forward_rows_split(*args, out=torch.zeros_like(d["q"]), **kw)
    out_na = ta.forward_rows_split_noalloc(*args, out=torch.zeros_like(d["q"]), **kw)
    torch.cuda.synchronize()
    return inp, out_ws, out_na


def test_noalloc_equals_the_workspace_entry_point():
    # 1) a decode step at the T=4096 shape: 13 key chunks, about 7 MiB of partial results
    big = mta_inputs.config("variant_bf16")
    _, ws1, na1 = _both(big, big.T - 1)
    assert torch.equal(ws1, na1)
    # 2) a smaller call on the same scratch: 3 rows of a shorter sequence, another placement
    small = mta_inputs.config("slice880m_bf16").replace(B=1, T=1500, M=4)
    inp, ws2, na2 = _both(small, small.T - 3)
    assert torch.equal(ws2, na2)
    # and the rows agree with the oracle (the bf16 bar of the other parity tests)
    rows = np.arange(small.T - 3, small.T, dtype=np.int32)
    want = oracle.forward_cfg(small, inp, rows=rows)[:, rows]
    got = na2.float().cpu().numpy().astype(np.float64)[:, rows]
    err = np.abs(got - want)
    log(f"  noalloc vs oracle: max|err| {err.max():.3e} mean|err| {err.mean():.3e}")
    assert np.isfinite(got).all() and err.max() <= 2e-2 and err.mean() <= 2e-3
    # rows before row_begin are untouched
    assert not torch.any(na2[:, : small.T - 3])
