"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bars (per workload): fp32 tensors max |err| <= 1e-5; bf16 tensors max |err| <= 2e-2
and mean |err| <= 2e-3 on the outputs. Both sides get the identical bf16-rounded
inputs. Small cases are checked on every output; the full-size workloads on
sampled rows (tile edges, both ends, seeded random rows), which the oracle
computes one by one.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import mta_inputs
import token_attention_amd as ta
from oracle import oracle

pytestmark = pytest.mark.gpu

TOL = {"fp32": (1e-5, None), "bf16": (2e-2, 2e-3)}


def log(msg):
    sys.__stdout__.write(msg + "\n")
    sys.__stdout__.flush()


def dev_inputs(cfg, inp):
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    d = {n: torch.from_numpy(inp[n]).to("cuda").to(dt).contiguous() for n in ("q", "k", "v")}
    for n in ("theta", "w", "gamma", "beta"):
        d[n] = torch.from_numpy(np.ascontiguousarray(inp[n], dtype=np.float32)).to("cuda")
    return d


def run(path, cfg, d, lam):
    kw = dict(c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
    args = (d["q"], d["k"], d["v"], d["theta"], d["w"], d["gamma"], d["beta"], lam)
    if path == "fused":
        out = ta.forward(*args, **kw)
    elif path == "materialized":
        out = ta.forward_materialized(*args, **kw)
    else:
        raise ValueError(path)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def compare(cfg, got, want, rows=None, what=""):
    if rows is not None:
        got, want = got[:, rows], want[:, rows]
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    log(f"  {what}: max|err| {mx:.3e}  mean|err| {mean:.3e}")
    tmax, tmean = TOL[cfg.dtype]
    assert mx <= tmax, f"{what}: max abs error {mx} > {tmax}"
    if tmean is not None:
        assert mean <= tmean, f"{what}: mean abs error {mean} > {tmean}"
    return mx, mean


@functools.lru_cache(maxsize=None)
def case(cfg):
    inp = mta_inputs.make_inputs(cfg)
    return inp


@functools.lru_cache(maxsize=None)
def oracle_full(cfg):
    return oracle.forward_cfg(cfg, case(cfg))


def output_rows_per_tile(cfg):
    """Output rows of one row tile of the fused bf16 kernel for this workload: 8 waves of 32 rows,
    8/c_h waves per head of the group (12 waves of 16 rows for the per-pair schedule of two-head
    groups at d = 96), less the query halo of c_q - 1 rows per convolution."""
    c_h = cfg.c_h if cfg.mix else 1
    halo = (cfg.c_q - 1) * {None: 0, "pre": 1, "post": 1, "both": 2}[cfg.kq]
    if cfg.d == 96 and c_h == 2 and cfg.kq == "pre" and cfg.mix == "post":
        return 16 * 6 - halo
    return 32 * (8 // c_h) - halo


@functools.lru_cache(maxsize=None)
def oracle_rows(cfg):
    # both ends, seeded random rows, and both sides of every tile edge of this workload's own
    # row tiles (and of the 59- and 27-row tiles of other shapes)
    rows = mta_inputs.sample_rows(cfg.T, row_tile=output_rows_per_tile(cfg), n_random=20)
    rows = np.unique(np.concatenate([rows, mta_inputs.sample_rows(cfg.T, row_tile=61, n_random=0),
                                     mta_inputs.sample_rows(cfg.T, row_tile=59, n_random=0),
                                     mta_inputs.sample_rows(cfg.T, row_tile=27, n_random=0)]))
    return rows, oracle.forward_cfg(cfg, case(cfg), rows=rows)


def small(cfg, **kw):
    """The workload's placement and kernel sizes at a size the oracle finishes in full."""
    base = dict(B=2, T=150, M=8 if cfg.M >= 8 else cfg.M)
    base.update(kw)
    return cfg.replace(name=cfg.name + "_small", **base)


# ---- the five workloads -------------------------------------------------------------
@pytest.mark.parametrize("path", ["fused", "materialized"])
def test_tiny_fp32_workload_full(path):
    cfg = mta_inputs.config(0)
    log(f"[{path}] {cfg}")
    compare(cfg, run(path, cfg, dev_inputs(cfg, case(cfg)), case(cfg)["lam"]), oracle_full(cfg), what=path)


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
@pytest.mark.parametrize("path", ["fused", "materialized"])
def test_workload_small_full_check(idx, path):
    cfg = small(mta_inputs.config(idx))
    log(f"[{path}] {cfg}")
    inp = case(cfg)
    compare(cfg, run(path, cfg, dev_inputs(cfg, inp), inp["lam"]), oracle_full(cfg), what=path)


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
@pytest.mark.parametrize("path", ["fused", "materialized"])
def test_workload_full_size_sampled_rows(idx, path):
    cfg = mta_inputs.config(idx)
    log(f"[{path}] full size {cfg}")
    rows, want = oracle_rows(cfg)
    inp = case(cfg)
    got = run(path, cfg, dev_inputs(cfg, inp), inp["lam"])
    compare(cfg, got, want, rows=rows, what=f"{path} rows={len(rows)}")
    assert np.isfinite(got).all()


def test_degenerate_kernels_equal_plain_attention():
    # delta kernel + identity mixing + no GroupNorm must reproduce plain causal attention
    cfg = mta_inputs.config(2)
    inp = case(cfg)
    d = dev_inputs(cfg, inp)
    mtaout = ta.forward(d["q"], d["k"], d["v"], d["theta"], d["w"], c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h,
                        kq=cfg.kq, mix=cfg.mix, gn=False)
    plain = ta.attention_plain(d["q"], d["k"], d["v"])
    torch.cuda.synchronize()
    a = mtaout.float().cpu().numpy()
    b = plain.float().cpu().numpy()
    err = np.abs(a - b)
    log(f"  mta vs plain: max {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


# ---- plain attention -----------------------------------------------------------------
@pytest.mark.parametrize("shape,dtype", [((2, 300, 4, 128), "bf16"), ((1, 77, 3, 64), "bf16"),
                                         ((2, 129, 2, 96), "bf16"), ((1, 64, 4, 16), "fp32"),
                                         ((1, 50, 2, 32), "fp32")])
def test_plain_attention(shape, dtype):
    B, T, M, d = shape
    cfg = mta_inputs.MTAConfig("plain", B, T, M, d, 1, 1, 1, None, None, False, dtype, 0.0, 0.0, seed=7)
    inp = case(cfg)
    dv = dev_inputs(cfg, inp)
    got = ta.attention_plain(dv["q"], dv["k"], dv["v"])
    torch.cuda.synchronize()
    compare(cfg, got.float().cpu().numpy().astype(np.float64), oracle_full(cfg), what="plain")


# ---- placements, kernel sizes, head sizes, ragged lengths -------------------------------
COMBOS = [("pre", "post"), ("post", "pre"), ("pre", None), ("post", None), (None, "post"), (None, "pre"),
          ("pre", "pre"), ("post", "post"), (None, None), ("both", None), ("both", "both"), ("both", "post"),
          ("both", "pre"), ("pre", "both"), ("post", "both"), (None, "both")]


@pytest.mark.parametrize("kq,mix", COMBOS)
@pytest.mark.parametrize("path", ["fused", "materialized"])
def test_every_placement(kq, mix, path):
    cfg = mta_inputs.MTAConfig("combo", 2, 97, 8, 64, 3, 7, 4, kq, mix, True, "bf16", 0.2, 0.3, 1.0, 0.0,
                               0.9, seed=11)
    inp = case(cfg)
    compare(cfg, run(path, cfg, dev_inputs(cfg, inp), inp["lam"]), oracle_full(cfg), what=f"{path} {kq}/{mix}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kq,mix,c_h", [(None, None, 1), ("pre", None, 1), ("post", None, 1), (None, "post", 4),
                                        (None, "pre", 2), ("pre", "post", 2), ("pre", "post", 4),
                                        ("post", "pre", 4)])
def test_late_dominant_key(kq, mix, c_h, d):
    """One key far past the first key tile whose logit for one query exceeds everything
    before it by ~130 (natural-log units, 2^187 as a weight against the first tile's
    maximum, past the fp32 range): the fused kernel's first-tile reference is then too
    small and the workgroup must take its exact fallback pass."""
    cfg = mta_inputs.MTAConfig("late", 1, 300, 8, d, 4, 9, c_h, kq, mix, True, "bf16", 0.05, 0.05, 1.0, 0.0,
                               0.8, seed=17)
    inp = dict(case(cfg))
    q, k = inp["q"].astype(np.float64), inp["k"].copy()
    jkey, iq = 200, 260
    for m in range(cfg.M):
        qv = q[0, iq, m]
        k[0, jkey, m] = 130.0 * np.sqrt(d) / float(qv @ qv) * qv
    inp["k"] = mta_inputs.round_bf16(k.astype(np.float32))
    logit = float(inp["q"][0, iq, 0].astype(np.float64) @ inp["k"][0, jkey, 0]) / np.sqrt(d)
    assert logit > 120.0
    want = oracle.forward_cfg(cfg, inp)
    compare(cfg, run("fused", cfg, dev_inputs(cfg, inp), inp["lam"]), want, what=f"late key {kq}/{mix}/{c_h} d={d}")


@pytest.mark.parametrize("kq,mix", [(None, "pre"), (None, "post"), ("pre", "post"), ("post", "pre"), ("post", "post"),
                                    (None, "both")])
@pytest.mark.parametrize("path", ["fused", "materialized"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_single_head_groups_scale(kq, mix, path, dtype):
    """c_h = 1: each head is its own group and the mixing weight is a scalar per head;
    without GroupNorm a negative weight must show up as a scaled (pre: sharpened or
    flattened and reversed) output."""
    cfg = mta_inputs.MTAConfig("ch1", 1, 90, 4, 64, 3, 5, 1, kq, mix, False, dtype, 0.1, 0.0, seed=19)
    inp = dict(case(cfg))
    inp["w"] = np.array([-0.7, 1.3, 0.4, -1.1], dtype=np.float32).reshape(4, 1, 1)
    if mix == "both":
        inp["w"] = np.stack([inp["w"], np.array([0.6, -1.2, 0.9, 1.4], dtype=np.float32).reshape(4, 1, 1)])
    # halved values keep the un-normalised outputs below 4, where half a bf16 ulp of the
    # stored output stays well inside the absolute bar
    inp["v"] = mta_inputs.round_bf16(inp["v"] * 0.5)
    want = oracle.forward_cfg(cfg, inp)
    compare(cfg, run(path, cfg, dev_inputs(cfg, inp), inp["lam"]), want, what=f"{path} c_h=1 {kq}/{mix}")


@pytest.mark.parametrize("c_q,c_k", [(1, 1), (1, 17), (8, 1), (8, 17), (2, 3), (5, 13)])
@pytest.mark.parametrize("kq", ["pre", "post"])
def test_kernel_sizes(c_q, c_k, kq):
    mix = "post" if kq == "pre" else "pre"
    cfg = mta_inputs.MTAConfig("ks", 1, 133, 4, 128, c_q, c_k, 2, kq, mix, True, "bf16", 0.2, 0.2, 1.0, 0.0,
                               0.8, seed=12)
    inp = case(cfg)
    compare(cfg, run("fused", cfg, dev_inputs(cfg, inp), inp["lam"]), oracle_full(cfg), what=f"{kq} {c_q}x{c_k}")


@pytest.mark.parametrize("T", [1, 2, 5, 16, 31, 64, 65, 200])
@pytest.mark.parametrize("placement", [("pre", "post", 2), ("post", "pre", 4)])
def test_ragged_lengths(T, placement):
    kq, mix, c_h = placement
    cfg = mta_inputs.MTAConfig("ragged", 2, T, 4, 32, 4, 9, c_h, kq, mix, True, "bf16", 0.2, 0.2, 1.0, 0.0,
                               0.8, seed=13)
    inp = case(cfg)
    compare(cfg, run("fused", cfg, dev_inputs(cfg, inp), inp["lam"]), oracle_full(cfg), what=f"T={T}")


@pytest.mark.parametrize("d,dtype", [(32, "bf16"), (64, "bf16"), (96, "bf16"), (16, "fp32"), (32, "fp32"),
                                     (64, "fp32")])
@pytest.mark.parametrize("placement", [("pre", "post", 2), ("post", "pre", 4), ("pre", "post", 4)])
def test_head_sizes(d, dtype, placement):
    kq, mix, c_h = placement
    cfg = mta_inputs.MTAConfig("hs", 1, 90, 4, d, 3, 5, c_h, kq, mix, True, dtype, 0.1, 0.1, 1.0, 0.0, 0.8,
                               seed=14)
    inp = case(cfg)
    for path in ("fused", "materialized"):
        compare(cfg, run(path, cfg, dev_inputs(cfg, inp), inp["lam"]), oracle_full(cfg), what=f"{path} d={d}")


def test_groupnorm_affine_values():
    cfg = mta_inputs.MTAConfig("gn", 1, 70, 4, 64, 3, 5, 2, "pre", "post", True, "bf16", 0.1, 0.1, seed=15)
    inp = dict(case(cfg))
    rng = np.random.default_rng(16)
    inp["gamma"] = rng.standard_normal(cfg.M * cfg.d).astype(np.float32)
    inp["beta"] = rng.standard_normal(cfg.M * cfg.d).astype(np.float32)
    inp["lam"] = 0.37
    want = oracle.forward_cfg(cfg, inp)
    compare(cfg, run("fused", cfg, dev_inputs(cfg, inp), inp["lam"]), want, what="gn affine")


# ---- properties on the GPU path --------------------------------------------------------
def test_deterministic():
    cfg = small(mta_inputs.config(4), T=300)
    d = dev_inputs(cfg, case(cfg))
    a = run("fused", cfg, d, 0.3)
    b = run("fused", cfg, d, 0.3)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("idx", [1, 4])
def test_causal_under_future_perturbation(idx):
    cfg = small(mta_inputs.config(idx), T=256)
    inp = case(cfg)
    d = dev_inputs(cfg, inp)
    base = run("fused", cfg, d, inp["lam"])
    cut = 100
    for n in ("q", "k", "v"):
        d[n][:, cut + 1:] = torch.randn_like(d[n][:, cut + 1:]) * 3
    pert = run("fused", cfg, d, inp["lam"])
    assert np.array_equal(pert[:, :cut + 1], base[:, :cut + 1])
    assert np.abs(pert[:, cut + 1:] - base[:, cut + 1:]).max() > 1e-3


def test_stream_argument():
    cfg = small(mta_inputs.config(1), T=64)
    inp = case(cfg)
    d = dev_inputs(cfg, inp)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = ta.forward(d["q"], d["k"], d["v"], d["theta"], d["w"], d["gamma"], d["beta"], inp["lam"],
                         c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn, stream=s)
    s.synchronize()
    compare(cfg, out.float().cpu().numpy().astype(np.float64), oracle_full(cfg), what="side stream")


def test_workspace_too_small_is_reported():
    cfg = small(mta_inputs.config(1), T=64)
    d = dev_inputs(cfg, case(cfg))
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ta.MTAError) as e:
        ta.forward_materialized(d["q"], d["k"], d["v"], d["theta"], d["w"], d["gamma"], d["beta"], 0.8,
                                c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn,
                                workspace=ws)
    assert e.value.status == 4


# ---- row ranges: decode step and prefill chunks ------------------------------------------
@pytest.mark.parametrize("row_begin", [0, 1, 97, 150, 299])
@pytest.mark.parametrize("kq,mix,c_h,dtype,d", [(None, None, 1, "bf16", 128), ("pre", "post", 2, "bf16", 96),
                                                ("post", "pre", 4, "bf16", 128), ("pre", "pre", 4, "bf16", 64),
                                                ("post", "post", 2, "bf16", 128), ("pre", "post", 2, "fp32", 32)])
def test_row_range_equals_full_forward(row_begin, kq, mix, c_h, dtype, d):
    """mta_forward_rows writes exactly rows row_begin.. of mta_forward (same values, bit for
    bit: every row is computed from the same keys in the same order) and leaves the rows
    before it untouched."""
    cfg = mta_inputs.MTAConfig("rows", 2, 300, 8, d, 4, 9, c_h, kq, mix, True, dtype, 0.1, 0.1, 1.0, 0.0, 0.8,
                               seed=21)
    inp = case(cfg)
    dv = dev_inputs(cfg, inp)
    kw = dict(c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
    args = (dv["q"], dv["k"], dv["v"], dv["theta"], dv["w"], dv["gamma"], dv["beta"], inp["lam"])
    full = ta.forward(*args, **kw)
    part = torch.full_like(full, 7.0)
    ta.forward_rows(*args, row_begin=row_begin, out=part, **kw)
    torch.cuda.synchronize()
    f, p = full.float().cpu(), part.float().cpu()
    log(f"  rows {row_begin}.. {kq}/{mix}/{c_h} {dtype}: max diff {float((f[:, row_begin:] - p[:, row_begin:]).abs().max()):.3e}")
    assert torch.equal(p[:, row_begin:], f[:, row_begin:])
    assert bool((p[:, :row_begin] == 7.0).all())


@pytest.mark.parametrize("row_begin", [4095, 3584])
def test_decode_step_and_chunk_at_full_size(row_begin):
    """Decode step (the last row) and a 512-row prefill chunk of the T=4096 workload
    against the oracle."""
    cfg = mta_inputs.config(4)
    inp = case(cfg)
    rows = np.arange(row_begin, cfg.T, dtype=np.int32)
    if len(rows) > 8:
        rows = np.unique(np.concatenate([rows[:4], rows[-4:], mta_inputs.sample_rows(cfg.T, row_tile=61, n_random=8)]))
        rows = rows[rows >= row_begin].astype(np.int32)
    want = oracle.forward_cfg(cfg, inp, rows=rows)
    dv = dev_inputs(cfg, inp)
    out = ta.forward_rows(dv["q"], dv["k"], dv["v"], dv["theta"], dv["w"], dv["gamma"], dv["beta"], inp["lam"],
                          row_begin=row_begin, c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix,
                          gn=cfg.gn)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    compare(cfg, got, want, rows=rows, what=f"rows {row_begin}.. ({len(rows)} checked)")


# ---- both sides of softmax ------------------------------------------------------------------
@pytest.mark.parametrize("c_q,c_k", [(1, 1), (2, 3), (4, 9), (6, 11), (8, 17), (5, 1)])
@pytest.mark.parametrize("mix,c_h", [(None, 1), ("both", 4), ("post", 2), ("pre", 4), ("both", 1)])
def test_both_convolutions_kernel_sizes(c_q, c_k, mix, c_h):
    cfg = mta_inputs.MTAConfig("dual", 1, 133, 4, 128, c_q, c_k, c_h, "both", mix, True, "bf16", 0.2, 0.2, 1.0,
                               0.0, 0.8, seed=23)
    inp = case(cfg)
    compare(cfg, run("fused", cfg, dev_inputs(cfg, inp), inp["lam"]), oracle_full(cfg),
            what=f"both {c_q}x{c_k} mix={mix}/{c_h}")


@pytest.mark.parametrize("T", [1, 2, 5, 16, 33, 64, 65, 200])
@pytest.mark.parametrize("d", [32, 96])
def test_both_sides_ragged_lengths_and_head_sizes(T, d):
    cfg = mta_inputs.MTAConfig("dual_ragged", 2, T, 4, d, 4, 9, 2, "both", "both", True, "bf16", 0.2, 0.2, 1.0,
                               0.0, 0.8, seed=24)
    inp = case(cfg)
    for path in ("fused", "materialized"):
        compare(cfg, run(path, cfg, dev_inputs(cfg, inp), inp["lam"]), oracle_full(cfg), what=f"{path} T={T} d={d}")


@pytest.mark.parametrize("mix,c_h", [(None, 1), ("both", 4), ("pre", 2)])
def test_both_sides_late_dominant_key(mix, c_h):
    """The exact fallback of the statistics phase with both convolutions: one key far past
    the lead-in tile dominates one query's softmax input by ~130 natural-log units."""
    d = 128
    cfg = mta_inputs.MTAConfig("dual_late", 1, 300, 8, d, 4, 9, c_h, "both", mix, True, "bf16", 0.05, 0.05, 1.0,
                               0.0, 0.8, seed=25)
    inp = dict(case(cfg))
    q, k = inp["q"].astype(np.float64), inp["k"].copy()
    jkey, iq = 200, 260
    for m in range(cfg.M):
        qv = q[0, iq, m]
        k[0, jkey, m] = 130.0 * np.sqrt(d) / float(qv @ qv) * qv
    inp["k"] = mta_inputs.round_bf16(k.astype(np.float32))
    want = oracle.forward_cfg(cfg, inp)
    compare(cfg, run("fused", cfg, dev_inputs(cfg, inp), inp["lam"]), want, what=f"late key both/{mix}/{c_h}")


@pytest.mark.parametrize("kq,c_h", [(None, 2), ("pre", 4), ("post", 2)])
def test_mixing_both_sides_fp32_fused(kq, c_h):
    cfg = mta_inputs.MTAConfig("mixboth_fp32", 1, 90, 4, 32, 3, 5, c_h, kq, "both", True, "fp32", 0.1, 0.2, 1.0, 0.0,
                               0.8, seed=45)
    inp = case(cfg)
    compare(cfg, run("fused", cfg, dev_inputs(cfg, inp), inp["lam"]), oracle_full(cfg), what=f"fp32 {kq}/both")


@pytest.mark.parametrize("c_q,c_k", [(1, 1), (2, 3), (3, 5), (4, 9), (8, 17), (5, 1)])
@pytest.mark.parametrize("mix,c_h", [(None, 1), ("both", 4), ("post", 2), ("pre", 4), ("both", 2), ("post", 1)])
def test_both_sides_fp32(c_q, c_k, mix, c_h):
    """fp32 tensors with convolutions on both sides: the fp32 fused kernel (its both-sides
    schedule: statistics of the convolved logits, then logits over both key halos -> weights
    ring -> second convolution) and the materialized chain, against the oracle at the fp32 bar."""
    cfg = mta_inputs.MTAConfig("dual_fp32", 1, 70, 4, 16, c_q, c_k, c_h, "both", mix, True, "fp32", 0.2, 0.2, 1.0,
                               0.0, 0.8, seed=26)
    inp = case(cfg)
    d = dev_inputs(cfg, inp)
    want = oracle_full(cfg)
    for path in ("fused", "materialized"):
        compare(cfg, run(path, cfg, d, inp["lam"]), want, what=f"{path} fp32 both {c_q}x{c_k} mix={mix}/{c_h}")


@pytest.mark.parametrize("T", [1, 2, 5, 16, 17, 33, 100])
@pytest.mark.parametrize("d,c_h", [(16, 4), (32, 2), (64, 4), (64, 1)])
def test_both_sides_fp32_ragged_lengths_and_head_sizes(T, d, c_h):
    """Both sides in fp32 at every fp32 head size (the d = 64, four-head tile is the largest
    LDS footprint of the schedule), lengths below, at and across one 16-key tile and one row
    tile (32 rows minus a halo of 2 (c_q - 1))."""
    cfg = mta_inputs.MTAConfig("dual_fp32_T", 2, T, 4, d, 4, 9, c_h, "both", "both" if c_h > 1 else None, True,
                               "fp32", 0.2, 0.2, 1.0, 0.0, 0.8, seed=28)
    inp = case(cfg)
    compare(cfg, run("fused", cfg, dev_inputs(cfg, inp), inp["lam"]), oracle_full(cfg), what=f"fp32 both T={T} d={d}")


def test_both_sides_fp32_largest_tile():
    """Both sides in fp32 at the schedule's largest LDS footprint and query halo: d = 64, four-head
    groups mixed on both sides, 8 x 17 kernels (a 14-row halo of a 32-row tile)."""
    cfg = mta_inputs.MTAConfig("dual_fp32_big", 1, 100, 8, 64, 8, 17, 4, "both", "both", True, "fp32", 0.1, 0.1,
                               1.0, 0.0, 0.8, seed=30)
    inp = case(cfg)
    compare(cfg, run("fused", cfg, dev_inputs(cfg, inp), inp["lam"]), oracle_full(cfg), what="fp32 both 8x17 d=64")


@pytest.mark.parametrize("row_begin", [0, 1, 37, 90])
def test_both_sides_fp32_row_range_equals_full_forward(row_begin):
    """mta_forward_rows of fp32 tensors on both sides writes exactly rows row_begin.. of
    mta_forward (bit for bit) and leaves the rows before it untouched."""
    cfg = mta_inputs.MTAConfig("dual_fp32_rows", 2, 100, 8, 32, 4, 9, 4, "both", "both", True, "fp32", 0.1, 0.1, 1.0,
                               0.0, 0.8, seed=29)
    inp = case(cfg)
    dv = dev_inputs(cfg, inp)
    kw = dict(c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
    args = (dv["q"], dv["k"], dv["v"], dv["theta"], dv["w"], dv["gamma"], dv["beta"], inp["lam"])
    full = ta.forward(*args, **kw)
    part = torch.full_like(full, 7.0)
    ta.forward_rows(*args, row_begin=row_begin, out=part, **kw)
    torch.cuda.synchronize()
    f, p = full.float().cpu(), part.float().cpu()
    assert torch.equal(p[:, row_begin:], f[:, row_begin:])
    assert bool((p[:, :row_begin] == 7.0).all())
    compare(cfg, f.numpy().astype(np.float64), oracle_full(cfg), what="fp32 both full")


@pytest.mark.parametrize("row_begin", [0, 1, 97, 299])
@pytest.mark.parametrize("mix,c_h", [("both", 4), (None, 1)])
def test_both_sides_row_range_equals_full_forward(row_begin, mix, c_h):
    cfg = mta_inputs.MTAConfig("dual_rows", 2, 300, 8, 128, 4, 9, c_h, "both", mix, True, "bf16", 0.1, 0.1, 1.0,
                               0.0, 0.8, seed=27)
    inp = case(cfg)
    dv = dev_inputs(cfg, inp)
    kw = dict(c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
    args = (dv["q"], dv["k"], dv["v"], dv["theta"], dv["w"], dv["gamma"], dv["beta"], inp["lam"])
    full = ta.forward(*args, **kw)
    part = torch.full_like(full, 7.0)
    ta.forward_rows(*args, row_begin=row_begin, out=part, **kw)
    torch.cuda.synchronize()
    f, p = full.float().cpu(), part.float().cpu()
    assert torch.equal(p[:, row_begin:], f[:, row_begin:])
    assert bool((p[:, :row_begin] == 7.0).all())


@pytest.mark.parametrize("path", ["fused", "materialized"])
def test_both_sides_full_size_sampled_rows(path):
    cfg = mta_inputs.config("both_sides_bf16")
    log(f"[{path}] full size {cfg}")
    rows, want = oracle_rows(cfg)
    inp = case(cfg)
    got = run(path, cfg, dev_inputs(cfg, inp), inp["lam"])
    compare(cfg, got, want, rows=rows, what=f"{path} rows={len(rows)}")
    assert np.isfinite(got).all()


# ---- row ranges with the key range split over workgroups -----------------------------------
SPLIT_PLACEMENTS = [(None, None, 1), ("pre", "post", 2), ("post", "pre", 4), ("pre", "pre", 4), ("post", "post", 2),
                    ("both", "both", 4), ("both", None, 1), (None, "post", 4), ("pre", None, 1)]


@pytest.mark.parametrize("row_begin", [299, 250, 0])
@pytest.mark.parametrize("kq,mix,c_h", SPLIT_PLACEMENTS)
def test_rows_split_against_oracle(row_begin, kq, mix, c_h):
    """mta_forward_rows_split (key chunks combined afterwards) against the oracle and the
    unsplit row range, for decode-like, chunk-like and whole ranges of every schedule."""
    cfg = mta_inputs.MTAConfig("rows_split", 2, 300, 8, 128, 4, 9, c_h, kq, mix, True, "bf16", 0.1, 0.1, 1.0, 0.0,
                               0.8, seed=41)
    inp = case(cfg)
    assert ta.rows_split_workspace_bytes(cfg.B, cfg.T, cfg.M, cfg.d, row_begin=row_begin, c_q=cfg.c_q, c_k=cfg.c_k,
                                         c_h=cfg.c_h, kq=kq, mix=mix, gn=True) > 0
    dv = dev_inputs(cfg, inp)
    kw = dict(c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
    args = (dv["q"], dv["k"], dv["v"], dv["theta"], dv["w"], dv["gamma"], dv["beta"], inp["lam"])
    part = torch.full_like(dv["q"], 7.0)
    ta.forward_rows_split(*args, row_begin=row_begin, out=part, **kw)
    ref = ta.forward_rows(*args, row_begin=row_begin, **kw)
    torch.cuda.synchronize()
    p = part.float().cpu()
    assert bool((p[:, :row_begin] == 7.0).all())
    got = p.numpy().astype(np.float64)
    rows = np.arange(row_begin, cfg.T)
    compare(cfg, got, oracle_full(cfg), rows=rows, what=f"split rows {row_begin}.. {kq}/{mix}/{c_h}")
    diff = float((p[:, row_begin:] - ref.float().cpu()[:, row_begin:]).abs().max())
    log(f"  vs unsplit: max diff {diff:.3e}")
    assert diff <= 2e-2


@pytest.mark.parametrize("kq,mix,c_h,c_q,c_k,nrows", [
    ("both", "both", 4, 8, 17, 2), ("both", "both", 4, 8, 17, 3),  # halo 14: 16-row tiles hold 2 rows
    ("post", "pre", 4, 4, 9, 13), ("post", "pre", 4, 4, 9, 14),    # halo 3
    ("pre", "post", 2, 6, 11, 11), ("pre", "post", 2, 6, 11, 12),  # halo 5
    (None, None, 1, 1, 1, 16), (None, None, 1, 1, 1, 17)])         # no halo
def test_rows_split_sixteen_row_tiles(kq, mix, c_h, c_q, c_k, nrows):
    """Key-split ranges that just fit one 16-row tile with its query halo (one wave per head)
    and ranges one row longer (the 8-wave shapes), against the oracle and the unsplit range."""
    cfg = mta_inputs.MTAConfig("rows_split16", 2, 200, 8, 128, c_q, c_k, c_h, kq, mix, True, "bf16", 0.1, 0.1, 1.0,
                               0.0, 0.8, seed=43)
    inp = case(cfg)
    row_begin = cfg.T - nrows
    dv = dev_inputs(cfg, inp)
    kw = dict(c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=cfg.gn)
    args = (dv["q"], dv["k"], dv["v"], dv["theta"], dv["w"], dv["gamma"], dv["beta"], inp["lam"])
    part = torch.full_like(dv["q"], 7.0)
    ta.forward_rows_split(*args, row_begin=row_begin, out=part, **kw)
    ref = ta.forward_rows(*args, row_begin=row_begin, **kw)
    torch.cuda.synchronize()
    p = part.float().cpu()
    assert bool((p[:, :row_begin] == 7.0).all())
    compare(cfg, p.numpy().astype(np.float64), oracle_full(cfg), rows=np.arange(row_begin, cfg.T),
            what=f"split {nrows} rows {kq}/{mix}/{c_h} {c_q}x{c_k}")
    diff = float((p[:, row_begin:] - ref.float().cpu()[:, row_begin:]).abs().max())
    log(f"  vs unsplit: max diff {diff:.3e}")
    assert diff <= 2e-2


def test_rows_split_many_row_tiles():
    """Several row tiles per sequence, each split into key chunks (the statistics of the rows a
    tile shares with its neighbour are written once)."""
    cfg = mta_inputs.MTAConfig("rows_split_tiles", 1, 600, 4, 128, 4, 9, 4, "both", "both", True, "bf16", 0.1, 0.1,
                               1.0, 0.0, 0.8, seed=42)
    inp = case(cfg)
    dv = dev_inputs(cfg, inp)
    out = ta.forward_rows_split(dv["q"], dv["k"], dv["v"], dv["theta"], dv["w"], dv["gamma"], dv["beta"], inp["lam"],
                                row_begin=0, c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix, gn=True)
    torch.cuda.synchronize()
    compare(cfg, out.float().cpu().numpy().astype(np.float64), oracle_full(cfg), what="split, 11 row tiles")


@pytest.mark.parametrize("kq,mix,c_h", [(None, None, 1), ("post", "pre", 4), ("both", "both", 4)])
def test_rows_split_late_dominant_key(kq, mix, c_h):
    """The exact fallback inside one key chunk: one key dominates one query's row by ~130."""
    d = 128
    cfg = mta_inputs.MTAConfig("split_late", 1, 300, 8, d, 4, 9, c_h, kq, mix, True, "bf16", 0.05, 0.05, 1.0, 0.0,
                               0.8, seed=43)
    inp = dict(case(cfg))
    q, k = inp["q"].astype(np.float64), inp["k"].copy()
    jkey, iq = 200, 299
    for m in range(cfg.M):
        qv = q[0, iq, m]
        k[0, jkey, m] = 130.0 * np.sqrt(d) / float(qv @ qv) * qv
    inp["k"] = mta_inputs.round_bf16(k.astype(np.float32))
    want = oracle.forward_cfg(cfg, inp, rows=[299])
    dv = dev_inputs(cfg, inp)
    out = ta.forward_rows_split(dv["q"], dv["k"], dv["v"], dv["theta"], dv["w"], dv["gamma"], dv["beta"], inp["lam"],
                                row_begin=299, c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=kq, mix=mix, gn=True)
    torch.cuda.synchronize()
    compare(cfg, out.float().cpu().numpy().astype(np.float64), want, rows=[299], what=f"split late {kq}/{mix}")


@pytest.mark.parametrize("row_begin", [4095, 3584])
def test_rows_split_at_full_size(row_begin):
    """Decode step and a 512-row chunk of the T=4096 workload, split over key chunks."""
    cfg = mta_inputs.config(4)
    inp = case(cfg)
    rows = np.arange(row_begin, cfg.T, dtype=np.int32)
    if len(rows) > 8:
        rows = np.unique(np.concatenate([rows[:4], rows[-4:], mta_inputs.sample_rows(cfg.T, row_tile=61, n_random=8)]))
        rows = rows[rows >= row_begin].astype(np.int32)
    want = oracle.forward_cfg(cfg, inp, rows=rows)
    dv = dev_inputs(cfg, inp)
    out = ta.forward_rows_split(dv["q"], dv["k"], dv["v"], dv["theta"], dv["w"], dv["gamma"], dv["beta"], inp["lam"],
                                row_begin=row_begin, c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=cfg.kq, mix=cfg.mix,
                                gn=cfg.gn)
    torch.cuda.synchronize()
    compare(cfg, out.float().cpu().numpy().astype(np.float64), want, rows=rows,
            what=f"split rows {row_begin}.. ({len(rows)} checked)")


def _split_chunks(nbytes, B, T, M, d, row_begin):
    """Key chunks of a split launch, read back from its workspace size (two statistics floats
    and d partial floats per chunk for each (b, row, head) of rows row_begin - 16 .. T-1, the
    statistics region rounded up to 64 floats)."""
    rows = B * (T - row_begin + 16) * M
    up = lambda x: (x + 63) // 64 * 64
    return next(n for n in range(2, 65) if 4 * (up(2 * n * rows) + n * rows * d) == nbytes)


@pytest.mark.parametrize("row_begin", [4095, 3900])
@pytest.mark.parametrize("kq,mix,c_h", [("post", "pre", 4), ("pre", "post", 4), (None, None, 1)])
def test_rows_split_sixty_four_chunks(kq, mix, c_h, row_begin):
    """The largest split: one head group at T=4096 takes 64 chunks of 64 keys, one per lane of
    the combining kernels. From row 3900 with a convolution or mixing, the first 64-row tile
    (output rows up to 3960) has no keys in the last two chunks."""
    cfg = mta_inputs.MTAConfig("split64", 1, 4096, 4, 128, 4, 9, c_h, kq, mix, True, "bf16", 0.1, 0.1, 1.0, 0.0,
                               0.8, seed=45)
    kw = dict(c_q=cfg.c_q, c_k=cfg.c_k, c_h=cfg.c_h, kq=kq, mix=mix, gn=True)
    need = ta.rows_split_workspace_bytes(cfg.B, cfg.T, cfg.M, cfg.d, row_begin=row_begin, **kw)
    assert _split_chunks(need, cfg.B, cfg.T, cfg.M, cfg.d, row_begin) == 64
    inp = case(cfg)
    rows = np.unique(np.r_[np.arange(row_begin, min(row_begin + 4, cfg.T)), 3960, 3961, cfg.T - 1])
    rows = rows[rows >= row_begin].astype(np.int32)
    want = oracle.forward_cfg(cfg, inp, rows=rows)
    dv = dev_inputs(cfg, inp)
    out = ta.forward_rows_split(dv["q"], dv["k"], dv["v"], dv["theta"], dv["w"], dv["gamma"], dv["beta"], inp["lam"],
                                row_begin=row_begin, **kw)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got[:, row_begin:]).all()
    compare(cfg, got, want, rows=rows, what=f"64 chunks rows {row_begin}.. {kq}/{mix}")


def test_rows_split_fp32_runs_unsplit():
    cfg = mta_inputs.MTAConfig("split_fp32", 1, 90, 4, 32, 3, 5, 2, "pre", "post", True, "fp32", 0.1, 0.1, 1.0, 0.0,
                               0.8, seed=44)
    assert ta.rows_split_workspace_bytes(1, 90, 4, 32, row_begin=89, c_q=3, c_k=5, c_h=2, kq="pre", mix="post",
                                         gn=True, fp32=True) == 0
    inp = case(cfg)
    dv = dev_inputs(cfg, inp)
    out = ta.forward_rows_split(dv["q"], dv["k"], dv["v"], dv["theta"], dv["w"], dv["gamma"], dv["beta"], inp["lam"],
                                row_begin=60, c_q=3, c_k=5, c_h=2, kq="pre", mix="post", gn=True)
    torch.cuda.synchronize()
    compare(cfg, out.float().cpu().numpy().astype(np.float64), oracle_full(cfg), rows=np.arange(60, 90),
            what="fp32 rows 60..")
