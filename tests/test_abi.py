"""C-ABI checks that need no GPU: the library loads, exports what include/mta.h
declares, its flag values match the binding, and argument validation (host-only,
``mta_check_args``) returns the documented status codes."""
import ctypes
import os
import re

import pytest

import token_attention_amd as ta
from token_attention_amd import mta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mta.h")

P = 0x10000  # a 16-byte aligned, never dereferenced pointer value


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mta_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = ta.lib()
    declared = _header_functions()
    assert set(declared) == set(mta.EXPORTED), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_flag_values_match_header():
    text = open(HEADER).read()
    for name in ("KQ_PRE", "KQ_POST", "MIX_PRE", "MIX_POST", "GN", "FP32"):
        m = re.search(r"#define MTA_%s (0x[0-9a-f]+)u" % name, text)
        assert m, name
        assert int(m.group(1), 16) == getattr(mta, name), name
    for name, val in (("MTA_OK", 0), ("MTA_ERR_INVALID_ARG", 1), ("MTA_ERR_UNSUPPORTED", 2),
                      ("MTA_ERR_HIP", 3), ("MTA_ERR_WORKSPACE", 4)):
        assert re.search(r"%s = %d" % (name, val), text), name


def _check(**kw):
    a = dict(q=P, k=P, v=P, theta=P, w=P, gamma=P, beta=P, out=P + 0x100, B=1, T=64, M=4, d=128, c_q=3,
             c_k=5, c_h=2, flags=mta.KQ_PRE | mta.MIX_POST | mta.GN)
    a.update(kw)
    return mta.check_args(a["q"], a["k"], a["v"], a["theta"], a["w"], a["gamma"], a["beta"], a["out"], a["B"],
                          a["T"], a["M"], a["d"], a["c_q"], a["c_k"], a["c_h"], a["flags"])


def test_valid_arguments_pass():
    assert _check() == mta.OK
    assert _check(flags=mta.KQ_POST | mta.MIX_PRE | mta.GN, c_q=4, c_k=9, c_h=4) == mta.OK
    assert _check(flags=0, theta=0, w=0, gamma=0, beta=0) == mta.OK  # plain attention
    assert _check(flags=mta.FP32 | mta.KQ_PRE, d=16, w=0) == mta.OK
    # both sides of softmax (parameters of the side before softmax first)
    assert _check(flags=mta.KQ_PRE | mta.KQ_POST | mta.MIX_PRE | mta.MIX_POST | mta.GN) == mta.OK
    assert _check(flags=mta.KQ_PRE | mta.KQ_POST, w=0) == mta.OK
    assert mta.last_error() == ""


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), mta.ERR_INVALID_ARG),
    (dict(T=-1), mta.ERR_INVALID_ARG),
    (dict(M=6, c_h=4), mta.ERR_INVALID_ARG),
    (dict(q=0), mta.ERR_INVALID_ARG),
    (dict(out=P + 8), mta.ERR_INVALID_ARG),               # misaligned
    (dict(out=P), mta.ERR_INVALID_ARG),                   # aliases q
    (dict(theta=0), mta.ERR_INVALID_ARG),                 # KQ flag without theta
    (dict(w=0), mta.ERR_INVALID_ARG),                     # MIX flag without w
    (dict(gamma=0), mta.ERR_INVALID_ARG),                 # GN without gamma
    (dict(flags=0x400), mta.ERR_INVALID_ARG),
    (dict(c_k=4), mta.ERR_UNSUPPORTED),                   # even key size
    (dict(c_q=9), mta.ERR_UNSUPPORTED),
    (dict(c_k=19), mta.ERR_UNSUPPORTED),
    (dict(c_h=8, M=8), mta.ERR_UNSUPPORTED),
    (dict(d=80), mta.ERR_UNSUPPORTED),
    (dict(d=128, flags=mta.FP32), mta.ERR_UNSUPPORTED),
    (dict(c_q=0), mta.ERR_INVALID_ARG),
    (dict(T=1 << 17, M=64, d=128), mta.ERR_UNSUPPORTED),  # one batch of q is 2 GiB
])
def test_invalid_arguments_are_rejected(kw, status):
    assert _check(**kw) == status
    assert mta.last_error() != ""


def test_ignored_arguments_without_flags():
    # without a KQ flag, theta/c_q/c_k are ignored; without MIX, w/c_h are ignored
    assert _check(flags=mta.GN, theta=0, w=0, c_q=0, c_k=4, c_h=3) == mta.OK


def test_status_strings_and_version():
    L = ta.lib()
    for s in range(5):
        assert L.mta_status_string(s).decode()
    assert L.mta_status_string(99).decode() == "unknown status"
    assert L.mta_version() >= 100


def test_workspace_size():
    assert ta.materialized_workspace_bytes(2, 64, 4) == 2 * 2 * 4 * 64 * 64 * 4
    assert ta.materialized_workspace_bytes(1, 65, 2) == 2 * 1 * 2 * 65 * 68 * 4
    assert ta.materialized_workspace_bytes(0, 64, 4) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 8, 1, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ta.attention_plain(q, q.clone(), q.clone())


@pytest.mark.parametrize("row_begin", [-1, 64, 1000])
def test_row_range_outside_the_sequence_is_rejected(row_begin):
    # validation happens before anything is launched, so this runs without a GPU
    st = mta.lib().mta_forward_rows(P, P, P, P, P, P, P, 1.0, P + 0x100, 1, 64, 4, 128, 3, 5, 2, row_begin,
                                    mta.KQ_PRE | mta.MIX_POST | mta.GN, None)
    assert st == mta.ERR_INVALID_ARG
    assert "row_begin" in mta.last_error()


def test_backward_workspace_size():
    # maps: S, P, G, G2 always; L with mixing before softmax, E with a convolution after it,
    # A with mixing after it; plus O and dO with GroupNorm, the transposed weights and partials
    B, T, M, d = 1, 64, 4, 32
    one_map = B * M * T * T * 4
    plain = ta.backward_workspace_bytes(B, T, M, d)
    assert 4 * one_map <= plain < 5 * one_map
    full = ta.backward_workspace_bytes(B, T, M, d, c_q=3, c_k=5, c_h=2, kq="both", mix="both", gn=True)
    assert 7 * one_map <= full < 8 * one_map
    assert ta.backward_workspace_bytes(0, T, M, d) == 0


@pytest.mark.parametrize("which", ["dout", "dtheta", "dw", "dgamma", "dlambda", "workspace"])
def test_backward_missing_buffers_are_rejected(which):
    # validation happens before anything is launched, so this runs without a GPU
    bufs = {n: P + 0x1000 * (i + 1) for i, n in enumerate(
        ["dout", "dq", "dk", "dv", "dtheta", "dw", "dgamma", "dbeta", "dlambda", "workspace"])}
    bufs[which] = 0
    st = mta.lib().mta_backward_materialized(
        P, P + 0x100, P + 0x200, P, P, P, P, 1.0, bufs["dout"], bufs["dq"], bufs["dk"], bufs["dv"], bufs["dtheta"],
        bufs["dw"], bufs["dgamma"], bufs["dbeta"], bufs["dlambda"], 1, 64, 4, 128, 3, 5, 2,
        mta.KQ_PRE | mta.MIX_POST | mta.GN, bufs["workspace"], 1 << 30, None)
    assert st == (mta.ERR_WORKSPACE if which == "workspace" else mta.ERR_INVALID_ARG)
    assert mta.last_error() != ""


def test_rows_split_workspace_size():
    kw = dict(c_q=4, c_k=9, c_h=4, kq="post", mix="pre", gn=True)
    decode = ta.rows_split_workspace_bytes(2, 4096, 32, 128, row_begin=4095, **kw)
    assert decode > 0
    # enough row tiles already (the whole sequence): no splitting, no workspace
    assert ta.rows_split_workspace_bytes(2, 4096, 32, 128, row_begin=0, **kw) == 0
    # fp32 tensors run the unsplit kernel
    assert ta.rows_split_workspace_bytes(1, 90, 4, 32, row_begin=89, c_q=3, c_k=5, c_h=2, kq="pre", mix="post",
                                         gn=True, fp32=True) == 0
    assert ta.rows_split_workspace_bytes(2, 4096, 32, 128, row_begin=4096, **kw) == 0


def _split_chunks(nbytes, B, T, M, d, row_begin):
    """Key chunks of a split launch, read back from its workspace size: per (b, row, head) two
    floats of statistics per chunk and d floats of AV partial per chunk (row_begin - 16 .. T-1:
    16 rows of query halo), the statistics region rounded up to 64 floats."""
    rows = B * (T - row_begin + 16) * M
    up = lambda x: (x + 63) // 64 * 64
    for n in range(2, 65):
        if 4 * (up(2 * n * rows) + n * rows * d) == nbytes:
            return n
    raise AssertionError(f"{nbytes} bytes match no chunk count")


def test_rows_split_plan_at_the_t4096_shape():
    # decode step, convolution after and mixing before softmax: 16 row tiles of 16 rows, four
    # waves each; 13 chunks of 320 keys (208 workgroups: a round of such workgroups is taken
    # as 7/8 of the 256 compute units)
    kw = dict(c_q=4, c_k=9, c_h=4, kq="post", mix="pre", gn=True)
    assert _split_chunks(ta.rows_split_workspace_bytes(2, 4096, 32, 128, row_begin=4095, **kw),
                         2, 4096, 32, 128, 4095) == 13
    # the default placement decodes the same way
    kw_default = dict(c_q=4, c_k=9, c_h=4, kq="pre", mix="post", gn=True)
    assert _split_chunks(ta.rows_split_workspace_bytes(2, 4096, 32, 128, row_begin=4095, **kw_default),
                         2, 4096, 32, 128, 4095) == 13
    # no convolution or mixing: 64 one-wave row tiles, 4 chunks fill the 256 units once
    assert _split_chunks(ta.rows_split_workspace_bytes(2, 4096, 32, 128, row_begin=4095, gn=True),
                         2, 4096, 32, 128, 4095) == 4
    # 512-row prefill chunk: 144 row tiles of 64 rows, 5 chunks of 832 keys
    assert _split_chunks(ta.rows_split_workspace_bytes(2, 4096, 32, 128, row_begin=3584, **kw),
                         2, 4096, 32, 128, 3584) == 5


@pytest.mark.parametrize("row_begin", [-1, 64])
def test_rows_split_outside_the_sequence_is_rejected(row_begin):
    st = mta.lib().mta_forward_rows_split(P, P + 0x100, P + 0x200, P, P, P, P, 1.0, P + 0x300, 1, 64, 4, 128, 3, 5,
                                          2, row_begin, mta.KQ_PRE | mta.MIX_POST | mta.GN, None, 0, None)
    assert st == mta.ERR_INVALID_ARG


def test_rows_split_plan_reads_the_compute_unit_count():
    # decode step at the T=4096 shape (16 row tiles of a four-head group, 16 rows each): with 256
    # compute units a round holds 224 such workgroups, so 13 chunks of 320 keys fill one round;
    # with 128 units (112 per round) 7 chunks of 640 keys do; with 64 units (56 per round) two
    # rounds of 7 chunks cost less than one round of 3 chunks of 1408 keys
    kw = dict(c_q=4, c_k=9, c_h=4, kq="post", mix="pre", gn=True)
    assert ta.rows_split_plan(2, 4096, 32, 128, row_begin=4095, compute_units=256, **kw) == (13, 320)
    assert ta.rows_split_plan(2, 4096, 32, 128, row_begin=4095, compute_units=128, **kw) == (7, 640)
    assert ta.rows_split_plan(2, 4096, 32, 128, row_begin=4095, compute_units=64, **kw) == (7, 640)
    # as many row tiles as compute units: no split
    assert ta.rows_split_plan(2, 4096, 32, 128, row_begin=0, compute_units=256, **kw) == (1, 4096)
    # the workspace query and the launch plan on the current device (256 units when none is
    # present): the query's chunk count is the plan's
    n, _ = ta.rows_split_plan(2, 4096, 32, 128, row_begin=4095, **kw)
    assert _split_chunks(ta.rows_split_workspace_bytes(2, 4096, 32, 128, row_begin=4095, **kw),
                         2, 4096, 32, 128, 4095) == n


def test_rows_split_plan_rejects_bad_arguments():
    n, keys = ctypes.c_int(0), ctypes.c_int(0)
    lib = mta.lib()
    assert lib.mta_forward_rows_split_plan(1, 64, 4, 128, 3, 5, 2, 64, mta.KQ_PRE, 0, ctypes.byref(n),
                                           ctypes.byref(keys)) == mta.ERR_INVALID_ARG
    assert lib.mta_forward_rows_split_plan(1, 64, 4, 128, 3, 5, 2, 0, mta.KQ_PRE, -1, ctypes.byref(n),
                                           ctypes.byref(keys)) == mta.ERR_INVALID_ARG
    assert lib.mta_forward_rows_split_plan(1, 64, 4, 128, 3, 5, 2, 0, mta.KQ_PRE, 0, None, None) == mta.ERR_INVALID_ARG


def test_noalloc_rejects_a_range_beyond_its_scratch():
    # a 512-row chunk at the T=4096 shape needs about 86 MB of partial results, more than the
    # library's scratch: refused before any GPU work
    need = ta.rows_split_workspace_bytes(2, 4096, 32, 128, row_begin=3584, c_q=4, c_k=9, c_h=4, kq="post",
                                         mix="pre", gn=True)
    assert need > mta.NOALLOC_SCRATCH_BYTES
    st = mta.lib().mta_forward_rows_split_noalloc(P, P + 0x100, P + 0x200, P, P, P, P, 1.0, P + 0x300, 2, 4096, 32,
                                                  128, 4, 9, 4, 3584, mta.KQ_POST | mta.MIX_PRE | mta.GN, None)
    assert st == mta.ERR_WORKSPACE
    assert "scratch" in mta.last_error()


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define MTA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == mta.NOALLOC_SCRATCH_BYTES
