"""The gradient oracle's pins catch plausible mistakes in it.

Each case plants one mistake in a copy of `oracle/backward.py` (the fp64 gradient oracle): a
dropped mask or gate, a wrong sign, lag or scale, a transposed mixing, swapped outputs. The pins
of `tests/test_oracle_backward_pins.py` then run against the copy in a child process. At least one
pin must fail for every mistake, and none for the unmodified copy. The pins tie the copy to things
outside it: the C++ oracle's forward, central finite differences of the C++ oracle, torch's scaled
dot-product attention and layer_norm under autograd, and log-sum-exps written out by plain loops.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "backward.py")

# name -> (text in the gradient oracle, replacement); each text occurs exactly once
MUTANTS = {
    "logit scale 1/d instead of 1/sqrt(d)": (
        "L = qh @ kh.transpose(-1, -2) / math.sqrt(d)", "L = qh @ kh.transpose(-1, -2) / d"),
    "convolution: key offset with the wrong sign": (
        "2 * h0 - e:2 * h0 - e + T]", "e:e + T]"),
    "convolution: query lag dropped": (
        "pad[..., c_q - 1 - a:c_q - 1 - a + T,", "pad[..., c_q - 1:c_q - 1 + T,"),
    "mixing with w transposed": ('"guv,bgvij->bguij"', '"gvu,bgvij->bguij"'),
    "Mask_0 before the convolution dropped": (
        "L = _conv(L.masked_fill(future, 0.0), th_pre)", "L = _conv(L, th_pre)"),
    "Mask_0 after the convolution after softmax dropped": (
        "A = _conv(A, th_post).masked_fill(future, 0.0)", "A = _conv(A, th_post)"),
    "softmax over future keys too": ("return L.masked_fill(future, -math.inf)", "return L"),
    "values taken from the queries": ("vh = v.permute(0, 2, 1, 3)", "vh = q.permute(0, 2, 1, 3)"),
    "GroupNorm with the unbiased variance": (
        "var = ((O - mu) ** 2).mean(dim=-1, keepdim=True)", "var = ((O - mu) ** 2).sum(dim=-1, keepdim=True) / (d - 1)"),
    "gate dropped": ("O = lam * (gamma.reshape(M, d)", "O = (gamma.reshape(M, d)"),
    "both sides share the first side's parameters": (
        "return params[0], params[1]", "return params[0], params[0]"),
    "output gradient scaled": (
        "out.backward(torch.tensor(np.asarray(dout, dtype=np.float64), dtype=_DT))",
        "out.backward(2.0 * torch.tensor(np.asarray(dout, dtype=np.float64), dtype=_DT))"),
    "key and value gradients swapped": ('"dk": grad(tk), "dv": grad(tv)', '"dk": grad(tv), "dv": grad(tk)'),
    "log-sum-exp over the query axis": (
        "torch.logsumexp(C, dim=-1)", "torch.logsumexp(C.masked_fill(torch.isinf(C), 0.0), dim=-2)"),
}

# runs the pins in a child process with the copy given on the command line as oracle.backward
_DRIVER = (
    "import sys, types; sys.path.insert(0, sys.argv[2]);"
    "import oracle;"
    "m = types.ModuleType('oracle.backward'); m.__file__ = sys.argv[1];"
    "exec(compile(open(sys.argv[1]).read(), sys.argv[1], 'exec'), m.__dict__);"
    "sys.modules['oracle.backward'] = m; oracle.backward = m;"
    "import pytest;"
    "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', sys.argv[2] + '/tests/test_oracle_backward_pins.py']))"
)


def _run(name, patch, workdir):
    src = open(SRC).read()
    if patch is not None:
        old, new = patch
        assert src.count(old) == 1, f"{name}: the text to replace must occur once"
        src = src.replace(old, new)
    tag = "".join(ch if ch.isalnum() else "_" for ch in name)[:60]
    path = os.path.join(workdir, tag + ".py")
    with open(path, "w") as f:
        f.write(src)
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", _DRIVER, path, ROOT], capture_output=True, text=True, env=env,
                       timeout=600)
    failed = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED")]
    return r.returncode, failed, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    workdir = str(tmp_path_factory.mktemp("backward_oracle_mutants"))
    cases = {"unmodified": None, **MUTANTS}
    with concurrent.futures.ThreadPoolExecutor(4) as ex:
        futs = {name: ex.submit(_run, name, patch, workdir) for name, patch in cases.items()}
        return {name: f.result() for name, f in futs.items()}


def test_unmodified_copy_passes_every_pin(outcomes):
    rc, failed, tail = outcomes["unmodified"]
    assert rc == 0, tail


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistake(outcomes, name):
    rc, failed, tail = outcomes[name]
    assert rc != 0, f"no pin fails when the gradient oracle has this mistake: {name}"
    assert rc == 1 and failed, tail
    print(f"{name}: caught by {failed[0][len('FAILED '):].split(' - ')[0]}")
