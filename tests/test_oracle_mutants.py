"""The oracle's pins catch plausible mistakes in it.

Each case plants one mistake in a copy of the C++ oracle (`oracle/mta_oracle.cpp`): a dropped
term or mask, a wrong sign or index, a transposed operand, a wrong constant. The copy is built
with g++ into a temporary directory, and the pins of `tests/test_oracle_pins.py` run against it
in a child process (a planted mistake may crash it without taking this process down). At least
one pin must fail for every mistake, and none for the unmodified copy.

The pin that compares the C++ oracle with its Python transcription is left out: that is a
second rendering of the same definitions, not a pin to something outside the oracle. What has
to catch each mistake is one of the others: scaled dot-product attention at identity kernels,
closed forms for shifted and lagged kernels, linearity, permutation and causality invariants,
torch's layer_norm for GroupNorm, and the hand-computed examples in `tests/golden/`.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mta_oracle.cpp")

# name -> (text in the oracle, replacement); each text occurs exactly once
MUTANTS = {
    "logit scale 1/d instead of 1/sqrt(d)": (
        "const double scale = 1.0 / std::sqrt((double)p.d);", "const double scale = 1.0 / (double)p.d;"),
    "pre-softmax mixing with w transposed": (
        "acc += wrow[u2] * raw[(size_t)u2 * p.T + j];",
        "acc += p.w_pre[((size_t)g * p.c_h + u2) * p.c_h + u] * raw[(size_t)u2 * p.T + j];"),
    "Mask_0 before the convolution dropped": (
        "if (r < 0 || s < 0 || s >= gm.T || s > r) return 0.0;", "if (r < 0 || s < 0 || s >= gm.T) return 0.0;"),
    "Mask_0 before the convolution also zeroes the diagonal": (
        "if (r < 0 || s < 0 || s >= gm.T || s > r) return 0.0;", "if (r < 0 || s < 0 || s >= gm.T || s >= r) return 0.0;"),
    "pre-softmax convolution: key offset with the wrong sign": (
        "masked_logit(gm, r - a, j - e + h0, u)", "masked_logit(gm, r - a, j + e - h0, u)"),
    "pre-softmax convolution: query lag dropped": (
        "masked_logit(gm, r - a, j - e + h0, u)", "masked_logit(gm, r, j - e + h0, u)"),
    "pre-softmax convolution: key axis not centred": (
        "const int T = p.T, h0 = (p.c_k - 1) / 2;", "const int T = p.T, h0 = 0;"),
    "pre-softmax convolution: kernel indexed [e][a]": (
        "acc += th[a * p.c_k + e] * masked_logit", "acc += th[e * p.c_q + a] * masked_logit"),
    "post-softmax convolution: key offset with the wrong sign": (
        "prob_at(gm, i - a, j - e + h0, u)", "prob_at(gm, i - a, j + e - h0, u)"),
    "post-softmax convolution: query lag dropped": (
        "prob_at(gm, i - a, j - e + h0, u)", "prob_at(gm, i, j - e + h0, u)"),
    "post-softmax convolution: key axis not centred": (
        "const int T = p.T, c_h = p.c_h, h0 = (p.c_k - 1) / 2;", "const int T = p.T, c_h = p.c_h, h0 = 0;"),
    "post-softmax mixing with w transposed": (
        "mixed[(size_t)u * T + j] += wrow[u2] * A[(size_t)u2 * T + j];",
        "mixed[(size_t)u * T + j] += p.w_post[((size_t)g * c_h + u2) * c_h + u] * A[(size_t)u2 * T + j];"),
    "softmax normaliser without the diagonal term": ("    sum += out[j];", "    if (j < i) sum += out[j];"),
    "values taken from the query row": (
        "o[c] += a_u[j] * p.v[idx4(p, b, j, m, c)];", "o[c] += a_u[j] * p.v[idx4(p, b, i, m, c)];"),
    "GroupNorm with the unbiased variance": ("    var /= d;", "    var /= (d - 1);"),
    "GroupNorm eps 1e-6": ("std::sqrt(var + 1e-5)", "std::sqrt(var + 1e-6)"),
    "GroupNorm mean not subtracted": ("gamma[(size_t)m * d + c] * (o[c] - mean) * inv", "gamma[(size_t)m * d + c] * o[c] * inv"),
    "GroupNorm scale indexed [c][m]": ("gamma[(size_t)m * d + c] *", "gamma[(size_t)c * p.M + m] *"),
    "gate dropped": ("dst[c] = lambda * (gamma", "dst[c] = (gamma"),
    "heads of a group strided instead of contiguous": (
        "    const int m = g * p.c_h + u;\n    for (int j = 0; j < p.T; ++j) {",
        "    const int m = u * (p.M / p.c_h) + g;\n    for (int j = 0; j < p.T; ++j) {"),
    "pre-softmax convolution: every head takes its group's first kernel": (
        "p.theta_pre + (size_t)(g * p.c_h + u) * p.c_q * p.c_k", "p.theta_pre + (size_t)(g * p.c_h) * p.c_q * p.c_k"),
    "post-softmax convolution: every head takes its group's first kernel": (
        "p.theta_post + (size_t)(g * c_h + u) * p.c_q * p.c_k", "p.theta_post + (size_t)(g * c_h) * p.c_q * p.c_k"),
    "pre-softmax mixing: every group takes the first group's weights": (
        "p.w_pre + ((size_t)g * p.c_h + u) * p.c_h", "p.w_pre + ((size_t)u) * p.c_h"),
    "post-softmax mixing: every group takes the first group's weights": (
        "p.w_post + ((size_t)g * c_h + u) * c_h", "p.w_post + ((size_t)u) * c_h"),
    "softmax normaliser over future keys too": (
        "for (int j = 0; j <= i; ++j) {\n    out[j] = std::exp(x[j] - mx);",
        "for (int j = 0; j < T; ++j) {\n    out[j] = std::exp(x[j] - mx);"),
    "both sides share the convolution kernels": (
        "const double* theta_post = (kq == 3) ? theta + th_size : theta;", "const double* theta_post = theta;"),
    "both sides share the mixing weights": (
        "const double* w_post = (mix == 3) ? w + w_size : w;", "const double* w_post = w;"),
}

# runs the pins in a child process against the oracle library given on the command line
_DRIVER = (
    "import sys; sys.path.insert(0, sys.argv[2]);"
    "from oracle import oracle; oracle._LIB = sys.argv[1]; oracle._lib = None;"
    "import pytest;"
    "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-k', 'not transcription',"
    " sys.argv[2] + '/tests/test_oracle_pins.py']))"
)


def _build_and_run(name, patch, workdir):
    src = open(SRC).read()
    if patch is not None:
        old, new = patch
        assert src.count(old) == 1, f"{name}: the text to replace must occur once"
        src = src.replace(old, new)
    tag = "".join(ch if ch.isalnum() else "_" for ch in name)[:60]
    cpp, lib = os.path.join(workdir, tag + ".cpp"), os.path.join(workdir, tag + ".so")
    with open(cpp, "w") as f:
        f.write(src)
    subprocess.run(["g++", "-O1", "-fopenmp", "-std=c++17", "-shared", "-fPIC", "-o", lib, cpp], check=True)
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", _DRIVER, lib, ROOT], capture_output=True, text=True, env=env,
                       timeout=300)
    failed = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED")]
    return r.returncode, failed, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    workdir = str(tmp_path_factory.mktemp("oracle_mutants"))
    cases = {"unmodified": None, **MUTANTS}
    with concurrent.futures.ThreadPoolExecutor(4) as ex:
        futs = {name: ex.submit(_build_and_run, name, patch, workdir) for name, patch in cases.items()}
        return {name: f.result() for name, f in futs.items()}


def test_unmodified_copy_passes_every_pin(outcomes):
    rc, failed, tail = outcomes["unmodified"]
    assert rc == 0, tail


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistake(outcomes, name):
    rc, failed, tail = outcomes[name]
    assert rc != 0, f"no pin fails when the oracle has this mistake: {name}"
    # a failing pin (exit status 1), not a crash or a collection error
    assert rc == 1 and failed, tail
    print(f"{name}: caught by {failed[0][len('FAILED '):].split(' - ')[0]}")
