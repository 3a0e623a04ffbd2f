"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (a flipped sign,
a dropped term, a transposed index, the other reading of an ambiguous step),
builds it, and runs the pin suite against it with the regression fixtures left
out, so that only checks against the mathematics count.  Every mutant must fail
at least one pin; the unmodified copy must pass them all.  CPU only."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "ttt_oracle.c")
# regression checks (stored values, determinism) say nothing about correctness
NOT_PINS = "not golden and not deterministic and not thread_count"

MUTANTS = {
    "update sign": (
        "G[i * d + j] += et * e[i] * k[j];", "G[i * d + j] -= et * e[i] * k[j];"),
    "read excludes the chunk's updates": (
        "s += (Ws[i * d + j] - G[i * d + j]) * q[j];", "s += Ws[i * d + j] * q[j];"),
    "error without the target": (
        "s += Ws[i * d + j] * k[j];\n                e[i] = s - v[i];",
        "s += Ws[i * d + j] * k[j];\n                e[i] = s;"),
    "MLP error without the target": (
        "s += W2s[(size_t)i * hd + u] * a[u];\n                e[i] = s - v[i];",
        "s += W2s[(size_t)i * hd + u] * a[u];\n                e[i] = s;"),
    "transposed state in the error": (
        "for (int j = 0; j < d; ++j) s += Ws[i * d + j] * k[j];",
        "for (int j = 0; j < d; ++j) s += Ws[j * d + i] * k[j];"),
    "mean over the chunk instead of the sum": (
        "for (int i = 0; i < d * d; ++i) W[i] = Ws[i] - G[i];",
        "for (int i = 0; i < d * d; ++i) W[i] = Ws[i] - G[i] / (c1 - c0);"),
    "gradient at the running state": (
        "for (int j = 0; j < d; ++j) s += Ws[i * d + j] * k[j];",
        "for (int j = 0; j < d; ++j) s += (Ws[i * d + j] - G[i * d + j]) * k[j];"),
    "gelu' without the density term": (
        "return 0.5 * (1.0 + erf(x / sqrt(2.0))) + x * inv_sqrt_2pi * exp(-0.5 * x * x);",
        "return 0.5 * (1.0 + erf(x / sqrt(2.0)));"),
    "tanh form of gelu": (
        "return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));",
        "return 0.5 * x * (1.0 + tanh(0.7978845608028654 * (x + 0.044715 * x * x * x)));"),
    "W2 gradient from the pre-activation": (
        "G2[(size_t)i * hd + u] += et * e[i] * a[u];", "G2[(size_t)i * hd + u] += et * e[i] * h[u];"),
    "b1 never updated": (
        "if (b1_0) for (int u = 0; u < hd; ++u) g1[u] += et * dl[u];", ""),
    "MLP read with the chunk-start W2": (
        "s += (W2s[(size_t)i * hd + u] - G2[(size_t)i * hd + u]) * hr[u];",
        "s += W2s[(size_t)i * hd + u] * hr[u];"),
    "MLP backward skips gelu'": (
        "dl[u] = s * ttt_oracle_gelu_prime(h[u]);", "dl[u] = s;"),
    "chunk-start read includes the chunk's updates": (
        "for (int j = 0; j < d; ++j) s += Ws[i * d + j] * q[j];",
        "for (int j = 0; j < d; ++j) s += (Ws[i * d + j] - G[i * d + j]) * q[j];"),
    "momentum weights swapped": (
        "Mom[i] = beta * Mom[i] + (1.0 - beta) * Gr[i];", "Mom[i] = (1.0 - beta) * Mom[i] + beta * Gr[i];"),
    "momentum not carried": (
        "Mom[i] = beta * Mom[i] + (1.0 - beta) * Gr[i];", "Mom[i] = (1.0 - beta) * Gr[i];"),
    "momentum read with the running state": (
        "sz += W[i * d + j] * q[j];", "sz += (W[i * d + j] - Gr[i * d + j]) * q[j];"),
    # TTT-Linear with the inner bias, LayerNorm and residual inside f
    "LN backward drops the mean term": (
        "gu[i] = rs * (gu[i] - mh - uh[i] * mhu);", "gu[i] = rs * (gu[i] - uh[i] * mhu);"),
    "LN backward drops the projection term": (
        "gu[i] = rs * (gu[i] - mh - uh[i] * mhu);", "gu[i] = rs * (gu[i] - mh);"),
    "LN loss without the residual": (
        "const double r = k[i] + lnw[i] * uh[i] + lnb[i] - v[i];",
        "const double r = lnw[i] * uh[i] + lnb[i] - v[i];"),
    "inner bias never updated": (
        "gb[i] += et * gu[i];", "gb[i] += 0.0 * gu[i];"),
    "LN output without the residual": (
        "for (int i = 0; i < d; ++i) z[i] = q[i] + lnw[i] * uh[i] + lnb[i];",
        "for (int i = 0; i < d; ++i) z[i] = lnw[i] * uh[i] + lnb[i];"),
    "LN without eps": (
        "const double rs = 1.0 / sqrt(var + eps);", "const double rs = 1.0 / sqrt(var);"),
    "bias read without the chunk's updates": (
        "double acc = bc[i] - gb[i];", "double acc = bc[i];"),
    # the vector-Jacobian product of the TTT-Linear scan
    "VJP: dq read at the chunk-start state": (
        "acc += (Wc[i * d + j] - G[i * d + j]) * dz[i];", "acc += Wc[i * d + j] * dz[i];"),
    "VJP: state cotangent not sent into the update": (
        "dG[i] = -dW[i];", "dG[i] = 0.0;"),
    "VJP: dv sign": (
        "dv[i] = -de[i];", "dv[i] = de[i];"),
    "VJP: dk misses the error path": (
        "dk[j] += acc;", "dk[j] += 0.0 * acc;"),
    "VJP: update not unwound between tokens": (
        "for (int j = 0; j < d; ++j) G[i * d + j] -= et * e[i] * k[j];", ";"),
    "VJP: deta scaled by eta": (
        "sdeta += e[i] * acc;", "sdeta += et * e[i] * acc;"),
    "VJP: transposed update cotangent in dk": (
        "for (int i = 0; i < d; ++i) acc += dG[i * d + j] * e[i];",
        "for (int i = 0; i < d; ++i) acc += dG[j * d + i] * e[i];"),
    "VJP: read cotangent skips the chunk-start state": (
        "dWc[i * d + j] += dz[i] * q[j];", "dWc[i * d + j] += 0.0;"),
}


def build_variant(tmp_path, name, old=None, new=None):
    src = open(SRC).read()
    if old is not None:
        assert src.count(old) == 1, "mutation site not found: %s" % name
        src = src.replace(old, new)
    d = tmp_path / name.replace(" ", "_").replace("'", "")
    d.mkdir()
    c = d / "ttt_oracle.c"
    c.write_text(src)
    lib = d / "libttt_oracle.so"
    subprocess.check_call(["gcc", "-O3", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off",
                           "-fno-fast-math", "-shared", "-fPIC",
                           "-I", os.path.join(ROOT, "oracle"), str(c), "-o", str(lib),
                           "-lm", "-lpthread"])
    return str(lib)


def run_pins(lib):
    env = dict(os.environ, TTT_ORACLE_LIB=lib)
    return subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_pins.py"),
                           os.path.join(HERE, "test_oracle_bwd_pins.py"),
                           os.path.join(HERE, "test_oracle_ln_pins.py"),
                           "-x", "-q", "-p", "no:cacheprovider", "-k", NOT_PINS],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_unmodified_copy_passes_the_pins(tmp_path):
    r = run_pins(build_variant(tmp_path, "control"))
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    r = run_pins(build_variant(tmp_path, name, old, new))
    assert r.returncode != 0, "no pin caught: %s" % name
    failed = [l for l in r.stdout.splitlines() if l.startswith("FAILED")]
    print(name, "->", failed[:1])
