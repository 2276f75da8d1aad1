"""The pins must catch plausible mistakes in the oracle.  Each case plants
one mistake (a sign flip, a swapped operand, a dropped term or factor, an
off-by-one bound, a wrong initial state) in a scratch copy of the oracle (its
C code or its Python layer) and runs the oracle's pin tests there; at least
one of them must fail.  CPU only; the repository's own oracle is not
touched."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_TESTS = ["tests/test_oracle_fwd.py", "tests/test_oracle_bwd.py",
             "tests/test_oracle_blockmask.py", "tests/test_oracle_ranges.py",
             "tests/test_oracle_diff.py"]

# (name, statement in oracle.c, the same statement with the mistake)
MUTATIONS = [
    ("bias sign",
     "return scale * dot_bf16(q + (size_t)r * d, k + (size_t)c * d, d) + beta;",
     "return scale * dot_bf16(q + (size_t)r * d, k + (size_t)c * d, d) - beta;"),
    ("sigmoid sign",
     "static real sigmoid(real x) { return (real)1 / ((real)1 + exp(-x)); }",
     "static real sigmoid(real x) { return (real)1 / ((real)1 + exp(x)); }"),
    ("key bound off by one", "return r < n && c < n &&", "return r < n && c <= n &&"),
    ("query and key swapped",
     "return scale * dot_bf16(q + (size_t)r * d, k + (size_t)c * d, d) + beta;",
     "return scale * dot_bf16(q + (size_t)c * d, k + (size_t)r * d, d) + beta;"),
    ("sigmoid derivative sign", "return dp * p * ((real)1 - p);", "return dp * p * ((real)1 + p);"),
    ("dK from K instead of Q",
     "gk[t] += scale * ds * widen(q[(size_t)r * d + t]);",
     "gk[t] += scale * ds * widen(k[(size_t)r * d + t]);"),
    ("softmax_1 without its unit term",
     "real l = variant == V_SOFTMAX1 ? (real)1 : (real)0;", "real l = (real)0;"),
    ("online rescale inverted", "real alpha = exp(m - mnew);", "real alpha = exp(mnew - m);"),
    ("softmax_1 zero logit sign", "denom = exp(-m);", "denom = exp(m);"),
    ("padded-length bias uses n",
     "if (mode == B_LOG_PADLEN) return -log((real)L);",
     "if (mode == B_LOG_PADLEN) return -log((real)n);"),
    ("dV from dP instead of P",
     "gv[t] += p * widen(dout[(size_t)r * d + t]);",
     "gv[t] += dp * widen(dout[(size_t)r * d + t]);"),
    ("D from K instead of V",
     "D += p * dot_bf16(dout + (size_t)r * d, v + (size_t)c * d, d);",
     "D += p * dot_bf16(dout + (size_t)r * d, k + (size_t)c * d, d);"),
    ("softmax dS sign", "return p * (dp - Dr);", "return p * (dp + Dr);"),
    ("block-mask tile loses its last column",
     "for (int c = j * bk; c < (j + 1) * bk && c < L; ++c)",
     "for (int c = j * bk; c < (j + 1) * bk - 1 && c < L; ++c)"),
    ("LSE without the maximum", "lse[r - r0] = m + log(denom);", "lse[r - r0] = log(denom);"),
    ("dQ without the scale",
     "for (int t = 0; t < d; ++t) g[t] += scale * ds * widen(k[(size_t)c * d + t]);",
     "for (int t = 0; t < d; ++t) g[t] += ds * widen(k[(size_t)c * d + t]);"),
]

# (name, statement in oracle/__init__.py, the same statement with the mistake)
PY_MUTATIONS = [
    ("key range end exclusive",
     "return ((kr[:, :, 0:1] <= c) & (c <= kr[:, :, 1:2])).astype(np.uint8)",
     "return ((kr[:, :, 0:1] <= c) & (c < kr[:, :, 1:2])).astype(np.uint8)"),
    ("key range start exclusive",
     "return ((kr[:, :, 0:1] <= c) & (c <= kr[:, :, 1:2])).astype(np.uint8)",
     "return ((kr[:, :, 0:1] < c) & (c <= kr[:, :, 1:2])).astype(np.uint8)"),
    ("key ranges ignored", "    return key_range_mask(key_range, L)\n", "    return mask\n"),
    ("differential sign", "return o1 - lam * o2, lse1, lse2", "return o1 + lam * o2, lse1, lse2"),
    ("differential map 2 gradient sign",
     "return g1[0], g1[1], -lam * g2[0], -lam * g2[1], g1[2] - lam * g2[2]",
     "return g1[0], g1[1], lam * g2[0], -lam * g2[1], g1[2] - lam * g2[2]"),
    ("differential dV drops map 2",
     "return g1[0], g1[1], -lam * g2[0], -lam * g2[1], g1[2] - lam * g2[2]",
     "return g1[0], g1[1], -lam * g2[0], -lam * g2[1], g1[2]"),
]


CASES = [("oracle.c",) + m for m in MUTATIONS] + [("__init__.py",) + m for m in PY_MUTATIONS]


@pytest.mark.parametrize("fname,name,orig,mutant", CASES, ids=[c[1] for c in CASES])
def test_planted_mistake_fails_a_pin(tmp_path, fname, name, orig, mutant):
    ignore = shutil.ignore_patterns("__pycache__", "*.so", "*.o")
    for sub in ("oracle", "tests", "synthetic"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub, ignore=ignore)
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path)
    src = tmp_path / "oracle" / fname
    text = src.read_text()
    assert text.count(orig) == 1, f"{name}: the statement to alter is not in {fname} once"
    src.write_text(text.replace(orig, mutant))
    res = subprocess.run([sys.executable, "-m", "pytest", *PIN_TESTS, "-x", "-q"], cwd=tmp_path,
                         capture_output=True, text=True, timeout=900)
    tail = res.stdout.strip().splitlines()[-1] if res.stdout.strip() else res.stderr[-500:]
    assert res.returncode == 1 and " failed" in tail, \
        f"{name}: no pin failed (exit {res.returncode}): {tail}"
