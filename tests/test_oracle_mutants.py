"""Mutation check of the oracle's pins: each plausible mistake below, planted
in a copy of oracle/oracle.c, must make the CPU pin suite fail, and the
unmutated copy must pass it.  This shows that the pins (golden examples,
brute force, closed forms, invariants, finite differences) pin the oracle's
arithmetic, not only its interface.  Everything runs on the CPU.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = ["tests/test_oracle_route.py", "tests/test_oracle_pft.py", "tests/test_oracle_ffn.py",
        "tests/test_oracle_backward.py"]

# (name, text in oracle.c, replacement, which occurrence: 1 = first)
MUTANTS = [
    ("silu derivative term dropped from dH1",
     "D1[j] = DA[j] * H3[j] * sg * (1.0 + H1[j] * (1.0 - sg));", "D1[j] = DA[j] * H3[j] * sg;", 1),
    ("1/tau missing from the gate gradient",
     "z[e] = z[e] * (gp[e] - c) * inv_tau;", "z[e] = z[e] * (gp[e] - c);", 1),
    ("sign of the softmax gradient's correction",
     "z[e] = z[e] * (gp[e] - c) * inv_tau;", "z[e] = z[e] * (gp[e] + c) * inv_tau;", 1),
    ("top-k ties to the higher expert index",
     "if (!taken[e] && (best < 0 || sel[e] > sel[best])) best = e;",
     "if (!taken[e] && (best < 0 || sel[e] >= sel[best])) best = e;", 1),
    ("combine weight copied from the token's first slot",
     "combine_weights[r] = topk_w ? topk_w[t * k + j] : 0.0f;",
     "combine_weights[r] = topk_w ? topk_w[t * k] : 0.0f;", 1),
    ("dH3 multiplied by W1 in dXs",
     "DX[i] = dot(D1, w1, w_dt, off, h) + dot(D3, w3, w_dt, off, h);",
     "DX[i] = dot(D1, w1, w_dt, off, h) + dot(D3, w1, w_dt, off, h);", 1),
    ("sigmoid in place of silu",
     "static double silu(double a) { return a / (1.0 + exp(-a)); }",
     "static double silu(double a) { return 1.0 / (1.0 + exp(-a)); }", 1),
    ("combine drops the routing weight",
     "y[t * d + c] += row_w[r] * ye[r * d + c];", "y[t * d + c] += ye[r * d + c];", 1),
    ("dW1 summed from dH3",
     "if (p1) p1[j] += X[i] * D1[j];", "if (p1) p1[j] += X[i] * D3[j];", 1),
    ("logit bias left out of the bf16 router's scores",
     "if (logit_bias) a = a + logit_bias[e];", "if (0) a = a + logit_bias[e];", 2),
    ("softmax over the selection keys (select bias in the weights)",
     "for (int e = 0; e < E; ++e) { p[e] = exp(s[e] - mx); den += p[e]; }",
     "for (int e = 0; e < E; ++e) { p[e] = exp(sel[e] - mx); den += p[e]; }", 1),
    ("tokens_per_expert off by one on expert 0",
     "if (tokens_per_expert) tokens_per_expert[e] = (int32_t)cnt;",
     "if (tokens_per_expert) tokens_per_expert[e] = (int32_t)cnt + (e == 0);", 1),
    ("the dispatch transpose ignores its addend",
     "dx[i] = dx_add ? ld(dx_add, add_dt, i) : 0.0;", "dx[i] = 0.0;", 1),
]


def _mutate(text, old, new, nth):
    at = -1
    for _ in range(nth):
        at = text.index(old, at + 1)
    return text[:at] + new + text[at + len(old):]


def _build_and_run(tmp, name, text):
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    src = os.path.join(tmp, name + ".c")
    with open(src, "w") as fh:
        fh.write(text)
    lib = ob.build(src=src, out=os.path.join(tmp, name + ".so"))
    env = dict(os.environ, XMOE_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + PINS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, (r.stdout + r.stderr)[-600:]


@pytest.mark.slow
def test_every_planted_mistake_is_caught(tmp_path):
    text = open(SRC).read()
    for _, old, _, nth in MUTANTS:
        assert text.count(old) >= nth, old
    jobs = [("control", text)] + [(f"m{i}", _mutate(text, old, new, nth))
                                  for i, (_, old, new, nth) in enumerate(MUTANTS)]
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        res = dict(zip([j[0] for j in jobs], ex.map(lambda j: _build_and_run(str(tmp_path), *j), jobs)))
    rc, log = res["control"]
    assert rc == 0, "the unmutated copy must pass the pins:\n" + log
    missed = [MUTANTS[i][0] for i in range(len(MUTANTS)) if res[f"m{i}"][0] == 0]
    assert not missed, f"planted mistakes no pin caught: {missed}"
