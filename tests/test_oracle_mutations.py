"""The oracle's pins must be able to fail.

Each case plants one plausible mistake in a private copy of the oracle's C source
(a wrong sign, a dropped term, an off-by-one index, a swapped operand, a reversed
tie rule), builds it with gcc on the CPU, and runs the pin suite against it: at
least one pin must fail for every planted mistake.  The shipped oracle is never
modified.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "fsl_oracle.c")

# (name, original text, planted text)
MUTATIONS = [
    ("prior sign", "erf(((double)i - p_c)", "erf((p_c - (double)i)"),
    ("prior scale sigma not 2 sigma", "/ (2.0 * cfg->sigma)", "/ (cfg->sigma)"),
    ("cell centre c+1", "((double)c + 0.5) * cfg->s", "((double)c + 1.0) * cfg->s"),
    ("score without 1/sqrt(d)", "return dot / sqrt((double)cfg->d) +", "return dot +"),
    ("prior without a_c", "cfg->lambda * a_c * g", "cfg->lambda * g"),
    ("readout without 1/sqrt(d)", "logit[x] = dot / sqrt((double)d);", "logit[x] = dot;"),
    ("availability off by one", "while ((n + 1) * (int64_t)s <= b_start)", "while (n * (int64_t)s <= b_start)"),
    ("eps outside the root", "sqrt(ms + cfg->eps)", "(sqrt(ms) + cfg->eps)"),
    ("eps dropped", "sqrt(ms + cfg->eps)", "sqrt(ms)"),
    ("tie rule id descending", "return (p->id < q->id) ? -1 : (p->id > q->id) ? 1 : 0;",
     "return (p->id > q->id) ? -1 : (p->id < q->id) ? 1 : 0;"),
    ("TopP by smallest norm", "if (p->val > q->val) return -1;\n    if (p->val < q->val) return 1;",
     "if (p->val < q->val) return -1;\n    if (p->val > q->val) return 1;"),
    ("recent taken from the oldest cells", "for (int64_t c = n_avail - n_recent; c < n_avail; ++c)",
     "for (int64_t c = 0; c < n_recent; ++c)"),
    ("mean over s-1", "kbar[c * d + f] = sum / s;", "kbar[c * d + f] = sum / (s - 1);"),
    ("min key norm instead of max", "if (j == c * s || nrm > best)", "if (j == c * s || nrm < best)"),
    ("values read from keys", "u += logit[x] * v[tok[x] * d + f];", "u += logit[x] * k[tok[x] * d + f];"),
    ("softmax not normalised", "        u /= z;\n", "\n"),
    ("one cell too few selected", "const int64_t nT = nA < K ? nA : K;", "const int64_t nT = nA < K ? nA : K - 1;"),
    ("block start of the next block", "const int64_t b_i = (int64_t)cfg->B * blk;",
     "const int64_t b_i = (int64_t)cfg->B * (blk + 1);"),
    ("gain ignored", "o[f] = (g ? g[f] : 1.0) * o[f] * inv;", "o[f] = o[f] * inv;"),
    ("query and key swapped in score", "dot += q_i[f] * kbar_c[f];", "dot += q_i[f] * q_i[f];"),
    ("rope rotation reversed", "y[2 * m] = x[2 * m] * c - x[2 * m + 1] * sn;", "y[2 * m] = x[2 * m] * c + x[2 * m + 1] * sn;"),
    ("rope frequency base^(-m/d)", "pow(rope_base, -2.0 * m / d)", "pow(rope_base, -1.0 * m / d)"),
    ("local window one short", "const int64_t lo = i - w > 0 ? i - w : 0;",
     "const int64_t lo = i - w + 1 > 0 ? i - w + 1 : 0;"),
    ("local logits without 1/sqrt(d)", "logit[j - lo] = dot / sqrt((double)d);", "logit[j - lo] = dot;"),
    ("alpha on the local branch", "o[f] = u / z + (o_lr ? alpha * o_lr[(i - i_lo) * d + f] : 0.0);",
     "o[f] = alpha * u / z + (o_lr ? o_lr[(i - i_lo) * d + f] : 0.0);"),
    ("gap_p one rank low", "*gap_p = relative_gap(order[cfg->P - 1].val, order[cfg->P].val);",
     "*gap_p = relative_gap(order[cfg->P].val, order[cfg->P + 1 < n_avail ? cfg->P + 1 : cfg->P].val);"),
    ("gap_p against the largest norm", "*gap_p = relative_gap(order[cfg->P - 1].val, order[cfg->P].val);",
     "*gap_p = relative_gap(order[0].val, order[cfg->P].val);"),
    ("readout reads the first selected cell for every cell", "for (int64_t j = T[t] * s; j < (T[t] + 1) * s; ++j)",
     "for (int64_t j = T[0] * s; j < (T[0] + 1) * s; ++j)"),
    ("gap_k term size without abs", "sum += fabs(q_i[f] * kbar_c[f]);", "sum += q_i[f] * kbar_c[f];"),
    ("gap_k term size without the prior",
     "return sum / sqrt((double)cfg->d) + cfg->lambda * a_c * fabs(prior_gate(cfg, i, c));",
     "return sum / sqrt((double)cfg->d);"),
    ("keys rotated at the query position", "rope_rotate(k + j * d, d, (double)j, rope_base",
     "rope_rotate(k + j * d, d, (double)i_lo, rope_base"),
]


def _pin_functions(golden):
    """Every pin as a zero-argument callable."""
    calls = []
    for name in dir(pins):
        fn = getattr(pins, name)
        if not name.startswith("test_") or not callable(fn):
            continue
        if name == "test_retention_brute_force":
            for P, W in [(0, 3), (3, 0), (4, 2), (7, 5)]:
                calls.append((f"{name}[{P},{W}]", lambda fn=fn, P=P, W=W: fn(P, W)))
        elif fn.__code__.co_argcount == 1:
            calls.append((name, lambda fn=fn: fn(golden)))
        else:
            calls.append((name, fn))
    return calls


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path, golden):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    mutated = tmp_path / "fsl_oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    inc = os.path.dirname(ORACLE_SRC)
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-I", inc, "-o", str(lib), str(mutated), "-lm"])
    failed = []
    with oracle.use_library(str(lib)):
        for pin_name, call in _pin_functions(golden):
            try:
                call()
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(pin_name)
    assert failed, f"no pin caught the planted mistake '{name}'"
