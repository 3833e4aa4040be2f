"""The oracle's pins must be able to fail.

Each case plants one plausible mistake in a private copy of one of the oracle's C
sources (fsl_oracle.c: FS / FS-L and the local branch; fsb_oracle.c: FS-B)
(a wrong sign, a dropped term, an off-by-one index, a swapped operand, a reversed
tie rule), builds it with gcc on the CPU, and runs the pin suite against it: at
least one pin must fail for every planted mistake.  The shipped oracle is never
modified.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_fsb_oracle_pins as fsb_pins
from tests import test_oracle_backward_pins as bwd_pins
from tests import test_oracle_pins as pins

ORACLE_DIR = os.path.dirname(oracle.__file__)
ORACLE_SRC = os.path.join(ORACLE_DIR, "fsl_oracle.c")
FSB_SRC = os.path.join(ORACLE_DIR, "fsb_oracle.c")

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
    ("gap_k at the boundary only", "for (int64_t t = 0; t < K && t + 1 < nA; ++t) { /* |r_t - r_t+1|",
     "for (int64_t t = K - 1; t < K && t + 1 < nA; ++t) { /* |r_t - r_t+1|"),
    ("keys rotated at the query position", "rope_rotate(k + j * d, d, (double)j, rope_base",
     "rope_rotate(k + j * d, d, (double)i_lo, rope_base"),
    # readout backward (Sec. 3.3 "Training"; App. D.4)
    ("backward: RMSNorm without the norm's own gradient", "du[f] = r * gf * dout[f] - r * r * r / d * sgu * u[f];",
     "du[f] = r * gf * dout[f];"),
    ("backward: RMSNorm correction r^2", "du[f] = r * gf * dout[f] - r * r * r / d * sgu * u[f];",
     "du[f] = r * gf * dout[f] - r * r / d * sgu * u[f];"),
    ("backward: gain dropped from du", "du[f] = r * gf * dout[f] -", "du[f] = r * dout[f] -"),
    ("backward: gain dropped from the correction", "sgu += gf * dout[f] * u[f];", "sgu += dout[f] * u[f];"),
    ("backward: eps dropped", "const double r = 1.0 / sqrt(ms / d + cfg->eps);", "const double r = 1.0 / sqrt(ms / d);"),
    ("backward: softmax without the mean term", "dl[x] = p[x] * (dl[x] - delta);", "dl[x] = p[x] * dl[x];"),
    ("backward: dq without 1/sqrt(d)", "dq[f] += dl[x] * k[tok[x] * d + f] / sd;", "dq[f] += dl[x] * k[tok[x] * d + f];"),
    ("backward: dq overwritten per token", "dq[f] += dl[x] * k[tok[x] * d + f] / sd;",
     "dq[f] = dl[x] * k[tok[x] * d + f] / sd;"),
    ("backward: dk from the key not the query", "dk[tok[x] * d + f] += dl[x] * q_i[f] / sd;",
     "dk[tok[x] * d + f] += dl[x] * k[tok[x] * d + f] / sd;"),
    ("backward: dv without the softmax weight", "dv[tok[x] * d + f] += p[x] * du[f];", "dv[tok[x] * d + f] += du[f];"),
    ("backward: dg without u", "dg[f] += r * dout[f] * u[f];", "dg[f] += r * dout[f];"),
    ("backward: softmax gradient from keys", "dp += du[f] * v[tok[x] * d + f];", "dp += du[f] * k[tok[x] * d + f];"),
    ("backward: dg size without the size of u", "dg_abs[f] += ra * fabs(dout[f] * u[f]) + r * fabs(dout[f]) * ua[f];",
     "dg_abs[f] += ra * fabs(dout[f] * u[f]);"),
]


# planted in fsb_oracle.c (FS-B: Sec. 3.4; App. E.1)
FSB_MUTATIONS = [
    ("chunks smallest first", "for (int k = 62; k >= 0; --k) /* powers of two of M, largest first */",
     "for (int k = 0; k <= 62; ++k) /* powers of two of M, largest first */"),
    ("split sorted descending", "    if (p->val < q->val) return -1;\n    if (p->val > q->val) return 1;\n    return (p->id",
     "    if (p->val > q->val) return -1;\n    if (p->val < q->val) return 1;\n    return (p->id"),
    ("node mean not divided by n", "mu[f] = s / (double)n;", "mu[f] = s;"),
    ("chunk radius from the first cell only", "        if (r > rho)\n            rho = r;",
     "        if (x == 0)\n            rho = r;"),
    ("join radius without the centre shift", "const double ra = F->rho[a_] + dist(F->mu + a_ * d, mu, d);",
     "const double ra = F->rho[a_];"),
    ("join centre unweighted", "mu[f] = (na * F->mu[a_ * d + f] + nb * F->mu[b_ * d + f]) / (na + nb);",
     "mu[f] = (F->mu[a_ * d + f] + F->mu[b_ * d + f]) / 2.0;"),
    ("node norm is the smallest", "        if (a[cells[x]] > A)\n            A = a[cells[x]];",
     "        if (A == -INFINITY || a[cells[x]] < A)\n            A = a[cells[x]];"),
    ("p_min from the latest cell", "        if (cells[x] < mn)\n            mn = cells[x];",
     "        if (cells[x] > mn)\n            mn = cells[x];"),
    ("priority without the radius term", "const double spread = fb->c * q_norm(q, d) * F->rho[v];",
     "const double spread = 0.0;"),
    ("priority prior taken two cells late", "const double g = erf(((double)i - F->pmin[v]) / (2.0 * cfg->sigma)); /* g_h(i - p_v^min) */",
     "const double g = erf(((double)i - F->pmin[v] - 2.0 * cfg->s) / (2.0 * cfg->sigma)); /* g_h(i - p_v^min) */"),
    ("leaves compete for their slots", "                leaves[n_leaf++] = beam[x]; /* a leaf keeps its slot */",
     "                kids[n_kid++] = beam[x];"),
    ("second forest admits above the threshold only", "if (a[c] >= fb->tau)", "if (a[c] > fb->tau)"),
    ("rerank without the log", "return mx + log(z) + cfg->lambda * a_c * g;", "return mx + z + cfg->lambda * a_c * g;"),
    ("rerank without the prior", "return mx + log(z) + cfg->lambda * a_c * g;", "return mx + log(z);"),
    ("rerank logits without 1/sqrt(d)", "        l[t] = dot / sqrt((double)d);", "        l[t] = dot;"),
    ("selection by the worst candidates", "while (y >= 0 && (rank[y].val < kv.val ||", "while (y >= 0 && (rank[y].val > kv.val ||"),
    ("rerank gap at the boundary only", "for (int64_t t = 0; t < K && t + 1 < nc; ++t) {",
     "for (int64_t t = K - 1; t < K && t + 1 < nc; ++t) {"),
    ("power iteration started at the nearest cell", "if (nrm > best || (nrm == best && cells[c] < bestid)) {",
     "if (best < 0 || nrm < best || (nrm == best && cells[c] < bestid)) {"),
]


def _pin_functions(golden):
    """Every pin of both suites as a zero-argument callable."""
    calls = []
    for mod in (pins, fsb_pins, bwd_pins):
        for name in dir(mod):
            fn = getattr(mod, name)
            if not name.startswith("test_") or not callable(fn):
                continue
            marks = getattr(fn, "pytestmark", [])
            params = [m for m in marks if m.name == "parametrize"]
            if params:
                argnames = [x.strip() for x in params[0].args[0].split(",")]
                for vals in params[0].args[1]:
                    vals = vals if isinstance(vals, tuple) else (vals,)
                    calls.append((f"{name}{vals}", lambda fn=fn, a=dict(zip(argnames, vals)): fn(**a)))
            elif fn.__code__.co_argcount == 1:
                calls.append((name, lambda fn=fn: fn(golden)))
            else:
                calls.append((name, fn))
    return calls


def _check_caught(src_path, name, old, new, tmp_path, golden):
    src = open(src_path).read()
    assert src.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    mutated = tmp_path / os.path.basename(src_path)
    mutated.write_text(src.replace(old, new))
    others = [s for s in oracle.SOURCES if os.path.basename(s) != os.path.basename(src_path)]
    lib = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-I", ORACLE_DIR, "-o", str(lib),
                           str(mutated), *others, "-lm"])
    failed = []
    with oracle.use_library(str(lib)):
        for pin_name, call in _pin_functions(golden):
            try:
                call()
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(pin_name)
    assert failed, f"no pin caught the planted mistake '{name}'"


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path, golden):
    _check_caught(ORACLE_SRC, name, old, new, tmp_path, golden)


@pytest.mark.parametrize("name,old,new", FSB_MUTATIONS, ids=[m[0] for m in FSB_MUTATIONS])
def test_fsb_pins_catch_planted_mistake(name, old, new, tmp_path, golden):
    _check_caught(FSB_SRC, name, old, new, tmp_path, golden)
