"""Mutation tests: every plausible mistake planted in a copy of the oracle must be caught.

The mistakes are planted in copies on the CPU (a rewritten C source compiled into a
temporary library, or a rewritten chunk step executed in a scratch namespace); the
oracle itself is never modified.  A mutant "survives" if every pin passes for it,
which would mean the pins could not tell that mistake from the truth.
"""
import functools
import inspect
import os
import re
import textwrap

import numpy as np
import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

# (name, original text, replacement).  Each original must occur in the source.
C_MUTANTS = [
    ("decay dropped from the state",
     "S[i * Dk + j] = a * S[i * Dk + j] - erase", "S[i * Dk + j] = S[i * Dk + j] - erase"),
    ("decay not applied to the erase term",
     "const double erase = a * b * Sk[i];", "const double erase = b * Sk[i];"),
    ("erase sign flipped", "- erase * kt[j]", "+ erase * kt[j]"),
    ("beta dropped from the write", "const double write = b * vt[i];",
     "const double write = vt[i];"),
    ("key index reversed in S k", "acc += S[i * Dk + j] * kt[j];",
     "acc += S[i * Dk + j] * kt[Dk - 1 - j];"),
    ("GQA head chosen by division", "hk = h % Hk", "hk = h / (Hv / Hk)"),
    ("initial state ignored", "if (initial_state)\n", "if (0)\n"),
    ("sequence start off by one", "for (int64_t t = cu_seqlens[n]; t",
     "for (int64_t t = cu_seqlens[n] + (n > 0); t"),
    ("gate read as log2 instead of natural log", "exp(g[t * Hv + h])", "exp2(g[t * Hv + h])"),
    ("query and key swapped",
     "const double *kt = k + (t * Hk + hk) * Dk;\n            const double *qt = q + (t * Hk + hk) * Dk;",
     "const double *kt = q + (t * Hk + hk) * Dk;\n            const double *qt = k + (t * Hk + hk) * Dk;"),
    ("output read before the update", None, None),   # block swap, handled below
]


def _mutate_c(src: str, name: str, orig, repl) -> str:
    if orig is not None:
        assert orig in src, f"mutation anchor for {name!r} not found in the oracle source"
        return src.replace(orig, repl)
    # move the output block ahead of the state update inside gdn_token_step
    upd = src.index("    /* S <- a*S")
    out = src.index("    /* o_t = S q_t")
    end = src.index("}\n", src.index("ot[i] = acc;")) + 2
    return src[:upd] + src[out:end] + src[upd:out] + src[end:]


def _pins_that_fail(rec, dec):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            if pin is oracle_pins.pin_decode:
                pin(rec, decode=dec)
            else:
                pin(rec)
        except (AssertionError, ValueError, FloatingPointError) as e:  # noqa: PERF203
            failed.append((pin.__name__, str(e).splitlines()[0][:100]))
    return failed


@pytest.mark.parametrize("name,orig,repl", C_MUTANTS, ids=[m[0] for m in C_MUTANTS])
def test_c_oracle_mutant_is_caught(tmp_path, name, orig, repl):
    with open(SRC) as f:
        src = f.read()
    mutated = _mutate_c(src, name, orig, repl)
    assert mutated != src
    msrc = tmp_path / "mutant.c"
    msrc.write_text(mutated)
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build(out_path=lib_path, src_path=str(msrc))
    lib = oracle.load_library(lib_path)
    rec = functools.partial(oracle.recurrent, lib=lib)
    dec = functools.partial(oracle.decode_step, lib=lib)
    with np.errstate(all="ignore"):
        failed = _pins_that_fail(rec, dec)
    assert failed, f"mutant {name!r} passed every pin"


# Mistakes planted in the chunked (Map-Reduce-Map) form; the pin comparing it with the
# recurrence must catch each.
CHUNK_MUTANTS = [
    ("beta of the column token used in A", "A = np.tril(bc[:, None] *", "A = np.tril(bc[None, :] *"),
    ("lambda dropped from the state update", "lam = np.exp(Gam[-1] - Gam)",
     "lam = np.ones_like(Gam)"),
    ("output mask drops the diagonal", "np.tril(Qc @ Kc.T)", "np.tril(Qc @ Kc.T, k=-1)"),
    ("chunk decay of the carried state dropped", "S_next = gamma[-1] * S", "S_next = S"),
    ("gamma dropped from W", "((bc * gamma)[:, None] * Kc)", "(bc[:, None] * Kc)"),
    ("decay matrix not masked", "D[r_idx, s_idx] = np.exp(Gam[r_idx] - Gam[s_idx])",
     "D[:, :] = np.exp(Gam[:, None] - Gam[None, :])"),
]


@pytest.mark.parametrize("name,orig,repl", CHUNK_MUTANTS, ids=[m[0] for m in CHUNK_MUTANTS])
def test_chunked_form_mutant_is_caught(monkeypatch, name, orig, repl):
    src = textwrap.dedent(inspect.getsource(oracle._chunk_step))
    assert orig in src, f"mutation anchor for {name!r} not found"
    ns = dict(oracle.__dict__)
    exec(compile(src.replace(orig, repl), "<mutant>", "exec"), ns)  # noqa: S102
    monkeypatch.setattr(oracle, "_chunk_step", ns["_chunk_step"])
    with np.errstate(all="ignore"), pytest.raises(AssertionError):
        oracle_pins.pin_chunked(oracle.recurrent)


# Mistakes planted in the per-key-channel (KDA) part of the C oracle only: the text is
# replaced after the KDA marker, so the gated delta rule above it is left intact.
KDA_MARK = "static void kda_token_step("
KDA_C_MUTANTS = [
    ("kda decay applied to value rows", "S[i * Dk + j] *= a[j];", "S[i * Dk + j] *= a[i % Dk];"),
    ("kda gate channels reversed", "a[j] = exp(gt[j]);", "a[j] = exp(gt[Dk - 1 - j]);"),
    ("kda gate read as log2", "a[j] = exp(gt[j]);", "a[j] = exp2(gt[j]);"),
    ("kda gate indexed per head", "g + (t * Hv + h) * Dk", "g + (t * Hv + h)"),
    ("kda decode gate indexed per head", "g + (b * Hv + h) * Dk", "g + (b * Hv + h)"),
    ("kda erase sign flipped", "- erase * kt[j]", "+ erase * kt[j]"),
    ("kda beta dropped from the erase", "const double erase = b * u[i];",
     "const double erase = u[i];"),
    ("kda erase reads the state before the decay", None, "decay-after-erase"),
    ("kda output read before the update", None, "output-first"),
]


def _mutate_kda(src: str, name: str, orig, repl) -> str:
    head, tail = src[:src.index(KDA_MARK)], src[src.index(KDA_MARK):]
    if orig is not None:
        assert orig in tail, f"mutation anchor for {name!r} not found in the KDA part"
        return head + tail.replace(orig, repl)
    dec = tail.index("    /* S <- S Diag(a)")
    ubl = tail.index("    /* u = (S Diag(a)) k_t */")
    upd = tail.index("    /* S <- S - b u k^T + b v k^T */")
    out = tail.index("    /* o_t = S q_t with the updated state */")
    end = tail.index("}\n", tail.index("ot[i] = acc;", out)) + 2
    if repl == "decay-after-erase":   # u = S k, then S <- S Diag(a), then the rank-1 terms
        tail = tail[:dec] + tail[ubl:upd] + tail[dec:ubl] + tail[upd:]
    else:                             # o = S q before any of the update
        tail = tail[:dec] + tail[out:end] + tail[dec:out] + tail[end:]
    return head + tail


@pytest.mark.parametrize("name,orig,repl", KDA_C_MUTANTS, ids=[m[0] for m in KDA_C_MUTANTS])
def test_kda_c_oracle_mutant_is_caught(tmp_path, name, orig, repl):
    with open(SRC) as f:
        src = f.read()
    mutated = _mutate_kda(src, name, orig, repl)
    assert mutated != src
    msrc = tmp_path / "mutant.c"
    msrc.write_text(mutated)
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build(out_path=lib_path, src_path=str(msrc))
    lib = oracle.load_library(lib_path)
    rec = functools.partial(oracle.recurrent, lib=lib)
    dec = functools.partial(oracle.decode_step, lib=lib)
    failed = []
    with np.errstate(all="ignore"):
        for pin in oracle_pins.KDA_PINS:
            try:
                pin(rec, decode=dec) if pin is oracle_pins.pin_kda_decode else pin(rec)
            except (AssertionError, ValueError, FloatingPointError) as e:  # noqa: PERF203
                failed.append((pin.__name__, str(e).splitlines()[0][:100]))
    assert failed, f"mutant {name!r} passed every KDA pin"


KDA_CHUNK_MUTANTS = [
    ("kda lambda dropped from the state update", "lam = np.exp(Gam[-1][None, :] - Gam)",
     "lam = np.ones_like(Gam)"),
    ("kda chunk decay of the carried state dropped", "S_next = S * gam[-1][None, :]",
     "S_next = S"),
    ("kda pairwise decay averaged over channels",
     "Dpair = np.exp(Gam[r_idx] - Gam[s_idx])",
     "Dpair = np.exp(Gam[r_idx] - Gam[s_idx]).mean(axis=1, keepdims=True)"),
    ("kda gamma dropped from W", "(bc[:, None] * (Kc * gam))", "(bc[:, None] * Kc)"),
    ("kda query decay dropped", "(Qc * gam) @ S.T", "Qc @ S.T"),
    ("kda cumulative gate exclusive", "Gam = np.cumsum(Gc, axis=0)",
     "Gam = np.cumsum(Gc, axis=0) - Gc"),
]


@pytest.mark.parametrize("name,orig,repl", KDA_CHUNK_MUTANTS, ids=[m[0] for m in KDA_CHUNK_MUTANTS])
def test_kda_chunked_form_mutant_is_caught(monkeypatch, name, orig, repl):
    src = textwrap.dedent(inspect.getsource(oracle._chunk_step_kda))
    assert orig in src, f"mutation anchor for {name!r} not found"
    ns = dict(oracle.__dict__)
    exec(compile(src.replace(orig, repl), "<mutant>", "exec"), ns)  # noqa: S102
    monkeypatch.setattr(oracle, "_chunk_step_kda", ns["_chunk_step_kda"])
    with np.errstate(all="ignore"), pytest.raises(AssertionError):
        oracle_pins.pin_kda_chunked(oracle.recurrent)


PROLOGUE_MUTANTS = [
    ("sigmoid of -x", "sigmoid", "return 1.0 / (1.0 + np.exp(-x))", "return 1.0 / (1.0 + np.exp(x))"),
    ("softplus without its max term", "softplus", "return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))",
     "return np.log1p(np.exp(-np.abs(x)))"),
    ("softplus as log(e^x) only", "softplus", "return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))",
     "return np.maximum(x, 0.0)"),
    ("L1 norm instead of L2", "l2_normalize", "norm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))",
     "norm = np.sum(np.abs(x), axis=-1, keepdims=True)"),
    ("norm over the head axis", "l2_normalize", "norm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))",
     "norm = np.sqrt(np.sum(x * x, axis=-2, keepdims=True))"),
    ("g = +softplus", "prologue", "g = -softplus(g)", "g = softplus(g)"),
    ("beta flag ignored", "prologue", "beta = sigmoid(beta)", "beta = beta"),
    # the bit-to-step mapping: a step keyed to another step's bit, or run whatever the bits
    ("softplus keyed to the sigmoid bit", "prologue", "if flags & PROLOGUE_G_SOFTPLUS:",
     "if flags & PROLOGUE_BETA_SIGMOID:"),
    ("sigmoid keyed to the norm bit", "prologue", "if flags & PROLOGUE_BETA_SIGMOID:",
     "if flags & PROLOGUE_QK_L2NORM:"),
    ("norm on any flag", "prologue", "if flags & PROLOGUE_QK_L2NORM:", "if flags:"),
    ("sigmoid always", "prologue", "if flags & PROLOGUE_BETA_SIGMOID:", "if True:"),
    ("norm of q only", "prologue", "q, k = l2_normalize(q), l2_normalize(k)", "q = l2_normalize(q)"),
]


@pytest.mark.parametrize("name,fn,orig,repl", PROLOGUE_MUTANTS, ids=[m[0] for m in PROLOGUE_MUTANTS])
def test_prologue_mutant_is_caught(monkeypatch, name, fn, orig, repl):
    src = textwrap.dedent(inspect.getsource(getattr(oracle, fn)))
    assert orig in src, f"mutation anchor for {name!r} not found"
    ns = dict(oracle.__dict__)
    exec(compile(src.replace(orig, repl), "<mutant>", "exec"), ns)  # noqa: S102
    monkeypatch.setattr(oracle, fn, ns[fn])
    failed = 0
    with np.errstate(all="ignore"):
        for pin in oracle_pins.PROLOGUE_PINS:
            try:
                pin()
            except (AssertionError, ValueError, FloatingPointError):
                failed += 1
    assert failed, f"mutant {name!r} passed every prologue pin"


def test_mutation_anchor_list_is_current():
    with open(SRC) as f:
        src = f.read()
    for name, orig, _ in C_MUTANTS:
        if orig is not None:
            assert src.count(orig) >= 1, name
    assert re.search(r"/\* o_t = S q_t", src) and re.search(r"/\* S <- a\*S", src)
