"""Pins that tie the CPU oracle to facts fixed by the pages and by mathematics.

Each pin takes a ``recurrent``-like callable (same signature as
``oracle.recurrent``) and raises AssertionError when the callable disagrees with
the fact it checks.  The pin tests run them against the real oracle; the mutation
tests run them against deliberately broken copies of the oracle and require every
copy to fail at least one pin.

None of these pins re-types the oracle's update formula: each compares against an
independent construction (a hand-worked example, the closed product form, a closed
form of a special case, an invariant, or the chunked reformulation).
"""
from __future__ import annotations

import json
import os
import re

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand_unit(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_case(seed, lengths, Hk, Hv, Dk, Dv, init=True, g_shift=0.0, kda=False):
    """kda: one gate per key channel, g [T, Hv, Dk], instead of one per head."""
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    q = _rand_unit(rng, (T, Hk, Dk))
    k = _rand_unit(rng, (T, Hk, Dk))
    v = rng.standard_normal((T, Hv, Dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, Hv))))
    x = rng.standard_normal((T, Hv, Dk) if kda else (T, Hv)) + g_shift
    g = -(np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x))))
    s0 = rng.standard_normal((len(lengths), Hv, Dv, Dk)) * 0.5 if init else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=s0, cu_seqlens=cu)


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


# 1. hand-worked example (tests/golden/hand_worked_d2_t2.json)
def pin_hand_example(rec, name="hand_worked_d2_t2.json"):
    with open(os.path.join(GOLDEN, name)) as f:
        gold = json.load(f)
    inp = {k_: np.array(v_, dtype=np.float64) for k_, v_ in gold["inputs"].items()}
    o, fs = rec(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["initial_state"])
    tol = gold["tolerance_abs"]
    _close(o, gold["expected"]["o"], tol, "hand example o")
    _close(fs, gold["expected"]["final_state"], tol, "hand example final state")
    # the state after the first token, from a one-token prefill
    o1, s1 = rec(inp["q"][:1], inp["k"][:1], inp["v"][:1], inp["g"][:1], inp["beta"][:1],
                 inp["initial_state"])
    _close(s1, gold["expected"]["state_after_t1"], tol, "hand example state after t=1")


# 2. closed product form with explicit transition matrices (tiny sizes), varlen + GQA
def pin_bruteforce(rec):
    for seed, lengths, Hk, Hv, Dk, Dv in [(1, [5], 1, 1, 3, 4), (2, [3, 0, 6], 2, 4, 5, 3),
                                          (3, [8, 2], 1, 2, 4, 4)]:
        c = random_case(seed, lengths, Hk, Hv, Dk, Dv)
        o, fs = rec(**c)
        ob, fb = oracle.bruteforce(**c)
        _close(o, ob, 1e-12, f"bruteforce o (seed {seed})")
        _close(fs, fb, 1e-12, f"bruteforce state (seed {seed})")


# 3. beta = 0: no erase and no write; the state only decays.
#    S_t = exp(Gamma_t) S_0 and o_t = exp(Gamma_t) S_0 q_t, Gamma_t = sum_{s<=t} g_s.
def pin_beta_zero(rec):
    c = random_case(4, [300], 2, 2, 6, 5, g_shift=0.5)
    c["beta"] = np.zeros_like(c["beta"])
    o, fs = rec(**c)
    Gam = np.cumsum(c["g"], axis=0)                       # [T, Hv]
    S0 = c["initial_state"][0]                            # [Hv, Dv, Dk]
    for h in range(2):
        exp_o = np.exp(Gam[:, h])[:, None] * (c["q"][:, h % 2] @ S0[h].T)
        _close(o[:, h], exp_o, 1e-12, "beta=0 outputs")
        _close(fs[0, h], np.exp(Gam[-1, h]) * S0[h], 1e-12, "beta=0 final state")
    assert np.all(np.exp(Gam[-1]) < 1e-100), "decay should underflow this long sequence"


# 4. orthonormal keys, zero initial state: the delta rule's erase term vanishes and the
#    recurrence is decayed linear attention,
#    o_t = sum_{s<=t} exp(Gamma_t - Gamma_s) beta_s (k_s . q_t) v_s.
def pin_orthonormal_keys(rec):
    rng = np.random.default_rng(5)
    T, D = 12, 16
    c = random_case(5, [T], 1, 1, D, 7, init=False)
    Qm, _ = np.linalg.qr(rng.standard_normal((D, D)))
    c["k"] = Qm[:, :T].T.reshape(T, 1, D).copy()         # orthonormal rows
    o, fs = rec(**c)
    Gam = np.cumsum(c["g"][:, 0])
    k, q, v, b = c["k"][:, 0], c["q"][:, 0], c["v"][:, 0], c["beta"][:, 0]
    for t in range(T):
        exp_o = sum(np.exp(Gam[t] - Gam[s]) * b[s] * (k[s] @ q[t]) * v[s] for s in range(t + 1))
        _close(o[t, 0], exp_o, 1e-12, f"orthonormal keys o[{t}]")
    exp_S = sum(np.exp(Gam[-1] - Gam[s]) * b[s] * np.outer(v[s], k[s]) for s in range(T))
    _close(fs[0, 0], exp_S, 1e-12, "orthonormal keys final state")


# 5. alpha = beta = 1 with unit keys: I - k k^T is the orthogonal projector off k, so
#    after token t:  S_t k_t = v_t,  S_t x = S_{t-1} x for x orthogonal to k_t, and a
#    query equal to the key reads back v_t.
def pin_projection(rec):
    rng = np.random.default_rng(6)
    c = random_case(6, [10], 1, 1, 8, 5)
    c["g"] = np.zeros_like(c["g"])
    c["beta"] = np.ones_like(c["beta"])
    c["q"] = c["k"].copy()
    o, _ = rec(**c)
    _close(o[:, 0], c["v"][:, 0], 1e-12, "q=k reads back v")
    prev = c["initial_state"]
    for t in range(1, 11):
        sub = {kk: (vv[:t] if kk in ("q", "k", "v", "g", "beta") else vv) for kk, vv in c.items()}
        sub["cu_seqlens"] = np.array([0, t])
        _, St = rec(**sub)
        kt = c["k"][t - 1, 0]
        _close(St[0, 0] @ kt, c["v"][t - 1, 0], 1e-12, f"S_t k_t = v_t at t={t}")
        x = rng.standard_normal(8)
        x -= (x @ kt) * kt
        _close(St[0, 0] @ x, prev[0, 0] @ x, 1e-12, f"orthogonal complement kept at t={t}")
        prev = St


# 6. the chunked reformulation equals the recurrence (~1e-11 at d=128, chunk 64 is the
#    agreement reported on "Exp 2026-07-13 -- Linear-Attention Scans on the NPU",
#    section 1), for several chunk sizes, ragged tails and strong decay.
def pin_chunked(rec, big=False):
    cases = [(7, [200], 1, 2, 32, 24, 0.0, (1, 7, 16, 64, 200)),
             (8, [70, 0, 129], 2, 2, 16, 16, 2.0, (16, 64)),
             (9, [150], 1, 1, 24, 24, 2.0, (64,)),
             # extreme decay (about -12 per token): unmasked exp(Gamma_r - Gamma_s) for r < s
             # overflows even in fp64 within one 64-token chunk
             (25, [100], 1, 1, 8, 8, 12.0, (64,))]
    if big:
        cases.append((10, [256], 1, 1, 128, 128, 0.0, (64,)))
    for seed, lengths, Hk, Hv, Dk, Dv, shift, chunk_sizes in cases:
        c = random_case(seed, lengths, Hk, Hv, Dk, Dv, g_shift=shift)
        o, fs = rec(**c)
        for cs in chunk_sizes:
            oc, fc = oracle.chunked(**c, chunk_size=cs)
            scale = max(1.0, float(np.max(np.abs(o))))
            _close(o / scale, oc / scale, 1e-11, f"chunked o (seed {seed}, C={cs})")
            _close(fs / scale, fc / scale, 1e-11, f"chunked state (seed {seed}, C={cs})")


# 7. state passing: prefill(x) == prefill(second part, init = final(prefill(first part)))
def pin_state_passing(rec, kda=False):
    c = random_case(11, [90], 2, 4, 8, 6, kda=kda)
    o, fs = rec(**c)
    cut = 37
    first = {kk: (vv[:cut] if kk in ("q", "k", "v", "g", "beta") else vv) for kk, vv in c.items()}
    first["cu_seqlens"] = np.array([0, cut])
    o1, s1 = rec(**first)
    second = {kk: (vv[cut:] if kk in ("q", "k", "v", "g", "beta") else vv) for kk, vv in c.items()}
    second["cu_seqlens"] = np.array([0, 90 - cut])
    second["initial_state"] = s1
    o2, s2 = rec(**second)
    _close(np.concatenate([o1, o2]), o, 1e-12, "state passing outputs")
    _close(s2, fs, 1e-12, "state passing final state")


# 8. prefill of T tokens == prefill of T-m tokens followed by m single-token decode steps
def pin_decode(rec, decode=None, kda=False):
    decode = decode or oracle.decode_step
    c = random_case(12, [40], 2, 4, 8, 6, kda=kda)
    o, fs = rec(**c)
    m = 5
    pre = {kk: (vv[:-m] if kk in ("q", "k", "v", "g", "beta") else vv) for kk, vv in c.items()}
    pre["cu_seqlens"] = np.array([0, 40 - m])
    _, st = rec(**pre)
    for i in range(40 - m, 40):
        od, st = decode(c["q"][i:i + 1], c["k"][i:i + 1], c["v"][i:i + 1], c["g"][i:i + 1],
                        c["beta"][i:i + 1], st)
        _close(od[0], o[i], 1e-12, f"decode step output at t={i}")
    _close(st, fs, 1e-12, "decode final state")


# 9. packed variable-length batch == each sequence run alone (zero-length included)
def pin_varlen(rec, kda=False):
    lengths = [13, 0, 29, 1, 20]
    c = random_case(13, lengths, 1, 2, 6, 5, kda=kda)
    o, fs = rec(**c)
    cu = c["cu_seqlens"]
    for n in range(len(lengths)):
        a, b = int(cu[n]), int(cu[n + 1])
        one = {kk: (vv[a:b] if kk in ("q", "k", "v", "g", "beta") else vv) for kk, vv in c.items()}
        one["cu_seqlens"] = np.array([0, b - a])
        one["initial_state"] = c["initial_state"][n:n + 1]
        on, sn = rec(**one)
        _close(o[a:b], on, 1e-12, f"varlen outputs of sequence {n}")
        _close(fs[n:n + 1], sn, 1e-12, f"varlen final state of sequence {n}")
    _close(fs[1], c["initial_state"][1], 0.0, "zero-length sequence keeps its initial state")


# 10. GQA: value head h reads key/query head h % Hk == the same run with keys/queries
#     replicated explicitly to Hv heads
def pin_gqa(rec, kda=False):
    c = random_case(14, [25], 2, 6, 5, 4, kda=kda)
    o, fs = rec(**c)
    rep = dict(c)
    idx = [h % 2 for h in range(6)]
    rep["q"] = c["q"][:, idx].copy()
    rep["k"] = c["k"][:, idx].copy()
    o2, f2 = rec(**rep)
    _close(o, o2, 1e-13, "GQA outputs")
    _close(fs, f2, 1e-13, "GQA final states")


# 11. linearity in (v, S_0) jointly, and value-channel permutation equivariance
def pin_linearity_and_permutation(rec, kda=False):
    c = random_case(15, [30], 1, 2, 6, 5, kda=kda)
    d = random_case(16, [30], 1, 2, 6, 5, kda=kda)
    oc, fc = rec(**c)
    mix = dict(c)
    mix["v"] = c["v"] - 2.5 * d["v"]
    mix["initial_state"] = c["initial_state"] - 2.5 * d["initial_state"]
    od, fd = rec(**{**c, "v": d["v"], "initial_state": d["initial_state"]})
    om, fm = rec(**mix)
    _close(om, oc - 2.5 * od, 1e-11, "linearity outputs")
    _close(fm, fc - 2.5 * fd, 1e-11, "linearity states")
    perm = np.random.default_rng(17).permutation(5)
    pc = dict(c)
    pc["v"] = c["v"][:, :, perm]
    pc["initial_state"] = c["initial_state"][:, :, perm, :]
    op, fp = rec(**pc)
    _close(op, oc[:, :, perm], 1e-13, "permuted value channels (outputs)")
    _close(fp, fc[:, :, perm, :], 1e-13, "permuted value channels (states)")


# 12. permuting the key channels (of q, k, a per-channel gate and the key index of S_0)
#     permutes the key index of the state and leaves the outputs unchanged
def pin_key_permutation(rec, kda=False):
    c = random_case(18, [40], 1, 2, 7, 5, kda=kda)
    o, fs = rec(**c)
    perm = np.random.default_rng(19).permutation(7)
    pc = dict(c)
    pc["q"], pc["k"] = c["q"][:, :, perm], c["k"][:, :, perm]
    if kda:
        pc["g"] = c["g"][:, :, perm]
    pc["initial_state"] = c["initial_state"][..., perm]
    op, fp = rec(**pc)
    _close(op, o, 1e-13, "permuted key channels (outputs)")
    _close(fp, fs[..., perm], 1e-13, "permuted key channels (states)")


ALL_PINS = [pin_hand_example, pin_bruteforce, pin_beta_zero, pin_orthonormal_keys,
            pin_projection, pin_chunked, pin_state_passing, pin_decode, pin_varlen, pin_gqa,
            pin_linearity_and_permutation, pin_key_permutation]


# --------------------------------------------------------------------------------------
# Per-key-channel gate (KDA).  The pages give this variant's gate only as one decay per
# key channel; the reading pinned here is S_t = S_{t-1} Diag(a_t) (I - b_t k_t k_t^T)
# + b_t v_t k_t^T, o_t = S_t q_t.
# --------------------------------------------------------------------------------------

# K1. hand-worked example (tests/golden/kda_hand_worked_d2_t2.json)
def pin_kda_hand_example(rec):
    pin_hand_example(rec, "kda_hand_worked_d2_t2.json")


# K2. closed product form with M_r = Diag(a_r) (I - b_r k_r k_r^T), varlen + GQA
def pin_kda_bruteforce(rec):
    for seed, lengths, Hk, Hv, Dk, Dv in [(31, [5], 1, 1, 3, 4), (32, [3, 0, 6], 2, 4, 5, 3)]:
        c = random_case(seed, lengths, Hk, Hv, Dk, Dv, kda=True)
        o, fs = rec(**c)
        ob, fb = oracle.bruteforce(**c)
        _close(o, ob, 1e-12, f"kda bruteforce o (seed {seed})")
        _close(fs, fb, 1e-12, f"kda bruteforce state (seed {seed})")


# K3. beta = 0: each key channel (column of S) decays on its own,
#     S_t = S_0 Diag(exp(Gamma_t)), o_t = S_0 (exp(Gamma_t) * q_t), Gamma_t = sum_{s<=t} g_s
def pin_kda_beta_zero(rec):
    c = random_case(33, [120], 1, 2, 6, 5, g_shift=0.5, kda=True)
    c["beta"] = np.zeros_like(c["beta"])
    o, fs = rec(**c)
    Gam = np.cumsum(c["g"], axis=0)                       # [T, Hv, Dk]
    S0 = c["initial_state"][0]
    for h in range(2):
        exp_o = (np.exp(Gam[:, h]) * c["q"][:, 0]) @ S0[h].T
        _close(o[:, h], exp_o, 1e-12, "kda beta=0 outputs")
        _close(fs[0, h], S0[h] * np.exp(Gam[-1, h])[None, :], 1e-12, "kda beta=0 final state")


# K4. one-hot keys on distinct channels, zero initial state: the erase term vanishes and
#     each token's write decays with its own channel's gate,
#     o_t = sum_{s<=t} beta_s exp(Gamma_t[j_s] - Gamma_s[j_s]) q_t[j_s] v_s
def pin_kda_onehot_keys(rec):
    T, D = 9, 12
    c = random_case(34, [T], 1, 1, D, 4, init=False, kda=True)
    ch = np.random.default_rng(35).permutation(D)[:T]
    c["k"] = np.zeros((T, 1, D))
    c["k"][np.arange(T), 0, ch] = 1.0
    o, fs = rec(**c)
    Gam = np.cumsum(c["g"][:, 0], axis=0)
    q, v, b = c["q"][:, 0], c["v"][:, 0], c["beta"][:, 0]
    for t in range(T):
        exp_o = sum(b[s] * np.exp(Gam[t, ch[s]] - Gam[s, ch[s]]) * q[t, ch[s]] * v[s]
                    for s in range(t + 1))
        _close(o[t, 0], exp_o, 1e-12, f"kda one-hot keys o[{t}]")
    exp_S = np.zeros((4, D))
    for s in range(T):
        exp_S[:, ch[s]] += b[s] * np.exp(Gam[-1, ch[s]] - Gam[s, ch[s]]) * v[s]
    _close(fs[0, 0], exp_S, 1e-12, "kda one-hot keys final state")


# K5. a gate that is the same on every key channel is the gated delta rule's scalar gate
def pin_kda_uniform_gate_is_gdn(rec):
    c = random_case(36, [50, 17], 1, 2, 8, 6)             # scalar gate [T, Hv]
    o, fs = rec(**c)
    wide = dict(c)
    wide["g"] = np.repeat(c["g"][:, :, None], 8, axis=2)
    ow, fw = rec(**wide)
    _close(ow, o, 1e-12, "uniform per-channel gate outputs")
    _close(fw, fs, 1e-12, "uniform per-channel gate states")


# K6. the chunked per-channel form equals the recurrence, for several chunk sizes, ragged
#     tails and strong decay (the pairwise per-channel decays are formed only as masked
#     differences, so |Gamma| far past exp's range inside one chunk is fine)
def pin_kda_chunked(rec, big=False):
    cases = [(37, [150], 1, 2, 16, 12, 0.0, (1, 7, 16, 64, 150)),
             (38, [70, 0, 129], 2, 2, 8, 8, 2.0, (16, 64)),
             (39, [100], 1, 1, 8, 8, 12.0, (64,))]
    if big:
        cases.append((40, [200], 1, 1, 128, 128, 0.0, (64,)))
    for seed, lengths, Hk, Hv, Dk, Dv, shift, chunk_sizes in cases:
        c = random_case(seed, lengths, Hk, Hv, Dk, Dv, g_shift=shift, kda=True)
        o, fs = rec(**c)
        for cs in chunk_sizes:
            oc, fc = oracle.chunked(**c, chunk_size=cs)
            scale = max(1.0, float(np.max(np.abs(o))))
            _close(o / scale, oc / scale, 1e-11, f"kda chunked o (seed {seed}, C={cs})")
            _close(fs / scale, fc / scale, 1e-11, f"kda chunked state (seed {seed}, C={cs})")


def pin_kda_state_passing(rec):
    pin_state_passing(rec, kda=True)


def pin_kda_decode(rec, decode=None):
    pin_decode(rec, decode=decode, kda=True)


def pin_kda_varlen(rec):
    pin_varlen(rec, kda=True)


def pin_kda_gqa(rec):
    pin_gqa(rec, kda=True)


def pin_kda_linearity_and_permutation(rec):
    pin_linearity_and_permutation(rec, kda=True)


def pin_kda_key_permutation(rec):
    pin_key_permutation(rec, kda=True)


KDA_PINS = [pin_kda_hand_example, pin_kda_bruteforce, pin_kda_beta_zero, pin_kda_onehot_keys,
            pin_kda_uniform_gate_is_gdn, pin_kda_chunked, pin_kda_state_passing, pin_kda_decode,
            pin_kda_varlen, pin_kda_gqa, pin_kda_linearity_and_permutation,
            pin_kda_key_permutation]


# --------------------------------------------------------------------------------------
# Input prologue: q/k L2 norm, beta = sigmoid, g = -softplus (the fused entry points).
# --------------------------------------------------------------------------------------

# P1. closed-form values and identities of the three maps
def pin_prologue_values(_rec=None):
    ln3 = np.log(3.0)
    _close(oracle.sigmoid(np.array([0.0, ln3, -ln3])), [0.5, 0.75, 0.25], 1e-15, "sigmoid values")
    _close(oracle.softplus(np.array([0.0, np.log(np.e - 1.0)])), [np.log(2.0), 1.0], 1e-15,
           "softplus values")
    x = np.linspace(-30.0, 30.0, 121)
    _close(oracle.softplus(x) - oracle.softplus(-x), x, 1e-12, "softplus(x) - softplus(-x) = x")
    _close(oracle.sigmoid(x) + oracle.sigmoid(-x), np.ones_like(x), 1e-15, "sigmoid symmetry")
    # far tails: softplus(x) -> x and e^x, relative to their size
    big = oracle.softplus(np.array([700.0, -700.0]))
    assert big[0] == 700.0 and abs(big[1] / np.exp(-700.0) - 1.0) < 1e-12, "softplus tails"
    rows = np.array([[3.0, 4.0, 0.0], [0.0, 0.0, 0.0], [1e-30, 0.0, 0.0]])
    _close(oracle.l2_normalize(rows), [[0.6, 0.8, 0.0], [0.0, 0.0, 0.0], [1e-18, 0.0, 0.0]], 1e-15,
           "l2 normalisation (3-4-5 row, zero row, a row below the 1e-12 floor)")
    rng = np.random.default_rng(42)
    y = rng.standard_normal((20, 3, 16))
    _close(np.linalg.norm(oracle.l2_normalize(y), axis=-1), np.ones((20, 3)), 1e-14, "unit norms")
    _close(oracle.l2_normalize(7.5 * y), oracle.l2_normalize(y), 1e-15, "scale invariance")


# P2. the prologue applied by the oracle to raw draws equals the input generator's own
#     recipe for the same draws (fp32 normalisation, fp64 sigmoid / softplus cast to fp32):
#     two independent implementations, agreeing to fp32 rounding
def pin_prologue_matches_generator(_rec=None):
    from linear_attention_chunked_gdn_amd import inputs
    for per_channel in (False, True):
        raw = inputs.make_custom(51, [40, 9], 2, 4, Dk=16, Dv=8, io="f32", g_shift=1.0,
                                 per_channel=per_channel, raw=True)
        ref = inputs.make_custom(51, [40, 9], 2, 4, Dk=16, Dv=8, io="f32", g_shift=1.0,
                                 per_channel=per_channel)
        q, k, g, b = oracle.prologue(raw.q, raw.k, raw.g, raw.beta, 7)
        _close(q, ref.q, 2e-7, "prologue q")
        _close(k, ref.k, 2e-7, "prologue k")
        _close(g, ref.g, 1e-6, "prologue g")
        _close(b, ref.beta, 1e-7, "prologue beta")
        _close(raw.v, ref.v, 0.0, "v is drawn the same")


# P3. each flag bit selects its own step and nothing else: flags = 0 is the identity, and
#     for every subset of the bits exactly the selected tensors change, to the generator's
#     recipe, while the others come back as drawn.  The bit values are the ones the C
#     header gives gdn_prologue_flags.
def pin_prologue_flag_subsets(_rec=None):
    from linear_attention_chunked_gdn_amd import inputs
    header = os.path.join(os.path.dirname(GOLDEN), os.pardir, "include", "gdn.h")
    with open(header) as f:
        bits = {n: int(b) for n, b in re.findall(r"GDN_PROLOGUE_(\w+)\s*=\s*(\d+)", f.read())}
    assert bits == {"QK_L2NORM": 1, "BETA_SIGMOID": 2, "G_SOFTPLUS": 4}, bits
    assert (oracle.PROLOGUE_QK_L2NORM, oracle.PROLOGUE_BETA_SIGMOID, oracle.PROLOGUE_G_SOFTPLUS) == \
        (bits["QK_L2NORM"], bits["BETA_SIGMOID"], bits["G_SOFTPLUS"]), "oracle flag values"
    for per_channel in (False, True):
        raw = inputs.make_custom(52, [33, 7], 2, 4, Dk=16, Dv=8, io="f32", g_shift=1.0,
                                 per_channel=per_channel, raw=True)
        ref = inputs.make_custom(52, [33, 7], 2, 4, Dk=16, Dv=8, io="f32", g_shift=1.0,
                                 per_channel=per_channel)
        # every step changes its tensors by far more than the tolerances below
        for a, b in ((raw.q, ref.q), (raw.k, ref.k), (raw.g, ref.g), (raw.beta, ref.beta)):
            assert np.min(np.abs(np.asarray(a, np.float64) - b)) > 1e-3 or np.max(np.abs(a - b)) > 0.1
        for flags in range(8):
            q, k, g, b = oracle.prologue(raw.q, raw.k, raw.g, raw.beta, flags)
            norm = bool(flags & bits["QK_L2NORM"])
            sig = bool(flags & bits["BETA_SIGMOID"])
            sp = bool(flags & bits["G_SOFTPLUS"])
            _close(q, ref.q if norm else raw.q, 2e-7 if norm else 0.0, f"flags={flags}: q")
            _close(k, ref.k if norm else raw.k, 2e-7 if norm else 0.0, f"flags={flags}: k")
            _close(b, ref.beta if sig else raw.beta, 1e-7 if sig else 0.0, f"flags={flags}: beta")
            _close(g, ref.g if sp else raw.g, 1e-6 if sp else 0.0, f"flags={flags}: g")


PROLOGUE_PINS = [pin_prologue_values, pin_prologue_matches_generator, pin_prologue_flag_subsets]
