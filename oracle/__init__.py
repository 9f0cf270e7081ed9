"""CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may import
this package.  It shares no code with the HIP library.

Three independent fp64 evaluations of the same function are provided:

* ``recurrent``  -- the definition, token by token (C, ``gdn_oracle.c``).  This is
  the oracle the GPU is compared against.
* ``chunked``    -- the chunkwise Map-Reduce-Map form (numpy), used only to pin the
  algebra of the chunked hot path against the definition.
* ``bruteforce`` -- the closed product form of the recurrence with explicit
  Dk x Dk transition matrices (numpy), for tiny sizes only.

Every function also takes a per-key-channel gate g of shape [T, Hv, Dk] (the KDA
variant: the head's scalar decay alpha_t becomes Diag(a_t) on the key index of S,
applied before the erase) and then evaluates that rule; a gate of shape [T, Hv] is
the gated delta rule.

Sources: "Empowering Hybrid Attention Models on NPUs" (section 2.1 for the
recurrence and the Map-Reduce-Map operators #1-#6, section 5 for the chunk-first
order "5-read, 6, 5-update" and the rewrite that factors the inverse out of the
W product), and "Exp 2026-07-13 -- Linear-Attention Scans on the NPU" (section 1:
chunk size 64, the (I+A)^-1 UT transform by forward substitution; section 4: GQA
head replication hv % Hk).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build(out_path: str = _LIB_PATH, src_path: str = _SRC, extra_flags=()) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP).  Returns the library path."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", *extra_flags,
           "-o", out_path, src_path, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.gdn_oracle_prefill_f64.argtypes = [dp, dp, dp, dp, dp, dp, lp, i64, i64, i64, i64,
                                           i64, i64, dp, dp, ctypes.c_int]
    lib.gdn_oracle_prefill_f64.restype = ctypes.c_int
    lib.gdn_oracle_decode_step_f64.argtypes = [dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, i64,
                                               dp, ctypes.c_int]
    lib.gdn_oracle_decode_step_f64.restype = ctypes.c_int
    lib.gdn_oracle_kda_prefill_f64.argtypes = lib.gdn_oracle_prefill_f64.argtypes
    lib.gdn_oracle_kda_prefill_f64.restype = ctypes.c_int
    lib.gdn_oracle_kda_decode_step_f64.argtypes = lib.gdn_oracle_decode_step_f64.argtypes
    lib.gdn_oracle_kda_decode_step_f64.restype = ctypes.c_int
    lib.gdn_oracle_max_threads.argtypes = []
    lib.gdn_oracle_max_threads.restype = ctypes.c_int
    return lib


def load_library(path: Optional[str] = None):
    """Load (building first if needed) the compiled C oracle."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if (not os.path.exists(_LIB_PATH)
                or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray], ctype=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _cu(cu_seqlens, T: int) -> np.ndarray:
    if cu_seqlens is None:
        return np.array([0, T], dtype=np.int64)
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))


def _per_channel(g, rows: int, Hv: int, Dk: int) -> bool:
    """True for a per-key-channel gate [rows, Hv, Dk], False for a per-head gate [rows, Hv]."""
    if g.shape == (rows, Hv):
        return False
    if g.shape == (rows, Hv, Dk):
        return True
    raise ValueError(f"gate shape {g.shape} is neither {(rows, Hv)} nor {(rows, Hv, Dk)}")


def recurrent(q, k, v, g, beta, initial_state=None, cu_seqlens=None, nthreads: int = 0,
              lib=None):
    """Token-by-token gated delta rule in fp64 (the definition).

    q, k: [T, Hk, Dk]; v: [T, Hv, Dv]; g: [T, Hv] (or [T, Hv, Dk] per key channel);
    beta: [T, Hv]; initial_state: [N, Hv, Dv, Dk] or None; cu_seqlens: [N+1] or None
    (one sequence).  Returns (o [T, Hv, Dv], final_state [N, Hv, Dv, Dk]) as fp64 arrays.
    """
    lib = lib if lib is not None else load_library()
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    cu = _cu(cu_seqlens, T)
    N = cu.shape[0] - 1
    s0 = None if initial_state is None else _f64(initial_state)
    if s0 is not None and s0.shape != (N, Hv, Dv, Dk):
        raise ValueError(f"initial_state shape {s0.shape} != {(N, Hv, Dv, Dk)}")
    fn = (lib.gdn_oracle_kda_prefill_f64 if _per_channel(g, T, Hv, Dk)
          else lib.gdn_oracle_prefill_f64)
    o = np.zeros((T, Hv, Dv), dtype=np.float64)
    fs = np.zeros((N, Hv, Dv, Dk), dtype=np.float64)
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
            _ptr(cu, ctypes.c_int64), N, T, Hk, Hv, Dk, Dv, _ptr(o), _ptr(fs), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle prefill returned {rc}")
    return o, fs


def decode_step(q, k, v, g, beta, state, nthreads: int = 0, lib=None):
    """One decode token per sequence.  q, k: [B, Hk, Dk]; v: [B, Hv, Dv]; g: [B, Hv] (or
    [B, Hv, Dk] per key channel); beta: [B, Hv]; state: [B, Hv, Dv, Dk].  Returns
    (o [B, Hv, Dv], new_state); the input is not modified."""
    lib = lib if lib is not None else load_library()
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    B, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    fn = (lib.gdn_oracle_kda_decode_step_f64 if _per_channel(g, B, Hv, Dk)
          else lib.gdn_oracle_decode_step_f64)
    o = np.zeros((B, Hv, Dv), dtype=np.float64)
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(st), B, Hk, Hv, Dk, Dv,
            _ptr(o), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle decode step returned {rc}")
    return o, st


def max_threads(lib=None) -> int:
    lib = lib if lib is not None else load_library()
    return int(lib.gdn_oracle_max_threads())


# --------------------------------------------------------------------------------------
# Input prologue (numpy, fp64): the steps that turn a linear-attention layer's projection
# outputs into the recurrence's inputs -- q, k scaled to unit L2 norm per (token, head),
# beta = sigmoid(x), g = -softplus(x) -- which the fused entry points apply while
# loading.  Flags as in include/gdn.h: 1 = q/k L2 norm, 2 = beta sigmoid, 4 = g softplus.
# Plain definitions: x / max(||x||_2, 1e-12); 1 / (1 + e^-x); softplus(x) = log(1 + e^x),
# evaluated as max(x, 0) + log1p(e^-|x|) so that it cannot overflow.
# --------------------------------------------------------------------------------------

PROLOGUE_QK_L2NORM = 1
PROLOGUE_BETA_SIGMOID = 2
PROLOGUE_G_SOFTPLUS = 4


def l2_normalize(x) -> np.ndarray:
    x = _f64(x)
    norm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(norm, 1e-12)


def sigmoid(x) -> np.ndarray:
    x = _f64(x)
    return 1.0 / (1.0 + np.exp(-x))


def softplus(x) -> np.ndarray:
    x = _f64(x)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def prologue(q, k, g, beta, flags: int):
    """(q, k, g, beta) after the prologue steps selected by flags (fp64)."""
    q, k, g, beta = map(_f64, (q, k, g, beta))
    if flags & PROLOGUE_QK_L2NORM:
        q, k = l2_normalize(q), l2_normalize(k)
    if flags & PROLOGUE_BETA_SIGMOID:
        beta = sigmoid(beta)
    if flags & PROLOGUE_G_SOFTPLUS:
        g = -softplus(g)
    return q, k, g, beta


# --------------------------------------------------------------------------------------
# Chunkwise form (numpy, fp64): the Map-Reduce-Map pipeline, used to pin the algebra the
# GPU kernels rely on.  Notation per chunk of n_c tokens, state S (Dv x Dk):
#   Gamma = cumsum(g)  (op #1, Gate);  gamma = exp(Gamma)
#   D[r, s] = exp(Gamma_r - Gamma_s) for r >= s, formed only where r >= s
#   A = strictly-lower( diag(beta) K K^T  (elementwise)  D )          (op #2, KKT)
#   T = (I + A)^-1 by forward substitution                            (op #3, Solve)
#   W = T diag(beta * gamma) K,  U = T diag(beta) V                   (op #4, W/U)
#   v_c = U - W S^T                                                   (op #5-read)
#   O   = diag(gamma) Q S^T + (lower-incl-diagonal(Q K^T) (.) D) v_c  (op #6, O)
#   S  <- gamma_last S + v_c^T diag(lambda) K, lambda_r = exp(Gamma_last - Gamma_r)
#                                                                     (op #5-update)
# The chunk-first order 5-read -> 6 -> 5-update lets op #6 read the chunk's incoming
# state before it is overwritten ("Empowering Hybrid Attention Models on NPUs",
# section 5, Figure 10).
# --------------------------------------------------------------------------------------

def forward_substitution_inverse(A: np.ndarray) -> np.ndarray:
    """(I + A)^-1 for strictly lower-triangular A, one row at a time:
    row r of X solves X[r] = e_r - sum_{s<r} A[r, s] X[s]."""
    n = A.shape[0]
    X = np.zeros((n, n), dtype=np.float64)
    for r in range(n):
        X[r] = -A[r, :r] @ X[:r]
        X[r, r] += 1.0
    return X


def _chunk_step(S, Qc, Kc, Vc, gc, bc):
    """One chunk of the Map-Reduce-Map pipeline.  Returns (O_c, S_next)."""
    n_c = gc.shape[0]
    Gam = np.cumsum(gc)                                   # op #1
    gamma = np.exp(Gam)
    r_idx, s_idx = np.tril_indices(n_c)                   # r >= s
    D = np.zeros((n_c, n_c), dtype=np.float64)
    D[r_idx, s_idx] = np.exp(Gam[r_idx] - Gam[s_idx])     # masked before the exponential
    A = np.tril(bc[:, None] * (Kc @ Kc.T) * D, k=-1)      # op #2
    T = forward_substitution_inverse(A)                   # op #3
    W = T @ ((bc * gamma)[:, None] * Kc)                  # op #4
    U = T @ (bc[:, None] * Vc)
    v_c = U - W @ S.T                                     # op #5-read
    O = gamma[:, None] * (Qc @ S.T) + (np.tril(Qc @ Kc.T) * D) @ v_c   # op #6
    lam = np.exp(Gam[-1] - Gam)
    S_next = gamma[-1] * S + v_c.T @ (lam[:, None] * Kc)  # op #5-update
    return O, S_next


# Per-key-channel gate (KDA).  Gamma = cumsum(g) is now [n_c, Dk] and every decay is a
# vector over key channels, formed only as differences Gamma_r - Gamma_s with r >= s:
#   A[r, s] = beta_r sum_j K[r, j] K[s, j] exp(Gamma[r, j] - Gamma[s, j])      (r > s)
#   P[r, s] = sum_j Q[r, j] K[s, j] exp(Gamma[r, j] - Gamma[s, j])             (r >= s)
#   W = T diag(beta) (K (.) exp(Gamma)),  U = T diag(beta) V,  v_c = U - W S^T
#   O = (Q (.) exp(Gamma)) S^T + P v_c
#   S <- S Diag(exp(Gamma_last)) + v_c^T (K (.) exp(Gamma_last - Gamma))
# With every channel's gate equal this is the chunk step above.

def _chunk_step_kda(S, Qc, Kc, Vc, Gc, bc):
    """One chunk with a per-key-channel gate Gc [n_c, Dk].  Returns (O_c, S_next)."""
    n_c = Gc.shape[0]
    Gam = np.cumsum(Gc, axis=0)                           # op #1, per channel
    r_idx, s_idx = np.tril_indices(n_c)                   # r >= s
    Dpair = np.exp(Gam[r_idx] - Gam[s_idx])               # [pairs, Dk], masked before exp
    P = np.zeros((n_c, n_c), dtype=np.float64)
    P[r_idx, s_idx] = np.einsum("pj,pj,pj->p", Qc[r_idx], Kc[s_idx], Dpair)
    KK = np.zeros((n_c, n_c), dtype=np.float64)
    KK[r_idx, s_idx] = np.einsum("pj,pj,pj->p", Kc[r_idx], Kc[s_idx], Dpair)
    A = np.tril(bc[:, None] * KK, k=-1)                   # op #2
    T = forward_substitution_inverse(A)                   # op #3
    gam = np.exp(Gam)                                     # [n_c, Dk]
    W = T @ (bc[:, None] * (Kc * gam))                    # op #4
    U = T @ (bc[:, None] * Vc)
    v_c = U - W @ S.T                                     # op #5-read
    O = (Qc * gam) @ S.T + P @ v_c                        # op #6
    lam = np.exp(Gam[-1][None, :] - Gam)                  # [n_c, Dk]
    S_next = S * gam[-1][None, :] + v_c.T @ (lam * Kc)    # op #5-update
    return O, S_next


def chunked(q, k, v, g, beta, initial_state=None, cu_seqlens=None, chunk_size: int = 64):
    """Chunkwise fp64 evaluation; chunks restart at every sequence start and the last
    chunk of a sequence may be short.  Same arguments and results as ``recurrent``."""
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    step = _chunk_step_kda if _per_channel(g, T, Hv, Dk) else _chunk_step
    cu = _cu(cu_seqlens, T)
    N = cu.shape[0] - 1
    o = np.zeros((T, Hv, Dv), dtype=np.float64)
    fs = np.zeros((N, Hv, Dv, Dk), dtype=np.float64)
    for n in range(N):
        for h in range(Hv):
            hk = h % Hk
            S = (np.zeros((Dv, Dk)) if initial_state is None
                 else np.array(initial_state[n, h], dtype=np.float64))
            for c0 in range(int(cu[n]), int(cu[n + 1]), chunk_size):
                c1 = min(c0 + chunk_size, int(cu[n + 1]))
                O, S = step(S, q[c0:c1, hk], k[c0:c1, hk], v[c0:c1, h],
                            g[c0:c1, h], beta[c0:c1, h])
                o[c0:c1, h] = O
            fs[n, h] = S
    return o, fs


# --------------------------------------------------------------------------------------
# Closed product form (numpy, fp64), tiny sizes only.  With M_r = alpha_r (I - beta_r k_r k_r^T)
# (per key channel: M_r = Diag(a_r) (I - beta_r k_r k_r^T)):
#   S_t = S_0 M_1 M_2 ... M_t + sum_{s<=t} beta_s v_s k_s^T M_{s+1} ... M_t,   o_t = S_t q_t.
# Each S_t is rebuilt from scratch from explicit Dk x Dk products, so nothing is carried
# from one token to the next.
# --------------------------------------------------------------------------------------

def bruteforce(q, k, v, g, beta, initial_state=None, cu_seqlens=None):
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    per_channel = _per_channel(g, T, Hv, Dk)
    cu = _cu(cu_seqlens, T)
    N = cu.shape[0] - 1
    o = np.zeros((T, Hv, Dv), dtype=np.float64)
    fs = np.zeros((N, Hv, Dv, Dk), dtype=np.float64)
    I = np.eye(Dk)
    for n in range(N):
        start, end = int(cu[n]), int(cu[n + 1])
        for h in range(Hv):
            hk = h % Hk
            S0 = (np.zeros((Dv, Dk)) if initial_state is None
                  else np.array(initial_state[n, h], dtype=np.float64))
            decay = ((lambda r: np.diag(np.exp(g[r, h]))) if per_channel
                     else (lambda r: np.exp(g[r, h]) * I))
            M = [decay(r) @ (I - beta[r, h] * np.outer(k[r, hk], k[r, hk]))
                 for r in range(start, end)]

            def prod(a, b):  # M_a ... M_b (1-based within the sequence), identity if empty
                P = np.eye(Dk)
                for r in range(a, b + 1):
                    P = P @ M[r - 1]
                return P

            St = S0.copy()
            for t in range(1, end - start + 1):
                St = S0 @ prod(1, t)
                for s in range(1, t + 1):
                    ts = start + s - 1
                    St = St + beta[ts, h] * np.outer(v[ts, h], k[ts, hk]) @ prod(s + 1, t)
                o[start + t - 1, h] = St @ q[start + t - 1, hk]
            fs[n, h] = St
    return o, fs
