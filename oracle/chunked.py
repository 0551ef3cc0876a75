"""Second float64 formulation of the KDA recurrence: the chunked WY/UT form.

Test infrastructure only (imported by ``tests/`` alone). It exists to pin the sequential
oracle in ``oracle/kda.py``: both are written from the rule

    S_t = Diag(a_t) S_{t-1} - b_t k_t k_t^T Diag(a_t) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t

but this one evaluates it a chunk of C tokens at a time, the way the pages' prefill does
("vLLM lifts Kimi K3 throughput by up to 2.8x", section "KDA checkpoints stay inside the
prefill": the prefill walks the prompt and exports state at block boundaries).

Derivation, for one chunk of n tokens (rows r, s = 1..n) entered with state S0. Write the
step as S_r = Diag(a_r) S_{r-1} + k_r w_r^T with the innovation
w_r = b_r (v_r - (Diag(a_r) S_{r-1})^T k_r). With g_r = sum_{s<=r} log a_s (per key channel),
unrolling gives S_r = Diag(e^{g_r}) S0 + sum_{s<=r} Diag(e^{g_r - g_s}) k_s w_s^T, hence

    A_kk[r,s] = sum_i k_ri k_si e^{g_ri - g_si}      (s <  r)
    A_qk[r,s] = sum_i q_ri k_si e^{g_ri - g_si}      (s <= r)
    (I + Diag(b) A_kk) W = Diag(b) (V - Kt S0),       Kt_r = k_r * e^{g_r}
    O   = Qt S0 + A_qk W,                            Qt_r = q_r * e^{g_r}
    S_n = Diag(e^{g_n}) S0 + Kb^T W,                 Kb_s = k_s * e^{g_n - g_s}

The triangular system is handed to ``numpy.linalg.solve``.
"""
from __future__ import annotations

import numpy as np


def kda_chunk(S0, q, k, v, a, b):
    """One chunk for one head. q, k, a [n, dk]; v [n, dv]; b [n]; S0 [dk, dv].
    Returns (S_n, O [n, dv])."""
    n = q.shape[0]
    g = np.cumsum(np.log(a), axis=0)                        # [n, dk]
    diff = g[:, None, :] - g[None, :, :]                   # g_r - g_s, [n, n, dk]
    lower_strict = np.tril(np.ones((n, n)), -1)
    lower = np.tril(np.ones((n, n)))
    with np.errstate(over="ignore"):
        decay = np.where(lower[:, :, None] > 0, np.exp(np.minimum(diff, 0.0)), 0.0)
    A_kk = np.einsum("ri,si,rsi->rs", k, k, decay) * lower_strict
    A_qk = np.einsum("ri,si,rsi->rs", q, k, decay) * lower
    Kt = k * np.exp(g)
    Qt = q * np.exp(g)
    Kb = k * np.exp(g[-1][None, :] - g)
    W = np.linalg.solve(np.eye(n) + b[:, None] * A_kk, b[:, None] * (v - Kt @ S0))
    O = Qt @ S0 + A_qk @ W
    S = np.exp(g[-1])[:, None] * S0 + Kb.T @ W
    return S, O


def kda_chunked(S0, q, k, v, a, b, C: int, snapshot_every: int = 0):
    """Whole sequence for one head, C tokens per chunk (the last chunk may be shorter).
    Returns (S_T, O [T, dv], snapshots every ``snapshot_every`` tokens, which must be a
    multiple of C)."""
    if snapshot_every and snapshot_every % C:
        raise ValueError("snapshot interval must be a multiple of the chunk")
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    O = np.zeros((T, S.shape[-1]))
    snaps = []
    for lo in range(0, T, C):
        hi = min(lo + C, T)
        S, O[lo:hi] = kda_chunk(S, q[lo:hi], k[lo:hi], v[lo:hi], a[lo:hi], b[lo:hi])
        if snapshot_every and hi % snapshot_every == 0:
            snaps.append(S.copy())
    return S, O, snaps
