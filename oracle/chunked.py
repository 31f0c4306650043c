"""Chunk-parallel form of the gated delta rule, fp64 numpy (tiny inputs only).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The "com.microsoft.GatedDeltaNet" README (Attributes, chunk_size) names a
chunk-parallel prefill algorithm whose chunk size never changes the result,
and (Inputs, key) a per-chunk linear system that needs unit keys.  The pages
do not print it; this is the form obtained by unrolling the README's
recurrence over one chunk.  In K-major notation (state M = S^T, dk x dv):

  within a chunk starting from state M0, with gamma_t = prod_{r<=t} alpha_r,
    M_t     = gamma_t M0 + sum_{s<=t} (gamma_t/gamma_s) k_s d_s^T
    d_t     = beta_t (v_t - gamma_t M0^T k_t - sum_{s<t} (gamma_t/gamma_s)(k_t.k_s) d_s)
  so, stacking d_t as the rows of D (C x dv):
    (I + A) D = diag(beta) (V - diag(gamma) K M0),   A_ts = beta_t (gamma_t/gamma_s) k_t.k_s  (s < t)
    D = U - W M0  with  W = (I+A)^-1 diag(beta gamma) K,  U = (I+A)^-1 diag(beta) V
    O = scale (diag(gamma) Q M0 + (Q K^T o Mask) D),  Mask_ts = gamma_t/gamma_s (s <= t)
    M_C = gamma_C M0 + (diag(gamma_C / gamma) K)^T D
Rules without retrieval (linear, gated) have D = V.  Every ratio of
cumulative decays is formed as exp(G_t - G_s) with s <= t, so no term
overflows.  The solve uses numpy's dense solver as a library step.
"""
from __future__ import annotations

import numpy as np

from . import RULES


def _softplus(x):
    return np.logaddexp(0.0, x)


def forward_chunked(q, k, v, *, gate=None, beta=None, a_log=None, dt_bias=None,
                    cu_seqlens=None, initial_state=None, update_rule="gated_delta",
                    gate_activation="none", beta_activation="none", qk_l2_norm=False,
                    scale=0.0, chunk_size=64, batch=None):
    """Rank-3 inputs (T,H,dk)/(T,HV,dv), scalar per-head decay.  Returns (o, state)
    with state V-major (B,HV,dv,dk), like ``oracle.forward``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, H, DK = q.shape
    HV, DV = v.shape[1:]
    rule = RULES[update_rule]
    if rule == RULES["gated_delta_v2"]:
        raise ValueError("the chunked form covers scalar-gate rules only")
    decayed = rule in (RULES["gated"], RULES["gated_delta"])
    retrieves = rule in (RULES["delta"], RULES["gated_delta"])
    if scale == 0.0:
        scale = 1.0 / np.sqrt(DK)
    if qk_l2_norm:
        q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + 1e-12)
        k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + 1e-12)
    g = np.zeros((T, HV))
    if decayed:
        g = np.asarray(gate, dtype=np.float64).reshape(T, HV)
        if gate_activation == "qwen":
            g = -np.exp(np.asarray(a_log, np.float64))[None, :] * _softplus(
                g + np.asarray(dt_bias, np.float64)[None, :])
    b = np.ones((T, HV))
    if retrieves:
        b = np.asarray(beta, dtype=np.float64).reshape(T, HV)
        if beta_activation == "sigmoid":
            b = 1.0 / (1.0 + np.exp(-b))

    if cu_seqlens is not None:
        cu = np.clip(np.asarray(cu_seqlens, dtype=np.int64), 0, T)
        B = len(cu) - 1
        ranges = [(int(cu[i]), int(max(cu[i], cu[i + 1]))) for i in range(B)]
    else:
        B = int(batch if batch is not None else
                (np.asarray(initial_state).shape[0] if initial_state is not None else 1))
        L = T // B
        ranges = [(i * L, (i + 1) * L) for i in range(B)]

    o = np.zeros((T, HV, DV))
    state = np.zeros((B, HV, DV, DK))
    for bi, (s, e) in enumerate(ranges):
        for h in range(HV):
            qh = h * H // HV
            M = np.zeros((DK, DV)) if initial_state is None else \
                np.asarray(initial_state, dtype=np.float64)[bi, h].T.copy()
            for c0 in range(s, e, chunk_size):
                c1 = min(c0 + chunk_size, e)
                Q, K, V = q[c0:c1, qh], k[c0:c1, qh], v[c0:c1, h]
                G = np.cumsum(g[c0:c1, h])            # log gamma_t
                bt = b[c0:c1, h]
                n = c1 - c0
                diff = G[:, None] - G[None, :]        # G_t - G_s
                lower = np.tril(np.ones((n, n), dtype=bool))
                ratio = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
                if retrieves:
                    strict = np.tril(np.ones((n, n), dtype=bool), -1)
                    A = np.where(strict, bt[:, None] * ratio * (K @ K.T), 0.0)
                    IA = np.eye(n) + A
                    W = np.linalg.solve(IA, (bt * np.exp(G))[:, None] * K)
                    U = np.linalg.solve(IA, bt[:, None] * V)
                    D = U - W @ M
                else:
                    D = V.copy()
                o[c0:c1, h] = scale * (np.exp(G)[:, None] * (Q @ M) + ((Q @ K.T) * ratio) @ D)
                M = np.exp(G[-1]) * M + (np.exp(G[-1] - G)[:, None] * K).T @ D
            state[bi, h] = M.T
    return o, state
