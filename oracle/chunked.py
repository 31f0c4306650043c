"""Chunk-parallel form of the gated delta rule, fp64 numpy (tiny inputs only).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The "com.microsoft.GatedDeltaNet" README (Attributes, chunk_size) names a
chunk-parallel prefill algorithm whose chunk size never changes the result,
and (Inputs, key) a per-chunk linear system that needs unit keys.  The pages
do not print it; this is the form obtained by unrolling the recurrence over
one chunk.  K-major notation (state M = S^T, dk x dv), decay per key channel
(a per-head decay is the same vector in every channel):

  one token:  M_t = Diag(alpha_t) M_{t-1} + k_t d_t^T,
              d_t = w_t v_t - (Diag(alpha_t) M_{t-1})^T l_t
  with (w_t, l_t) = (beta_t, beta_t k_t) for the delta rules (README,
  Description), (1, b_t o k_t) for the Gated DeltaNet-2 erase gate (ONNX issue
  "Spec gap ... Gated DeltaNet-2", "The GDN-2 recurrence": the erase gate acts
  on the key axis inside the second k_t), and (1, 0) for the rules without
  retrieval (linear, gated).  The per-key decay is the Ascend
  "aclnnRecurrentGatedDeltaRule" Formula's Diag(alpha).

  within a chunk starting from M0, with G_t = sum_{r<=t} log alpha_r (a dk
  vector) and E_ts = exp(G_t - G_s) (elementwise, s <= t):
    M_t = Diag(e^{G_t}) M0 + sum_{s<=t} Diag(E_ts) k_s d_s^T
    d_t = w_t v_t - M0^T (e^{G_t} o l_t) - sum_{s<t} (l_t . (E_ts o k_s)) d_s
  so, stacking d_t as the rows of D (C x dv):
    (I + A) D = diag(w) V - (L o e^G) M0,   A_ts = l_t . (E_ts o k_s)  (s < t)
    D = U - W M0  with  W = (I+A)^-1 (L o e^G),  U = (I+A)^-1 diag(w) V
    O = scale ((Q o e^G) M0 + P D),          P_ts = q_t . (E_ts o k_s)  (s <= t)
    M_C = Diag(e^{G_C}) M0 + (K o e^{G_C - G})^T D
Every exponential is of G_t - G_s with s <= t (or of G_t itself), so no term
overflows.  The solve uses numpy's dense solver as a library step.
"""
from __future__ import annotations

import numpy as np

from . import RULES


def _softplus(x):
    return np.logaddexp(0.0, x)


def forward_chunked(q, k, v, *, gate=None, beta=None, erase=None, a_log=None, dt_bias=None,
                    cu_seqlens=None, initial_state=None, update_rule="gated_delta",
                    gate_activation="none", beta_activation="none", qk_l2_norm=False,
                    scale=0.0, chunk_size=64, batch=None, gate_scale=None):
    """Rank-3 inputs (T,H,dk)/(T,HV,dv); gate (T,HV) per head or (T,HV,dk) per
    key; erase (T,HV,dk) for gated_delta_v2.  Returns (o, state) with state
    V-major (B,HV,dv,dk), like ``oracle.forward``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, H, DK = q.shape
    HV, DV = v.shape[1:]
    rule = RULES[update_rule]
    v2 = rule == RULES["gated_delta_v2"]
    decayed = rule in (RULES["gated"], RULES["gated_delta"], RULES["gated_delta_v2"])
    has_beta = rule in (RULES["delta"], RULES["gated_delta"])
    if scale == 0.0:
        scale = 1.0 / np.sqrt(DK)
    if qk_l2_norm:
        q = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + 1e-12)
        k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + 1e-12)
    # log decay per (token, head, key channel)
    g = np.zeros((T, HV, DK))
    if decayed:
        gg = np.asarray(gate, dtype=np.float64)
        per_key = gg.size == T * HV * DK and gg.size != T * HV
        gg = gg.reshape(T, HV, DK) if per_key else gg.reshape(T, HV)
        if gate_activation == "qwen":
            # gate_scale is the once-folded -exp(a_log); the bias is (HV, dk)
            # beside a per-key gate (CLIKA "gatedDeltaUpdate")
            gs = (np.asarray(gate_scale, np.float64) if gate_scale is not None
                  else -np.exp(np.asarray(a_log, np.float64)))
            db = np.asarray(dt_bias, np.float64)
            if per_key:
                gg = gs[None, :, None] * _softplus(gg + db.reshape(HV, DK)[None, :, :])
            else:
                gg = gs[None, :] * _softplus(gg + db[None, :])
        g = gg if per_key else np.repeat(gg[:, :, None], DK, axis=2)
    b = np.ones((T, HV))
    if has_beta:
        b = np.asarray(beta, dtype=np.float64).reshape(T, HV)
        if beta_activation == "sigmoid":
            b = 1.0 / (1.0 + np.exp(-b))
    er = np.asarray(erase, dtype=np.float64).reshape(T, HV, DK) if v2 else None

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
                n = c1 - c0
                Q, K, V = q[c0:c1, qh], k[c0:c1, qh], v[c0:c1, h]
                G = np.cumsum(g[c0:c1, h], axis=0)           # (n, dk) log decay products
                # weights and retrieval keys of the chunk's tokens
                if v2:
                    w, Lk = np.ones(n), er[c0:c1, h] * K
                elif has_beta:
                    w, Lk = b[c0:c1, h], b[c0:c1, h][:, None] * K
                else:
                    w, Lk = np.ones(n), np.zeros_like(K)
                lower = np.tril(np.ones((n, n), dtype=bool))
                diff = G[:, None, :] - G[None, :, :]         # G_t - G_s, (t, s, key)
                E = np.where(lower[:, :, None], np.exp(np.where(lower[:, :, None], diff, 0.0)), 0.0)
                A = np.tril(np.einsum("tj,sj,tsj->ts", Lk, K, E), -1)
                P = np.einsum("tj,sj,tsj->ts", Q, K, E)      # zero above the diagonal
                IA = np.eye(n) + A
                W = np.linalg.solve(IA, Lk * np.exp(G))
                U = np.linalg.solve(IA, w[:, None] * V)
                D = U - W @ M
                o[c0:c1, h] = scale * ((Q * np.exp(G)) @ M + P @ D)
                M = np.exp(G[-1])[:, None] * M + (K * np.exp(G[-1][None, :] - G)).T @ D
            state[bi, h] = M.T
    return o, state
