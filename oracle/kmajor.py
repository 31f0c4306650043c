"""Independent K-major numpy transcription of the gated delta rule (tiny inputs).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Written from the ONNX issue "Spec gap: LinearAttention (opset 27) cannot
represent Gated DeltaNet-2's channel-wise erase gate":
  * section "What LinearAttention currently does (gated_delta)" states the step
    on a K-major state M (dk x dv): decay M by exp(g), replace v by
    beta (v - M^T k), add the outer product k v^T; the decay may be one scalar
    per head or one value per key dimension (a diagonal acting on M's rows);
  * section "The GDN-2 recurrence" writes the Gated DeltaNet-2 step as
    M_t = (I - k_t (b_t o k_t)^T) D_t M_{t-1} + k_t v_t^T with D_t the
    diagonal of per-key decays and the erase gate b_t on the key axis;
plus the readout o = scale M^T q of the "com.microsoft.GatedDeltaNet" README.
It keeps its own loop structure (one matrix per head, whole-matrix numpy
operations) and shares nothing with ``gdr_oracle.c`` beyond the definition.
Uniform packing, f64 only.
"""
from __future__ import annotations

import numpy as np


def forward_kmajor(q, k, v, g, beta, initial_state_kmajor=None, scale=None, erase=None):
    """q, k: (B,L,H,dk); v: (B,L,HV,dv); g: log decays (B,L,HV) per head or
    (B,L,HV,dk) per key dimension; beta: (B,L,HV) update rates (already
    activated), or None with ``erase``.  erase: (B,L,HV,dk) key-axis erase gate
    of Gated DeltaNet-2 (then the write is the ungated k v^T).

    initial_state_kmajor: (B,HV,dk,dv).  Returns o (B,L,HV,dv) and the K-major
    final state (B,HV,dk,dv)."""
    Bn, L, H, dk = q.shape
    HV, dv = v.shape[2:]
    group = HV // H
    if scale is None:
        scale = dk ** -0.5
    per_key = np.ndim(g) == 4
    o = np.zeros((Bn, L, HV, dv))
    out_state = np.zeros((Bn, HV, dk, dv))
    for b in range(Bn):
        for hv in range(HV):
            h = hv // group
            M = np.zeros((dk, dv)) if initial_state_kmajor is None else \
                np.array(initial_state_kmajor[b, hv], dtype=np.float64)
            for t in range(L):
                kt, qt, vt = k[b, t, h], q[b, t, h], v[b, t, hv]
                D = np.diag(np.exp(g[b, t, hv])) if per_key else np.exp(g[b, t, hv]) * np.eye(dk)
                M = D @ M
                if erase is None:
                    vt = beta[b, t, hv] * (vt - M.T @ kt)
                    M = M + np.outer(kt, vt)
                else:
                    E = np.eye(dk) - np.outer(kt, erase[b, t, hv] * kt)
                    M = E @ M + np.outer(kt, vt)
                o[b, t, hv] = scale * (M.T @ qt)
            out_state[b, hv] = M
    return o, out_state
