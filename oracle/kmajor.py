"""Independent K-major numpy transcription of the gated delta rule (tiny inputs).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Written from the ONNX issue "Spec gap: LinearAttention (opset 27) cannot
represent Gated DeltaNet-2's channel-wise erase gate", section "What
LinearAttention currently does (gated_delta)", which states the step on a
K-major state (dk x dv): decay the state by exp(g), replace v by
beta (v - state^T k), add the outer product k v^T; plus the readout
o = scale state^T q of the "com.microsoft.GatedDeltaNet" README.  It keeps its
own loop structure (one matrix per head, whole-matrix numpy operations) and
shares nothing with ``gdr_oracle.c`` beyond the definition.  Scalar decay,
uniform packing, f64 only.
"""
from __future__ import annotations

import numpy as np


def forward_kmajor(q, k, v, g, beta, initial_state_kmajor=None, scale=None):
    """q, k: (B,L,H,dk); v: (B,L,HV,dv); g, beta: (B,L,HV) (already activated).

    initial_state_kmajor: (B,HV,dk,dv).  Returns o (B,L,HV,dv) and the K-major
    final state (B,HV,dk,dv)."""
    Bn, L, H, dk = q.shape
    HV, dv = v.shape[2:]
    group = HV // H
    if scale is None:
        scale = dk ** -0.5
    o = np.zeros((Bn, L, HV, dv))
    out_state = np.zeros((Bn, HV, dk, dv))
    for b in range(Bn):
        for hv in range(HV):
            h = hv // group
            M = np.zeros((dk, dv)) if initial_state_kmajor is None else \
                np.array(initial_state_kmajor[b, hv], dtype=np.float64)
            for t in range(L):
                kt, qt, vt = k[b, t, h], q[b, t, h], v[b, t, hv]
                M = M * np.exp(g[b, t, hv])
                vt = beta[b, t, hv] * (vt - M.T @ kt)
                M = M + np.outer(kt, vt)
                o[b, t, hv] = scale * (M.T @ qt)
            out_state[b, hv] = M
    return o, out_state
