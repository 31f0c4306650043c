"""Pins for the fp64 oracle: checks against facts that do not come from the
oracle itself.

Each pin takes ``fwd`` (``oracle.forward`` or a copy of it built from a
deliberately broken source) and raises AssertionError when the oracle
disagrees with what the pages or the mathematics fix.  ``test_oracle_pins``
runs every pin on the real oracle; ``test_oracle_mutants`` plants mistakes in
copies of the oracle source and shows that each one is caught.

Sources of truth used here:
  * the hand-worked example in tests/golden/hand_worked_2x2.json;
  * closed forms of the recurrence on the "com.microsoft.GatedDeltaNet" README
    (Description): the linear rule is a causal sum of (q_t.k_s) v_s, the
    gated rule weights it by exp(G_t - G_s), beta = 0 only decays the state;
    orthonormal keys decouple the delta retrievals;
  * the delta invariant: beta = 1 and a unit key store v_t exactly under k_t;
  * structural facts: grouped heads read q/k head floor(h*H/HV) (README,
    Description), packed requests are independent (README, Inputs
    cu_seqlens), an empty request copies its state (README, Outputs), a slot
    slab is updated in place at the addressed rows (CLIKA "gatedDeltaUpdate");
  * gate arms in closed form (README, Attributes; "LinearAttentionGate",
    Description), computed here with numpy's own routines;
  * the Gated DeltaNet-2 reductions of the ONNX issue ("Proposed
    extension": b = beta * 1 recovers the v1 rule);
  * brute-force equivalence with the chunk-parallel form and with an
    independent K-major transcription.
"""
from __future__ import annotations

import json
import os

import numpy as np

from oracle.chunked import forward_chunked
from oracle.kmajor import forward_kmajor

HERE = os.path.dirname(os.path.abspath(__file__))


def _rng(seed):
    return np.random.Generator(np.random.PCG64(1000 + seed))


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, "%s: shape %s vs %s" % (what, a.shape, b.shape)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 0.0)
    assert err <= tol * scale, "%s: max abs err %.3e > %.1e" % (what, err, tol * scale)


def _softplus(x):
    return np.logaddexp(0.0, x)


def _expit(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


# ---------------------------------------------------------------- golden
def pin_golden_hand(fwd):
    with open(os.path.join(HERE, "golden", "hand_worked_2x2.json")) as f:
        gold = json.load(f)
    inp = gold["inputs"]
    k = np.array(inp["k"])[:, None, :]
    q = np.array(inp["q"])[:, None, :]
    v = np.array(inp["v"])[:, None, :]
    T = k.shape[0]
    g = np.full((T, 1), np.log(inp["alpha"]))
    beta = np.full((T, 1), inp["beta"])
    for rule, exp in gold["expected"].items():
        kw = dict(update_rule=rule, scale=1.0)
        if rule in ("gated", "gated_delta"):
            kw["gate"] = g
        if rule in ("delta", "gated_delta"):
            kw["beta"] = beta
        if rule == "gated_delta_v2":
            kw["gate"] = np.tile(np.log(np.array(inp["alpha_per_key_v2"])), (T, 1, 1))
            kw["erase"] = np.tile(np.array(inp["erase_v2"]), (T, 1, 1))
        o, st = fwd(q, k, v, **kw)
        _close(o[:, 0], exp["o"], 1e-12, "golden %s o" % rule)
        _close(st[0, 0], exp["state"], 1e-12, "golden %s state" % rule)
    # the same alpha = beta = 0.5 through the raw-gate and sigmoid arms
    exp = gold["expected"]["gated_delta"]
    o, st = fwd(q, k, v, update_rule="gated_delta", scale=1.0, gate=np.zeros((T, 1)),
                a_log=np.zeros(1), dt_bias=np.zeros(1), gate_activation="qwen",
                beta=np.zeros((T, 1)), beta_activation="sigmoid")
    _close(o[:, 0], exp["o"], 1e-12, "golden qwen/sigmoid o")
    _close(st[0, 0], exp["state"], 1e-12, "golden qwen/sigmoid state")


# ---------------------------------------------------------------- closed forms
def pin_linear_closed_form(fwd):
    r = _rng(1)
    T, DK, DV = 9, 5, 4
    q, k, v = r.standard_normal((T, 1, DK)), r.standard_normal((T, 1, DK)), r.standard_normal((T, 1, DV))
    S0 = r.standard_normal((1, 1, DV, DK))
    scale = 0.7
    o, st = fwd(q, k, v, update_rule="linear", initial_state=S0, scale=scale)
    for t in range(T):
        ref = S0[0, 0] @ q[t, 0] + sum((q[t, 0] @ k[s, 0]) * v[s, 0] for s in range(t + 1))
        _close(o[t, 0], scale * ref, 1e-12, "linear o[%d]" % t)
    _close(st[0, 0], S0[0, 0] + sum(np.outer(v[s, 0], k[s, 0]) for s in range(T)), 1e-12,
           "linear state")


def pin_gated_closed_form(fwd):
    r = _rng(2)
    T, DK, DV = 11, 6, 3
    q, k, v = r.standard_normal((T, 1, DK)), r.standard_normal((T, 1, DK)), r.standard_normal((T, 1, DV))
    S0 = r.standard_normal((1, 1, DV, DK))
    g = -r.uniform(0.0, 1.0, (T, 1))
    G = np.cumsum(g[:, 0])
    o, st = fwd(q, k, v, update_rule="gated", gate=g, initial_state=S0)
    sc = DK ** -0.5
    for t in range(T):
        ref = np.exp(G[t]) * (S0[0, 0] @ q[t, 0]) + sum(
            np.exp(G[t] - G[s]) * (q[t, 0] @ k[s, 0]) * v[s, 0] for s in range(t + 1))
        _close(o[t, 0], sc * ref, 1e-12, "gated o[%d]" % t)
    ref_state = np.exp(G[-1]) * S0[0, 0] + sum(
        np.exp(G[-1] - G[s]) * np.outer(v[s, 0], k[s, 0]) for s in range(T))
    _close(st[0, 0], ref_state, 1e-12, "gated state")


def pin_delta_invariant(fwd):
    """beta = 1 and |k| = 1: after the step, S_t k_t = v_t for any decay, so with
    q = k the output is scale * v_t."""
    r = _rng(3)
    T, DK, DV = 12, 8, 5
    k = _unit(r.standard_normal((T, 1, DK)))
    v = r.standard_normal((T, 1, DV))
    S0 = r.standard_normal((1, 1, DV, DK))
    for rule in ("delta", "gated_delta"):
        kw = dict(update_rule=rule, beta=np.ones((T, 1)), initial_state=S0, scale=1.0)
        if rule == "gated_delta":
            kw["gate"] = -r.uniform(0.0, 2.0, (T, 1))
        o, st = fwd(k, k, v, **kw)
        _close(o[:, 0], v[:, 0], 1e-12, "%s invariant o" % rule)
        _close(st[0, 0] @ k[-1, 0], v[-1, 0], 1e-12, "%s invariant state" % rule)


def pin_beta_zero(fwd):
    r = _rng(4)
    T, DK, DV = 7, 6, 4
    q, k, v = r.standard_normal((T, 1, DK)), r.standard_normal((T, 1, DK)), r.standard_normal((T, 1, DV))
    S0 = r.standard_normal((1, 1, DV, DK))
    g = -r.uniform(0.0, 1.0, (T, 1))
    G = np.cumsum(g[:, 0])
    o, st = fwd(q, k, v, update_rule="gated_delta", gate=g, beta=np.zeros((T, 1)),
                initial_state=S0, scale=1.0)
    for t in range(T):
        _close(o[t, 0], np.exp(G[t]) * (S0[0, 0] @ q[t, 0]), 1e-12, "beta=0 o[%d]" % t)
    _close(st[0, 0], np.exp(G[-1]) * S0[0, 0], 1e-12, "beta=0 state")


def pin_orthonormal_keys(fwd):
    """Mutually orthonormal keys (T <= dk): every retrieval sees only the
    decayed initial state, so
    o_t = scale (e^{G_t} S0 q_t + sum_{s<=t} e^{G_t-G_s} beta_s (q_t.k_s)(v_s - e^{G_s} S0 k_s))."""
    r = _rng(5)
    T, DK, DV = 6, 8, 5
    Qm, _ = np.linalg.qr(r.standard_normal((DK, DK)))
    k = Qm[:, :T].T[:, None, :]
    q, v = r.standard_normal((T, 1, DK)), r.standard_normal((T, 1, DV))
    S0 = r.standard_normal((1, 1, DV, DK))
    beta = r.uniform(0.1, 0.9, (T, 1))
    for rule in ("delta", "gated_delta"):
        g = -r.uniform(0.0, 1.0, (T, 1)) if rule == "gated_delta" else np.zeros((T, 1))
        G = np.cumsum(g[:, 0])
        kw = dict(update_rule=rule, beta=beta, initial_state=S0, scale=1.0)
        if rule == "gated_delta":
            kw["gate"] = g
        o, st = fwd(q, k, v, **kw)
        for t in range(T):
            ref = np.exp(G[t]) * (S0[0, 0] @ q[t, 0])
            for s in range(t + 1):
                d = beta[s, 0] * (v[s, 0] - np.exp(G[s]) * (S0[0, 0] @ k[s, 0]))
                ref = ref + np.exp(G[t] - G[s]) * (q[t, 0] @ k[s, 0]) * d
            _close(o[t, 0], ref, 1e-12, "%s orthonormal o[%d]" % (rule, t))


# ---------------------------------------------------------------- structure
def pin_gqa_mapping(fwd):
    """Value head h reads q/k head floor(h*H/HV): equal to the HV=H call on
    q/k with each head repeated HV/H times in a row, and not to the
    h mod H interleave."""
    r = _rng(6)
    T, H, HV, DK, DV = 5, 2, 6, 4, 3
    q, k = r.standard_normal((T, H, DK)), _unit(r.standard_normal((T, H, DK)))
    v = r.standard_normal((T, HV, DV))
    g, beta = -r.uniform(0, 1, (T, HV)), r.uniform(0, 1, (T, HV))
    S0 = r.standard_normal((1, HV, DV, DK))
    kw = dict(gate=g, beta=beta, initial_state=S0)
    o, st = fwd(q, k, v, **kw)
    rep = HV // H
    o2, st2 = fwd(np.repeat(q, rep, axis=1), np.repeat(k, rep, axis=1), v, **kw)
    _close(o, o2, 0.0, "gqa o")
    _close(st, st2, 0.0, "gqa state")
    o3, _ = fwd(np.tile(q, (1, rep, 1)), np.tile(k, (1, rep, 1)), v, **kw)
    assert np.max(np.abs(o3 - o)) > 1e-3, "interleaved head map must differ"


def pin_varlen_packing(fwd):
    r = _rng(7)
    lengths = [3, 0, 5, 1]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, HV, DK, DV = int(cu[-1]), 1, 2, 4, 3
    q, k = r.standard_normal((T, H, DK)), _unit(r.standard_normal((T, H, DK)))
    v = r.standard_normal((T, HV, DV))
    g, beta = -r.uniform(0, 1, (T, HV)), r.uniform(0, 1, (T, HV))
    S0 = r.standard_normal((len(lengths), HV, DV, DK))
    o, st = fwd(q, k, v, gate=g, beta=beta, initial_state=S0, cu_seqlens=cu)
    for b, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
        ob, sb = fwd(q[s:e], k[s:e], v[s:e], gate=g[s:e], beta=beta[s:e],
                     initial_state=S0[b:b + 1], cu_seqlens=[0, e - s])
        _close(o[s:e], ob, 0.0, "varlen o request %d" % b)
        _close(st[b], sb[0], 0.0, "varlen state request %d" % b)
    _close(st[1], S0[1], 0.0, "empty request copies its state")
    # clamped offsets: an entry past T ends at T, a decreasing entry is empty
    o_c, st_c = fwd(q, k, v, gate=g, beta=beta, initial_state=S0[:3],
                    cu_seqlens=[0, 4, 2, 100])
    o_a, st_a = fwd(q[:4], k[:4], v[:4], gate=g[:4], beta=beta[:4],
                    initial_state=S0[:1], cu_seqlens=[0, 4])
    o_b, st_b = fwd(q[2:], k[2:], v[2:], gate=g[2:], beta=beta[2:],
                    initial_state=S0[2:3], cu_seqlens=[0, T - 2])
    _close(st_c[0], st_a[0], 0.0, "clamp request 0")
    _close(st_c[1], S0[1], 0.0, "decreasing entry -> empty request")
    _close(st_c[2], st_b[0], 0.0, "entry past T is clamped to T")


def pin_seq_lens(fwd):
    """seq_lens bounds each uniform-packed request to its first tokens (CLIKA
    "gatedDeltaUpdate"): the same as packing those prefixes with cu_seqlens;
    padding rows keep whatever o held; a zero length copies the state; lengths
    outside [0, L] clamp."""
    r = _rng(17)
    B, L, H, HV, DK, DV = 4, 7, 1, 2, 5, 3
    q, k = r.standard_normal((B, L, H, DK)), _unit(r.standard_normal((B, L, H, DK)))
    v = r.standard_normal((B, L, HV, DV))
    g, beta = -r.uniform(0, 1, (B, L, HV)), r.uniform(0, 1, (B, L, HV))
    S0 = r.standard_normal((B, HV, DV, DK))
    lens = np.array([12, 3, 0, 6], dtype=np.int32)      # 12 clamps to 7
    sentinel = np.full((B, L, HV, DV), 5.5)
    o, st = fwd(q, k, v, gate=g, beta=beta, initial_state=S0, seq_lens=lens, o_init=sentinel)
    eff = np.minimum(np.maximum(lens, 0), L)
    flat = lambda x: np.concatenate([x[b, :eff[b]] for b in range(B)])
    cu = np.concatenate([[0], np.cumsum(eff)]).astype(np.int32)
    o2, st2 = fwd(flat(q), flat(k), flat(v), gate=flat(g), beta=flat(beta), initial_state=S0,
                  cu_seqlens=cu)
    _close(flat(o), o2, 1e-14, "seq_lens o")
    _close(st, st2, 1e-14, "seq_lens state")
    for b in range(B):
        assert np.array_equal(o[b, eff[b]:], sentinel[b, eff[b]:]), "padding rows must keep o"
    _close(st[2], S0[2], 0.0, "zero-length request copies its state")


def pin_slots(fwd):
    r = _rng(8)
    B, L, H, HV, DK, DV, NS = 3, 4, 1, 2, 4, 3, 7
    q, k = r.standard_normal((B, L, H, DK)), _unit(r.standard_normal((B, L, H, DK)))
    v = r.standard_normal((B, L, HV, DV))
    g, beta = -r.uniform(0, 1, (B, L, HV)), r.uniform(0, 1, (B, L, HV))
    slab = r.standard_normal((NS, HV, DV, DK))
    ids = np.array([5, 0, 3], dtype=np.int32)
    o, new = fwd(q, k, v, gate=g, beta=beta, slot_ids=ids, slab=slab)
    o2, st2 = fwd(q, k, v, gate=g, beta=beta, initial_state=slab[ids])
    _close(o, o2, 0.0, "slab o == gather")
    _close(new[ids], st2, 0.0, "slab rows == scatter")
    untouched = np.setdiff1d(np.arange(NS), ids)
    _close(new[untouched], slab[untouched], 0.0, "untouched slots")
    # an id outside [0, num_slots) skips its request
    bad = np.array([5, 9, 3], dtype=np.int32)
    o3, new3 = fwd(q, k, v, gate=g, beta=beta, slot_ids=bad, slab=slab)
    _close(new3[[5, 3]], new[[5, 3]], 0.0, "valid slots unaffected by a bad id")
    _close(new3[0], slab[0], 0.0, "slot of the skipped request untouched")
    assert np.all(o3[1] == 0.0), "skipped request writes no output"


def pin_gate_arms(fwd):
    r = _rng(9)
    T, H, HV, DK, DV = 6, 1, 3, 4, 4
    q, k = r.standard_normal((T, H, DK)), _unit(r.standard_normal((T, H, DK)))
    v = r.standard_normal((T, HV, DV))
    a = 3.0 * r.standard_normal((T, HV))
    a[0, 0], a[1, 1] = 40.0, -40.0  # far tails of softplus
    a_log, dt_bias = np.log(r.uniform(1, 16, HV)), r.uniform(0, 1, HV)
    braw = 2.0 * r.standard_normal((T, HV))
    o, st = fwd(q, k, v, gate=a, a_log=a_log, dt_bias=dt_bias, gate_activation="qwen",
                beta=braw, beta_activation="sigmoid")
    decay = -np.exp(a_log)[None, :] * _softplus(a + dt_bias[None, :])
    o2, st2 = fwd(q, k, v, gate=decay, beta=_expit(braw))
    _close(o, o2, 1e-13, "qwen/sigmoid arms o")
    _close(st, st2, 1e-13, "qwen/sigmoid arms state")
    # the folded scale (CLIKA "gatedDeltaUpdate": gate_scale = -exp(A_log)) is the same arm
    o3, st3 = fwd(q, k, v, gate=a, gate_scale=-np.exp(a_log), dt_bias=dt_bias,
                  gate_activation="qwen", beta=braw, beta_activation="sigmoid")
    _close(o3, o2, 1e-13, "gate_scale arm o")
    _close(st3, st2, 1e-13, "gate_scale arm state")
    # per-key raw gate with its [HV, K] bias (same page): decay per key channel
    ak = 3.0 * r.standard_normal((T, HV, DK))
    bias_k = r.uniform(-1, 1, (HV, DK))
    o4, st4 = fwd(q, k, v, gate=ak, a_log=a_log, dt_bias=bias_k, gate_activation="qwen",
                  beta=braw, beta_activation="sigmoid")
    dk_ = -np.exp(a_log)[None, :, None] * _softplus(ak + bias_k[None, :, :])
    o5, st5 = fwd(q, k, v, gate=dk_, beta=_expit(braw))
    _close(o4, o5, 1e-13, "per-key qwen arm o")
    _close(st4, st5, 1e-13, "per-key qwen arm state")


def pin_zero_vectors_normalise_to_zero(fwd):
    """qk L2-norm with an all-zero q or k row: the epsilon under the square
    root (README, Attributes qk_l2_norm) keeps the result finite and zero, so
    a zero key writes nothing and a zero query reads out nothing."""
    r = _rng(18)
    T, H, HV, DK, DV = 4, 1, 2, 6, 3
    q, k = r.standard_normal((T, H, DK)), r.standard_normal((T, H, DK))
    q[1] = 0.0
    k[2] = 0.0
    v = r.standard_normal((T, HV, DV))
    S0 = r.standard_normal((1, HV, DV, DK))
    beta = r.uniform(0, 1, (T, HV))
    o, st = fwd(q, k, v, update_rule="delta", beta=beta, qk_l2_norm=True, initial_state=S0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(st))
    _close(o[1], np.zeros_like(o[1]), 0.0, "zero query reads out zero")
    o2, st2 = fwd(q[:2], k[:2], v[:2], update_rule="delta", beta=beta[:2], qk_l2_norm=True, initial_state=S0)
    _, st3 = fwd(q[:3], k[:3], v[:3], update_rule="delta", beta=beta[:3], qk_l2_norm=True, initial_state=S0)
    _close(st3, st2, 0.0, "zero key leaves the state as it was")


def pin_l2_norm(fwd):
    r = _rng(10)
    T, H, HV, DK, DV = 5, 2, 2, 6, 3
    q, k = 3.0 * r.standard_normal((T, H, DK)), 0.2 * r.standard_normal((T, H, DK))
    v = r.standard_normal((T, HV, DV))
    g, beta = -r.uniform(0, 1, (T, HV)), r.uniform(0, 1, (T, HV))
    o, st = fwd(q, k, v, gate=g, beta=beta, qk_l2_norm=True)
    o2, st2 = fwd(_unit(q), _unit(k), v, gate=g, beta=beta)
    # the 1e-12 epsilon under the square root shifts a key of squared norm ~0.2
    # by ~3e-12 relative; 1e-10 leaves room for that and nothing more
    _close(o, o2, 1e-10, "l2 norm o")
    _close(st, st2, 1e-10, "l2 norm state")


def pin_scale(fwd):
    r = _rng(11)
    T, DK, DV = 4, 9, 2
    q, k, v = r.standard_normal((T, 1, DK)), _unit(r.standard_normal((T, 1, DK))), r.standard_normal((T, 1, DV))
    beta = r.uniform(0, 1, (T, 1))
    o0, _ = fwd(q, k, v, update_rule="delta", beta=beta)
    o1, _ = fwd(q, k, v, update_rule="delta", beta=beta, scale=1.0)
    _close(o0, o1 / 3.0, 1e-14, "default scale is 1/sqrt(dk)")


def pin_rule_reductions(fwd):
    r = _rng(12)
    T, H, HV, DK, DV = 6, 1, 2, 4, 3
    q, k = r.standard_normal((T, H, DK)), _unit(r.standard_normal((T, H, DK)))
    v = r.standard_normal((T, HV, DV))
    beta = r.uniform(0, 1, (T, HV))
    S0 = r.standard_normal((1, HV, DV, DK))
    z = np.zeros((T, HV))
    a, _ = fwd(q, k, v, update_rule="gated_delta", gate=z, beta=beta, initial_state=S0)
    b, _ = fwd(q, k, v, update_rule="delta", beta=beta, initial_state=S0)
    _close(a, b, 0.0, "gated_delta(g=0) == delta")
    a, _ = fwd(q, k, v, update_rule="gated", gate=z, initial_state=S0)
    b, _ = fwd(q, k, v, update_rule="linear", initial_state=S0)
    _close(a, b, 0.0, "gated(g=0) == linear")
    g = -r.uniform(0, 1, (T, HV))
    a, sa = fwd(q, k, v, update_rule="gated_delta", gate=g, beta=beta, initial_state=S0)
    b, sb = fwd(q, k, v, update_rule="gated_delta", gate=np.repeat(g[:, :, None], DK, 2),
                beta=beta, initial_state=S0)
    _close(a, b, 0.0, "per-key decay constant over dk == scalar decay")
    _close(sa, sb, 0.0, "per-key decay constant over dk == scalar decay (state)")


# ---------------------------------------------------------------- GDN-2
def pin_v2_reductions(fwd):
    r = _rng(13)
    T, H, HV, DK, DV = 7, 1, 2, 5, 4
    q, k = r.standard_normal((T, H, DK)), _unit(r.standard_normal((T, H, DK)))
    v = r.standard_normal((T, HV, DV))
    S0 = r.standard_normal((1, HV, DV, DK))
    g = -r.uniform(0, 1, (T, HV))
    beta = r.uniform(0, 1, (T, HV))
    # erase = beta * 1 with v scaled by beta recovers the v1 rule
    o1, s1 = fwd(q, k, v, update_rule="gated_delta", gate=g, beta=beta, initial_state=S0)
    o2, s2 = fwd(q, k, beta[:, :, None] * v, update_rule="gated_delta_v2",
                 gate=np.repeat(g[:, :, None], DK, 2),
                 erase=np.repeat(beta[:, :, None], DK, 2), initial_state=S0)
    _close(o2, o1, 1e-12, "v2 with erase = beta recovers gated_delta")
    _close(s2, s1, 1e-12, "v2 with erase = beta recovers gated_delta (state)")
    # erase = 0: per-key gated closed form
    gk = -r.uniform(0, 1, (T, HV, DK))
    o3, s3 = fwd(q, k, v, update_rule="gated_delta_v2", gate=gk, erase=np.zeros((T, HV, DK)),
                 initial_state=S0, scale=1.0)
    G = np.cumsum(gk, axis=0)
    for t in range(T):
        for h in range(HV):
            ref = S0[0, h] @ (np.exp(G[t, h]) * q[t, 0])
            for s in range(t + 1):
                ref = ref + ((q[t, 0] * np.exp(G[t, h] - G[s, h])) @ k[s, 0]) * v[s, h]
            _close(o3[t, h], ref, 1e-12, "v2 erase=0 closed form o[%d,%d]" % (t, h))
    # erase = 1 with unit keys stores v_t under k_t exactly
    o4, _ = fwd(k, k, v, update_rule="gated_delta_v2", gate=gk, erase=np.ones((T, HV, DK)),
                initial_state=S0, scale=1.0)
    _close(o4, v, 1e-12, "v2 erase=1 invariant")
    # the key-axis erase differs from the value-axis parse on random b
    b = r.uniform(0, 1, (T, HV, DK))
    ok, _ = fwd(q, k, v, update_rule="gated_delta_v2", gate=gk, erase=b, initial_state=S0)
    ov, _ = fwd(q, k, v, update_rule="gated_delta_v2", gate=gk, erase=b, initial_state=S0,
                erase_axis="value")
    assert np.max(np.abs(ok - ov)) > 1e-3, "key- and value-axis erase readings must differ"


# ---------------------------------------------------------------- cross forms
def pin_chunked_equivalence(fwd):
    """The chunk-parallel form equals the recurrence for every chunk size,
    including chunks that straddle no request boundary and a ragged tail."""
    r = _rng(14)
    lengths = [13, 1, 0, 22]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, HV, DK, DV = int(cu[-1]), 2, 4, 8, 6
    q, k = r.standard_normal((T, H, DK)), _unit(r.standard_normal((T, H, DK)))
    v = r.standard_normal((T, HV, DV))
    g = -r.uniform(0, 3, (T, HV))
    beta = r.uniform(0, 1, (T, HV))
    S0 = 0.3 * r.standard_normal((len(lengths), HV, DV, DK))
    for rule in ("gated_delta", "delta", "gated", "linear"):
        kw = dict(update_rule=rule, initial_state=S0, cu_seqlens=cu)
        if rule in ("gated", "gated_delta"):
            kw["gate"] = g
        if rule in ("delta", "gated_delta"):
            kw["beta"] = beta
        o_ref, s_ref = fwd(q, k, v, **kw)
        for c in (1, 2, 4, 16, 64):
            o_c, s_c = forward_chunked(q, k, v, chunk_size=c, **kw)
            _close(o_c, o_ref, 1e-10, "chunked %s C=%d o" % (rule, c))
            _close(s_c, s_ref, 1e-10, "chunked %s C=%d state" % (rule, c))
    # per-key-channel decay (Ascend Formula) and the key-axis erase gate of
    # Gated DeltaNet-2, with the raw-gate arm on a per-key gate as well
    gk = -r.uniform(0, 2, (T, HV, DK))
    erase = r.uniform(0, 1, (T, HV, DK))
    raw = r.standard_normal((T, HV, DK))
    a_log, dt_bias = np.log(r.uniform(1, 16, HV)), r.uniform(0, 1, HV)
    bias_k = r.uniform(-1, 1, (HV, DK))
    cases = [
        ("gated_delta per-key", dict(update_rule="gated_delta", gate=gk, beta=beta)),
        ("gated per-key", dict(update_rule="gated", gate=gk)),
        ("gated_delta_v2 per-key", dict(update_rule="gated_delta_v2", gate=gk, erase=erase)),
        ("gated_delta_v2 per-head", dict(update_rule="gated_delta_v2", gate=g, erase=erase)),
        ("gated_delta per-key qwen", dict(update_rule="gated_delta", gate=raw, beta=beta,
                                          gate_activation="qwen", a_log=a_log, dt_bias=bias_k)),
        ("gated_delta_v2 per-key folded scale", dict(update_rule="gated_delta_v2", gate=raw, erase=erase,
                                                     gate_activation="qwen", gate_scale=-np.exp(a_log),
                                                     dt_bias=bias_k)),
    ]
    for name, kw in cases:
        kw.update(initial_state=S0, cu_seqlens=cu)
        o_ref, s_ref = fwd(q, k, v, **kw)
        for c in (1, 3, 16, 64):
            o_c, s_c = forward_chunked(q, k, v, chunk_size=c, **kw)
            _close(o_c, o_ref, 1e-10, "chunked %s C=%d o" % (name, c))
            _close(s_c, s_ref, 1e-10, "chunked %s C=%d state" % (name, c))


def pin_segment_composition(fwd):
    """The recurrence maps the state affinely: over a run of tokens each
    V-major row goes s -> s M + c, where row r of M is the run started from
    row r of the identity with every value zero, and c the run started from
    zero.  Cutting a request into segments and composing (M, c) in order
    must therefore give the one-pass final state (the reading the segmented
    chunk scan relies on)."""
    r = _rng(17)
    T, H, HV, D = 23, 1, 2, 5
    q, k = r.standard_normal((T, H, D)), _unit(r.standard_normal((T, H, D)))
    v = r.standard_normal((T, HV, D))
    S0 = r.standard_normal((1, HV, D, D))
    eye = np.broadcast_to(np.eye(D), (1, HV, D, D)).copy()
    cases = [
        ("gated_delta", dict(update_rule="gated_delta", gate=-r.uniform(0, 0.3, (T, HV)), beta=r.uniform(0, 1, (T, HV)))),
        ("linear", dict(update_rule="linear")),
        ("gated_delta_v2 per-key", dict(update_rule="gated_delta_v2", gate=-r.uniform(0, 0.3, (T, HV, D)),
                                        erase=r.uniform(0, 1, (T, HV, D)))),
    ]
    cuts = [0, 7, 8, 19, T]
    for name, kw in cases:
        _, s_ref = fwd(q, k, v, initial_state=S0, **kw)
        s = S0
        for a, b in zip(cuts[:-1], cuts[1:]):
            seg = {key: (val[a:b] if isinstance(val, np.ndarray) else val) for key, val in kw.items()}
            _, M = fwd(q[a:b], k[a:b], np.zeros_like(v[a:b]), initial_state=eye, **seg)
            _, c = fwd(q[a:b], k[a:b], v[a:b], initial_state=np.zeros_like(S0), **seg)
            s = np.einsum("bhij,bhjk->bhik", s, M) + c
        _close(s, s_ref, 1e-12, "segment composition %s" % name)
        # and the map really depends on the start (M is not zero)
        _, s_zero = fwd(q, k, v, initial_state=np.zeros_like(S0), **kw)
        assert np.max(np.abs(s_ref - s_zero)) > 1e-3, name


def pin_kmajor_cross(fwd):
    """The V-major oracle against the independent K-major transcription: a
    per-head decay, a decay per key dimension, and the Gated DeltaNet-2
    key-axis erase gate with a per-key and with a per-head decay."""
    r = _rng(15)
    B, L, H, HV, DK, DV = 2, 6, 2, 4, 5, 3
    q, k = r.standard_normal((B, L, H, DK)), _unit(r.standard_normal((B, L, H, DK)))
    v = r.standard_normal((B, L, HV, DV))
    g, beta = -r.uniform(0, 1, (B, L, HV)), r.uniform(0, 1, (B, L, HV))
    gk = -r.uniform(0, 1, (B, L, HV, DK))
    erase = r.uniform(0, 1, (B, L, HV, DK))
    S0 = r.standard_normal((B, HV, DV, DK))
    S0k = np.swapaxes(S0, 2, 3)
    cases = [
        ("per-head decay", dict(gate=g, beta=beta), (g, beta, None)),
        ("per-key decay", dict(gate=gk, beta=beta), (gk, beta, None)),
        ("erase, per-key decay", dict(update_rule="gated_delta_v2", gate=gk, erase=erase), (gk, None, erase)),
        ("erase, per-head decay", dict(update_rule="gated_delta_v2", gate=g, erase=erase), (g, None, erase)),
    ]
    for name, kw, (kg, kb, ke) in cases:
        o, st = fwd(q, k, v, initial_state=S0, **kw)
        o2, st2 = forward_kmajor(q, k, v, kg, kb, S0k, erase=ke)
        _close(o, o2, 1e-12, "K-major cross o (%s)" % name)
        _close(st, np.swapaxes(st2, 2, 3), 1e-12, "K-major cross state (%s)" % name)


def pin_row_split_invariance(fwd):
    r = _rng(16)
    T, H, HV, DK, DV = 5, 1, 1, 4, 10
    q, k = r.standard_normal((T, H, DK)), _unit(r.standard_normal((T, H, DK)))
    v = r.standard_normal((T, HV, DV))
    g, beta = -r.uniform(0, 1, (T, HV)), r.uniform(0, 1, (T, HV))
    a = fwd(q, k, v, gate=g, beta=beta, row_block=1)
    b = fwd(q, k, v, gate=g, beta=beta, row_block=16)
    _close(a[0], b[0], 0.0, "row split o")
    _close(a[1], b[1], 0.0, "row split state")


# ---------------------------------------------------------------- standalone gate
# ("com.microsoft.LinearAttentionGate", Description and Outputs)
def pin_gate_closed_points(gate, fwd):
    """softplus(0) = ln 2 and sigmoid(0) = 1/2 at every head (a = -dt_bias
    exactly, so a wrong head index or bias sign moves the argument off zero);
    the far tails softplus(40) = 40 + ln(1 + e^-40), softplus(-40) =
    ln(1 + e^-40) ~ e^-40, sigmoid(+-40) = 1 / (1 + e^-+40)."""
    import math
    heads = 5
    r = _rng(20)
    dt_bias = r.uniform(-2, 2, heads)
    dscale = -r.uniform(1, 16, heads)
    a = np.tile(-dt_bias, (3, 1))
    d, b = gate(a, dt_bias, dscale, b=np.zeros_like(a), want_beta=True)
    _close(d, np.tile(dscale * math.log(2.0), (3, 1)), 1e-15, "gate at softplus(0)")
    _close(b, np.full_like(a, 0.5), 0.0, "sigmoid(0)")
    e40 = math.exp(-40.0)
    a = np.array([[40.0, -40.0]])
    d, b = gate(a, np.zeros(2), np.array([-1.0, -2.0]), b=a, want_beta=True)
    _close(d, [[-(40.0 + math.log1p(e40)), -2.0 * e40]], 1e-15, "softplus tails")
    assert abs(d[0, 1] / (-2.0 * e40) - 1.0) < 1e-12, "softplus(-40) keeps its relative precision"
    _close(b, [[1.0 / (1.0 + e40), e40 / (1.0 + e40)]], 1e-15, "sigmoid tails")
    assert abs(b[0, 1] / e40 - 1.0) < 1e-12


def pin_gate_matches_forward(gate, fwd):
    """The standalone gate's decay and rate drive the recurrence exactly as
    the forward pass's fused raw-gate arm and sigmoid (README, Attributes
    gate_activation / beta_activation): two independent code paths."""
    r = _rng(21)
    T, H, HV, DK, DV = 7, 1, 3, 4, 4
    q, k = r.standard_normal((T, H, DK)), _unit(r.standard_normal((T, H, DK)))
    v = r.standard_normal((T, HV, DV))
    a = 3.0 * r.standard_normal((T, HV))
    braw = 2.0 * r.standard_normal((T, HV))
    a_log, dt_bias = np.log(r.uniform(1, 16, HV)), r.uniform(0, 1, HV)
    decay, beta = gate(a, dt_bias, -np.exp(a_log), b=braw, want_beta=True)
    o, st = fwd(q, k, v, gate=a, a_log=a_log, dt_bias=dt_bias, gate_activation="qwen",
                beta=braw, beta_activation="sigmoid")
    o2, st2 = fwd(q, k, v, gate=decay, beta=beta)
    _close(o2, o, 1e-14, "gate output drives the recurrence like the fused arm (o)")
    _close(st2, st, 1e-14, "gate output drives the recurrence like the fused arm (state)")
    # an unconsumed b is allowed and changes nothing (Description)
    d2, none = gate(a, dt_bias, -np.exp(a_log), b=braw, want_beta=False)
    assert none is None
    _close(d2, decay, 0.0, "decay without beta")


GATE_PINS = [pin_gate_closed_points, pin_gate_matches_forward]


ALL_PINS = [
    pin_golden_hand, pin_linear_closed_form, pin_gated_closed_form, pin_delta_invariant,
    pin_beta_zero, pin_orthonormal_keys, pin_gqa_mapping, pin_varlen_packing, pin_seq_lens, pin_slots,
    pin_gate_arms, pin_zero_vectors_normalise_to_zero, pin_l2_norm, pin_scale, pin_rule_reductions, pin_v2_reductions,
    pin_chunked_equivalence, pin_segment_composition, pin_kmajor_cross, pin_row_split_invariance,
]
