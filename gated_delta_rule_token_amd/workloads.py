"""Seeded synthetic inputs for the gated delta-rule engine.

This module only draws inputs: it holds none of the recurrence's arithmetic
and is shared by the tests, the benchmark and the smoke check, which feed
the same arrays to the HIP path and to the CPU oracle.  All draws use
``numpy.random.Generator(PCG64(seed))``; values are drawn in float32/float64
and cast to the activation dtype with round-to-nearest-even.

The five named workloads mirror the shapes the pages' operator contract is
exercised at (rank-3 varlen packing, rank-4 batches, a state slab addressed
by slot ids, grouped heads, dk = dv = 128).  No public dataset or benchmark
suite is involved; these arrays are the whole workload.

Each case is a plain dict:
  q, k, v, gate, beta, erase, a_log, dt_bias, cu_seqlens, slot_ids,
  initial_state, slab, gate_scale, seq_lens  -- numpy arrays or None
  update_rule, gate_activation, beta_activation, qk_l2_norm, scale,
  chunk_size, act_dtype, name -- attributes
"""
from __future__ import annotations

import numpy as np

ATTR_KEYS = ("update_rule", "gate_activation", "beta_activation", "qk_l2_norm", "scale",
             "chunk_size")
ARRAY_KEYS = ("q", "k", "v", "gate", "beta", "erase", "a_log", "dt_bias", "cu_seqlens",
              "slot_ids", "initial_state", "slab", "gate_scale", "seq_lens")


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng, shape, dtype=np.float32, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x.astype(dtype)


def unit_rows(rng, shape, dtype):
    """N(0,1) vectors along the last axis, scaled to unit length in float32 and
    then cast (keys that arrive already normalised from upstream)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / n.astype(np.float32)).astype(dtype)


def bf16_grid(x):
    """float32 array rounded to the nearest bfloat16 value (ties to even), kept
    as float32: numpy has no bfloat16, and these values convert to bfloat16
    exactly on the device."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def _draw(rng, shape, dtype, unit=False):
    """N(0,1) draw (unit rows with unit=True) in fp32/fp16, or on the bf16 grid."""
    if dtype == "bf16":
        x = unit_rows(rng, shape, np.float32) if unit else _normal(rng, shape, np.float32)
        return bf16_grid(x)
    return unit_rows(rng, shape, dtype) if unit else _normal(rng, shape, dtype)


def _log_uniform_alog(rng, n):
    # A_log = log U(1, 16): the per-head log decay rate
    return np.log(rng.uniform(1.0, 16.0, size=n)).astype(np.float32)


def _logistic(x):
    # input recipe only: a logistic draw for precomputed update rates
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _neg_softplus_scaled(x, factor):
    # input recipe only: a log decay drawn as -log(1 + e^x) * factor
    return (-np.logaddexp(0.0, x.astype(np.float64)) * factor).astype(np.float32)


def base(**kw):
    case = {key: None for key in ARRAY_KEYS}
    case.update(update_rule="gated_delta", gate_activation="none", beta_activation="none",
                qk_l2_norm=0, scale=0.0, chunk_size=64, act_dtype="f32", name="case")
    case.update(kw)
    return case


def tiny_varlen(seed: int = 0):
    """T=16 tokens as two requests (cu_seqlens [0,5,16]), H=2 q/k heads, HV=4
    value heads, dk=dv=32, fp32.  q,k,v ~ N(0,1) with qk_l2_norm=1; raw-gate
    arm with a ~ N(0,1), dt_bias ~ U(0,1), A_log = log U(1,16); update rate
    sigmoid(b), b ~ N(0,1); zero initial state; scale 1/sqrt(dk)."""
    rng = rng_for(seed)
    T, H, HV, D = 16, 2, 4, 32
    return base(
        name="tiny_varlen_T16_H2_HV4_d32_f32",
        q=_normal(rng, (T, H, D)), k=_normal(rng, (T, H, D)), v=_normal(rng, (T, HV, D)),
        gate=_normal(rng, (T, HV)),
        dt_bias=rng.uniform(0.0, 1.0, size=HV).astype(np.float32),
        a_log=_log_uniform_alog(rng, HV),
        beta=_normal(rng, (T, HV)),
        cu_seqlens=np.array([0, 5, 16], dtype=np.int32),
        update_rule="gated_delta", gate_activation="qwen", beta_activation="sigmoid",
        qk_l2_norm=1, act_dtype="f32")


def decode_slab(seed: int = 1, B=256, H=16, HV=32, D=128, num_slots=512, with_slab=True, L=1):
    """One decode step: B requests of L tokens (rank-4 (B,L,...); L = 1 is
    plain decode, a few tokens the speculative / multi-token verify shape), H=16
    q/k heads, HV=32 value heads, dk=dv=128, fp16 q/k/v (keys unit length), a
    fp32 state slab of num_slots slots ~ N(0, 0.05) updated in place at B
    distinct random slot ids; raw-gate arm (fp16 a ~ N(0,1), per-head dt_bias
    ~ U(0,1), A_log = log U(1,16)), update rate sigmoid(b), b ~ N(0,1)."""
    rng = rng_for(seed)
    slot_ids = rng.choice(num_slots, size=B, replace=False).astype(np.int32)
    q = _normal(rng, (B, L, H, D), np.float16)
    k = unit_rows(rng, (B, L, H, D), np.float16)
    v = _normal(rng, (B, L, HV, D), np.float16)
    a = _normal(rng, (B, L, HV), np.float16)
    dt_bias = rng.uniform(0.0, 1.0, size=HV).astype(np.float32)
    a_log = _log_uniform_alog(rng, HV)
    b = _normal(rng, (B, L, HV))
    slab = _normal(rng, (num_slots, HV, D, D), np.float32, std=0.05) if with_slab else None
    return base(
        name=("decode_B%d_H%d_HV%d_d%d_slab%d_f16" % (B, H, HV, D, num_slots)) if L == 1 else
             ("decode_B%d_L%d_H%d_HV%d_d%d_slab%d_f16" % (B, L, H, HV, D, num_slots)),
        q=q, k=k, v=v, gate=a, dt_bias=dt_bias, a_log=a_log, beta=b, slot_ids=slot_ids,
        slab=slab, update_rule="gated_delta", gate_activation="qwen",
        beta_activation="sigmoid", qk_l2_norm=0, act_dtype="f16", num_slots=num_slots)


def varlen_prefill(seed: int = 2, n_req=8, lo=512, hi=8192, H=16, HV=32, D=128, lengths=None):
    """n_req requests with lengths uniform in [lo, hi], packed via cu_seqlens;
    H=16, HV=32, dk=dv=128, fp16 q/k/v with qk_l2_norm=1; raw-gate arm as the
    decode case; random fp32 initial state ~ N(0, 0.05) per request; the
    final state goes to a separate buffer."""
    rng = rng_for(seed)
    if lengths is None:
        lengths = rng.integers(lo, hi + 1, size=n_req)
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    return base(
        name="varlen_prefill_%dreq_T%d_H%d_HV%d_d%d_f16" % (len(lengths), T, H, HV, D),
        q=_normal(rng, (T, H, D), np.float16), k=_normal(rng, (T, H, D), np.float16),
        v=_normal(rng, (T, HV, D), np.float16),
        gate=_normal(rng, (T, HV), np.float16),
        dt_bias=rng.uniform(0.0, 1.0, size=HV).astype(np.float32),
        a_log=_log_uniform_alog(rng, HV),
        beta=_normal(rng, (T, HV)),
        initial_state=_normal(rng, (len(lengths), HV, D, D), np.float32, std=0.05),
        cu_seqlens=cu, update_rule="gated_delta", gate_activation="qwen",
        beta_activation="sigmoid", qk_l2_norm=1, act_dtype="f16")


def long_prefill(seed: int = 3, T=65536, H=16, HV=16, D=128, chunk_size=64):
    """One sequence of T tokens (rank-4 (1,T,...)), H=HV=16, dk=dv=128, fp16
    q/k/v with unit keys; log decay g = -softplus(x) * A_h with x ~ N(0,1)
    per (t,h) and A_h ~ U(1,16) per head (fp32, no gate activation); update
    rate precomputed as sigmoid(N(0,1)) (no beta activation); zero initial
    state; chunk size 64."""
    rng = rng_for(seed)
    q = _normal(rng, (1, T, H, D), np.float16)
    k = unit_rows(rng, (1, T, H, D), np.float16)
    v = _normal(rng, (1, T, HV, D), np.float16)
    A = rng.uniform(1.0, 16.0, size=HV).astype(np.float32)
    g = _neg_softplus_scaled(_normal(rng, (1, T, HV)), A[None, None, :])
    beta = _logistic(_normal(rng, (1, T, HV)))
    return base(
        name="long_prefill_T%d_H%d_HV%d_d%d_f16" % (T, H, HV, D),
        q=q, k=k, v=v, gate=g, beta=beta, update_rule="gated_delta",
        gate_activation="none", beta_activation="none", qk_l2_norm=0,
        chunk_size=chunk_size, act_dtype="f16")


def perkey_erase(seed: int = 4, B=4, L=4096, H=8, HV=32, D=128):
    """B=4 requests of L=4096 tokens (rank-4), H=8, HV=32, dk=dv=128, fp16
    q/k/v with unit keys; per-key log decay (B,L,HV,dk) = -softplus(N(0,1))*0.1
    and a key-axis erase gate (B,L,HV,dk) = sigmoid(N(0,1)), both fp32; the
    Gated DeltaNet-2 rule (no update rate); zero initial state."""
    rng = rng_for(seed)
    q = _normal(rng, (B, L, H, D), np.float16)
    k = unit_rows(rng, (B, L, H, D), np.float16)
    v = _normal(rng, (B, L, HV, D), np.float16)
    decay = _neg_softplus_scaled(_normal(rng, (B, L, HV, D)), 0.1)
    erase = _logistic(_normal(rng, (B, L, HV, D)))
    return base(
        name="perkey_erase_B%d_L%d_H%d_HV%d_d%d_f16" % (B, L, H, HV, D),
        q=q, k=k, v=v, gate=decay, erase=erase, update_rule="gated_delta_v2",
        gate_activation="none", beta_activation="none", qk_l2_norm=0, act_dtype="f16")


def odd_shape(seed: int = 5, dtype=np.float32):
    """The README usage example's shapes: T=4 tokens, one q/k head of dk=12,
    two value heads of dv=9, one request, with decay and beta given
    directly (no activations) and an explicit initial state."""
    rng = rng_for(seed)
    T, H, HV, DK, DV = 4, 1, 2, 12, 9
    return base(
        name="odd_T4_H1_HV2_dk12_dv9",
        q=_normal(rng, (T, H, DK), dtype), k=unit_rows(rng, (T, H, DK), dtype),
        v=_normal(rng, (T, HV, DV), dtype),
        gate=_neg_softplus_scaled(_normal(rng, (T, HV)), 1.0),
        beta=_logistic(_normal(rng, (T, HV))),
        initial_state=_normal(rng, (1, HV, DV, DK), np.float32, std=0.1),
        act_dtype="f32" if dtype == np.float32 else "f16")


def as_bf16(case):
    """The same case with bf16 activations: q, k, v (and a raw gate given in
    the activation dtype) rounded onto the bf16 grid, held as float32."""
    out = dict(case, act_dtype="bf16", name=case["name"].replace("_f16", "") + "_bf16")
    keys = ("q", "k", "v") + (("gate",) if case["gate_activation"] == "qwen" else ())
    for key in keys:
        if out[key] is not None:
            out[key] = bf16_grid(out[key].astype(np.float32))
    return out


def random_case(seed, *, T=None, lengths=None, H=2, HV=4, DK=32, DV=32, dtype=np.float32,
                update_rule="gated_delta", gate_activation="none", beta_activation="none",
                qk_l2_norm=0, per_key=False, with_initial=True, unit_keys=True,
                rank4_batch=None, slots=None, seq_lens=None, folded_scale=False):
    """Generic small case for parity tests.  ``lengths`` gives varlen packing
    (cu_seqlens); ``rank4_batch`` gives a uniform (B, L) batch, optionally
    bounded per request by ``seq_lens``; ``slots`` = (num_slots,) addresses a
    slab at distinct random ids.  The raw-gate arm draws a per-head (or, with
    a per-key gate, per (head, key channel)) bias; ``folded_scale`` passes
    gate_scale = -exp(A_log) instead of A_log."""
    rng = rng_for(seed)
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        T = int(cu[-1])
        B = len(lengths)
        lead = (T,)
    elif rank4_batch is not None:
        B, L = rank4_batch
        cu = None
        T = B * L
        lead = (B, L)
    else:
        B, cu = 1, None
        lead = (T,)
    act = "bf16" if dtype == "bf16" else ("f32" if dtype == np.float32 else "f16")
    q = _draw(rng, lead + (H, DK), dtype)
    k = _draw(rng, lead + (H, DK), dtype, unit=unit_keys)
    v = _draw(rng, lead + (HV, DV), dtype)
    case = base(name="random_%s_s%d" % (update_rule, seed), q=q, k=k, v=v, cu_seqlens=cu,
                update_rule=update_rule, gate_activation=gate_activation,
                beta_activation=beta_activation, qk_l2_norm=qk_l2_norm, act_dtype=act)
    if update_rule in ("gated", "gated_delta", "gated_delta_v2"):
        gshape = lead + ((HV, DK) if per_key else (HV,))
        if gate_activation == "qwen":
            case["gate"] = _draw(rng, gshape, dtype)
            case["a_log"] = _log_uniform_alog(rng, HV)
            case["dt_bias"] = rng.uniform(0.0, 1.0, size=(HV, DK) if per_key else HV).astype(np.float32)
            if folded_scale:
                case["gate_scale"] = (-np.exp(case["a_log"].astype(np.float64))).astype(np.float32)
                case["a_log"] = None
        else:
            case["gate"] = _neg_softplus_scaled(_normal(rng, gshape), 0.5)
    if update_rule in ("delta", "gated_delta"):
        raw = _normal(rng, lead + (HV,))
        case["beta"] = raw if beta_activation == "sigmoid" else _logistic(raw)
    if update_rule == "gated_delta_v2":
        case["erase"] = _logistic(_normal(rng, lead + (HV, DK)))
    if slots is not None:
        (num_slots,) = slots
        case["slot_ids"] = rng.choice(num_slots, size=B, replace=False).astype(np.int32)
        case["slab"] = _normal(rng, (num_slots, HV, DV, DK), np.float32, std=0.1)
    elif with_initial:
        case["initial_state"] = _normal(rng, (B, HV, DV, DK), np.float32, std=0.1)
    if seq_lens is not None:
        case["seq_lens"] = np.asarray(seq_lens, dtype=np.int32)
    return case


NAMED = {
    "tiny_varlen": tiny_varlen,
    "decode_slab": decode_slab,
    "varlen_prefill": varlen_prefill,
    "long_prefill": long_prefill,
    "perkey_erase": perkey_erase,
}
