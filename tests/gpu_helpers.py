"""Helpers for the GPU parity tests: run one seeded case through the C-ABI
(HIP kernels) and through the fp64 oracle, restrict a case to a sample of
(request, value head) pairs the oracle can finish quickly, and compare."""
from __future__ import annotations

import sys

import numpy as np

import oracle

# tolerances of the parity bar: max |gpu - ref| / max |ref| per tensor
TOL_F32 = 1e-4
TOL_F16 = 2e-3
TOL_CHUNKED = 2e-3
# bf16 outputs: one round-to-nearest-even store costs up to 2^-9 (1.95e-3) of
# an element, so the max-error / max-value metric stays below 2^-8; the state
# stays fp32 and its inputs are exact, so it keeps the fp16 bound
TOL_BF16_O = 4e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(case):
    import torch
    dev = {}
    for key in ("q", "k", "v", "gate", "beta", "erase", "a_log", "dt_bias", "cu_seqlens",
                "slot_ids", "initial_state", "slab", "gate_scale", "seq_lens"):
        x = case.get(key)
        dev[key] = None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()
    if case.get("act_dtype") == "bf16":
        # bf16 activations are drawn on the bf16 grid and held as fp32 in numpy
        for key in ("q", "k", "v") + (("gate",) if case["gate_activation"] == "qwen" else ()):
            if dev[key] is not None:
                dev[key] = dev[key].to(torch.bfloat16)
    return dev


def gpu_forward(case, algo="auto", dev=None, **over):
    """Returns (o, state) as numpy float64; in slab mode the state is the
    updated slab (a fresh copy of the input slab is updated)."""
    import torch
    from gated_delta_rule_token_amd import api
    d = dev if dev is not None else to_dev(case)
    slab = None if d["slab"] is None else d["slab"].clone()
    kw = dict(gate=d["gate"], beta=d["beta"], erase=d["erase"], a_log=d["a_log"],
              dt_bias=d["dt_bias"], cu_seqlens=d["cu_seqlens"], initial_state=d["initial_state"],
              slot_ids=d["slot_ids"], state=slab, update_rule=case["update_rule"],
              gate_activation=case["gate_activation"], beta_activation=case["beta_activation"],
              qk_l2_norm=case["qk_l2_norm"], scale=case["scale"],
              chunk_size=case.get("chunk_size", 64), algo=algo,
              gate_scale=d.get("gate_scale"), seq_lens=d.get("seq_lens"))
    kw.update(over)
    o, st = api.forward(d["q"], d["k"], d["v"], **kw)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), st.double().cpu().numpy()


def oracle_forward(case, **over):
    kw = dict(gate=case["gate"], beta=case["beta"], erase=case["erase"], a_log=case["a_log"],
              dt_bias=case["dt_bias"], cu_seqlens=case["cu_seqlens"],
              initial_state=case["initial_state"], slot_ids=case["slot_ids"], slab=case["slab"],
              update_rule=case["update_rule"], gate_activation=case["gate_activation"],
              beta_activation=case["beta_activation"], qk_l2_norm=case["qk_l2_norm"],
              scale=case["scale"], gate_scale=case.get("gate_scale"), seq_lens=case.get("seq_lens"))
    kw.update(over)
    return oracle.forward(case["q"], case["k"], case["v"], **kw)


def request_ranges(case):
    T = case["q"].shape[0] if case["q"].ndim == 3 else case["q"].shape[0] * case["q"].shape[1]
    if case["cu_seqlens"] is not None:
        cu = np.clip(case["cu_seqlens"].astype(np.int64), 0, T)
        return [(int(cu[i]), int(max(cu[i], cu[i + 1]))) for i in range(len(cu) - 1)]
    if case["q"].ndim == 4:
        B, L = case["q"].shape[:2]
    else:
        B = case["initial_state"].shape[0] if case["initial_state"] is not None else 1
        L = T // B
    lens = case.get("seq_lens")
    if lens is not None:
        return [(b * L, b * L + int(min(max(lens[b], 0), L))) for b in range(B)]
    return [(b * L, (b + 1) * L) for b in range(B)]


def sub_case(case, b, heads):
    """Case restricted to request b and value heads ``heads`` (each with its
    own q/k head), as a rank-3 single request; exact because requests and
    heads evolve independently (README: grouped heads read q/k head
    floor(h*H/HV))."""
    s, e = request_ranges(case)[b]
    q, k, v = case["q"], case["k"], case["v"]
    rank4 = q.ndim == 4

    def tok(x):
        if x is None:
            return None
        return x.reshape((-1,) + x.shape[2:])[s:e] if rank4 else x[s:e]

    H, HV = q.shape[-2], v.shape[-2]
    qh = [h * H // HV for h in heads]
    out = dict(case)
    out["q"] = np.ascontiguousarray(tok(q)[:, qh])
    out["k"] = np.ascontiguousarray(tok(k)[:, qh])
    out["v"] = np.ascontiguousarray(tok(v)[:, heads])
    for key in ("gate", "beta", "erase"):
        x = tok(case[key])
        out[key] = None if x is None else np.ascontiguousarray(x[:, heads])
    for key in ("a_log", "dt_bias", "gate_scale"):
        out[key] = None if case.get(key) is None else case[key][heads]
    out["seq_lens"] = None
    out["cu_seqlens"] = np.array([0, e - s], dtype=np.int32)
    if case["slab"] is not None:
        init = case["slab"][case["slot_ids"][b]][None]
    elif case["initial_state"] is not None:
        init = case["initial_state"][b:b + 1]
    else:
        init = None
    out["initial_state"] = None if init is None else np.ascontiguousarray(init[:, heads])
    out["slab"] = None
    out["slot_ids"] = None
    return out, (s, e)


def rel_err(got, ref):
    return oracle.max_rel_err(got, ref)


def assert_close(got, ref, tol, what):
    err = rel_err(got, ref)
    say("  %-48s max rel err %.3e (tol %.0e)" % (what, err, tol))
    assert np.all(np.isfinite(got)), "%s: non-finite values" % what
    assert err <= tol, "%s: max rel err %.3e > %.1e" % (what, err, tol)
