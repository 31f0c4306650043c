"""fp64 CPU oracle for the gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``; never by the product package.
It shares no code with the HIP path.

* ``forward`` -- the plain per-token recurrence (``gdr_oracle.c``), written
  from the "com.microsoft.GatedDeltaNet" README (Description, Inputs,
  Outputs, Attributes), the Ascend "aclnnRecurrentGatedDeltaRule" Formula
  (per-key decay) and the ONNX "Spec gap ... Gated DeltaNet-2" issue (erase
  gate).  Every input is upcast exactly to float64 before the call.
* ``oracle.chunked.forward_chunked`` -- the chunk-parallel form of the same
  recurrence (fp64 numpy), checked against ``forward`` by brute force.
* ``oracle.kmajor.forward_kmajor`` -- an independent numpy transcription in
  the K-major orientation of the ONNX issue (sections "What LinearAttention
  currently does" and "The GDN-2 recurrence"), for tiny cross-checks.
* ``gate`` -- the standalone gate of the "com.microsoft.LinearAttentionGate"
  README (``gdro_gate`` in ``gdr_oracle.c``).

Parity pins for all three live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "libgdr_oracle.so")
_lock = threading.Lock()
_lib = None

RULES = {"linear": 0, "gated": 1, "delta": 2, "gated_delta": 3, "gated_delta_v2": 4}


class _Problem(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64),
        ("B", ctypes.c_int32),
        ("L", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("HV", ctypes.c_int32),
        ("DK", ctypes.c_int32),
        ("DV", ctypes.c_int32),
        ("rule", ctypes.c_int32),
        ("gate_qwen", ctypes.c_int32),
        ("beta_sigmoid", ctypes.c_int32),
        ("qk_l2_norm", ctypes.c_int32),
        ("per_key", ctypes.c_int32),
        ("erase_value_axis", ctypes.c_int32),
        ("num_slots", ctypes.c_int32),
        ("row_block", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("gate", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("erase", ctypes.c_void_p),
        ("a_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p),
        ("slot_ids", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("state", ctypes.c_void_p),
        ("gate_scale", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
    ]


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (fp64, -O2, no fast-math, OpenMP)."""
    with _lock:
        stale = (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)
        if force or stale:
            tmp = _LIB + ".tmp%d" % os.getpid()
            subprocess.check_call(
                ["gcc", "-O2", "-fopenmp", "-std=c99", "-shared", "-fPIC", "-Wall",
                 "-o", tmp, _SRC, "-lm"])
            os.replace(tmp, _LIB)
    return _LIB


def _open(path):
    lib = ctypes.CDLL(path)
    lib.gdro_forward.argtypes = [ctypes.POINTER(_Problem)]
    lib.gdro_forward.restype = ctypes.c_int
    lib.gdro_num_threads.restype = ctypes.c_int
    lib.gdro_gate.argtypes = [ctypes.c_int64, ctypes.c_int32] + [ctypes.c_void_p] * 6
    lib.gdro_gate.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _open(_LIB)
    return _lib


def compile_variant(src_text: str, out_path: str):
    """Compile a modified copy of the oracle source (used by the tests that plant
    mistakes in the oracle to show the pins catch them) and return its handle,
    to be passed as ``forward(..., lib=handle)``."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-std=c99", "-shared", "-fPIC",
                           "-o", out_path, src, "-lm"])
    return _open(out_path)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def num_threads() -> int:
    """OpenMP threads the oracle runs on (honours OMP_NUM_THREADS)."""
    return int(_load().gdro_num_threads())


def _f64(x):
    if x is None:
        return None
    a = np.asarray(x)
    if a.dtype not in (np.float16, np.float32, np.float64):
        raise TypeError("oracle inputs must be fp16/fp32/fp64, got %s" % a.dtype)
    return np.ascontiguousarray(a, dtype=np.float64)  # exact upcast


def _i32(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x), dtype=np.int32)


def _ptr(a):
    return None if a is None else a.ctypes.data


def forward(q, k, v, *, gate=None, beta=None, erase=None, a_log=None, dt_bias=None,
            cu_seqlens=None, initial_state=None, slot_ids=None, slab=None,
            update_rule="gated_delta", gate_activation="none", beta_activation="none",
            qk_l2_norm=False, scale=0.0, batch=None, erase_axis="key", o_init=None,
            row_block=16, lib=None, gate_scale=None, seq_lens=None):
    """Run the fp64 recurrence.

    q, k: (T,H,dk) or (B,L,H,dk); v: (T,HV,dv) or (B,L,HV,dv).
    gate: (T,HV) or (T,HV,dk) per-key (leading axes as q); beta: (T,HV);
    erase: (T,HV,dk).  cu_seqlens: (B+1) int.  initial_state: (B,HV,dv,dk).
    slot_ids + slab: slab (num_slots,HV,dv,dk) is updated in a copy that is
    returned as the state.  Raw-gate arm: dt_bias (HV,) or (HV,dk) beside a
    per-key gate, with a_log (HV,) or the folded gate_scale (HV,).  seq_lens
    (B,) bounds each uniform-packed request to its first seq_lens[b] tokens.  Returns (o, state) as float64 arrays; o has q's
    leading axes with (HV, dv) trailing.  Tokens no request covers keep
    ``o_init`` (zeros by default).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    rank4 = q.ndim == 4
    if rank4:
        B, L = q.shape[0], q.shape[1]
        q = q.reshape(B * L, *q.shape[2:])
        k = k.reshape(B * L, *k.shape[2:])
        v = v.reshape(B * L, *v.shape[2:])
    T, H, DK = q.shape
    HV, DV = v.shape[1], v.shape[2]
    lead = (B, L) if rank4 else (T,)

    def flat(x, tail):
        x = _f64(x)
        return None if x is None else x.reshape((T,) + tail)

    per_key = gate is not None and np.asarray(gate).ndim == len(lead) + 2
    gate = flat(gate, (HV, DK) if per_key else (HV,))
    if beta is not None and np.asarray(beta).shape[-1] == 1 and HV > 1:
        # (..., 1): one update rate per token for every value head
        beta = np.broadcast_to(np.asarray(beta), lead + (HV,))
    beta = flat(beta, (HV,))
    erase = flat(erase, (HV, DK))
    cu = _i32(cu_seqlens)
    sl = _i32(slot_ids)
    lens = _i32(seq_lens)

    if cu is not None:
        if rank4:
            raise ValueError("cu_seqlens requires the rank-3 spelling")
        B = len(cu) - 1
        L = 0
    elif not rank4:
        if batch is None:
            if initial_state is not None:
                batch = np.asarray(initial_state).shape[0]
            elif sl is not None:
                batch = len(sl)
            elif lens is not None:
                batch = len(lens)
            else:
                batch = 1
        B = int(batch)
        if B == 0 or T % B:
            raise ValueError("uniform packing needs T % B == 0")
        L = T // B

    if slab is not None:
        state = np.array(_f64(slab), dtype=np.float64, copy=True)
        num_slots = state.shape[0]
        init = None
    else:
        state = np.zeros((B, HV, DV, DK), dtype=np.float64)
        num_slots = 0
        init = _f64(initial_state)
    o = np.zeros((T, HV, DV), dtype=np.float64) if o_init is None else \
        np.array(_f64(o_init).reshape(T, HV, DV), copy=True)

    keep = [q, k, v, gate, beta, erase, cu, sl, init, o, state]
    a_log = _f64(a_log)
    dt_bias = _f64(dt_bias)
    gscale = _f64(gate_scale)
    keep += [a_log, dt_bias, gscale, lens]
    p = _Problem(
        T=T, B=B, L=L, H=H, HV=HV, DK=DK, DV=DV,
        rule=RULES[update_rule],
        gate_qwen=int(gate_activation == "qwen"),
        beta_sigmoid=int(beta_activation == "sigmoid"),
        qk_l2_norm=int(bool(qk_l2_norm)),
        per_key=int(per_key),
        erase_value_axis=int(erase_axis == "value"),
        num_slots=num_slots,
        row_block=int(row_block),
        scale=float(scale),
        q=_ptr(q), k=_ptr(k), v=_ptr(v), gate=_ptr(gate), beta=_ptr(beta),
        erase=_ptr(erase), a_log=_ptr(a_log), dt_bias=_ptr(dt_bias),
        cu_seqlens=_ptr(cu), slot_ids=_ptr(sl), initial_state=_ptr(init),
        o=_ptr(o), state=_ptr(state), gate_scale=_ptr(gscale), seq_lens=_ptr(lens))
    rc = (lib if lib is not None else _load()).gdro_forward(ctypes.byref(p))
    del keep
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    return o.reshape(lead + (HV, DV)), state


def gate(a, dt_bias, decay_scale, b=None, want_beta=False, lib=None):
    """Standalone gate ("com.microsoft.LinearAttentionGate", Description), fp64:
    decay = decay_scale * softplus(a + dt_bias), beta = sigmoid(b) if wanted.
    The last axis of ``a`` is the head axis (dt_bias and decay_scale have one
    entry per head).  Returns (decay, beta or None) as float64 arrays of a's
    shape."""
    a = _f64(a)
    heads = a.shape[-1] if a.ndim else 1
    dt_bias = _f64(dt_bias).reshape(-1)
    decay_scale = _f64(decay_scale).reshape(-1)
    if dt_bias.size != heads or decay_scale.size != heads:
        raise ValueError("dt_bias and decay_scale need one entry per head")
    bb = _f64(b)
    if bb is not None and bb.shape != a.shape:
        raise ValueError("b must have a's shape")
    if want_beta and bb is None:
        raise ValueError("beta requested without b")
    decay = np.zeros(a.shape, dtype=np.float64)
    beta = np.zeros(a.shape, dtype=np.float64) if want_beta else None
    rc = (lib if lib is not None else _load()).gdro_gate(
        a.size, heads, _ptr(a), _ptr(dt_bias), _ptr(decay_scale), _ptr(bb), _ptr(decay), _ptr(beta))
    if rc != 0:
        raise ValueError("oracle gate rejected the arguments (code %d)" % rc)
    return decay, beta


def max_rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| over the whole tensor (0 when both are 0)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den
