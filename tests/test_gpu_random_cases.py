"""Seeded random sweep of the operator contract on the GPU: update rule,
per-head or per-key decay, gate arm, update-rate activation, activation
dtype, head dimensions, grouped heads, varlen or uniform packing with
ragged lengths (empty requests included), initial state, state slab and
the kernel family (AUTO or a forced one), each case against the fp64
oracle.  The cases are drawn from fixed seeds, so every run checks the
same 128 problems (64 over every kernel family, 64 with 16-bit activations
at dk = dv = 128 on AUTO or the chunked kernels); the targeted tests
elsewhere cover each feature alone."""
import numpy as np
import pytest

from gated_delta_rule_token_amd import workloads
from tests.gpu_helpers import (TOL_BF16_O, TOL_CHUNKED, TOL_F16, TOL_F32, assert_close, gpu_forward, oracle_forward,
                               request_ranges, say)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RULES = ["linear", "gated", "delta", "gated_delta", "gated_delta_v2"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_token_amd import api
    api.load_library()


def draw(i, chunked=False):
    """Case i of the sweep: (random_case keyword arguments, algo).  With
    ``chunked`` the case has 16-bit activations, dk = dv = 128 and longer
    requests, and runs on AUTO or the chunked kernels."""
    r = np.random.default_rng((2000 if chunked else 1000) + i)
    rule = RULES[r.integers(len(RULES))]
    gated = rule in ("gated", "gated_delta", "gated_delta_v2")
    dtype = [np.float16, "bf16"][r.integers(2)] if chunked else [np.float32, np.float16, "bf16"][r.integers(3)]
    d128 = chunked or dtype != np.float32 or r.random() < 0.5
    DK, DV = (128, 128) if d128 else [(64, 48), (32, 32), (96, 128)][r.integers(3)]
    H = int(r.choice([1, 2, 4]))
    HV = H * int(r.choice([1, 2]))
    short = not chunked and d128 and r.random() < 0.25  # decode-sized requests
    B = int(r.integers(1, 6))
    lengths = r.integers(0, 9 if short else (700 if chunked else 301), size=B)
    if B > 1 and r.random() < 0.3:
        lengths[r.integers(B)] = 0
    kw = dict(H=H, HV=HV, DK=DK, DV=DV, dtype=dtype, update_rule=rule,
              gate_activation=("qwen" if gated and r.random() < 0.5 else "none"),
              beta_activation=("sigmoid" if r.random() < 0.5 else "none"),
              qk_l2_norm=int(rule in ("delta", "gated_delta", "gated_delta_v2") or r.random() < 0.5),
              per_key=bool(gated and r.random() < 0.4),
              with_initial=bool(r.random() < 0.7))
    if r.random() < 0.25:
        kw["slots"] = (B + int(r.integers(1, 4)),)
    if not short and r.random() < 0.25:
        L = int(r.integers(1, 200))
        kw["rank4_batch"] = (B, L)
        kw["seq_lens"] = r.integers(0, L + 1, size=B).tolist()
    else:
        kw["lengths"] = lengths.tolist()
    algos = ["auto", "chunked"] if chunked else ["auto", "recurrent"]
    if not chunked and d128 and dtype != np.float32:
        algos.append("chunked")
    if short:
        algos.append("decode")
    return kw, algos[r.integers(len(algos))]


@pytest.mark.parametrize("chunked", [False, True], ids=["any", "chunked"])
@pytest.mark.parametrize("i", range(64))
def test_random_case(i, chunked):
    kw, algo = draw(i, chunked)
    case = workloads.random_case(5000 + i, **kw)
    act = case["act_dtype"]
    say("random case %d: %s %s dk=%d dv=%d H=%d HV=%d per_key=%s gate=%s algo=%s" % (
        i, case["update_rule"], act, kw["DK"], kw["DV"], kw["H"], kw["HV"], kw["per_key"],
        kw["gate_activation"], algo))
    o, st = gpu_forward(case, algo)
    ro, rs = oracle_forward(case)
    tol_state = TOL_F32 if act == "f32" else (TOL_CHUNKED if algo == "chunked" else TOL_F16)
    tol_o = TOL_BF16_O if act == "bf16" else tol_state
    # o rows of the requests (rows past a request's seq_lens are the
    # caller's: left as they are, README-style output contract)
    rows = np.zeros(o.shape[0] * (o.shape[1] if o.ndim == 4 else 1), bool)
    for s, e in request_ranges(case):
        rows[s:e] = True
    flat = lambda x: x.reshape((-1,) + x.shape[-2:])
    assert_close(flat(o)[rows], flat(ro)[rows], tol_o, "case %d o" % i)
    assert_close(st, rs, tol_state, "case %d state" % i)
