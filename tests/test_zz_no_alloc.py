"""gdr_forward_noalloc, the entry point for callers that cannot allocate:
through the C ABI it must give what gdr_forward gives with a caller
workspace (the same kernels on the same inputs: bit for bit) on consecutive
calls that share the library's scratch array, the second smaller than the
first, and refuse a problem whose workspace exceeds that array before
enqueueing anything."""
import numpy as np
import pytest

from gated_delta_rule_token_amd import workloads
from tests.gpu_helpers import TOL_CHUNKED, TOL_F16, assert_close, oracle_forward, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_token_amd import api
    api.load_library()


def _kw(case, d):
    return dict(gate=d["gate"], beta=d["beta"], erase=d["erase"], a_log=d["a_log"], dt_bias=d["dt_bias"],
                cu_seqlens=d["cu_seqlens"], initial_state=d["initial_state"], slot_ids=d["slot_ids"],
                update_rule=case["update_rule"], gate_activation=case["gate_activation"],
                beta_activation=case["beta_activation"], qk_l2_norm=case["qk_l2_norm"], scale=case["scale"])


def _both(case, tol):
    """The call through gdr_forward_noalloc and through gdr_forward, compared
    bit for bit, and the first against the oracle."""
    from gated_delta_rule_token_amd import api
    d = to_dev(case)
    kw = _kw(case, d)
    prob = api.build_problem(d["q"], d["k"], d["v"], **kw)
    algo, need = api.selected_algo(prob), api.workspace_size(prob)
    say("case %s: AUTO runs %s, workspace %d bytes" % (case["name"], algo, need))
    o1, s1 = api.forward_noalloc(d["q"], d["k"], d["v"], **kw)
    o2, s2 = api.forward(d["q"], d["k"], d["v"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2), "noalloc differs from the workspace call"
    ro, rs = oracle_forward(case)
    assert_close(o1.double().cpu().numpy(), ro, tol, "%s noalloc o" % case["name"])
    assert_close(s1.double().cpu().numpy(), rs, tol, "%s noalloc state" % case["name"])
    return need


def test_noalloc_equals_forward_on_consecutive_calls():
    base = dict(H=2, HV=4, DK=128, DV=128, dtype=np.float16, update_rule="gated_delta",
                gate_activation="qwen", beta_activation="sigmoid", qk_l2_norm=1)
    big = workloads.random_case(61, lengths=[700, 300, 500], **base)
    small = workloads.random_case(62, lengths=[200, 150], **base)
    n_big = _both(big, TOL_CHUNKED)
    n_small = _both(small, TOL_CHUNKED)  # second call, smaller input, same scratch
    assert 0 < n_small < n_big
    # the per-key form (its own record layout) in the same array
    pk = workloads.random_case(63, lengths=[400, 260], update_rule="gated_delta_v2", per_key=True,
                               **{k: v for k, v in base.items() if k not in ("update_rule", "gate_activation",
                                                                         "beta_activation")})
    assert _both(pk, TOL_CHUNKED) > 0
    # a decode step needs no workspace and goes through unchanged
    dec = workloads.random_case(64, lengths=[1] * 8, **base)
    assert _both(dec, TOL_F16) == 0


def test_noalloc_refuses_a_workspace_beyond_its_array():
    from gated_delta_rule_token_amd import api
    T, H = 32768, 16  # records of 34 KB per (chunk, head): ~300 MB of workspace
    q = torch.zeros((T, H, 128), dtype=torch.float16, device="cuda")
    v = torch.zeros((T, H, 128), dtype=torch.float16, device="cuda")
    g = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    p = api.build_problem(q, q, v, gate=g, beta=g)
    assert api.selected_algo(p) == "chunked" and api.workspace_size(p) > api.NOALLOC_SCRATCH_BYTES
    out = torch.full((T, H, 128), 5.0, dtype=torch.float16, device="cuda")
    with pytest.raises(api.GDRError, match="GDR_E_WORKSPACE"):
        api.forward_noalloc(q, q, v, gate=g, beta=g, out=out)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 5.0)), "a refused call enqueues nothing"
