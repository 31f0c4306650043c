"""GPU parity: the HIP kernels, called through the C ABI, against the fp64
oracle on the same seeded inputs.  Bar: max |gpu - ref| / max |ref| per
output tensor <= 1e-4 for fp32 activations on the recurrent kernels, 2e-3
for fp16 activations; addressing (slot ids, cu_seqlens, empty requests,
state hand-off) bit-exact between equivalent GPU calls."""
import zlib

import numpy as np
import pytest

from gated_delta_rule_token_amd import workloads
from tests.gpu_helpers import (TOL_BF16_O, TOL_CHUNKED, TOL_F16, TOL_F32, assert_close, gpu_forward, oracle_forward,
                               rel_err, say, sub_case, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_token_amd import api
    api.load_library()


def _tol(case):
    return TOL_F32 if case["act_dtype"] == "f32" else TOL_F16


def _tol_o(case):
    return TOL_BF16_O if case["act_dtype"] == "bf16" else _tol(case)


def _check_full(case, algo, what):
    say("case %s algo=%s" % (case["name"], algo))
    o, st = gpu_forward(case, algo)
    ro, rs = oracle_forward(case)
    assert_close(o, ro, _tol_o(case), "%s o" % what)
    assert_close(st, rs, _tol(case), "%s state" % what)
    return o, st


# ------------------------------------------------------------------ small cases
def test_tiny_varlen_workload():
    case = workloads.tiny_varlen()
    o, st = _check_full(case, "recurrent", "tiny_varlen")
    z = dict(case, initial_state=np.zeros((2, 4, 32, 32), np.float32))
    o2, st2 = gpu_forward(z, "recurrent")
    assert np.array_equal(o, o2) and np.array_equal(st, st2), "explicit zero state must equal absent state"


@pytest.mark.parametrize("dtype", [np.float32, np.float16], ids=["f32", "f16"])
def test_readme_usage_shape(dtype):
    _check_full(workloads.odd_shape(dtype=dtype), "recurrent", "odd dk=12 dv=9")


RULES = [("linear", False), ("gated", False), ("gated", True), ("delta", False),
         ("gated_delta", False), ("gated_delta", True), ("gated_delta_v2", False),
         ("gated_delta_v2", True)]
SHAPES = [("recurrent", 32, 32), ("recurrent", 128, 128), ("recurrent", 64, 48),
          ("recurrent", 256, 100), ("decode", 128, 128)]


@pytest.mark.parametrize("rule,per_key", RULES, ids=["%s%s" % (r, "_pk" if p else "") for r, p in RULES])
@pytest.mark.parametrize("dtype", [np.float32, np.float16], ids=["f32", "f16"])
@pytest.mark.parametrize("algo,dk,dv", SHAPES, ids=["%s_%dx%d" % s for s in SHAPES])
def test_rules_and_shapes(rule, per_key, dtype, algo, dk, dv):
    seed = zlib.crc32(("%s/%s/%d/%d/%s" % (rule, per_key, dk, dv, algo)).encode()) % 1000
    arms = {}
    if rule in ("gated", "gated_delta") and not per_key and seed % 2 == 0:
        arms["gate_activation"] = "qwen"
    if rule in ("delta", "gated_delta") and seed % 3 != 0:
        arms["beta_activation"] = "sigmoid"
    # several staged token blocks, a ragged tail, a one-token and an empty request
    lengths = [70, 1, 0, 33] if algo == "recurrent" else [1, 3, 0, 8, 1]
    case = workloads.random_case(seed, lengths=lengths, H=2, HV=4, DK=dk, DV=dv, dtype=dtype,
                                 update_rule=rule, per_key=per_key, qk_l2_norm=seed % 2,
                                 unit_keys=True, **arms)
    _check_full(case, algo, "%s %s %s" % (rule, algo, dtype.__name__))


def test_gqa_ratio_and_scale():
    case = workloads.random_case(7, lengths=[40, 9], H=2, HV=8, DK=128, DV=64,
                                 update_rule="gated_delta", beta_activation="sigmoid")
    case["scale"] = 0.37
    _check_full(case, "recurrent", "HV/H=4 explicit scale")


def test_decode_kernel_multi_token_requests():
    case = workloads.random_case(11, rank4_batch=(16, 4), H=4, HV=8, DK=128, DV=128,
                                 dtype=np.float16, update_rule="gated_delta",
                                 gate_activation="qwen", beta_activation="sigmoid",
                                 slots=(40,))
    _check_full(case, "decode", "decode L=4 slab")


@pytest.mark.parametrize("rule,per_key", [("gated_delta", False), ("gated_delta_v2", True)],
                         ids=["gated_delta_qwen", "gated_delta_v2_pk"])
def test_decode_kernel_staged_token_blocks(rule, per_key):
    """The decode kernel forced on varlen requests of 0 to 20 tokens: the
    token inputs go through LDS in blocks of 8, so requests cross one, two or
    three blocks, with a ragged last block and an empty request."""
    kw = dict(gate_activation="none" if per_key else "qwen",
              beta_activation="none" if per_key else "sigmoid")
    case = workloads.random_case(zlib.crc32(("stage/" + rule).encode()) % 1000,
                                 lengths=[1, 8, 9, 0, 16, 20, 5, 17], H=2, HV=4, DK=128, DV=128,
                                 dtype=np.float16, update_rule=rule, per_key=per_key, **kw)
    _check_full(case, "decode", "decode staged %s" % rule)


# ------------------------------------------------------------------ the five workloads, full size
def test_decode_workload_full():
    case = workloads.decode_slab()
    d = to_dev(case)
    slab0 = d["slab"].clone()
    say("case %s: decode kernel" % case["name"])
    o, new_slab = gpu_forward(case, "auto", dev=d)
    ids = case["slot_ids"]
    gath = dict(case, slab=None, slot_ids=None, initial_state=case["slab"][ids])
    ro, rs = oracle_forward(gath)
    assert_close(o, ro, TOL_F16, "decode o")
    assert_close(new_slab[ids], rs, TOL_F16, "decode slab rows")
    untouched = np.setdiff1d(np.arange(case["slab"].shape[0]), ids)
    assert np.array_equal(new_slab[untouched], case["slab"][untouched].astype(np.float64)), \
        "untouched slots must be bit-identical"
    # the rank-3 spelling with cu_seqlens = [0, 1, ..., B] is the same call
    B = len(ids)
    r3 = dict(case, q=case["q"].reshape(B, 16, 128), k=case["k"].reshape(B, 16, 128),
              v=case["v"].reshape(B, 32, 128), gate=case["gate"].reshape(B, 32),
              beta=case["beta"].reshape(B, 32), cu_seqlens=np.arange(B + 1, dtype=np.int32))
    o3, slab3 = gpu_forward(r3, "auto")
    assert np.array_equal(o3.reshape(o.shape), o) and np.array_equal(slab3, new_slab)
    # the recurrent kernel on the same step agrees with the oracle too
    o4, slab4 = gpu_forward(case, "recurrent")
    assert_close(o4, ro, TOL_F16, "decode via recurrent o")
    assert_close(slab4[ids], rs, TOL_F16, "decode via recurrent slab rows")
    del slab0


def _sampled(case, algo, pairs, tol, label, tol_state=None):
    tol_state = tol if tol_state is None else tol_state
    say("case %s algo=%s (GPU full, oracle on %d sampled request-head pairs)" % (case["name"], algo, len(pairs)))
    o, st = gpu_forward(case, algo)
    T = o.shape[0] * (o.shape[1] if o.ndim == 4 else 1)
    of = o.reshape(T, o.shape[-2], o.shape[-1])
    for b, heads in pairs:
        sc, (s, e) = sub_case(case, b, heads)
        ro, rs = oracle_forward(sc)
        assert_close(of[s:e][:, heads], ro, tol, "%s o req %d heads %s" % (label, b, heads))
        assert_close(st[b][heads], rs[0], tol_state, "%s state req %d heads %s" % (label, b, heads))


def test_decode_workload_four_tokens_per_request():
    """The decode step at its full shape with 4 tokens per request (the
    multi-token verify shape): AUTO keeps the decode kernel, which holds the
    state rows in registers across the tokens."""
    case = workloads.decode_slab(L=4)
    say("case %s: decode kernel, 4 tokens per request" % case["name"])
    o, new_slab = gpu_forward(case, "auto")
    ids = case["slot_ids"]
    gath = dict(case, slab=None, slot_ids=None, initial_state=case["slab"][ids])
    ro, rs = oracle_forward(gath)
    assert_close(o, ro, TOL_F16, "decode L=4 o")
    assert_close(new_slab[ids], rs, TOL_F16, "decode L=4 slab rows")
    untouched = np.setdiff1d(np.arange(case["slab"].shape[0]), ids)
    assert np.array_equal(new_slab[untouched], case["slab"][untouched].astype(np.float64))


def test_varlen_prefill_workload_full():
    case = workloads.varlen_prefill()
    _sampled(case, "recurrent", [(0, [0, 31]), (3, [5]), (7, [16, 17])], TOL_F16, "varlen")


def test_long_prefill_workload_full_recurrent():
    case = workloads.long_prefill()
    _sampled(case, "recurrent", [(0, [0]), (0, [11])], TOL_F16, "long")


def test_perkey_erase_workload_full():
    case = workloads.perkey_erase()
    _sampled(case, "recurrent", [(0, [0, 3]), (3, [31])], TOL_F16, "perkey+erase")


# ------------------------------------------------------------------ bit-exact addressing
def _small(seed, **kw):
    base = dict(H=2, HV=4, DK=128, DV=128, dtype=np.float16, update_rule="gated_delta",
                gate_activation="qwen", beta_activation="sigmoid", qk_l2_norm=1)
    base.update(kw)
    return workloads.random_case(seed, **base)


@pytest.mark.parametrize("algo", ["recurrent", "decode"])
def test_slots_equal_gather_scatter(algo):
    case = _small(21, rank4_batch=(6, 5), slots=(13,))
    o, slab = gpu_forward(case, algo)
    ids = case["slot_ids"]
    g = dict(case, slab=None, slot_ids=None, initial_state=case["slab"][ids])
    o2, st2 = gpu_forward(g, algo)
    assert np.array_equal(o, o2)
    assert np.array_equal(slab[ids], st2)
    rest = np.setdiff1d(np.arange(13), ids)
    assert np.array_equal(slab[rest], case["slab"][rest].astype(np.float64))


@pytest.mark.parametrize("tokens", [1, 3])
def test_decode_step_replays_in_a_hip_graph(tokens):
    """A decode step on a slot slab (updated in place), captured once in a HIP
    graph the way a serving loop would, and replayed: after every replay the
    output and the slab equal the same step run eagerly on a second copy, with
    eager work and synchronisations between the replays."""
    import torch
    from gated_delta_rule_token_amd import api
    case = _small(41 + tokens, rank4_batch=(6, tokens), slots=(11,))
    d = to_dev(case)
    common = dict(gate=d["gate"], beta=d["beta"], a_log=d["a_log"], dt_bias=d["dt_bias"],
                  slot_ids=d["slot_ids"], update_rule=case["update_rule"],
                  gate_activation=case["gate_activation"], beta_activation=case["beta_activation"],
                  qk_l2_norm=case["qk_l2_norm"], scale=case["scale"], algo="decode")
    slab_e, slab_g = d["slab"].clone(), d["slab"].clone()
    eager = api.prepare(d["q"], d["k"], d["v"], state=slab_e, **common)
    graphed = api.prepare(d["q"], d["k"], d["v"], state=slab_g, **common)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.run()
    torch.cuda.synchronize()
    assert torch.equal(slab_g, d["slab"]), "capture must not run the step"
    for i in range(4):
        eager.run()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(graphed.o, eager.o), "replay %d: o differs from the eager step" % i
        assert torch.equal(slab_g, slab_e), "replay %d: slab differs from the eager step" % i
        if i == 0:
            # one step from the input slab: the fp64 oracle's step
            ro, rs = oracle_forward(case)
            assert_close(graphed.o.double().cpu().numpy(), ro, TOL_F16, "graph replay o")
            assert_close(slab_g.double().cpu().numpy(), rs, TOL_F16, "graph replay slab")


def test_out_of_range_slot_is_skipped():
    case = _small(22, rank4_batch=(4, 3), slots=(9,))
    case["slot_ids"] = np.array([2, 9, -1, 5], dtype=np.int32)
    d = to_dev(case)
    sentinel = torch.full((4, 3, 4, 128), 7.0, dtype=torch.float16, device="cuda")
    o, slab = gpu_forward(case, "recurrent", dev=d, out=sentinel)
    assert np.all(o[1] == 7.0) and np.all(o[2] == 7.0), "skipped requests write no output"
    for s in (0, 1, 3, 4, 6, 7, 8):
        assert np.array_equal(slab[s], case["slab"][s].astype(np.float64))
    ro, rs = oracle_forward(case)
    assert_close(o[[0, 3]], ro[[0, 3]], TOL_F16, "valid requests o")


def test_packed_equals_separate_and_empty_copies():
    case = _small(23, lengths=[37, 0, 64, 5], DV=64)
    o, st = gpu_forward(case, "recurrent")
    cu = case["cu_seqlens"]
    for b in range(4):
        s, e = int(cu[b]), int(cu[b + 1])
        sc, _ = sub_case(case, b, [0, 1, 2, 3])
        sc["q"], sc["k"] = case["q"][s:e], case["k"][s:e]  # keep the grouped q/k heads
        ob, sb = gpu_forward(sc, "recurrent")
        assert np.array_equal(o[s:e], ob), "request %d o differs when run alone" % b
        assert np.array_equal(st[b], sb[0]), "request %d state differs when run alone" % b
    assert np.array_equal(st[1], case["initial_state"][1].astype(np.float64)), "empty request copies its state"


def test_clamped_cu_seqlens():
    case = _small(24, lengths=[10, 10, 10], DV=32)
    case["cu_seqlens"] = np.array([0, 12, 7, 1000], dtype=np.int32)
    o, st = gpu_forward(case, "recurrent")
    ro, rs = oracle_forward(case)
    assert_close(st, rs, TOL_F16, "clamped cu_seqlens states")
    assert np.array_equal(st[1], case["initial_state"][1].astype(np.float64))


@pytest.mark.parametrize("split", [1, 31, 32, 45])
def test_resume_split_is_bit_exact(split):
    case = _small(25, lengths=[90], DV=64)
    o, st = gpu_forward(case, "recurrent")
    a = dict(case, q=case["q"][:split], k=case["k"][:split], v=case["v"][:split],
             gate=case["gate"][:split], beta=case["beta"][:split],
             cu_seqlens=np.array([0, split], np.int32))
    oa, sa = gpu_forward(a, "recurrent")
    b = dict(case, q=case["q"][split:], k=case["k"][split:], v=case["v"][split:],
             gate=case["gate"][split:], beta=case["beta"][split:],
             cu_seqlens=np.array([0, 90 - split], np.int32), initial_state=sa.astype(np.float32))
    ob, sb = gpu_forward(b, "recurrent")
    assert np.array_equal(np.concatenate([oa, ob]), o)
    assert np.array_equal(sb, st)


def test_deterministic():
    case = workloads.varlen_prefill(lengths=[700, 300])
    a = gpu_forward(case, "recurrent")
    b = gpu_forward(case, "recurrent")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rule_reduction_gated_delta_zero_gate():
    # fp32 activations so the comparison is not blurred by fp16 output rounding;
    # the two paths differ only in fp32 rounding of the (exactly 1) decay
    case = _small(26, lengths=[50], DV=32, gate_activation="none", dtype=np.float32)
    case["gate"] = np.zeros_like(case["gate"])
    a = gpu_forward(case, "recurrent")
    b = gpu_forward(dict(case, gate=None, update_rule="delta"), "recurrent")
    assert_close(a[0], b[0], 1e-5, "gated_delta(g=0) vs delta o")
    assert_close(a[1], b[1], 1e-5, "gated_delta(g=0) vs delta state")


# ------------------------------------------------------------------ standalone gate
@pytest.mark.parametrize("dtype", [np.float32, np.float16, "bf16"], ids=["f32", "f16", "bf16"])
def test_gate_kernel(dtype):
    """gdr_gate ("com.microsoft.LinearAttentionGate") against the oracle's
    fp64 gate on the same inputs, including far softplus / sigmoid tails.
    Bound per element, relative: the one rounding of the store (2^-24 for
    f32, 2^-11 for f16, 2^-8 for bf16) plus the fp32 arithmetic before it --
    the argument x = a + dt_bias (or b) rounds once, and softplus(x) and
    sigmoid(x) carry that relative error times up to |x| (their relative
    condition numbers), plus a few ulps of exp / log1p / the scale product:
    (|x| + 4) 2^-24.  Absolute: f16's subnormal spacing 2^-24 for values
    that small."""
    import oracle
    from gated_delta_rule_token_amd import api
    rng = np.random.Generator(np.random.PCG64(31))
    a = (3 * rng.standard_normal((37, 5))).astype(np.float32 if dtype == "bf16" else dtype)
    a[0, 0], a[1, 1], a[2, 2], a[3, 3] = 30.0, -30.0, 40.0, -40.0
    b = rng.standard_normal((37, 5)).astype(np.float32 if dtype == "bf16" else dtype)
    b[4, 4], b[5, 0] = 40.0, -40.0
    if dtype == "bf16":
        a, b = workloads.bf16_grid(a), workloads.bf16_grid(b)
    dt_bias = rng.uniform(0, 1, 5).astype(np.float32)
    dscale = -np.exp(np.log(rng.uniform(1, 16, 5))).astype(np.float32)
    tt = lambda x: torch.from_numpy(x).cuda()
    ta = (lambda x: tt(x).to(torch.bfloat16)) if dtype == "bf16" else tt
    decay, beta = api.gate(ta(a), tt(dt_bias), tt(dscale), b=ta(b), want_beta=True)
    ref_decay, ref_beta = oracle.gate(a, dt_bias, dscale, b=b, want_beta=True)
    store = {np.float32: 2.0 ** -24, np.float16: 2.0 ** -11, "bf16": 2.0 ** -8}[dtype]
    tiny = {np.float32: 1e-38, np.float16: 2.0 ** -24, "bf16": 1e-38}[dtype]
    x_decay = np.abs(a.astype(np.float64) + dt_bias.astype(np.float64))
    x_beta = np.abs(b.astype(np.float64))
    for got, ref, x, what in ((decay, ref_decay, x_decay, "decay"), (beta, ref_beta, x_beta, "beta")):
        got = got.double().cpu().numpy()
        bound = (store + (x + 4.0) * 2.0 ** -24) * np.abs(ref) + tiny
        worst = float(np.max(np.abs(got - ref) / bound))
        say("  gate %s %s: worst error %.3f of the bound" % (dtype if isinstance(dtype, str) else dtype.__name__,
                                                           what, worst))
        assert worst <= 1.0, "%s off the oracle by more than one store rounding" % what


# ------------------------------------------------------------------ slab stream
@pytest.mark.parametrize("shape", [(12, 3, 16, 20), (6, 2, 128, 128)], ids=["ragged", "d128"])
def test_slab_stream_touches_only_addressed_rows(shape):
    """gdr_slab_stream scales exactly the addressed state matrices (every head
    of slab[slot_ids[b]]) by the factor -- one fp32 multiply per element, so
    bit for bit what torch's fp32 multiply gives -- and leaves every other
    slot, and requests with a slot id outside [0, num_slots), untouched.
    Covers a matrix that is not a whole number of 16 KB pieces (320 floats)
    and one of four pieces (128 x 128)."""
    from gated_delta_rule_token_amd import api
    g = torch.Generator().manual_seed(5)
    slab = torch.randn(shape, generator=g).cuda()
    before = slab.clone()
    n = shape[0]
    ids = torch.tensor([n - 1, -1, 2, 0, n, 2 * n], dtype=torch.int32).cuda()
    api.slab_stream(slab, ids, 1.5)
    torch.cuda.synchronize()
    want = before.clone()
    for s in (n - 1, 2, 0):
        want[s] = before[s] * 1.5
    assert torch.equal(slab, want)
    api.slab_stream(slab, ids, 1.0)  # factor 1 leaves the values as they are
    torch.cuda.synchronize()
    assert torch.equal(slab, want)


# ------------------------------------------------------------------ chunked prefill
CHUNK_RULES = ["linear", "gated", "delta", "gated_delta"]


@pytest.mark.parametrize("rule", CHUNK_RULES)
@pytest.mark.parametrize("arms", ["plain", "qwen_sigmoid_l2"])
def test_chunked_rules(rule, arms):
    kw = {}
    if arms != "plain":
        kw["qk_l2_norm"] = 1
        if rule in ("gated", "gated_delta"):
            kw["gate_activation"] = "qwen"
        if rule in ("delta", "gated_delta"):
            kw["beta_activation"] = "sigmoid"
    # several chunks, a ragged tail, an exact multiple of 64, one token, an empty request
    case = workloads.random_case(zlib.crc32(("chunk/%s/%s" % (rule, arms)).encode()) % 1000,
                                 lengths=[200, 1, 0, 64, 130], H=2, HV=4, DK=128, DV=128,
                                 dtype=np.float16, update_rule=rule, unit_keys=(arms == "plain"), **kw)
    _check_full(case, "chunked", "chunked %s %s" % (rule, arms))


def test_chunked_gqa_and_slab():
    case = workloads.random_case(41, rank4_batch=(3, 150), H=2, HV=8, DK=128, DV=128,
                                 dtype=np.float16, update_rule="gated_delta",
                                 gate_activation="qwen", beta_activation="sigmoid", slots=(7,))
    say("case chunked slab")
    o, slab = gpu_forward(case, "chunked")
    ro, rs = oracle_forward(case)
    assert_close(o, ro, TOL_CHUNKED, "chunked slab o")
    ids = case["slot_ids"]
    assert_close(slab[ids], rs[ids], TOL_CHUNKED, "chunked slab rows")
    rest = np.setdiff1d(np.arange(7), ids)
    assert np.array_equal(slab[rest], case["slab"][rest].astype(np.float64))


def test_chunked_matches_recurrent():
    case = workloads.varlen_prefill(lengths=[700, 65, 300])
    a = gpu_forward(case, "chunked")
    b = gpu_forward(case, "recurrent")
    assert_close(a[0], b[0], TOL_CHUNKED, "chunked vs recurrent o")
    assert_close(a[1], b[1], TOL_CHUNKED, "chunked vs recurrent state")


def test_chunked_deterministic():
    case = workloads.varlen_prefill(lengths=[333, 129])
    a = gpu_forward(case, "chunked")
    b = gpu_forward(case, "chunked")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _mild(case, seed, per_key=False):
    """Weak decay and small update rates (input recipe only), so that a long
    segment's transition matrix stays far from zero and a mistake in how the
    segments are composed shows in the result."""
    rng = workloads.rng_for(seed)
    lead = case["v"].shape[:-2]
    HV = case["v"].shape[-2]
    if case["gate"] is not None:
        shape = lead + ((HV, case["k"].shape[-1]) if per_key else (HV,))
        case["gate"] = (-0.001 * rng.random(shape)).astype(np.float32)
        case["gate_activation"], case["a_log"], case["dt_bias"] = "none", None, None
    if case["beta"] is not None:
        case["beta"] = (0.01 + 0.05 * rng.random(lead + (HV,))).astype(np.float32)
        case["beta_activation"] = "none"
    if case["erase"] is not None:
        case["erase"] = (0.05 * rng.random(case["erase"].shape)).astype(np.float32)
    for key in ("initial_state", "slab"):
        if case[key] is not None:
            case[key] = case[key] * np.float32(10.0)
    return case


def _start_matters(case, label):
    # the final state must depend on the initial state, or segment composition is untested
    _, rs = oracle_forward(case)
    _, rz = oracle_forward(dict(case, initial_state=None))
    d = np.max(np.abs(rs - rz)) / np.max(np.abs(rs))
    say("  %s: initial state moves the final state by %.2f (relative)" % (label, d))
    assert d > 0.05


@pytest.mark.parametrize("nseg", [2, 3, 5, 16])
def test_chunked_segmented_scan(nseg):
    """The chain of chunk steps cut into nseg composed segments (two scan
    passes around the combine step) against the oracle and the one-pass scan,
    on one request of 38 chunks with a ragged tail."""
    case = _mild(workloads.random_case(71, lengths=[64 * 37 + 19], H=1, HV=2, DK=128, DV=128,
                                       dtype=np.float16, update_rule="gated_delta"), 72)
    if nseg == 2:
        _start_matters(case, "segmented scan")
    say("case segmented scan nseg=%d" % nseg)
    o, st = gpu_forward(case, "chunked", scan_segments=nseg)
    ro, rs = oracle_forward(case)
    assert_close(o, ro, TOL_CHUNKED, "segmented o")
    assert_close(st, rs, TOL_CHUNKED, "segmented state")
    o1, st1 = gpu_forward(case, "chunked", scan_segments=1)
    assert_close(o, o1, TOL_CHUNKED, "segmented vs one pass o")
    assert_close(st, st1, TOL_CHUNKED, "segmented vs one pass state")
    assert np.array_equal(gpu_forward(case, "chunked", scan_segments=nseg)[1], st), "deterministic"


@pytest.mark.parametrize("nseg,per_key", [(4, False), (5, False), (5, True)])
def test_chunked_segmented_wide_pass1(nseg, per_key):
    """16 (request, head) pairs in 4 or 5 segments: pass 1 then runs in 64-row
    tiles (192 or 256 workgroups), per head and per key, against the oracle
    and the one-pass scan."""
    rule = "gated_delta_v2" if per_key else "gated_delta"
    case = _mild(workloads.random_case(80 + nseg + 2 * per_key, lengths=[64 * 26 + 41], H=4, HV=16, DK=128,
                                       DV=128, dtype=np.float16, update_rule=rule, per_key=per_key),
                 86, per_key=per_key)
    say("case segmented scan, 64-row pass 1: nseg=%d per_key=%s" % (nseg, per_key))
    o, st = gpu_forward(case, "chunked", scan_segments=nseg)
    ro, rs = oracle_forward(case)
    assert_close(o, ro, TOL_CHUNKED, "wide pass 1 o")
    assert_close(st, rs, TOL_CHUNKED, "wide pass 1 state")
    o1, st1 = gpu_forward(case, "chunked", scan_segments=1)
    assert_close(st, st1, TOL_CHUNKED, "wide pass 1 vs one pass state")


@pytest.mark.parametrize("rule", ["linear", "gated", "delta", "gated_delta"])
def test_chunked_segmented_varlen_slab(rule):
    """Segmented scans over varlen requests in a slot slab: requests shorter
    than the segment count (empty segments), an empty request, a ragged tail,
    an out-of-range slot (skipped: no output, no state touched)."""
    case = _mild(workloads.random_case(zlib.crc32(("seg/" + rule).encode()) % 1000,
                                       lengths=[700, 0, 5, 130, 1500], H=2, HV=4, DK=128, DV=128,
                                       dtype=np.float16, update_rule=rule, slots=(9,)), 73)
    ids = case["slot_ids"].copy()
    ids[3] = 9  # out of range
    case["slot_ids"] = ids
    d = to_dev(case)
    T = case["q"].shape[0]
    sentinel = torch.full((T, 4, 128), 7.0, dtype=torch.float16, device="cuda")
    say("case segmented varlen slab %s" % rule)
    o, slab = gpu_forward(case, "chunked", dev=d, out=sentinel, scan_segments=3)
    cu = case["cu_seqlens"]
    assert np.all(o[cu[3]:cu[4]] == 7.0), "the skipped request writes no output"
    keep = np.setdiff1d(np.arange(9), ids[[0, 1, 2, 4]])
    assert np.array_equal(slab[keep], case["slab"][keep].astype(np.float64)), "unaddressed slots untouched"
    ro, rs = oracle_forward(case)
    rows = np.r_[cu[0]:cu[3], cu[4]:cu[5]]
    assert_close(o[rows], ro[rows], TOL_CHUNKED, "segmented varlen o")
    live = ids[[0, 1, 2, 4]]
    assert_close(slab[live], rs[live], TOL_CHUNKED, "segmented varlen slab rows")
    assert np.array_equal(slab[ids[1]], case["slab"][ids[1]].astype(np.float64)), "empty request copies its state"


@pytest.mark.parametrize("rule", ["gated_delta", "gated_delta_v2"])
def test_chunked_segmented_per_key(rule):
    """The per-key chunked form (decay per key channel; the erase gate) with
    a segmented scan."""
    case = _mild(workloads.random_case(74 if rule == "gated_delta" else 75, lengths=[64 * 21 + 33, 400],
                                       H=1, HV=2, DK=128, DV=128, dtype=np.float16,
                                       update_rule=rule, per_key=True), 76, per_key=True)
    _start_matters(case, "per-key segmented scan")
    say("case segmented per-key %s" % rule)
    o, st = gpu_forward(case, "chunked", scan_segments=4)
    ro, rs = oracle_forward(case)
    assert_close(o, ro, TOL_CHUNKED, "segmented per-key o")
    assert_close(st, rs, TOL_CHUNKED, "segmented per-key state")


def test_long_prefill_workload_full_chunked():
    case = workloads.long_prefill()
    _sampled(case, "chunked", [(0, [0]), (0, [7]), (0, [15])], TOL_CHUNKED, "long chunked")


def test_varlen_prefill_workload_full_chunked():
    case = workloads.varlen_prefill()
    _sampled(case, "chunked", [(0, [0, 31]), (2, [9]), (5, [20, 21])], TOL_CHUNKED, "varlen chunked")


# ------------------------------------------------------------------ chunked prefill, per-key form
PK_RULES = [("gated_delta", True), ("gated", True), ("gated_delta_v2", True), ("gated_delta_v2", False)]


@pytest.mark.parametrize("rule,per_key", PK_RULES, ids=["%s%s" % (r, "_pk" if p else "") for r, p in PK_RULES])
@pytest.mark.parametrize("arms", ["plain", "sigmoid_l2"])
def test_chunked_per_key_rules(rule, per_key, arms):
    kw = {}
    if arms != "plain":
        kw["qk_l2_norm"] = 1
        if rule == "gated_delta":
            kw["beta_activation"] = "sigmoid"
    case = workloads.random_case(zlib.crc32(("chunkpk/%s/%d/%s" % (rule, per_key, arms)).encode()) % 1000,
                                 lengths=[200, 1, 0, 64, 130], H=2, HV=4, DK=128, DV=128,
                                 dtype=np.float16, update_rule=rule, per_key=per_key,
                                 unit_keys=(arms == "plain"), **kw)
    _check_full(case, "chunked", "chunked per-key %s%s %s" % (rule, "_pk" if per_key else "", arms))


@pytest.mark.parametrize("rule", ["gated_delta", "gated_delta_v2"])
def test_chunked_per_key_strong_decay(rule):
    """Channels that decay by 8 nats per token exceed the bound the chunk
    prologue's block split allows inside a 16-token block, so those diagonal
    blocks are summed term by term; the rest of the channels stay mild."""
    case = workloads.random_case(77, lengths=[150, 64, 37], H=2, HV=4, DK=128, DV=128,
                                 dtype=np.float16, update_rule=rule, per_key=True)
    g = case["gate"].copy()
    g[:, :, ::5] = -8.0
    g[:90, 1, 3::7] = -0.001
    case["gate"] = g
    _check_full(case, "chunked", "chunked per-key strong decay %s" % rule)


def test_chunked_per_key_growing_channels():
    """Channels whose log decay alternates +5 / -5 per token grow by more than
    80 nats inside a chunk in total (while their state stays bounded), which
    sends every Gram block of those chunks to the term-by-term path."""
    case = workloads.random_case(78, lengths=[150, 70], H=2, HV=4, DK=128, DV=128,
                                 dtype=np.float16, update_rule="gated_delta_v2", per_key=True)
    g = case["gate"].copy()
    sign = np.where(np.arange(g.shape[0]) % 2 == 0, 5.0, -5.0).astype(np.float32)
    g[:, :, 3::9] = sign[:, None, None]
    case["gate"] = g
    _check_full(case, "chunked", "chunked per-key growing channels")


def test_chunked_per_key_gqa_and_slab():
    case = workloads.random_case(43, rank4_batch=(3, 150), H=2, HV=8, DK=128, DV=128,
                                 dtype=np.float16, update_rule="gated_delta_v2", per_key=True,
                                 slots=(7,))
    say("case chunked per-key slab")
    o, slab = gpu_forward(case, "chunked")
    ro, rs = oracle_forward(case)
    assert_close(o, ro, TOL_CHUNKED, "chunked per-key slab o")
    ids = case["slot_ids"]
    assert_close(slab[ids], rs[ids], TOL_CHUNKED, "chunked per-key slab rows")
    rest = np.setdiff1d(np.arange(7), ids)
    assert np.array_equal(slab[rest], case["slab"][rest].astype(np.float64))


def test_chunked_per_key_matches_recurrent_and_is_deterministic():
    case = workloads.perkey_erase(B=2, L=700)
    a = gpu_forward(case, "chunked")
    b = gpu_forward(case, "recurrent")
    assert_close(a[0], b[0], TOL_CHUNKED, "per-key chunked vs recurrent o")
    assert_close(a[1], b[1], TOL_CHUNKED, "per-key chunked vs recurrent state")
    c = gpu_forward(case, "chunked")
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def test_perkey_erase_workload_full_chunked():
    case = workloads.perkey_erase()
    _sampled(case, "chunked", [(0, [0, 3]), (2, [17]), (3, [31])], TOL_CHUNKED, "perkey+erase chunked")


# ------------------------------------------------------------------ raw per-key gate, folded scale, seq_lens
# (CLIKA "gatedDeltaUpdate": gate_bias [HV, K] beside a [B, T, HV, K] gate,
# gate_scale = the once-folded -exp(A_log), seq_lens bounding ragged rows)
RAW_GATE_CASES = [("decode", 1), ("recurrent", 70), ("chunked", 150)]


@pytest.mark.parametrize("algo,L", RAW_GATE_CASES, ids=[c[0] for c in RAW_GATE_CASES])
@pytest.mark.parametrize("rule", ["gated_delta", "gated_delta_v2"])
def test_per_key_raw_gate_folded_scale(algo, L, rule):
    case = workloads.random_case(zlib.crc32(("rawpk/%s/%s" % (algo, rule)).encode()) % 1000,
                                 rank4_batch=(3, L), H=2, HV=4, DK=128, DV=128, dtype=np.float16,
                                 update_rule=rule, per_key=True, gate_activation="qwen",
                                 beta_activation="sigmoid" if rule == "gated_delta" else "none",
                                 folded_scale=True)
    assert case["gate"].dtype == np.float16 and case["dt_bias"].shape == (4, 128)
    _check_full(case, algo, "per-key raw gate %s %s" % (rule, algo))


SEQ_LEN_CASES = [("decode", 6, [6, 0, 3, 9]), ("recurrent", 90, [90, 1, 0, 37]),
                 ("chunked", 200, [200, 64, 0, 129]), ("chunked_pk", 200, [130, 0, 199, 65])]


@pytest.mark.parametrize("algo,L,lens", SEQ_LEN_CASES, ids=[c[0] for c in SEQ_LEN_CASES])
def test_seq_lens_bound_uniform_requests(algo, L, lens):
    per_key = algo == "chunked_pk"
    case = workloads.random_case(zlib.crc32(("seqlens/%s" % algo).encode()) % 1000,
                                 rank4_batch=(4, L), H=2, HV=4, DK=128, DV=128, dtype=np.float16,
                                 update_rule="gated_delta_v2" if per_key else "gated_delta",
                                 per_key=per_key, gate_activation="none" if per_key else "qwen",
                                 beta_activation="none" if per_key else "sigmoid",
                                 seq_lens=lens, slots=(9,) if algo == "decode" else None)
    import torch
    sentinel = np.full(case["v"].shape, 3.0, dtype=np.float16)
    out = torch.from_numpy(sentinel.copy()).cuda()
    say("case %s seq_lens %s" % (case["name"], lens))
    o, st = gpu_forward(case, "chunked" if per_key else algo, out=out)
    ro, rs = oracle_forward(case, o_init=sentinel)
    assert_close(o, ro, TOL_F16 if algo in ("decode", "recurrent") else TOL_CHUNKED, "seq_lens o")
    if case["slab"] is not None:
        ids = case["slot_ids"]
        assert_close(st[ids], rs[ids], TOL_F16, "seq_lens slab rows")
    else:
        assert_close(st, rs, TOL_F16 if algo == "recurrent" else TOL_CHUNKED, "seq_lens state")
    for b, n in enumerate(lens):
        n = min(max(n, 0), L)
        assert np.all(o[b, n:] == 3.0), "rows past seq_lens[%d] must stay unwritten" % b
    if case["initial_state"] is not None:
        z = lens.index(0)
        assert np.array_equal(st[z], case["initial_state"][z].astype(np.float64)), \
            "a zero-length request copies its state"


# beta (..., 1): one update rate per token for every value head (the ONNX
# issue quotes LinearAttention's schema: beta's last axis in {kv_num_heads, 1})
BETA_TOK_CASES = [("decode", 2, False), ("recurrent", 50, False), ("chunked", 140, False),
                  ("chunked", 140, True)]


@pytest.mark.parametrize("algo,L,per_key", BETA_TOK_CASES,
                         ids=["%s%s" % (c[0], "_pk" if c[2] else "") for c in BETA_TOK_CASES])
def test_beta_one_per_token(algo, L, per_key):
    case = workloads.random_case(zlib.crc32(("betatok/%s/%d" % (algo, per_key)).encode()) % 1000,
                                 rank4_batch=(3, L), H=2, HV=4, DK=128, DV=128, dtype=np.float16,
                                 update_rule="gated_delta", per_key=per_key,
                                 beta_activation="sigmoid")
    case["beta"] = np.ascontiguousarray(case["beta"][..., :1])
    assert case["beta"].shape == (3, L, 1)
    _check_full(case, algo, "beta per token %s%s" % (algo, " per-key" if per_key else ""))


# ------------------------------------------------------------------ bf16 activations
# (beyond the pages' type list; loads widen bf16 exactly, o is rounded on store)
BF16_CASES = [("decode", 128, 128, 2), ("recurrent", 128, 128, 70), ("recurrent", 64, 48, 33)]


@pytest.mark.parametrize("algo,dk,dv,L", BF16_CASES, ids=["%s_%dx%d" % c[:3] for c in BF16_CASES])
@pytest.mark.parametrize("rule,per_key", [("gated_delta", False), ("gated_delta_v2", True)],
                         ids=["gated_delta_qwen", "gated_delta_v2_pk"])
def test_bf16_activations(algo, dk, dv, L, rule, per_key):
    case = workloads.random_case(zlib.crc32(("bf16/%s/%d/%s" % (algo, dk, rule)).encode()) % 1000,
                                 rank4_batch=(3, L), H=2, HV=4, DK=dk, DV=dv, dtype="bf16",
                                 update_rule=rule, per_key=per_key,
                                 gate_activation="none" if per_key else "qwen",
                                 beta_activation="none" if per_key else "sigmoid", qk_l2_norm=1)
    _check_full(case, algo, "bf16 %s %s" % (rule, algo))


BF16_CHUNK_RULES = [("linear", False), ("gated", False), ("gated", True), ("delta", False),
                    ("gated_delta", False), ("gated_delta", True), ("gated_delta_v2", False),
                    ("gated_delta_v2", True)]


@pytest.mark.parametrize("rule,per_key", BF16_CHUNK_RULES,
                         ids=["%s%s" % (r, "_pk" if k else "") for r, k in BF16_CHUNK_RULES])
def test_bf16_chunked(rule, per_key):
    """bf16 activations on the chunked kernels (every rule takes the per-key
    form): several chunks, a ragged tail, one token, an empty request; raw
    gate in bf16 and sigmoid update rate where the rule has them."""
    kw = dict(qk_l2_norm=1)
    if rule in ("gated", "gated_delta", "gated_delta_v2") and not per_key:
        kw["gate_activation"] = "qwen"
    if rule in ("delta", "gated_delta"):
        kw["beta_activation"] = "sigmoid"
    case = workloads.random_case(zlib.crc32(("bf16chunk/%s/%d" % (rule, per_key)).encode()) % 1000,
                                 lengths=[200, 1, 0, 64, 130], H=2, HV=4, DK=128, DV=128, dtype="bf16",
                                 update_rule=rule, per_key=per_key, **kw)
    o, st = _check_full(case, "chunked", "bf16 chunked %s" % rule)
    o2, st2 = gpu_forward(case, "recurrent")
    # each side rounds o to bf16 on its own, so the two may differ by both roundings
    assert_close(o, o2, 2 * TOL_BF16_O, "bf16 chunked vs recurrent o")
    assert_close(st, st2, TOL_CHUNKED, "bf16 chunked vs recurrent state")


def test_bf16_chunked_segmented():
    """bf16 on the chunked kernels with the chain cut into segments."""
    case = _mild(workloads.random_case(77, lengths=[64 * 30 + 5], H=1, HV=2, DK=128, DV=128, dtype="bf16",
                                       update_rule="gated_delta"), 78)
    say("case bf16 segmented scan")
    o, st = gpu_forward(case, "chunked", scan_segments=4)
    ro, rs = oracle_forward(case)
    assert_close(o, ro, TOL_BF16_O, "bf16 segmented o")
    assert_close(st, rs, TOL_CHUNKED, "bf16 segmented state")


def test_bf16_varlen_prefill_workload_full_chunked():
    """The varlen prefill workload (8 requests, 29,273 tokens, H=16, HV=32)
    with its activations on the bf16 grid: AUTO runs the chunked kernels."""
    case = workloads.as_bf16(workloads.varlen_prefill())
    _sampled(case, "auto", [(0, [0, 31]), (5, [20])], TOL_BF16_O, "bf16 varlen chunked", TOL_CHUNKED)


# ------------------------------------------------------------------ sizes past 32-bit byte offsets
def test_decode_slab_beyond_4gib():
    """A 4.3 GiB slab (2,200 slots x 32 heads x 64 KiB) addressed at slots past
    the 4 GiB mark: offsets are 64-bit, untouched slots keep their bytes."""
    import torch
    case = workloads.decode_slab(B=64, num_slots=2200, with_slab=False)
    rng = workloads.rng_for(202)
    ids = (2200 - 1 - rng.permutation(150)[:64]).astype(np.int32)   # slots 2050 .. 2199
    rows = workloads._normal(rng, (64, 32, 128, 128), np.float32, std=0.05)
    say("case decode slab 4.3 GiB, slots %d..%d" % (ids.min(), ids.max()))
    slab = torch.full((2200, 32, 128, 128), 0.25, dtype=torch.float32, device="cuda")
    slab[torch.from_numpy(ids).long().cuda()] = torch.from_numpy(rows).cuda()
    d = to_dev(dict(case, slab=None))
    d["slot_ids"] = torch.from_numpy(ids).cuda()
    d["slab"] = slab
    from gated_delta_rule_token_amd import api
    o, st = api.forward(d["q"], d["k"], d["v"], gate=d["gate"], beta=d["beta"], a_log=d["a_log"],
                        dt_bias=d["dt_bias"], slot_ids=d["slot_ids"], state=slab,
                        update_rule="gated_delta", gate_activation="qwen", beta_activation="sigmoid")
    torch.cuda.synchronize()
    ro, rs = oracle_forward(dict(case, slab=None, slot_ids=None, initial_state=rows))
    assert_close(o.double().cpu().numpy(), ro, TOL_F16, "decode 4.3 GiB slab o")
    assert_close(st[torch.from_numpy(ids).long().cuda()].double().cpu().numpy(), rs, TOL_F16,
                 "decode 4.3 GiB slab rows")
    mask = torch.ones(2200, dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(ids).long().cuda()] = False
    assert bool(torch.all(st[mask] == 0.25)), "untouched slots must keep their bytes"


def test_chunked_workspace_beyond_4gib():
    """262,144 tokens x 16 heads: a 7.6 GB chunk workspace (64-bit record
    offsets) and 1 GiB q/k/v; the oracle checks sampled heads."""
    case = workloads.long_prefill(T=262144)
    _sampled(case, "chunked", [(0, [0]), (0, [15])], TOL_CHUNKED, "chunked 262k tokens")


@pytest.mark.parametrize("algo", ["recurrent", "decode"])
def test_l2_norm_epsilon_placement(algo):
    """qk L2-norm of rows whose squared norm is the size of the epsilon
    (README, Attributes qk_l2_norm: epsilon 1e-12).  The kernels follow the
    oracle's reading x / sqrt(sum x^2 + 1e-12): a key or query scaled to
    squared norm 1e-12 normalises to length 1/sqrt(2).  x / max(|x|, 1e-12)
    would give length 1 here; the check below shows that this case tells the
    two readings apart by far more than the bar."""
    lengths = [1] * 8 if algo == "decode" else [40, 23]
    case = _small(60, lengths=lengths, dtype=np.float32)
    T = case["q"].shape[0]
    tiny = [0, T - 1]
    for arr in ("k", "q"):
        x = case[arr][tiny].astype(np.float64)
        case[arr][tiny] = (x / np.linalg.norm(x, axis=-1, keepdims=True) * 1e-6).astype(np.float32)
    say("case l2-norm epsilon placement algo=%s" % algo)
    o, st = gpu_forward(case, algo)
    ro, rs = oracle_forward(case)
    assert_close(o, ro, TOL_F32, "epsilon placement o")
    assert_close(st, rs, TOL_F32, "epsilon placement state")
    # the other reading: those rows at full length
    alt = dict(case)
    for arr in ("k", "q"):
        alt[arr] = case[arr].copy()
        x = alt[arr][tiny].astype(np.float64)
        alt[arr][tiny] = (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)
    ao, ast = oracle_forward(alt)
    assert max(rel_err(ao, ro), rel_err(ast, rs)) > 100 * TOL_F32, "the case separates the two readings"
