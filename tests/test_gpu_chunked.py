"""GPU parity of the chunk-parallel prefill beyond the plain workloads:
requests whose cu_seqlens ranges overlap (the README's decreasing entries),
packed == separate calls, a request resumed from its own final state at and
off chunk boundaries (the state is the checkpoint: README, Inputs
initial_state and Outputs final_state), state magnitudes far from 1, and the
three prefill workloads at full size with every (request, head) pair compared
with the fp64 oracle.  Every call goes through the C ABI."""
import json
import os
import zlib

import numpy as np
import pytest

from gated_delta_rule_token_amd import workloads
from tests.gpu_helpers import (TOL_BF16_O, TOL_CHUNKED, assert_close, gpu_forward, oracle_forward, rel_err, say,
                               sub_case, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_token_amd import api
    api.load_library()


def _case(seed, lengths, **kw):
    base = dict(H=2, HV=4, DK=128, DV=128, dtype=np.float16, update_rule="gated_delta",
                gate_activation="qwen", beta_activation="sigmoid", qk_l2_norm=1)
    base.update(kw)
    return workloads.random_case(seed, lengths=lengths, **base)


def _log_errors(name, **errs):
    """Append the measured errors of a full-size check to the file named by
    GDR_PARITY_LOG (one JSON object per line), when set."""
    path = os.environ.get("GDR_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(dict(name=name, **errs)) + "\n")


# ------------------------------------------------------------------ overlapping requests
OVERLAP_CASES = [
    # three full-length requests restarting at token 0: 48 chunks against a
    # budget of 22, so requests 2 and 4 go to the recurrent kernel
    ("restart_three_times", 1024, [0, 1024, 0, 1024, 0, 1024, 0]),
    # two overlapping requests fit the budget; the last one, which no other
    # request overlaps, does not
    ("overlap_then_tail", 1100, [0, 600, 0, 600, 600, 1100, 0]),
    # out-of-range and negative entries as well
    ("out_of_range", 700, [-5, 300, 9999, 0, 700, 200, 700]),
]


@pytest.mark.parametrize("algo", ["chunked", "auto"])
@pytest.mark.parametrize("name,T,cu", OVERLAP_CASES, ids=[c[0] for c in OVERLAP_CASES])
def test_overlapping_requests(name, T, cu, algo):
    """Every request's final state matches the oracle run on that request
    alone; an output row that several requests write holds one of their
    values (which one is unspecified), every other row the oracle's."""
    B = len(cu) - 1
    case = _case(zlib.crc32(name.encode()) % 1000, [T] + [0] * (B - 1))
    case["cu_seqlens"] = np.array(cu, dtype=np.int32)
    say("case overlapping cu_seqlens %s algo=%s" % (cu, algo))
    d = to_dev(case)
    sentinel = torch.full((T, 4, 128), 3.0, dtype=torch.float16, device="cuda")
    o, st = gpu_forward(case, algo, dev=d, out=sentinel)
    HV = 4
    cover = [[] for _ in range(T)]
    refs = []
    for b in range(B):
        sc, (s, e) = sub_case(case, b, list(range(HV)))
        ro, rs = oracle_forward(sc)
        refs.append((s, e, ro))
        assert_close(st[b], rs[0], TOL_CHUNKED, "%s final state of request %d" % (name, b))
        for t in range(s, e):
            cover[t].append(b)
    scale = max(float(np.max(np.abs(ro))) for _, _, ro in refs if ro.size)
    for t in range(T):
        if not cover[t]:
            assert np.all(o[t] == 3.0), "row %d belongs to no request and must stay unwritten" % t
            continue
        err = np.min([np.abs(o[t] - refs[b][2][t - refs[b][0]]) for b in cover[t]], axis=0)
        assert np.max(err) <= TOL_CHUNKED * scale, \
            "row %d (requests %s): max err %.3e" % (t, cover[t], float(np.max(err)) / scale)


# ------------------------------------------------------------------ request order
@pytest.mark.parametrize("B", [900, 1100], ids=["ranked", "batch_order"])
def test_many_requests_any_order(B):
    """The scans take requests longest first (ranked by chunk count, ties by
    index) up to 1,024 requests and in batch order past that: ragged lengths
    0-300 with many ties, empty requests included; every request's o rows
    and final state against the oracle."""
    rng = np.random.default_rng(B)
    lengths = rng.integers(0, 301, size=B)
    lengths[rng.integers(0, B, size=B // 10)] = 0
    case = _case(52 + B, lengths.tolist(), H=1, HV=2)
    say("case %d requests, %d tokens" % (B, int(lengths.sum())))
    o, st = gpu_forward(case, "chunked")
    ro, rs = oracle_forward(case)
    assert_close(o, ro, TOL_CHUNKED, "%d requests o" % B)
    assert_close(st, rs, TOL_CHUNKED, "%d requests state" % B)


# ------------------------------------------------------------------ packing and hand-off
@pytest.mark.parametrize("per_key", [False, True], ids=["per_head", "per_key_form"])
def test_chunked_packed_equals_separate(per_key):
    """Each request of a packed chunked call gives, bit for bit, what the same
    request gives alone (its chunks start at its own first token either way);
    an empty request copies its state."""
    kw = dict(update_rule="gated_delta_v2", per_key=True, gate_activation="none",
              beta_activation="none") if per_key else {}
    lengths = [300, 0, 70, 200]
    case = _case(41 + per_key, lengths, **kw)
    o, st = gpu_forward(case, "chunked", scan_segments=1)
    cu = case["cu_seqlens"]
    for b in range(len(lengths)):
        s, e = int(cu[b]), int(cu[b + 1])
        sc, _ = sub_case(case, b, [0, 1, 2, 3])
        sc["q"], sc["k"] = case["q"][s:e], case["k"][s:e]  # keep the grouped q/k heads
        ob, sb = gpu_forward(sc, "chunked", scan_segments=1)
        assert np.array_equal(o[s:e], ob), "request %d o differs when run alone" % b
        assert np.array_equal(st[b], sb[0]), "request %d state differs when run alone" % b
    assert np.array_equal(st[1], case["initial_state"][1].astype(np.float64)), "empty request copies its state"
    ro, rs = oracle_forward(case)
    assert_close(o, ro, TOL_CHUNKED, "packed chunked o")
    assert_close(st, rs, TOL_CHUNKED, "packed chunked state")


@pytest.mark.parametrize("split", [64, 128, 100, 257])
def test_chunked_resume_split(split):
    """A request cut in two, the second call starting from the first call's
    final state, at and off chunk boundaries: within the chunked bar of one
    call and of the oracle.  (Each call scales its state tiles by a power of
    two taken from its own inputs, which moves the rounding of the split
    operands' low parts, so even a cut at a chunk boundary is not bit-exact.)"""
    T = 300
    case = _case(43, [T])
    o, st = gpu_forward(case, "chunked", scan_segments=1)
    cut = lambda x, a, b: None if x is None else x[a:b]
    first = dict(case, cu_seqlens=np.array([0, split], np.int32),
                 **{k: cut(case[k], 0, split) for k in ("q", "k", "v", "gate", "beta")})
    oa, sa = gpu_forward(first, "chunked", scan_segments=1)
    second = dict(case, cu_seqlens=np.array([0, T - split], np.int32), initial_state=sa.astype(np.float32),
                  **{k: cut(case[k], split, T) for k in ("q", "k", "v", "gate", "beta")})
    ob, sb = gpu_forward(second, "chunked", scan_segments=1)
    both = np.concatenate([oa, ob])
    assert_close(both, o, TOL_CHUNKED, "resumed at %d vs one call: o" % split)
    assert_close(sb, st, TOL_CHUNKED, "resumed at %d vs one call: state" % split)
    ro, rs = oracle_forward(case)
    assert_close(both, ro, TOL_CHUNKED, "resumed at %d: o" % split)
    assert_close(sb, rs, TOL_CHUNKED, "resumed at %d: state" % split)


@pytest.mark.parametrize("H,HV", [(8, 64), (4, 24), (16, 48)], ids=["ratio8", "ratio6", "ratio3"])
def test_chunked_grouped_heads_on_one_xcd(H, HV):
    """Single-pass scans place the value heads of one q/k head in a row on one
    XCD (2, 4 or 8 of them, the largest power of two dividing HV / H): ragged
    requests over 128 pairs or more (the T form) with 8, 6 and 3 value heads
    per q/k head, so the grid's last round is partly empty."""
    case = _case(90 + HV, [150, 333, 0, 64, 97], H=H, HV=HV)
    say("case grouped heads H=%d HV=%d" % (H, HV))
    o, st = gpu_forward(case, "chunked", scan_segments=1)
    ro, rs = oracle_forward(case)
    assert_close(o, ro, TOL_CHUNKED, "H=%d HV=%d o" % (H, HV))
    assert_close(st, rs, 1e-4, "H=%d HV=%d state" % (H, HV))


@pytest.mark.parametrize("rule,per_key", [("gated_delta", False), ("gated_delta_v2", True)],
                         ids=["per_head", "per_key_form"])
def test_chunked_wide_tiles(rule, per_key):
    """128 (request, head) pairs or more take 64-row state tiles in the scan
    (and two 16-byte output stores per lane): ragged chunk tails, an empty
    request and grouped heads on that path."""
    kw = dict(update_rule=rule, per_key=per_key, gate_activation="none", beta_activation="none") if per_key else {}
    case = _case(45 + per_key, [150, 0, 70, 200], H=16, HV=64, **kw)  # 4 x 64 = 256 pairs
    o, st = gpu_forward(case, "chunked", scan_segments=1)
    ro, rs = oracle_forward(case)
    assert_close(o, ro, TOL_CHUNKED, "64-row tiles o")
    assert_close(st, rs, TOL_CHUNKED, "64-row tiles state")
    assert np.array_equal(st[1], case["initial_state"][1].astype(np.float64)), "empty request copies its state"


# ------------------------------------------------------------------ state precision
# (form, lengths, q/k heads, value heads, per-key decay)
PRECISION_FORMS = [("t_form", [700, 300, 1000, 64], 16, 64, False), ("wu_form", [1500, 700], 2, 4, False),
                   ("per_key_form", [900, 500], 2, 4, True), ("wu_form_one_chunk", [64], 16, 64, False),
                   ("per_key_raw_gate", [700, 64, 300], 4, 16, True)]


@pytest.mark.parametrize("form,lengths,H,HV,per_key", PRECISION_FORMS, ids=[f[0] for f in PRECISION_FORMS])
def test_chunked_state_precision(form, lengths, H, HV, per_key):
    """The final state of the chunked forms matches the oracle to 1e-4 of
    its largest entry.  Two things keep it there: the scan multiplies fp32
    operands as fp16 (hi, lo) pairs that hold about 22 bits (single fp16
    operands, 11 bits, would miss by several times the bar), and the decay
    factors between tokens come from the cumulative log decay without the
    cancellation of two large fp32 prefix sums (the qwen gate of these
    inputs decays some heads by hundreds of nats per chunk).  o is stored in
    fp16 and keeps the 2e-3 bar."""
    kw = dict(update_rule="gated_delta_v2", per_key=True, gate_activation="none",
              beta_activation="none") if per_key else {}
    if form == "per_key_raw_gate":
        # the raw-gate arm per key channel: some channels decay by tens of nats per token
        kw = dict(update_rule="gated_delta_v2", per_key=True, gate_activation="qwen", beta_activation="none")
    case = _case(67 if not per_key else 73, lengths, H=H, HV=HV, **kw)
    if form == "wu_form_one_chunk":
        # request 3 of the T-form case on its own: 64 pairs take W and U in the records
        case = _case(67, [700, 300, 1000, 64], H=H, HV=HV)
        case, _ = sub_case(case, 3, list(range(HV)))
    say("case state precision %s" % form)
    o, st = gpu_forward(case, "chunked", scan_segments=1)
    ro, rs = oracle_forward(case)
    say("  %s: o %.3e state %.3e" % (form, rel_err(o, ro), rel_err(st, rs)))
    assert_close(o, ro, TOL_CHUNKED, "%s o" % form)
    assert_close(st, rs, 1e-4, "%s state" % form)


# ------------------------------------------------------------------ NaN in v
@pytest.mark.parametrize("form,H,HV", [("t_form", 16, 64), ("wu_form", 2, 4)], ids=["t_form", "wu_form"])
def test_chunked_nan_value_hand_over(form, H, HV):
    """A NaN in one value channel c of token t: token by token (the README
    recurrence) it reaches only row c of the state, so only channel c of o
    from t on.  The chunk products would spread it to the earlier tokens of
    the chunk (zero entries of T times NaN), so the prologue hands the pair
    to the recurrent kernel: every other output and state entry stays finite
    and matches the oracle."""
    case = _case(88, [300, 200], H=H, HV=HV)
    t, h, c = 150, 1, 5
    case["v"] = case["v"].copy()
    case["v"][t, h, c] = np.float16(np.nan)
    say("case NaN value %s" % form)
    o, st = gpu_forward(case, "chunked", scan_segments=1)
    ro, rs = oracle_forward(case)
    bad_o = np.zeros(o.shape, bool)
    bad_o[t:300, h, c] = True
    bad_s = np.zeros(st.shape, bool)
    bad_s[0, h, c, :] = True
    assert np.all(np.isnan(o[bad_o])) and np.all(np.isnan(st[bad_s])), "the NaN reaches what the recurrence sends it to"
    assert np.all(np.isfinite(o[~bad_o])) and np.all(np.isfinite(st[~bad_s])), "and nothing else"
    assert rel_err(np.where(bad_o, 0.0, o), np.where(bad_o, 0.0, ro)) <= TOL_CHUNKED
    assert rel_err(np.where(bad_s, 0.0, st), np.where(bad_s, 0.0, rs)) <= TOL_CHUNKED


# ------------------------------------------------------------------ state magnitude
@pytest.mark.parametrize("magnitude", [1e4, 1e-5])
@pytest.mark.parametrize("rule", ["gated_delta", "gated"])
def test_chunked_state_magnitude(magnitude, rule):
    """States and values far from 1 on the chunked path AUTO picks: entries
    near 1e4 and near 1e-5 (where fp16 (hi, lo) split operands of the state
    would turn subnormal unless the tile is scaled).  The state is fp32 and
    keeps the 2e-3 bar; o is stored in fp16, whose spacing below 2^-14 is
    2^-24, so o may also differ by the half spacing of that one rounding."""
    kw = {} if rule == "gated_delta" else dict(beta_activation="none")
    case = _case(44, [500, 300], update_rule=rule, **kw)
    case["v"] = (case["v"].astype(np.float32) * np.float32(magnitude)).astype(np.float16)
    case["initial_state"] = (case["initial_state"] * np.float32(magnitude * 5.0)).astype(np.float32)
    say("case state magnitude %.0e rule %s" % (magnitude, rule))
    o, st = gpu_forward(case, "auto")
    ro, rs = oracle_forward(case)
    assert float(np.max(np.abs(rs))) > 0.1 * magnitude, "the states reach the intended magnitude"
    assert_close(st, rs, TOL_CHUNKED, "magnitude %.0e %s state" % (magnitude, rule))
    bound = TOL_CHUNKED * float(np.max(np.abs(ro))) + 2.0 ** -25
    worst = float(np.max(np.abs(o - ro)))
    say("  magnitude %.0e %s o: max abs err %.3e, bound %.3e" % (magnitude, rule, worst, bound))
    assert np.all(np.isfinite(o)) and worst <= bound


# ------------------------------------------------------------------ operands past the fp16 range
def _check_heads(case, o, st, heads, tol_o, what):
    """o and the final state of every request on value heads ``heads``
    against the oracle run on those heads alone (requests and heads evolve
    independently)."""
    if case["slab"] is not None:
        st = st[case["slot_ids"]]
    for b in range(len(case["cu_seqlens"]) - 1):
        sc, (s, e) = sub_case(case, b, heads)
        ro, rs = oracle_forward(sc)
        assert_close(o[s:e][:, heads], ro, tol_o, "%s request %d o" % (what, b))
        assert_close(st[b][heads], rs[0], TOL_CHUNKED, "%s request %d state" % (what, b))
        yield rs


# (name, slots, scan segments, grown request's tokens, q/k heads, value heads):
# 8 pairs take the form with W and U in the records; 128 pairs the T form
GROWTH = [("plain", None, 1, 16384, 2, 4), ("slab", (5,), 1, 16384, 2, 4), ("segmented", None, 2, 32768, 2, 4),
          ("t_form", None, 1, 16384, 16, 64), ("t_form_slab", (5,), 1, 16384, 16, 64)]


@pytest.mark.parametrize("name,slots,segs,T0,H,HV", GROWTH, ids=[g[0] for g in GROWTH])
def test_chunked_state_growth_hand_over(name, slots, segs, T0, H, HV):
    """A state that grows past what the scan's fp16 (hi, lo) operands hold: the
    linear rule (README, update rules: no decay, no erase) with one key
    repeated for T0 tokens and v = 1 builds a state column of T0 times the
    value, 2^14 times max |v| or more (with two segments, each segment's own
    carry grows that far).  The scan flags those (request, head) pairs and the
    recurrent kernel recomputes them in fp32; the second request stays on the
    chunked path.  In slab mode the final states of the unflagged pairs go
    through the staging area and the flagged ones are recomputed from the
    intact slab."""
    case = _case(47, [T0, 300], update_rule="linear", gate_activation="none", beta_activation="none",
                 slots=slots, H=H, HV=HV)
    key = np.zeros(128, np.float16)
    key[5] = 1.0
    case["k"][:T0] = key
    case["v"][:T0] = np.float16(1.0)
    say("case state growth %s segments=%d pairs=%d" % (name, segs, 2 * HV))
    o, st = gpu_forward(case, "chunked", scan_segments=segs)
    heads = [0, 1, HV - 1]
    states = list(_check_heads(case, o, st, heads, TOL_CHUNKED, name))
    assert float(np.max(np.abs(states[0]))) > 16000.0, "the state reaches the intended size"


# (form, q/k heads, value heads)
PROLOGUE = [("per_head_scores", 2, 4), ("t_form_scores", 16, 64), ("per_key_bf16_values", 2, 4),
            ("per_head_bf16_values", 2, 4), ("t_form_bf16_tiny_keys", 16, 64)]


@pytest.mark.parametrize("form,H,HV", PROLOGUE, ids=[f[0] for f in PROLOGUE])
def test_chunked_prologue_hand_over(form, H, HV):
    """Operands the prologue splits into fp16 (hi, lo) past the fp16 range:
    scores scale q.k of unnormalised keys near 1e5 (per-head form, gated
    rule; 8 pairs with W and U in the records, 128 pairs in the T form), and
    bf16 values near 5e5 (per-key form, Gated DeltaNet-2 rule).  And bf16
    activations the per-head form cannot read as fp16 exactly: values near
    5e5, keys near 1e-7 (below fp16's exact range; L2-normalised, so the
    method itself is indifferent to their size).  The prologue flags the
    request's pairs and the recurrent kernel computes them; the other request
    stays on the chunked path."""
    T0 = 400
    if form == "per_head_bf16_values":
        case = _case(50, [T0, 200], dtype="bf16", H=H, HV=HV)
        case["v"][:T0] = case["v"][:T0] * np.float32(2.0 ** 17)  # stays on the bf16 grid
        assert float(np.max(np.abs(case["v"][:T0]))) > 65504.0
    elif form == "t_form_bf16_tiny_keys":
        case = _case(51, [T0, 200], dtype="bf16", H=H, HV=HV)
        case["k"][:T0] = case["k"][:T0] * np.float32(2.0 ** -23)  # stays on the bf16 grid
        assert float(np.max(np.abs(case["k"][:T0]))) < 2.0 ** -17
    elif form != "per_key_bf16_values":
        case = _case(48, [T0, 200], update_rule="gated", gate_activation="none", beta_activation="none",
                     qk_l2_norm=0, H=H, HV=HV)
        rng = np.random.default_rng(48)
        for hq in range(H):
            u = rng.standard_normal(128)
            u = 1000.0 * u / np.linalg.norm(u)
            case["q"][:T0, hq] = u.astype(np.float16)
            case["k"][:T0, hq] = u.astype(np.float16)
        case["v"][:T0] = (case["v"][:T0].astype(np.float32) * np.float32(1e-3)).astype(np.float16)
        assert float((case["scale"] or 128 ** -0.5) * 1000.0 ** 2) > 65504.0
    else:
        case = _case(49, [T0, 200], dtype="bf16", update_rule="gated_delta_v2", per_key=True,
                     gate_activation="none", beta_activation="none")
        case["v"][:T0] = case["v"][:T0] * np.float32(2.0 ** 17)  # stays on the bf16 grid
        assert float(np.max(np.abs(case["v"][:T0]))) > 65504.0
    say("case prologue hand-over %s pairs=%d" % (form, 2 * HV))
    o, st = gpu_forward(case, "chunked", scan_segments=1)
    tol_o = TOL_BF16_O if case["act_dtype"] == "bf16" else TOL_CHUNKED
    list(_check_heads(case, o, st, [0, 1, HV - 1], tol_o, form))


# ------------------------------------------------------------------ the workloads, every pair
FULL = [("varlen_prefill", lambda: workloads.varlen_prefill()),
        ("long_prefill", lambda: workloads.long_prefill()),
        ("perkey_erase", lambda: workloads.perkey_erase()),
        ("varlen_prefill_bf16", lambda: workloads.as_bf16(workloads.varlen_prefill()))]


@pytest.mark.parametrize("name,make", FULL, ids=[f[0] for f in FULL])
def test_workload_every_pair(name, make):
    """The prefill workload at its full size on the path AUTO runs (the
    chunked kernels), every (request, value head) pair of o and of the final
    state against the fp64 oracle."""
    case = make()
    say("case %s: AUTO path, all pairs against the oracle" % case["name"])
    o, st = gpu_forward(case, "auto")
    ro, rs = oracle_forward(case)
    tol_o = TOL_BF16_O if case["act_dtype"] == "bf16" else TOL_CHUNKED
    eo, es = rel_err(o, ro), rel_err(st, rs)
    _log_errors(case["name"], o=eo, state=es, tol_o=tol_o, tol_state=TOL_CHUNKED)
    assert_close(o, ro, tol_o, "%s o (all pairs)" % name)
    assert_close(st, rs, TOL_CHUNKED, "%s state (all pairs)" % name)
