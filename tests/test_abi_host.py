"""The C-ABI library on the host: it loads, exports every function that
include/gdr.h declares, and rejects invalid arguments before touching the
GPU (gdr_validate / gdr_workspace_size / gdr_select_algo make no HIP call and
read no tensor memory, so fake, aligned pointer values are enough here)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_token_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "gdr.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(gdr_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(api.library_path()):
        from gated_delta_rule_token_amd import build
        build.build()
    return api.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == set(api.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), name
    assert lib.gdr_abi_version() == api.ABI_VERSION == 3


def test_status_strings(lib):
    for code, name in enumerate(["GDR_OK", "GDR_E_INVALID", "GDR_E_UNSUPPORTED", "GDR_E_ALIAS",
                                 "GDR_E_WORKSPACE", "GDR_E_HIP"]):
        assert lib.gdr_status_str(code).decode() == name


# fake device addresses: distinct, 1 MiB apart, 256-byte aligned; never dereferenced
_BASE = 0x7F0000000000


def _fake(i):
    return _BASE + i * (1 << 28)


def _good(**over):
    T, B, H, HV, D = 16, 2, 2, 4, 32
    p = api.Problem(total_tokens=T, batch=B, seq_len=0, num_heads_qk=H, num_heads_v=HV,
                    head_dim_k=D, head_dim_v=D, num_slots=0, act_dtype=api.F32,
                    gate_dtype=api.F32, update_rule=api.RULES["gated_delta"],
                    gate_activation=api.GATES["qwen"], beta_activation=api.BETAS["sigmoid"],
                    qk_l2_norm=1, decay_per_key=0, rank4=0, chunk_size=64, algo=0,
                    state_update_capacity=0, scale=0.0)
    t = api.Tensors(q=_fake(1), k=_fake(2), v=_fake(3), o=_fake(4), gate=_fake(5), beta=_fake(6),
                    erase=None, a_log=_fake(7), dt_bias=_fake(8), cu_seqlens=_fake(9),
                    slot_ids=None, initial_state=None, final_state=_fake(10))
    for key, val in over.items():
        if hasattr(p, key) and key not in ("q", "k", "v", "o"):
            setattr(p, key, val)
        else:
            setattr(t, key, val)
    return p, t


def _validate(lib, p, t):
    return lib.gdr_validate(ctypes.byref(p), ctypes.byref(t) if t is not None else None)


def test_good_problem_validates(lib):
    p, t = _good()
    assert _validate(lib, p, t) == api.GDR_OK, lib.gdr_last_error()


BAD = [
    ("capacity", dict(state_update_capacity=4), api.GDR_E_UNSUPPORTED),
    ("act_dtype", dict(act_dtype=7), api.GDR_E_INVALID),
    ("rule", dict(update_rule=9), api.GDR_E_INVALID),
    ("gate_act", dict(gate_activation=5), api.GDR_E_INVALID),
    ("beta_act", dict(beta_activation=5), api.GDR_E_INVALID),
    ("algo", dict(algo=11), api.GDR_E_INVALID),
    ("hv_not_multiple", dict(num_heads_v=3), api.GDR_E_INVALID),
    ("dk_too_big", dict(head_dim_k=257), api.GDR_E_INVALID),
    ("dv_zero", dict(head_dim_v=0), api.GDR_E_INVALID),
    ("rank4_with_cu", dict(rank4=1, seq_len=8), api.GDR_E_INVALID),
    ("missing_gate", dict(gate=None), api.GDR_E_INVALID),
    ("missing_beta", dict(beta=None), api.GDR_E_INVALID),
    ("a_log_without_dt_bias", dict(dt_bias=None), api.GDR_E_INVALID),
    ("qwen_without_params", dict(a_log=None, dt_bias=None), api.GDR_E_INVALID),
    ("params_without_qwen", dict(gate_activation=0), api.GDR_E_INVALID),
    ("erase_for_v1", dict(erase=_fake(11)), api.GDR_E_INVALID),
    ("slots_without_ids", dict(num_slots=8), api.GDR_E_INVALID),
    ("ids_without_slots", dict(slot_ids=_fake(12)), api.GDR_E_INVALID),
    ("missing_final_state", dict(final_state=None), api.GDR_E_INVALID),
    ("missing_q", dict(q=None), api.GDR_E_INVALID),
    ("misaligned", dict(v=_fake(3) + 4), api.GDR_E_INVALID),
    ("o_aliases_q", dict(o=_fake(1)), api.GDR_E_ALIAS),
    ("state_aliases_v", dict(final_state=_fake(3) + 256), api.GDR_E_ALIAS),
    ("a_log_and_gate_scale", dict(gate_scale=_fake(13)), api.GDR_E_INVALID),
    ("gate_scale_without_qwen", dict(gate_activation=0, a_log=None, dt_bias=None,
                                     gate_scale=_fake(13)), api.GDR_E_INVALID),
    ("seq_lens_with_cu_seqlens", dict(seq_lens=_fake(14)), api.GDR_E_INVALID),
    ("beta_per_token_without_beta", dict(update_rule=api.RULES["gated"], beta=None, beta_activation=0,
                                         beta_per_token=1), api.GDR_E_INVALID),
    ("beta_per_token_value", dict(beta_per_token=2), api.GDR_E_INVALID),
    ("dt_bias_aliases_o_per_key", dict(decay_per_key=1, o=_fake(8) + 256), api.GDR_E_ALIAS),
    ("decode_needs_128", dict(algo=api.ALGOS["decode"]), api.GDR_E_UNSUPPORTED),
    ("chunked_needs_128_f16", dict(algo=api.ALGOS["chunked"]), api.GDR_E_UNSUPPORTED),
    ("gate_dtype", dict(gate_dtype=api.F16), api.GDR_E_INVALID),
]


@pytest.mark.parametrize("name,over,status", BAD, ids=[b[0] for b in BAD])
def test_rejects(lib, name, over, status):
    p, t = _good(**over)
    got = _validate(lib, p, t)
    assert got == status, (name, got, lib.gdr_last_error())
    assert lib.gdr_last_error().decode() != ""


def test_rule_presence_rules(lib):
    # linear: no gate, no beta
    p, t = _good(update_rule=api.RULES["linear"], gate_activation=0, gate=None, beta=None,
                 a_log=None, dt_bias=None)
    assert _validate(lib, p, t) == api.GDR_OK, lib.gdr_last_error()
    t.beta = _fake(6)
    assert _validate(lib, p, t) == api.GDR_E_INVALID
    # gated_delta_v2: gate + erase, no beta
    p, t = _good(update_rule=api.RULES["gated_delta_v2"], gate_activation=0, a_log=None,
                 dt_bias=None, beta=None, erase=_fake(11), decay_per_key=1)
    assert _validate(lib, p, t) == api.GDR_OK, lib.gdr_last_error()
    t.beta = _fake(6)
    assert _validate(lib, p, t) == api.GDR_E_INVALID


def test_raw_gate_spellings_and_seq_lens(lib):
    # the folded gate_scale replaces a_log (CLIKA "gatedDeltaUpdate": gate_bias + gate_scale)
    p, t = _good(a_log=None, gate_scale=_fake(13))
    assert _validate(lib, p, t) == api.GDR_OK, lib.gdr_last_error()
    # a per-key raw gate (fp32 or the activations' dtype) with a (HV, dk) bias
    p, t = _good(decay_per_key=1)
    assert _validate(lib, p, t) == api.GDR_OK, lib.gdr_last_error()
    p, t = _good(decay_per_key=1, act_dtype=api.F16, gate_dtype=api.F16)
    assert _validate(lib, p, t) == api.GDR_OK, lib.gdr_last_error()
    # seq_lens with uniform packing, rank-3 or rank-4
    p, t = _good(cu_seqlens=None, seq_len=8, seq_lens=_fake(14))
    assert _validate(lib, p, t) == api.GDR_OK, lib.gdr_last_error()
    p.rank4 = 1
    assert _validate(lib, p, t) == api.GDR_OK, lib.gdr_last_error()
    # beta (T, 1) shared by the value heads
    p, t = _good(beta_per_token=1)
    assert _validate(lib, p, t) == api.GDR_OK, lib.gdr_last_error()


def test_in_place_state_allowed_partial_overlap_rejected(lib):
    p, t = _good(cu_seqlens=None, seq_len=8)
    t.initial_state = _fake(10)
    t.final_state = _fake(10)
    assert _validate(lib, p, t) == api.GDR_OK, lib.gdr_last_error()
    t.final_state = _fake(10) + 1024
    assert _validate(lib, p, t) == api.GDR_E_ALIAS


def test_uniform_packing_needs_consistent_sizes(lib):
    p, t = _good(cu_seqlens=None, seq_len=7)
    assert _validate(lib, p, t) == api.GDR_E_INVALID
    p.seq_len = 8
    assert _validate(lib, p, t) == api.GDR_OK, lib.gdr_last_error()


def test_slab_forbids_initial_state(lib):
    p, t = _good(num_slots=16, slot_ids=_fake(12))
    assert _validate(lib, p, t) == api.GDR_OK, lib.gdr_last_error()
    t.initial_state = _fake(13)
    assert _validate(lib, p, t) == api.GDR_E_INVALID


def test_workspace_and_algo_selection(lib):
    p, _ = _good()
    n = ctypes.c_size_t(99)
    assert lib.gdr_workspace_size(ctypes.byref(p), ctypes.byref(n)) == api.GDR_OK
    assert n.value == 0
    assert api.selected_algo(p) == "recurrent"
    p.head_dim_k = p.head_dim_v = 128
    p.total_tokens, p.batch = 256, 256
    assert api.selected_algo(p) == "decode"
    # long fp16 requests at dk = dv = 128 take the chunked kernels and need a workspace
    p.total_tokens, p.batch, p.act_dtype, p.gate_dtype = 4096, 2, api.F16, api.F16
    assert api.selected_algo(p) == "chunked"
    assert lib.gdr_workspace_size(ctypes.byref(p), ctypes.byref(n)) == api.GDR_OK
    assert n.value >= (4096 // 64) * 4 * 64 * 128 * 4
    # a per-key decay takes the per-key chunked form, whose record is larger
    n_head = n.value
    p.decay_per_key, p.gate_activation, p.gate_dtype = 1, 0, api.F32
    assert api.selected_algo(p) == "chunked"
    assert lib.gdr_workspace_size(ctypes.byref(p), ctypes.byref(n)) == api.GDR_OK
    assert n.value > n_head
    # short requests stay on the recurrent kernel, and so do fp32 activations
    p.total_tokens = 2 * 100
    assert api.selected_algo(p) == "recurrent"
    p.total_tokens, p.act_dtype = 4096, api.F32
    assert api.selected_algo(p) == "recurrent"
    # bf16 with a per-head decay takes the per-head chunked form (the fp16
    # problem's layout); the erase gate takes the per-key form
    p.decay_per_key, p.gate_activation, p.gate_dtype, p.update_rule = 0, 0, api.F32, api.RULES["gated_delta"]
    p.act_dtype = api.BF16
    assert api.selected_algo(p) == "chunked"
    assert lib.gdr_workspace_size(ctypes.byref(p), ctypes.byref(n)) == api.GDR_OK
    assert n.value == n_head
    p.update_rule = api.RULES["gated_delta_v2"]
    assert lib.gdr_workspace_size(ctypes.byref(p), ctypes.byref(n)) == api.GDR_OK
    assert n.value > n_head
    p.update_rule = api.RULES["gated_delta"]
    p.act_dtype = api.F32
    p.algo = api.ALGOS["chunked"]
    assert lib.gdr_validate(ctypes.byref(p), None) == api.GDR_E_UNSUPPORTED


def test_scan_segments_workspace(lib):
    """A segmented chunk scan keeps per (request, head) segment states in the
    workspace; the count is validated on the host."""
    p, _ = _good()
    p.head_dim_k = p.head_dim_v = 128
    p.total_tokens, p.batch, p.act_dtype, p.gate_dtype = 4096, 2, api.F16, api.F16
    n1, n4 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    p.scan_segments = 1
    assert lib.gdr_workspace_size(ctypes.byref(p), ctypes.byref(n1)) == api.GDR_OK
    p.scan_segments = 4
    assert lib.gdr_workspace_size(ctypes.byref(p), ctypes.byref(n4)) == api.GDR_OK
    heads = p.batch * p.num_heads_v
    assert n4.value - n1.value >= heads * 3 * 4 * 128 * 128 * 4
    for bad in (-1, 17):
        p.scan_segments = bad
        assert lib.gdr_validate(ctypes.byref(p), None) == api.GDR_E_INVALID
        assert b"scan_segments" in lib.gdr_last_error()
    # the automatic choice splits one long request over few heads, not many short ones
    p.scan_segments, p.batch, p.num_heads_qk, p.num_heads_v = 0, 1, 16, 16
    p.total_tokens = 65536
    assert lib.gdr_workspace_size(ctypes.byref(p), ctypes.byref(n4)) == api.GDR_OK
    p.scan_segments = 1
    assert lib.gdr_workspace_size(ctypes.byref(p), ctypes.byref(n1)) == api.GDR_OK
    assert n4.value > n1.value


@pytest.mark.parametrize("tokens,heads,nseg", [(65536, 16, 5), (65536, 8, 9), (32768, 4, 9), (65536, 1, 9),
                                                (16384, 16, 5), (12000, 16, 1), (65536, 32, 1)])
def test_scan_segments_automatic_choice(lib, tokens, heads, nseg):
    """The segment count AUTO picks for one long request over few heads,
    read back from the workspace size (each segment adds three 64 KiB states
    per (request, head)): pass 2 gets about 64 (request, head, segment)
    groups, at most 16 segments, none for short requests or many pairs."""
    p, _ = _good()
    p.head_dim_k = p.head_dim_v = 128
    p.act_dtype, p.gate_dtype = api.F16, api.F16
    p.batch, p.num_heads_qk, p.num_heads_v, p.total_tokens, p.seq_len = 1, heads, heads, tokens, tokens
    sizes = {}
    for forced in (0, 1):
        p.scan_segments = forced
        n = ctypes.c_size_t(0)
        assert lib.gdr_workspace_size(ctypes.byref(p), ctypes.byref(n)) == api.GDR_OK
        sizes[forced] = n.value
    extra = sizes[0] - sizes[1]
    assert extra == (0 if nseg == 1 else heads * 3 * nseg * 128 * 128 * 4)


def test_gate_argument_checks(lib):
    assert lib.gdr_gate(10, 3, 0, _fake(1), _fake(2), _fake(3), None, _fake(4), None, None) \
        == api.GDR_E_INVALID  # 10 not a multiple of 3 heads
    assert lib.gdr_gate(12, 3, 0, _fake(1), _fake(2), _fake(3), None, _fake(4), _fake(5), None) \
        == api.GDR_E_INVALID  # beta without b
    assert lib.gdr_gate(12, 3, 9, _fake(1), _fake(2), _fake(3), None, _fake(4), None, None) \
        == api.GDR_E_INVALID  # bad dtype


def test_slab_stream_argument_checks(lib):
    f = ctypes.c_float(1.0)
    assert lib.gdr_slab_stream(_fake(1), _fake(2), 4, 0, 16, 8, f, None) == api.GDR_E_INVALID  # no heads
    assert lib.gdr_slab_stream(_fake(1), _fake(2), 4, 2, 18, 8, f, None) == api.GDR_E_INVALID  # not 4k floats
    assert lib.gdr_slab_stream(_fake(1), _fake(2), 4, 2, 16, 0, f, None) == api.GDR_E_INVALID  # no slots
    assert lib.gdr_slab_stream(None, _fake(2), 4, 2, 16, 8, f, None) == api.GDR_E_INVALID
    assert lib.gdr_slab_stream(_fake(1) + 4, _fake(2), 4, 2, 16, 8, f, None) == api.GDR_E_INVALID  # misaligned
    # 2^20 requests x 2^10 heads x 4 pieces of 64 KB: 2^32 workgroups, past one launch
    assert lib.gdr_slab_stream(_fake(1), _fake(2), 1 << 20, 1 << 10, 1 << 16, 8, f, None) \
        == api.GDR_E_INVALID
    assert lib.gdr_slab_stream(None, None, 0, 2, 16, 8, f, None) == api.GDR_OK  # nothing to do


def test_forward_rejects_a_short_workspace(lib):
    """gdr_forward compares the workspace size it is given with what the
    problem needs and returns GDR_E_WORKSPACE before anything is enqueued."""
    p, t = _good()
    p.head_dim_k = p.head_dim_v = 128
    p.total_tokens, p.act_dtype, p.gate_dtype = 4096, api.F16, api.F16
    need = ctypes.c_size_t(0)
    assert lib.gdr_workspace_size(ctypes.byref(p), ctypes.byref(need)) == api.GDR_OK and need.value > 0
    assert lib.gdr_forward(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(_fake(11)),
                           need.value - 1, None) == api.GDR_E_WORKSPACE
    assert lib.gdr_forward(ctypes.byref(p), ctypes.byref(t), None, 0, None) == api.GDR_E_WORKSPACE


def _cpu_problem(**kw):
    import torch
    T, H, HV, dk, dv, B = 40, 2, 4, 32, 16, 2
    q = torch.zeros(T, H, dk)
    v = torch.zeros(T, HV, dv)
    args = dict(gate=torch.zeros(T, HV), beta=torch.zeros(T, HV), a_log=torch.zeros(HV),
                dt_bias=torch.zeros(HV), cu_seqlens=torch.zeros(B + 1, dtype=torch.int32),
                initial_state=torch.zeros(B, HV, dv, dk), gate_activation="qwen")
    args.update(kw)
    p = api.build_problem(q, q, v, **args)
    shapes = {k: (None if x is None else tuple(x.shape)) for k, x in args.items()
              if k in ("gate", "beta", "a_log", "dt_bias", "cu_seqlens", "initial_state")}
    return p, (T,), shapes


def test_binding_shape_checks():
    """The binding checks every tensor's shape against the problem before the
    call (the kernels take raw pointers, so a short buffer would otherwise be
    read or written out of bounds)."""
    import torch
    p, lead, shapes = _cpu_problem()
    api.check_shapes(p, lead, shapes)  # consistent
    api.check_shapes(p, lead, dict(shapes, beta=(40, 1), out=(40, 4, 16), final_state=(2, 4, 16, 32)))
    bad = [("gate", (40, 3)), ("gate", (39, 4)), ("beta", (40, 2)), ("a_log", (3,)),
           ("dt_bias", (4, 32)), ("cu_seqlens", (2,)), ("initial_state", (2, 4, 32, 16)),
           ("initial_state", (1, 4, 16, 32)), ("out", (40, 4, 32)), ("final_state", (3, 4, 16, 32)),
           ("erase", (40, 4)), ("seq_lens", (3,)), ("slot_ids", (1,)), ("gate_scale", (5,))]
    for name, shape in bad:
        with pytest.raises(api.GDRError, match=name):
            api.check_shapes(p, lead, dict(shapes, **{name: shape}))
    # a per-key gate takes (T, HV, dk) and a (HV, dk) bias
    pk, lead, sh = _cpu_problem(gate=torch.zeros(40, 4, 32), dt_bias=torch.zeros(4, 32))
    assert pk.decay_per_key == 1
    api.check_shapes(pk, lead, sh)
    with pytest.raises(api.GDRError, match="dt_bias"):
        api.check_shapes(pk, lead, dict(sh, dt_bias=(4,)))
    # the slab: (num_slots, HV, dv, dk)
    ps = api.build_problem(torch.zeros(2, 1, 2, 32), torch.zeros(2, 1, 2, 32), torch.zeros(2, 1, 4, 16),
                           state=torch.zeros(7, 4, 16, 32), slot_ids=torch.zeros(2, dtype=torch.int32),
                           update_rule="delta", beta=torch.zeros(2, 1, 4))
    api.check_shapes(ps, (2, 1), {"state": (7, 4, 16, 32), "slot_ids": (2,), "beta": (2, 1, 4)})
    with pytest.raises(api.GDRError, match="state"):
        api.check_shapes(ps, (2, 1), {"state": (7, 4, 32, 16)})
