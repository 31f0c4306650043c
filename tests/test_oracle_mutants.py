"""Plant plausible mistakes in copies of the oracle source and show that the
pins catch every one of them (CPU only; the copies are built with gcc in a
temporary directory and never touch the GPU path).  Each mutant runs in its
own interpreter so a broken copy cannot disturb the test process."""
import functools
import json
import os
import subprocess
import sys

import pytest

import oracle
from tests.oracle_pins import ALL_PINS, GATE_PINS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in gdr_oracle.c, replacement)
MUTANTS = [
    ("no_decay", "Si[j] *= alpha[j];", "(void)alpha;"),
    ("retrieval_sign", "vprime = beta * (vt[i] - r);", "vprime = beta * (vt[i] + r);"),
    ("beta_outside", "vprime = beta * (vt[i] - r);", "vprime = beta * vt[i] - r;"),
    ("readout_before_write", "acc += Si[j] * qn[j];", "acc += (Si[j] - vprime * kn[j]) * qn[j];"),
    ("retrieve_before_decay", "r += Si[j] * kn[j];", "r += Si[j] / alpha[j] * kn[j];"),
    ("retrieve_with_query", "r += Si[j] * kn[j];", "r += Si[j] * qn[j];"),
    ("gqa_modulo", "(int)(((int64_t)h * H) / HV);", "h % H;"),
    ("softplus_bias_sign", "softplus(raw + bias)", "softplus(raw - bias)"),
    ("decay_scale_no_exp", ": -exp(p->a_log[h]);", ": -p->a_log[h];"),
    ("per_key_bias_per_head", "p->dt_bias[(size_t)h * DK + j]", "p->dt_bias[h]"),
    ("gate_scale_ignored", "p->gate_scale ? p->gate_scale[h]", "p->gate_scale ? -1.0"),
    ("seq_lens_ignored", "len = p->seq_lens[b];", "len = p->L;"),
    ("seq_lens_no_upper_clamp", "if (len > p->L) len = p->L;", "if (len > 100000) len = p->L;"),
    ("sigmoid_sign", "1.0 / (1.0 + exp(-x))", "1.0 / (1.0 + exp(x))"),
    ("l2_no_sqrt", "1.0 / sqrt(qss + 1e-12)", "1.0 / (qss + 1e-12)"),
    ("erase_value_axis", "if (bt && !p->erase_value_axis)", "if (bt && p->erase_value_axis)"),
    ("v2_no_erase", "vprime = vt[i] - r;", "vprime = vt[i];"),
    ("cu_end_off_by_one", "*e = z > a ? z : a;", "*e = z > a ? z - 1 : a;"),
    ("cu_clamp_short", "if (z > p->T) z = p->T;", "if (z > p->T) z = p->T - 1;"),
    ("scale_default", "1.0 / sqrt((double)DK)", "1.0 / (double)DK"),
    ("initial_state_ignored", "S[(size_t)i * DK + j] = S0 ? S0[(size_t)i * DK + j] : 0.0;",
     "S[(size_t)i * DK + j] = 0.0;"),
    ("slot_addressed_by_batch_row", "((size_t)slot * HV + h)", "((size_t)b * HV + h)"),
    ("perkey_first_channel_only", "p->gate[((size_t)t * HV + h) * DK + j]",
     "p->gate[((size_t)t * HV + h) * DK]"),
    ("write_uses_query", "Si[j] += vprime * kn[j];", "Si[j] += vprime * qn[j];"),
    # the standalone gate
    ("gate_head_by_row", "const int64_t head = n % heads;", "const int64_t head = (n / heads) % heads;"),
    ("gate_bias_dropped", "softplus(a[n] + dt_bias[head])", "softplus(a[n])"),
    ("gate_bias_sign", "softplus(a[n] + dt_bias[head])", "softplus(a[n] - dt_bias[head])"),
    ("gate_scale_dropped", "decay[n] = decay_scale[head] *", "decay[n] = -1.0 *"),
    ("gate_beta_sign", "if (beta) beta[n] = sigmoid(b[n]);", "if (beta) beta[n] = sigmoid(-b[n]);"),
    ("gate_beta_from_a", "if (beta) beta[n] = sigmoid(b[n]);", "if (beta) beta[n] = sigmoid(a[n]);"),
    # the L2 norm of a zero row
    ("l2_eps_dropped", "1.0 / sqrt(kss + 1e-12)", "1.0 / sqrt(kss)"),
]


def run_pins_on_variant(src_text, lib_path):
    """Compile ``src_text`` and return the names of the pins it fails."""
    lib = oracle.compile_variant(src_text, lib_path)
    fwd = functools.partial(oracle.forward, lib=lib)
    gate = functools.partial(oracle.gate, lib=lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(fwd)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    for pin in GATE_PINS:
        try:
            pin(gate, fwd)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    return caught


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = oracle.source_text()
    assert src.count(old) == 1, "mutation anchor for %s must occur exactly once" % name
    src_path = tmp_path / "mutant.c"
    src_path.write_text(src.replace(old, new))
    code = ("import json,sys; sys.path.insert(0, %r); "
            "from tests.test_oracle_mutants import run_pins_on_variant; "
            "print(json.dumps(run_pins_on_variant(open(%r).read(), %r)))"
            % (ROOT, str(src_path), str(tmp_path / "libmutant.so")))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=300, env=env, cwd=ROOT)
    assert res.returncode == 0, "mutant %s crashed: %s" % (name, res.stderr[-2000:])
    caught = json.loads(res.stdout.strip().splitlines()[-1])
    assert caught, "planted mistake %r passed every pin" % name
