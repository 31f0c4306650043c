"""Benchmark of the gated delta-rule engine on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline (the JSON line's ``value``): the decode state update -- B=256
requests of one token each, H=16 q/k heads, HV=32 value heads, dk=dv=128,
fp16 q/k/v, raw-gate arm, a 512-slot fp32 state slab updated in place at 256
distinct slot ids -- reported as HBM GB/s of algorithmic traffic.  A step is
one gdr_forward call over that batch.  Consecutive steps alternate between
two disjoint sets of 256 slot ids (each a full decode batch of the same
workload), so a step never finds the previous step's state in the 256 MB
Infinity Cache.

Also reported: prefill tokens/s on the varlen workload (8 requests of
512..8192 tokens, H=16, HV=32, dk=dv=128, fp16, raw-gate arm, qk L2-norm,
fp32 initial/final states), on one 65,536-token sequence (H=HV=16), on
the per-key-decay / erase-gate workload (4 x 4096 tokens, H=8, HV=32) and on
the varlen workload with bf16 activations, each with its HBM roofline
(algorithmic bytes of the call against 8 TB/s, with the counter-measured
bytes when the committed counter summary matches the kernel source), the
executed matrix-core rate when known, the recurrence-equivalent flop rate
against the fp32 vector peak, and the fp64 CPU oracle timed on a bounded
sample of the same workload; the decode step's own oracle baseline is the
line's ``cpu_baseline``.

``value`` is the wall-clock rate over exactly ``steps`` launches between two
device synchronisations; per-launch durations come from HIP events recorded
on the stream the kernels run on (torch's current stream), around each of as
many launches again after that region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published
METRIC = "decode state-update HBM GB/s (% peak); prefill tokens/s at dk=dv=128"


def _t(x):
    import torch
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


def decode_bytes(B, H, HV, dk, dv, L=1, act_bytes=2):
    """Algorithmic bytes of one decode step of L tokens per request: each
    addressed state row is read and written once; q, k, v, o, gate, beta of
    every token, slot ids and per-head params once."""
    state = 2 * B * HV * dv * dk * 4
    acts = B * L * ((2 * H * dk + 2 * HV * dv) * act_bytes + HV * (act_bytes + 4)) + B * 4 + 2 * HV * 4
    return state + acts, state


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


CSRC = "gated_delta_rule_token_amd/csrc/"
DECODE_SOURCES = [CSRC + f for f in ("gdr_decode.hip", "gdr_device.hpp", "gdr_chunk_plan.hpp")]
CHUNKED_SOURCES = [CSRC + f for f in ("gdr_chunked.hpp", "gdr_chunked.hip", "gdr_chunked_bf16.hip",
                                      "gdr_recurrent.hip", "gdr_device.hpp", "gdr_chunk_plan.hpp")]


def committed_counters(summary, digest, workload=None):
    """Per-launch figures from a committed rocprofv3 counter summary: the
    ``key: value`` lines of the block whose ``kernel_source_digest`` matches
    (and, for a summary that covers several workloads, whose ``workload``
    matches).  None when the summary is missing or was taken on other source."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    blocks = re.split(r"\n(?=kernel_source_digest:)", open(path).read())
    for blk in blocks:
        vals = dict(re.findall(r"^([a-z_]+):\s*(\S+)\s*$", blk, re.M))
        if vals.get("kernel_source_digest") != digest:
            continue
        if workload is not None and vals.get("workload") != workload:
            continue
        return vals
    return None


def committed_traffic(digest):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    or None when that summary is missing or was taken on other kernel source."""
    vals = committed_counters("decode_hbm_counters.md", digest)
    return None if vals is None or "hbm_bytes_per_launch" not in vals else float(vals["hbm_bytes_per_launch"])


def time_wall(calls, steps, warmup):
    """Run ``calls`` round-robin: ``warmup`` untimed launches, then exactly
    ``steps`` launches bracketed by a device synchronisation on both sides
    (nothing else in the timed region).  Returns the wall seconds."""
    import torch
    for i in range(warmup):
        calls[i % len(calls)].run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        calls[i % len(calls)].run()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def time_events(calls, reps):
    """Mean duration in ms of one launch, from a HIP event pair recorded on the
    launch's own stream (torch's current stream) around each of ``reps``
    launches, after the wall-clock region."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record()
        calls[i % len(calls)].run()
        ev[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def time_calls(calls, steps, warmup):
    """Wall seconds over exactly ``steps`` launches, then the mean event-timed
    launch duration in ms over as many launches again."""
    wall = time_wall(calls, steps, warmup)
    return wall, time_events(calls, steps)


def bench_decode(args, L=1):
    import torch
    from gated_delta_rule_token_amd import api, workloads
    case = workloads.decode_slab(L=L)
    B, H = case["q"].shape[0], case["q"].shape[2]
    HV, dv, dk = case["v"].shape[2], case["v"].shape[3], case["q"].shape[3]
    ids_a = case["slot_ids"]
    rng = workloads.rng_for(101)
    ids_b = rng.permutation(np.setdiff1d(np.arange(case["slab"].shape[0]), ids_a)).astype(np.int32)
    slab = _t(case["slab"])
    common = dict(gate=_t(case["gate"]), beta=_t(case["beta"]), a_log=_t(case["a_log"]),
                  dt_bias=_t(case["dt_bias"]), state=slab, update_rule="gated_delta",
                  gate_activation="qwen", beta_activation="sigmoid", algo=args.decode_algo)
    q, k, v = _t(case["q"]), _t(case["k"]), _t(case["v"])
    calls = [api.prepare(q, k, v, slot_ids=_t(ids), **common) for ids in (ids_a, ids_b)]
    steps = args.steps if L == 1 else max(20, args.steps // 4)
    wall, kms = time_calls(calls, steps, args.warmup)
    total_b, state_b = decode_bytes(B, H, HV, dk, dv, L)
    digest = source_digest(DECODE_SOURCES)
    traffic = committed_traffic(digest)
    achieved = total_b / (kms * 1e-3) / 1e9
    out = {
        "wall_s": wall, "kernel_ms": kms, "bytes_per_step": total_b, "state_bytes": state_b,
        "gbs_wall": total_b * steps / wall / 1e9, "gbs_kernel": achieved,
        "algo": calls[0].algo, "tokens": B * L, "traffic": traffic, "digest": digest,
    }
    if L == 1:
        # the same steps' state bytes moved by a plain in-place copy (no compute),
        # alternating the two slot sets as the decode steps do: the ceiling of
        # this access pattern (random 2 MiB slots), measured after the timed region
        class Floor:
            def __init__(self, ids):
                self.ids = ids

            def run(self):
                api.slab_stream(slab, self.ids, 1.0)
        floors = [Floor(_t(ids)) for ids in (ids_a, ids_b)]
        for i in range(args.warmup):
            floors[i % 2].run()
        fms = time_events(floors, steps)
        out["slab_stream_ms"] = fms
        out["slab_stream_gbs"] = state_b / (fms * 1e-3) / 1e9
    return case, out


PREFILL_CASES = {
    "varlen": lambda w: w.varlen_prefill(),
    "long": lambda w: w.long_prefill(),
    "perkey": lambda w: w.perkey_erase(),
    "varlen_bf16": lambda w: w.as_bf16(w.varlen_prefill()),
}
CLOCK_HZ = 2.4e9    # MI355X peak engine clock
SIMDS = 256 * 4     # 256 CUs x 4 SIMDs


def prefill_bytes(case):
    """Algorithmic HBM bytes of one prefill call: q, k, v, o, the gate, beta
    and erase rows once, the incoming state read once (when given) and the
    final state written once."""
    q, v = case["q"], case["v"]
    T = q.shape[0] * (q.shape[1] if q.ndim == 4 else 1)
    H, dk, HV, dv = q.shape[-2], q.shape[-1], v.shape[-2], v.shape[-1]
    act = 2 if case["act_dtype"] in ("f16", "bf16") else 4
    n = T * (2 * H * dk + 2 * HV * dv) * act
    for key in ("gate", "beta", "erase"):
        x = case.get(key)
        if x is not None:
            n += x.size * (act if key == "gate" and case["gate_activation"] == "qwen" else 4)
    B = len(case["cu_seqlens"]) - 1 if case["cu_seqlens"] is not None else q.shape[0]
    state = B * HV * dv * dk * 4
    return n + state * (2 if case["initial_state"] is not None else 1)


def bench_prefill(args, which):
    """Prefill throughput on one workload: the varlen batch (8 requests,
    cu_seqlens, qk L2-norm, raw gate, random initial states), the long single
    sequence (65,536 tokens, H=HV=16), the per-key decay / erase-gate batch
    (4 x 4,096 tokens) or the varlen batch in bf16.  One call is the whole hot
    path (chunk table, prologue and scan kernels, and the recurrent kernel for
    pairs the chunked form hands over)."""
    import torch
    from gated_delta_rule_token_amd import api, workloads
    case = PREFILL_CASES[which](workloads)
    q, k, v = case["q"], case["k"], case["v"]
    T = q.shape[0] * (q.shape[1] if q.ndim == 4 else 1)
    dk, HV, dv = q.shape[-1], v.shape[-2], v.shape[-1]
    act = (lambda x: _t(x).to(torch.bfloat16)) if case["act_dtype"] == "bf16" else _t
    gate = act(case["gate"]) if case["gate_activation"] == "qwen" else _t(case["gate"])
    call = api.prepare(act(q), act(k), act(v), gate=gate, beta=_t(case["beta"]),
                       erase=_t(case["erase"]),
                       a_log=_t(case["a_log"]), dt_bias=_t(case["dt_bias"]),
                       cu_seqlens=_t(case["cu_seqlens"]), initial_state=_t(case["initial_state"]),
                       update_rule=case["update_rule"], gate_activation=case["gate_activation"],
                       beta_activation=case["beta_activation"], qk_l2_norm=case["qk_l2_norm"],
                       algo=args.prefill_algo)
    steps = max(1, args.prefill_steps)
    wall, kms = time_calls([call], steps, max(1, args.warmup // 2))
    nbytes = prefill_bytes(case)
    gbs = nbytes / (kms * 1e-3) / 1e9
    flops = 7.0 * dk * dv * HV * T  # decay, two dot products, rank-1 write per state element
    tflops = flops / (kms * 1e-3) / 1e12
    digest = source_digest(CHUNKED_SOURCES)
    counters = committed_counters("prefill_hbm_counters.md", digest, case["name"]) if call.algo == "chunked" else None
    traffic = float(counters["hbm_bytes_per_call"]) if counters and "hbm_bytes_per_call" in counters else None
    out = {
        "workload": case["name"], "tokens": int(T), "algo": call.algo, "steps": steps,
        "ms_per_call": kms, "tokens_per_s": T / (kms * 1e-3), "tokens_per_s_wall": T * steps / wall,
        # the HBM roofline of the whole call: its algorithmic bytes at 8 TB/s
        # take longer than its executed matrix-core flops at 2.5 PFLOP/s
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes": nbytes,
                     "scope": "whole call"},
        # the method's own count (7 dk dv flops per token and value head)
        # against the fp32 vector peak: a reference figure, not the kernels' unit
        "recurrence_equivalent": {"tflops": tflops, "frac_of_fp32_vector_peak": tflops / FP32_VECTOR_PEAK_TFLOPS},
        "kernel_source_digest": digest,
    }
    if counters and "mfma_busy_cycles_per_call" in counters:
        # matrix-core busy SIMD-cycles of the call's kernels (committed counter
        # summary) over the SIMD-cycles of the call at the nominal clock
        busy = float(counters["mfma_busy_cycles_per_call"])
        out["mfma"] = {"busy_frac": busy / (kms * 1e-3 * CLOCK_HZ * SIMDS), "busy_cycles": busy}
    if case["cu_seqlens"] is not None:
        out["lengths"] = np.diff(case["cu_seqlens"]).tolist()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = prefill_cpu_baseline(case)
    return out


def prefill_cpu_baseline(case):
    """The fp64 oracle on the whole workload (every request and value head),
    once, on the host cores, in tokens/s."""
    import oracle
    from tests.gpu_helpers import oracle_forward
    oracle.build()
    q = case["q"]
    T = q.shape[0] * (q.shape[1] if q.ndim == 4 else 1)
    t0 = time.perf_counter()
    oracle_forward(case)
    elapsed = time.perf_counter() - t0
    return {"value": T / elapsed, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "the whole workload (%d tokens, every request and value head) once, fp64 oracle "
                      "incl. input upcast, %.1f s" % (T, elapsed)}


def cpu_baseline(case, total_bytes):
    """The fp64 oracle on the same decode step (all 256 requests x 32 heads),
    on the host cores."""
    import oracle
    ids = case["slot_ids"]
    g = dict(gate=case["gate"], beta=case["beta"], a_log=case["a_log"], dt_bias=case["dt_bias"],
             initial_state=case["slab"][ids], update_rule="gated_delta", gate_activation="qwen",
             beta_activation="sigmoid")
    oracle.build()
    cores = oracle.num_threads()
    reps, elapsed = 0, 0.0
    while elapsed < 10.0 and reps < 200:
        t0 = time.perf_counter()
        oracle.forward(case["q"], case["k"], case["v"], **g)
        elapsed += time.perf_counter() - t0
        reps += 1
    return {"value": total_bytes * reps / elapsed / 1e9, "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": "%d run(s) of the full decode step (256 requests x 32 heads, 1 token each), "
                      "fp64 oracle incl. input upcast, %.1f s total" % (reps, elapsed)}


def stream_ceiling(reps=20):
    """What plain streaming kernels reach on this device for the decode step's
    byte count: PyTorch's own elementwise kernels reading and writing 512 MiB
    of fp32 (in place, and into a second buffer), median over ``reps``
    event-timed launches.  A reference for the HBM roofline, not part of the
    engine."""
    import torch
    n = 512 * 1024 * 1024 // 4
    x = torch.ones(n, device="cuda")
    y = torch.empty_like(x)
    out = {}
    for name, fn in (("inplace_mul_512MiB", lambda: x.mul_(1.0000001)),
                     ("add_out_512MiB", lambda: torch.add(x, 1.0, out=y))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
        out[name] = {"ms": ms, "GB/s": 2 * n * 4 / (ms * 1e-3) / 1e9}
    del x, y
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--decode-algo", default="auto")
    ap.add_argument("--prefill-algo", default="auto")
    ap.add_argument("--only", choices=["decode", "mtp", "prefill", "varlen", "long", "perkey", "bf16", "ceiling"],
                    default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 256 MiB -> 256 MiB device copy three times, as the "
                         "known-size reference for hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the engine has no multi-GPU path "
              "(requests and heads shard with no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    result = {"metric": METRIC}
    if args.only in (None, "decode"):
        case, d = bench_decode(args)
        pct = d["gbs_kernel"] / HBM_PEAK_GBS
        # value: bytes of exactly `steps` launches over the wall time between two
        # device synchronisations (launch gaps included); roofline.achieved: the
        # same bytes over the mean event-timed duration of one launch
        result.update({
            "value": d["gbs_wall"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": d["wall_s"] * 1e3 / args.steps,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": case["name"], "batch": 256, "tokens_per_request": 1,
                       "num_heads_qk": 16, "num_heads_v": 32, "dk": 128, "dv": 128,
                       "num_slots": 512, "activations": "f16", "state": "f32",
                       "update_rule": "gated_delta", "gate": "qwen raw gate + sigmoid beta",
                       "kernel": d["algo"]},
            "decode": {"kernel_ms": d["kernel_ms"], "gbs_kernel": d["gbs_kernel"],
                       "pct_of_8tbs": 100 * pct, "gbs_wall": d["gbs_wall"],
                       "pct_of_8tbs_wall": 100 * d["gbs_wall"] / HBM_PEAK_GBS,
                       "ms_per_step_wall": d["wall_s"] * 1e3 / args.steps,
                       "tokens_per_s": d["tokens"] / (d["kernel_ms"] * 1e-3),
                       "bytes_per_step": d["bytes_per_step"], "state_bytes_per_step": d["state_bytes"],
                       "kernel_source_digest": d["digest"]},
            "roofline": {"bound": "hbm", "achieved": d["gbs_kernel"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": pct, "traffic": d["traffic"]},
        })
        # the practical reference on this device: plain elementwise kernels that
        # read and write the step's byte count (not part of the timed region)
        ceil = stream_ceiling()
        best = max(x["GB/s"] for x in ceil.values())
        result["decode"]["stream_ceiling_gbs"] = best
        result["decode"]["frac_of_stream_ceiling"] = d["gbs_kernel"] / best
        # the same slots' state bytes with no compute (gdr_slab_stream): a plain
        # copy over the step's own access pattern
        result["decode"]["slab_stream_gbs"] = d["slab_stream_gbs"]
        result["decode"]["slab_stream_ms"] = d["slab_stream_ms"]
        result["decode"]["kernel_ms_over_slab_stream_ms"] = d["kernel_ms"] / d["slab_stream_ms"]
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = cpu_baseline(case, d["bytes_per_step"])
        del case
    if args.only in (None, "mtp"):
        # the same step with 4 tokens per request (speculative / multi-token verify):
        # the state crosses HBM once for all four tokens
        case, d = bench_decode(args, L=4)
        result["decode_mtp"] = {
            "workload": case["name"], "tokens_per_request": 4, "kernel": d["algo"],
            "kernel_ms": d["kernel_ms"], "tokens_per_s": d["tokens"] / (d["kernel_ms"] * 1e-3),
            "gbs_kernel": d["gbs_kernel"], "pct_of_8tbs": 100 * d["gbs_kernel"] / HBM_PEAK_GBS,
            "bytes_per_step": d["bytes_per_step"]}
        del case
    if args.only in (None, "prefill", "varlen"):
        result["prefill"] = bench_prefill(args, "varlen")
    if args.only in (None, "prefill", "long"):
        result["prefill_long"] = bench_prefill(args, "long")
    if args.only in (None, "prefill", "perkey"):
        result["prefill_perkey_erase"] = bench_prefill(args, "perkey")
    if args.only in (None, "prefill", "bf16"):
        # the varlen workload with bf16 activations (beyond the pages' type list)
        result["prefill_bf16"] = bench_prefill(args, "varlen_bf16")
    if args.only == "ceiling":
        result["stream_ceiling"] = stream_ceiling()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
