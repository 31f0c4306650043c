"""CPU check of the chunked prefill's chunk plan (which requests get chunk
records, and where), built with g++ from the same header the chunk-table
kernel uses (``csrc/gdr_chunk_plan.hpp``) and run on adversarial cu_seqlens.

The README's cu_seqlens row ("com.microsoft.GatedDeltaNet", Inputs) allows
decreasing and out-of-range entries: each request is clamped to [0, T] and
is empty when its end is not past its start.  After a decreasing entry a
later request can start again from an earlier token, so request ranges can
overlap and their chunk counts can exceed the budget that sizes the
workspace (ceil(T/64) + B).  The plan must never hand out a chunk index at
or past that budget, every chunk it hands out must lie inside its request,
and every request with tokens must either own all of its chunks or be
marked for the recurrent kernel.
"""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_token_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "host", "chunk_plan_check.cpp")


@pytest.fixture(scope="module")
def plan_exe(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("plan") / "chunk_plan_check")
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-Wall", "-I" + CSRC, SRC, "-o", exe])
    return exe


def run_plan(exe, cases):
    text = "".join("%d %d %s\n" % (T, len(cu) - 1, " ".join(str(int(c)) for c in cu)) for T, cu in cases)
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout.splitlines()
    res = []
    for line in out:
        left, right = line.split("|")
        nums = [int(x) for x in left.split()]
        res.append((nums[0], np.array(nums[1:], dtype=np.int64), np.array([int(x) for x in right.split()], dtype=np.int64)))
    return res


def ranges(T, cu):
    """Request ranges by the README rule, written out independently."""
    out = []
    for b in range(len(cu) - 1):
        s = min(max(int(cu[b]), 0), T)
        e = min(max(int(cu[b + 1]), 0), T)
        out.append((s, max(s, e)))
    return out


def check_plan(T, cu, budget, off, denied):
    B = len(cu) - 1
    rr = ranges(T, cu)
    n = [-(-(e - s) // 64) for s, e in rr]
    assert budget == -(-T // 64) + B
    assert off[0] == 0 and np.all(np.diff(off) >= 0), "chunk offsets must not decrease"
    assert off[B] <= budget, "chunk table past the budget: %d > %d" % (off[B], budget)
    for b in range(B):
        if denied[b]:
            assert n[b] > 0, "only requests with tokens are handed over"
            assert off[b + 1] == off[b], "a handed-over request owns no chunk"
        else:
            assert off[b + 1] - off[b] == n[b], "request %d must own all %d of its chunks" % (b, n[b])
    # the prologue's view: chunk ci belongs to the largest b with off[b] <= ci;
    # the first and last chunk of every owner map back to it and start inside it
    for owner in range(B):
        if off[owner + 1] == off[owner]:
            continue
        for ci in (int(off[owner]), int(off[owner + 1]) - 1):
            b = int(np.searchsorted(off[:B], ci, side="right")) - 1
            assert b == owner and not denied[b]
            s, e = rr[b]
            t0 = s + (ci - off[b]) * 64
            assert s <= t0 < e, "chunk %d of request %d starts outside it" % (ci, b)
    if all(cu[i] <= cu[i + 1] for i in range(B)):
        assert not np.any(denied), "a monotone cu_seqlens hands nothing over"
    return n


def test_overlapping_requests_stay_within_budget(plan_exe):
    # three full-length requests restarting at token 0: 48 chunks against a 22-chunk budget
    T, cu = 1024, [0, 1024, 0, 1024, 0, 1024, 0]
    (budget, off, denied), = run_plan(plan_exe, [(T, cu)])
    n = check_plan(T, cu, budget, off, denied)
    assert sum(n) == 48 and budget == 22
    assert list(denied) == [0, 0, 1, 0, 1, 0] and list(off) == [0, 16, 16, 16, 16, 16, 16]


def test_adversarial_cu_seqlens(plan_exe):
    rng = np.random.Generator(np.random.PCG64(2024))
    cases = []
    for T in (1, 63, 64, 65, 1000, 4096, 65536):
        for B in (1, 2, 7, 64, 300, 700):
            cases.append((T, rng.integers(-T // 2, 3 * T // 2 + 2, B + 1)))  # anything goes
            cases.append((T, np.sort(rng.integers(0, T + 1, B + 1))))        # monotone
            zig = np.where(np.arange(B + 1) % 2 == 0, 0, T)
            cases.append((T, zig))                                            # full overlaps
            cases.append((T, np.maximum.accumulate(rng.integers(0, T + 1, B + 1)) - rng.integers(0, 2, B + 1) * 70))
    results = run_plan(plan_exe, cases)
    handed = 0
    for (T, cu), (budget, off, denied) in zip(cases, results):
        check_plan(T, list(cu), budget, off, denied)
        handed += int(denied.sum())
    assert handed > 0, "the adversarial inputs must exercise the hand-over"


def test_large_overlap_sums_do_not_wrap(plan_exe):
    # 3000 requests each covering all of a 2^30-token range: the uncapped sum
    # of chunk counts (3000 * 2^24) is far past 32 bits
    T = 1 << 30
    cu = [0 if i % 2 == 0 else T for i in range(3001)]
    (budget, off, denied), = run_plan(plan_exe, [(T, cu)])
    assert off[-1] <= budget
    assert denied[0] == 0 and denied[2] == 1 and all(denied[2::2])
