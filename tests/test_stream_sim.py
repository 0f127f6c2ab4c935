"""The serving leg's continuous-batching bookkeeping, on the host with made-up step times:
time to first token and inter-token latency are counted as the request-stream measurement
defines them (the pages' scheduling-stability comparison, Technical Summary 3.2)."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_one_request_by_hand():
    # arrives at 5 ms; 1024 prompt tokens in chunks of 512; 3 output tokens; 10 ms per step
    res = bench.simulate_stream([(5.0, 1024, 3)], lambda n: 512, lambda c, n: 10.0)
    assert res["ttft"] == [20.0]           # two chunk steps after the arrival
    assert res["itl"] == [10.0, 10.0]      # two more tokens, one step each
    assert res["steps"] == 4 and res["makespan_ms"] == 45.0
    assert res["chunks"] == {512: 2}


def test_chunk_is_capped_by_the_prompt_left():
    res = bench.simulate_stream([(0.0, 768, 1)], lambda n: 512, lambda c, n: float(c))
    assert res["chunks"] == {512: 1, 256: 1}
    assert res["ttft"] == [768.0] and res["itl"] == []


def test_two_requests_overlap_decode_with_prefill():
    # step time = 1 ms per 256 prompt tokens + 0.5 ms per decoding request
    step = lambda c, n: c / 256.0 + 0.5 * n  # noqa: E731
    res = bench.simulate_stream([(0.0, 512, 3), (0.0, 512, 2)], lambda n: 256, step)
    # r0: prefill steps at t = 1, 2 -> first token at 2.  r1: prefill steps (with r0
    # decoding) at 3.5, 5 -> first token at 5; r0's tokens at 3.5 and 5 (done).
    # r1's last token one decode step later at 5.5.
    assert res["ttft"] == [2.0, 5.0]
    assert res["itl"] == [1.5, 1.5, 0.5]
    assert res["makespan_ms"] == 5.5 and res["steps"] == 5


def test_batch_cap_holds_back_prefill():
    calls = []

    def step(c, n):
        calls.append((c, n))
        return 1.0
    bench.simulate_stream([(0.0, 256, 3), (0.0, 256, 2)], lambda n: 256, step, max_batch=1)
    # the second prompt waits until the first request has finished decoding
    assert calls == [(256, 0), (0, 1), (0, 1), (256, 0), (0, 1)]


def test_policy_sees_the_decode_count():
    seen = []

    def choose(n):
        seen.append(n)
        return 1024 if n == 0 else 256
    bench.simulate_stream([(0.0, 512, 2), (0.0, 1024, 2)], choose, lambda c, n: 1.0)
    assert seen[0] == 0 and 1 in seen


def test_summary_counts_slo_violations():
    res = {"ttft": [10.0, 30.0], "itl": [5.0, 20.0, 25.0, 10.0], "steps": 6, "makespan_ms": 100.0,
           "chunks": {512: 3}}
    s = bench.stream_summary(res, (16.0, 22.0), [(0.0, 512, 3), (0.0, 1024, 3)])
    assert s["itl_over_16ms_pct"] == 50.0 and s["itl_over_22ms_pct"] == 25.0
    assert s["ttft_ms_mean"] == 20.0 and s["tokens_per_s"] == pytest.approx(1e3 * 1542 / 100.0)
