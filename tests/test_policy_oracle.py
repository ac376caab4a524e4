"""The oracle's chunk policy against the pages' printed chunk plan."""
import json
import os

import numpy as np
import pytest

from oracle import policy

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "chunk_plan_qwen3_tts.json")))


def test_printed_chunk_plan():
    ramp, steady = tuple(GOLD["ramp"]), GOLD["steady"]
    n = sum(GOLD["new_frames_per_decode"])
    plan = policy.chunk_plan(n, ramp, steady)
    assert plan == GOLD["new_frames_per_decode"]
    pts = policy.decode_points(plan)
    assert pts[:6] == GOLD["decode_points_first_six"]
    ms = [k * GOLD["frame_ms"] for k in plan[:6]]
    assert ms == GOLD["segment_ms_first_six"]
    assert [p * GOLD["frame_ms"] for p in pts[:6]] == GOLD["cumulative_ms_first_six"]


def test_printed_window_counts():
    got = policy.window_frame_counts(GOLD["left_context"], tuple(GOLD["ramp"]), GOLD["steady"])
    assert list(got) == GOLD["window_frame_counts"]


@pytest.mark.parametrize("total,expect", [
    (1, [1]), (2, [1, 1]), (3, [1, 2]), (50, [1, 2, 4, 8, 8, 8, 8, 8, 3]),
    (200, [1, 2, 4] + [8] * 24 + [1]),
])
def test_final_chunk_takes_remainder(total, expect):
    assert policy.chunk_plan(total) == expect


def test_ramp_entries_clamped_to_steady_and_override():
    assert policy.chunk_plan(20, (1, 16, 4), 8) == [1, 8, 4, 7]
    assert policy.chunk_plan(20, (1, 2, 4), 8, initial=5) == [5, 2, 4, 8, 1]
    assert policy.chunk_plan(20, (1, 2, 4), 8, initial=50) == [8, 2, 4, 6]


def test_initial_chunk_size():
    # no request: the fallback; requests above the steady size are capped
    assert policy.initial_chunk_size(None, 8) == 0
    assert policy.initial_chunk_size(None, 8, fallback=3) == 3
    assert policy.initial_chunk_size(5, 8) == 5
    assert policy.initial_chunk_size(np.int64(6), 8) == 6
    assert policy.initial_chunk_size(0, 8) == 0
    assert policy.initial_chunk_size(40, 8) == 8
    assert policy.initial_chunk_size(8, 8) == 8
    with pytest.raises(ValueError):
        policy.initial_chunk_size(3, 0)
    with pytest.raises(ValueError):
        policy.initial_chunk_size(-1, 8)
    with pytest.raises(ValueError):
        policy.initial_chunk_size(None, 8, fallback=-2)
    for bad in ("5", 2.5, True, [1]):
        with pytest.raises(TypeError):
            policy.initial_chunk_size(bad, 8)
