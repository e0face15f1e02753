"""Request-slot schedules (host logic, CPU only)."""
import math

import pytest

from shared_prefix_stream_amd.batching import continuous_schedule, static_schedule


def _visits(steps, answer_lens):
    seen = {}
    for i, step in enumerate(steps):
        for b, x in enumerate(step):
            if x is not None:
                assert x not in seen, f"{x} scheduled twice"
                seen[x] = (i, b)
    assert set(seen) == {(r, t) for r, a in enumerate(answer_lens) for t in range(a)}
    # a request stays in one slot and takes one step per decode step
    for r, a in enumerate(answer_lens):
        pos = [seen[(r, t)] for t in range(a)]
        assert len({b for _, b in pos}) == 1
        assert [i for i, _ in pos] == list(range(pos[0][0], pos[0][0] + a))
    return seen


LENS = [[8, 128] * 8, [3, 1, 4, 1, 5, 9, 2, 6, 5, 3, 5], [7], [2, 2, 2, 2]]


@pytest.mark.parametrize("lens", LENS)
@pytest.mark.parametrize("B", [1, 2, 4])
def test_schedules_visit_every_request_step_once(lens, B):
    s = static_schedule(lens, B)
    c = continuous_schedule(lens, B)
    _visits(s, lens)
    _visits(c, lens)
    assert all(len(step) == B for step in s + c)
    # static: each group of B lasts as long as its longest answer
    assert len(s) == sum(max(lens[g:g + B]) for g in range(0, len(lens), B))
    # continuous: never longer than static, never shorter than the work allows
    assert math.ceil(sum(lens) / B) <= len(c) <= len(s)
    assert len(c) >= max(lens)


def test_continuous_refills_the_moment_a_slot_frees():
    c = continuous_schedule([1, 3, 2, 2], 2)
    assert c == [[(0, 0), (1, 0)], [(2, 0), (1, 1)], [(2, 1), (1, 2)], [(3, 0), None], [(3, 1), None]]


def test_short_and_long_answers_save_steps():
    # every other request asks for a long answer
    lens = [8, 128] * 8
    assert len(static_schedule(lens, 4)) == 4 * 128
    assert len(continuous_schedule(lens, 4)) < 0.7 * 4 * 128


def test_bad_arguments():
    with pytest.raises(ValueError):
        static_schedule([1, 0], 2)
    with pytest.raises(ValueError):
        continuous_schedule([1], 0)
