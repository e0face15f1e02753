"""Request-slot schedules for serving several Parallel Prompting requests.

A server keeps B request slots in one pp_attn_decode_multi launch.  Every
decode step advances each busy slot's request by one answer token per stream.
Two ways to refill the slots (Parallel Prompting project page, "Continuous
batching"):

* static: B requests start together and the next B start only when the
  slowest of them has finished;
* continuous: a slot takes the next waiting request as soon as its own
  request has finished, so short answers never wait for long ones.

Only the bookkeeping lives here (which request sits in which slot at which
of its steps); the attention of each step is one library call whose per-slot
lengths (and retired streams) follow from this schedule.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

__all__ = ["Step", "static_schedule", "continuous_schedule"]

# One decode step: per slot, (request, its answer step t) or None for an
# idle slot.  At its step t a request has t + 1 answer tokens per stream in
# the cache (the step's own token is appended before it attends).
Step = List[Optional[Tuple[int, int]]]


def _check(answer_lens: Sequence[int], B: int) -> None:
    if B < 1:
        raise ValueError("B must be >= 1")
    if any(a < 1 for a in answer_lens):
        raise ValueError("every request decodes at least one token")


def static_schedule(answer_lens: Sequence[int], B: int) -> List[Step]:
    """Requests in order, B at a time; a group runs until its longest answer
    is done, finished slots idling meanwhile."""
    _check(answer_lens, B)
    steps: List[Step] = []
    for g in range(0, len(answer_lens), B):
        group = list(range(g, min(g + B, len(answer_lens))))
        for t in range(max(answer_lens[r] for r in group)):
            steps.append([(r, t) if t < answer_lens[r] else None for r in group] + [None] * (B - len(group)))
    return steps


def continuous_schedule(answer_lens: Sequence[int], B: int) -> List[Step]:
    """Requests in order; a slot whose request finished takes the next one
    before the following step."""
    _check(answer_lens, B)
    nxt = 0
    slot: List[Optional[List[int]]] = [None] * B  # [request, next step]
    steps: List[Step] = []
    while True:
        for b in range(B):
            if slot[b] is None and nxt < len(answer_lens):
                slot[b] = [nxt, 0]
                nxt += 1
        if all(x is None for x in slot):
            return steps
        steps.append([None if x is None else (x[0], x[1]) for x in slot])
        for b in range(B):
            x = slot[b]
            if x is not None:
                x[1] += 1
                if x[1] == answer_lens[x[0]]:
                    slot[b] = None
