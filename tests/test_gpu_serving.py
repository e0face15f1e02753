"""GPU parity of continuous batching over request slots: retired streams,
idle slots and requests refilled into freed slots, step by step against
the oracle on each request's own data."""
import numpy as np
import pytest
import torch

import shared_prefix_stream_amd as pp
from oracle import oracle_decode
from shared_prefix_stream_amd.batching import continuous_schedule, static_schedule
from tests.gpu_helpers import assert_close, say
from workloads import multi_case, serving_pool

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_retired_streams_give_zeros_and_leave_the_others_alone():
    case = multi_case(8, 2, 128, 11, [900, 400], q_range=(2, 30), a_len=6, seed=21, name="retire")
    q, k, v, sid = (t.to(DEV) for t in (case.q, case.k, case.v, case.stream_id))
    lens = torch.tensor(case.seq_lens, dtype=torch.int32, device=DEV)
    active = torch.ones(2, 11, dtype=torch.int32, device=DEV)
    active[0, [0, 5, 10]] = 0
    active[1, 3] = 0
    for batched in (False, True):
        say(f"  gpu: retire streams batched={batched}")
        full = pp.pp_attn_decode_multi(q, k, v, sid, lens, scale=case.scale, batched=batched)
        part = pp.pp_attn_decode_multi(q, k, v, sid, lens, scale=case.scale, batched=batched, active=active)
        torch.cuda.synchronize()
        on = active.bool()
        assert torch.count_nonzero(part[~on]).item() == 0
        assert torch.equal(part[on].view(torch.int16), full[on].view(torch.int16))


@pytest.mark.parametrize("policy", ["continuous", "static"])
def test_slot_schedule_step_by_step(policy):
    lens = [2, 5, 1, 3, 2]
    B = 2
    pool = serving_pool(lens, P=3, Hq=4, Hkv=2, D=128, seed=23)
    steps = (continuous_schedule if policy == "continuous" else static_schedule)(lens, B)
    T = max(len(x) for x in pool.ids)
    K = torch.zeros(B, T, pool.Hkv, pool.D, dtype=torch.bfloat16, device=DEV)
    V = torch.zeros_like(K)
    sid = torch.full((B, T), -1, dtype=torch.int32, device=DEV)
    q = torch.zeros(B, pool.P, pool.Hq, pool.D, dtype=torch.bfloat16, device=DEV)
    placed = [None] * B
    scale = 1 / np.sqrt(pool.D)
    for i, step in enumerate(steps):
        seq = []
        for b, x in enumerate(step):
            if x is None:
                seq.append(0)
                continue
            r, t = x
            if placed[b] != r:  # the request enters this slot
                n = len(pool.ids[r])
                K[b, :n] = pool.k[r].to(DEV)
                V[b, :n] = pool.v[r].to(DEV)
                sid[b, :n] = torch.from_numpy(pool.ids[r]).to(DEV)
                placed[b] = r
            q[b] = pool.queries(r, t).to(DEV)
            seq.append(pool.base[r] + (t + 1) * pool.P)
        say(f"  gpu: step {i} slots {step} lens {seq}")
        out = pp.pp_attn_decode_multi(q, K, V, sid, torch.tensor(seq, dtype=torch.int32, device=DEV), scale=scale)
        torch.cuda.synchronize()
        for b, x in enumerate(step):
            if x is None:
                assert torch.count_nonzero(out[b]).item() == 0
                continue
            r, t = x
            ref = oracle_decode(pool.queries(r, t), pool.k[r], pool.v[r], pool.ids[r], seq[b], scale)
            assert_close(out[b], ref, what=f"step {i} slot {b} request {r} t {t}")
