"""GPU parity of several requests per launch with grouped key/value heads
(pp_attn_decode_multi and its per-question baseline) against the oracle,
request by request."""
import numpy as np
import pytest
import torch

import shared_prefix_stream_amd as pp
from oracle import oracle_decode
from tests.gpu_helpers import assert_close, say
from workloads import multi_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(case, batched=False, lens=None):
    q, k, v, sid = (t.to(DEV) for t in (case.q, case.k, case.v, case.stream_id))
    seq_lens = torch.tensor(case.seq_lens if lens is None else lens, dtype=torch.int32, device=DEV)
    say(f"  gpu: pp_attn_decode_multi{'_batched' if batched else ''} {case.name} B={q.shape[0]} P={case.P} "
        f"Hq={case.Hq} Hkv={case.Hkv} D={case.D} T={k.shape[1]} lens={seq_lens.tolist()}")
    out = pp.pp_attn_decode_multi(q, k, v, sid, seq_lens, scale=case.scale, batched=batched)
    torch.cuda.synchronize()
    return out


def _check(case, out, lens=None, streams=None, what=""):
    lens = case.seq_lens if lens is None else lens
    for b in range(case.q.shape[0]):
        n = max(0, min(lens[b], case.k.shape[1]))
        if n == 0:
            assert torch.count_nonzero(out[b]).item() == 0, f"{what} request {b}: empty request must give zeros"
            continue
        ref = oracle_decode(case.q[b], case.k[b, :n], case.v[b, :n], case.stream_id[b].numpy(), n, case.scale,
                            streams=streams)
        assert_close(out[b], ref, streams, what=f"{what} request {b}")


CASES = {
    # name: (Hq, Hkv, D, P, doc_lens, dtype)
    "gqa4_one_request": (8, 2, 128, 13, [700], torch.bfloat16),
    "gqa7_qwen_shape": (28, 4, 128, 64, [2100], torch.bfloat16),
    "three_requests_mha": (4, 4, 128, 9, [0, 1500, 333], torch.bfloat16),
    "three_requests_gqa4": (8, 2, 64, 21, [260, 1000, 64], torch.bfloat16),
    "f32_two_requests_gqa2": (4, 2, 64, 6, [300, 129], torch.float32),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("batched", [False, True])
def test_multi_matches_the_oracle(name, batched):
    Hq, Hkv, D, P, docs, dtype = CASES[name]
    case = multi_case(Hq, Hkv, D, P, docs, q_range=(1, 40), a_len=7, dtype=dtype, seed=len(name), name=name)
    _check(case, _run(case, batched), what=f"{name} {'baseline' if batched else 'parallel'}")


def test_single_request_equals_pp_attn_decode():
    case = multi_case(8, 8, 128, 17, [1200], q_range=(4, 30), a_len=5, seed=3, name="b1")
    out = _run(case)
    n = case.seq_lens[0]
    ref = pp.pp_attn_decode(case.q[0].to(DEV), case.k[0, :n].contiguous().to(DEV), case.v[0, :n].contiguous().to(DEV),
                            case.stream_id[0, :n].contiguous().to(DEV), seq_len=n, scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out[0].view(torch.int16), ref.view(torch.int16))


def test_device_lengths_are_clamped():
    # a request of length 0 (its streams see nothing) and one whose length
    # exceeds the cache (clamped to it)
    case = multi_case(4, 2, 128, 5, [400, 300, 200], q_range=(2, 9), a_len=3, seed=4, name="clamp")
    T = case.k.shape[1]
    lens = [0, 10**9, case.seq_lens[2]]
    # the clamped request reads every row of the cache: give it finite rows
    k = case.k.clone()
    v = case.v.clone()
    k[1] = torch.nan_to_num(k[1], nan=0.25)
    v[1] = torch.nan_to_num(v[1], nan=-0.5)
    case.k, case.v = k, v
    out = _run(case, lens=lens)
    _check(case, out, lens=[0, T, case.seq_lens[2]], what="clamped lengths")


def test_multi_full_size_sampled():
    # four requests of 64 streams on 16k-token documents, 28 query heads
    # sharing 4 key/value heads
    case = multi_case(28, 4, 128, 64, [16384, 16384, 12000, 16384], q_range=(8, 48), a_len=31, seed=1007,
                      name="qwen_shape_4x64")
    out = _run(case)
    streams = [0, 17, 40, 63]
    _check(case, out, streams=streams, what="4 requests x 64 streams, 28/4 heads")


def test_single_stream_single_head_requests():
    case = multi_case(1, 1, 64, 1, [5, 0, 130, 1, 64], q_range=(1, 3), a_len=2, seed=31, name="p1h1")
    _check(case, _run(case), what="P=1 H=1")
    _check(case, _run(case, batched=True), what="P=1 H=1 baseline")
