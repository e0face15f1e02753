"""Steps whose keys and values exceed the 256 MB last-level cache load the
rows each workgroup reads once with the non-temporal hint (the document
kernel with one query tile per head, the gather without grouped heads).
Parity of each such kernel variant -- every query-tile shape, both head
sizes, fp32 -- against the fp64 oracle on sampled streams, at the agreed
tolerance."""
import numpy as np
import pytest
import torch

import shared_prefix_stream_amd as pp
from oracle import oracle_decode
from tests.gpu_helpers import assert_close, reference, run
from workloads import make_case, multi_case

pytestmark = pytest.mark.gpu

LLC_BYTES = 256 * 1024 * 1024

LARGE = [
    # (P, H, D, doc, dtype): 16-query tiles of 4 waves (P <= 64), 4 waves of
    # 32 queries (P <= 128), 8 waves of 32 (P <= 256); fp32 takes the vector
    # kernel for the document and the gather's fp32 variant
    (48, 32, 64, 33000, torch.bfloat16),
    (100, 32, 64, 33000, torch.bfloat16),
    (200, 32, 64, 33000, torch.bfloat16),
    (48, 32, 128, 17000, torch.bfloat16),
    (100, 32, 128, 17000, torch.bfloat16),
    (16, 32, 128, 9000, torch.float32),
]


@pytest.mark.parametrize("P,H,D,doc,dtype", LARGE)
def test_steps_past_the_last_level_cache(P, H, D, doc, dtype):
    rng = np.random.default_rng(P * 7 + D + doc)
    case = make_case(H, D, doc, rng.integers(1, 21, P).tolist(), rng.integers(0, 11, P).tolist(), dtype=dtype,
                     seed=P + doc, name=f"llc_p{P}_h{H}_d{D}_doc{doc}")
    es = torch.empty(0, dtype=dtype).element_size()
    assert 2 * case.seq_len * H * D * es > LLC_BYTES  # the non-temporal variants run
    streams = sorted({0, P - 1, *rng.choice(P, 4, replace=False).tolist()})
    assert_close(run(case, "decode"), reference(case, streams=streams), streams=streams, what=case.name)


def test_two_requests_past_the_last_level_cache():
    # several requests per launch (each its own caches, request strides in
    # the kernels' addressing) with the non-temporal variants
    case = multi_case(32, 32, 128, 60, [9000, 8000], q_range=(1, 40), a_len=7, seed=21, name="llc_two_requests")
    B, T = case.k.shape[0], case.k.shape[1]
    assert 2 * B * T * 32 * 128 * 2 > LLC_BYTES
    q, k, v, sid = (t.to("cuda:0") for t in (case.q, case.k, case.v, case.stream_id))
    lens = torch.tensor(case.seq_lens, dtype=torch.int32, device="cuda:0")
    out = pp.pp_attn_decode_multi(q, k, v, sid, lens, scale=case.scale)
    torch.cuda.synchronize()
    streams = [0, 17, 38, 59]
    for b in range(B):
        n = case.seq_lens[b]
        ref = oracle_decode(case.q[b], case.k[b, :n], case.v[b, :n], case.stream_id[b].numpy(), n, case.scale,
                            streams=streams)
        assert_close(out[b], ref, streams, what=f"{case.name} request {b}")
