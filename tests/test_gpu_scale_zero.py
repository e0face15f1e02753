"""GPU parity at a zero scale (+0 and -0), through the C ABI.

With scale 0 every visible key gets the same logit, so each output row is
the plain mean of the stream's visible V rows (the header's definition of
the softmax over the visible set).  Masked keys must still get weight 0:
the document length 4097 leaves a ragged last tile in a document split, and
the prefill masks keys above the diagonal of every causal tile, so these
cases check that no masked score is scaled into NaN."""
import numpy as np
import pytest
import torch

import shared_prefix_stream_amd as pp
from oracle import oracle_append_step, oracle_prefill
from tests.gpu_helpers import assert_close, reference, run, say
from workloads import canonical_layout, make_case, prefill_case

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALES = [0.0, -0.0]


def _sign(x):
    return "-0" if np.signbit(x) else "+0"


def _decode_case(scale, dtype=torch.bfloat16, D=128):
    rng = np.random.default_rng(4097)
    P = 37
    case = make_case(4, D, 4097, rng.integers(1, 30, P).tolist(), rng.integers(0, 9, P).tolist(), dtype=dtype,
                     seed=4097, name=f"scale{_sign(scale)}_doc4097_p{P}_{str(dtype)[6:]}_d{D}")
    case.scale = scale
    return case


@pytest.mark.parametrize("entry", ["decode", "batched"])
@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 64)])
def test_decode_at_zero_scale(entry, scale, dtype, D):
    case = _decode_case(scale, dtype, D)
    ref = reference(case)
    # the oracle's own closed form here: the mean of the visible V rows
    v = case.v.double().numpy()
    ids = case.stream_id.numpy()[: case.seq_len]
    for s in (0, case.P - 1):
        vis = np.nonzero((ids == 0) | (ids == s + 1))[0]
        np.testing.assert_allclose(ref[s], v[vis].mean(axis=0), rtol=1e-12, atol=1e-12)
    assert_close(run(case, entry), ref, what=case.name)


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_at_zero_scale(scale, dtype):
    q_lens = np.random.default_rng(5).integers(1, 60, 11).tolist()
    case = prefill_case(2, 128 if dtype == torch.bfloat16 else 64, 4097, q_lens, dtype=dtype, seed=4098,
                        name=f"prefill_scale{_sign(scale)}")
    q, k, v, sid = (t.to(DEV) for t in (case.q, case.k, case.v, case.stream_id))
    say(f"  gpu: pp_attn_prefill {case.name} T={case.seq_len} {dtype}")
    out = pp.pp_attn_prefill(q, k, v, sid, seq_len=case.seq_len, scale=scale)
    torch.cuda.synchronize()
    # every query slot of the document, its first and last causal tile, and every question slot
    rows = sorted(set(list(range(0, 300)) + list(range(3800, case.seq_len))))
    ref = oracle_prefill(case.q, case.k, case.v, case.stream_id.numpy(), case.seq_len, scale, rows=rows)
    got = out[: case.seq_len].double().cpu().numpy()
    assert np.isfinite(got).all(), "non-finite prefill output"
    assert_close(got[rows], ref[rows], what=case.name)


@pytest.mark.parametrize("scale", SCALES)
def test_appending_step_at_zero_scale(scale):
    P, H, D = 9, 4, 128
    rng = np.random.default_rng(4099)
    ids0, _ = canonical_layout(4097, rng.integers(1, 40, P).tolist(), rng.integers(0, 12, P).tolist())
    T0 = len(ids0)
    cap = T0 + P + 3
    g = torch.Generator().manual_seed(4099)
    k = torch.randn(cap, H, D, generator=g).to(torch.bfloat16)
    v = torch.randn(cap, H, D, generator=g).to(torch.bfloat16)
    q = torch.randn(P, H, D, generator=g).to(torch.bfloat16)
    kn, vn = (torch.randn(P, H, D, generator=g).to(torch.bfloat16) for _ in range(2))
    ids = np.concatenate([ids0, np.zeros(cap - T0, dtype=np.int32)]).astype(np.int32)
    kg, vg = k.to(DEV), v.to(DEV)
    sid = torch.from_numpy(ids).to(DEV)
    say(f"  gpu: pp_attn_decode_append scale {_sign(scale)} T0={T0} P={P}")
    plan = pp.pp_step_plan(sid, torch.tensor([T0], dtype=torch.int32, device=DEV), P, max_seq_len=cap)
    out = pp.pp_attn_decode_append(q.to(DEV), kn.to(DEV), vn.to(DEV), kg, vg, sid, plan, scale=scale,
                                   rope_base=1e4)
    torch.cuda.synchronize()
    r = oracle_append_step(q, kn, vn, k, v, ids, T0, scale, 1e4, store_bf16=True)
    assert_close(out, r["out"], what=f"append scale {_sign(scale)}")
