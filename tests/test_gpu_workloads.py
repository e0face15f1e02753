"""GPU parity on the ragged stress sweep and on the multi-step decode loop.

Ragged sweep: H=32, d=128, bf16, document lengths {1, 4097, 32768} x
streams {1, 7, 128, 512}, questions uniform 1-128, answers uniform 0-64,
1% of K elements x50 (peaked softmax).  Checked on every stream up to 64
streams and on 64 sampled streams past that, all heads.

Long answers: an 8k-token document with 128 questions and 128 to 1,024
answer tokens per stream already in the cache, sampled streams, both entry
points.

Decode loop: 32 answer steps; at each step every stream appends one K/V
slot (its own id) and then attends, over independent layers.  A reduced copy
(512-token document, 16 streams, 4 layers) is checked at every step; the
full-size loop (12000-token document, 256 streams) at sampled (layer, step)
points and streams."""
import numpy as np
import pytest
import torch

import shared_prefix_stream_amd as pp
from oracle import oracle_decode
from tests.gpu_helpers import assert_close, reference, run, say
from workloads import decode_loop_layout, decode_loop_step_inputs, long_answer_case, ragged_case

pytestmark = pytest.mark.gpu


def _sample_streams(P, rng, n=8):
    if P <= n:
        return list(range(P))
    pick = set([0, P - 1]) | set(rng.choice(P, n - 2, replace=False).tolist())
    return sorted(pick)


@pytest.mark.parametrize("doc", [1, 4097, 32768])
@pytest.mark.parametrize("P", [1, 7, 128, 512])
def test_ragged_sweep(doc, P):
    case = ragged_case(doc, P, seed=5000 + doc + P)
    # every stream up to 64; 64 sampled ones (first and last included) past that
    streams = _sample_streams(P, np.random.default_rng(doc * 7 + P), n=64)
    ref = reference(case, streams)
    for entry in ("decode", "batched"):
        assert_close(run(case, entry), ref, streams, what=f"{case.name} {entry}")


@pytest.mark.parametrize("answer_len", [128, 1024])
def test_long_answers(answer_len):
    case = long_answer_case(answer_len, seed=6000 + answer_len)
    streams = _sample_streams(case.P, np.random.default_rng(answer_len), n=6)
    ref = reference(case, streams)
    for entry in ("decode", "batched"):
        assert_close(run(case, entry), ref, streams, what=f"{case.name} {entry}")


def _decode_loop(doc, P, steps, layers, H, D, seed, check, sample):
    ids, q_lens, base = decode_loop_layout(doc, P, steps, seed)
    cap = len(ids)
    sid = torch.from_numpy(ids).cuda()
    scale = 1.0 / np.sqrt(D)
    rng = np.random.default_rng(seed)
    for layer in layers:
        K = torch.empty(cap, H, D, dtype=torch.bfloat16, device="cuda")
        V = torch.empty_like(K)
        for t in range(steps):
            inp = decode_loop_step_inputs(H, D, P, cap, layer, t, seed, base_len=base)
            if t == 0:
                K[:base] = inp["k0"].cuda()
                V[:base] = inp["v0"].cuda()
            K[base + t * P: base + (t + 1) * P] = inp["k_new"].cuda()
            V[base + t * P: base + (t + 1) * P] = inp["v_new"].cuda()
            seq_len = base + (t + 1) * P
            q = inp["q"].cuda()
            out = pp.pp_attn_decode(q, K, V, sid, seq_len=seq_len, scale=scale)
            if check(layer, t):
                torch.cuda.synchronize()
                streams = sample(P, rng)
                say(f"  check layer {layer} step {t} seq_len {seq_len} streams {len(streams)}")
                ref = oracle_decode(inp["q"], K[:seq_len].cpu(), V[:seq_len].cpu(), ids, seq_len, scale,
                                    streams=streams)
                assert_close(out, ref, streams, what=f"layer {layer} step {t}")
                if t in (0, steps - 1):
                    outb = pp.pp_attn_decode_batched(q, K, V, sid, seq_len=seq_len, scale=scale)
                    torch.cuda.synchronize()
                    assert_close(outb, ref, streams, what=f"batched layer {layer} step {t}")


def test_decode_loop_reduced_every_step():
    _decode_loop(doc=512, P=16, steps=32, layers=range(4), H=32, D=128, seed=77,
                 check=lambda layer, t: True, sample=lambda P, rng: list(range(P)))


def test_decode_loop_full_size_sampled():
    picks = {(0, 0), (0, 31), (31, 31), (31, 0), (0, 13), (31, 22)}
    _decode_loop(doc=12000, P=256, steps=32, layers=[0, 31], H=32, D=128, seed=1003,
                 check=lambda layer, t: (layer, t) in picks, sample=lambda P, rng: _sample_streams(P, rng, 6))
