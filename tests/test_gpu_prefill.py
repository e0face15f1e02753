"""GPU parity of the prefill (every slot of the packed request a query,
causal under the stream rule) against the prefill oracle: every row at sizes
that span several query and key tiles with ragged ends, sampled rows at the
16k-document shape."""
import numpy as np
import pytest
import torch

import shared_prefix_stream_amd as pp
from oracle import oracle_prefill
from tests.gpu_helpers import assert_close, say
from workloads import prefill_case, prefill_doc16k_p256

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(case):
    q, k, v, sid = (t.to(DEV) for t in (case.q, case.k, case.v, case.stream_id))
    say(f"  gpu: pp_attn_prefill {case.name} T={case.seq_len} doc={case.doc_len} H={case.H} D={case.D} "
        f"{case.q.dtype}")
    out = pp.pp_attn_prefill(q, k, v, sid, seq_len=case.seq_len, scale=case.scale)
    torch.cuda.synchronize()
    return out


def _ref(case, rows=None):
    return oracle_prefill(case.q, case.k, case.v, case.stream_id.numpy(), case.seq_len, case.scale, rows=rows)


def _rng_lens(seed, P, lo, hi):
    return np.random.default_rng(seed).integers(lo, hi + 1, P).tolist()


CASES = {
    # name: (H, D, doc, P, q range, dtype, shuffle, answers)
    "bf16_d128_doc700": (4, 128, 700, 13, (1, 40), torch.bfloat16, False, None),
    "bf16_d128_doc700_shuffled": (4, 128, 700, 13, (1, 40), torch.bfloat16, True, None),
    "bf16_d64_doc300_answers": (2, 64, 300, 7, (1, 20), torch.bfloat16, False, 5),
    "bf16_d128_no_document": (2, 128, 0, 9, (3, 50), torch.bfloat16, False, None),
    "bf16_d128_document_only": (2, 128, 777, 0, (1, 1), torch.bfloat16, False, None),
    "bf16_d128_small_t40": (2, 128, 17, 3, (2, 9), torch.bfloat16, False, None),
    "bf16_d128_small_t100": (2, 128, 60, 4, (2, 12), torch.bfloat16, False, None),
    "f32_d64_doc500": (2, 64, 500, 6, (1, 30), torch.float32, False, None),
    "f32_d128_doc300_shuffled": (2, 128, 300, 5, (1, 30), torch.float32, True, 3),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_matches_the_oracle(name):
    H, D, doc, P, (lo, hi), dtype, shuffle, ans = CASES[name]
    q_lens = _rng_lens(len(name), P, lo, hi)
    case = prefill_case(H, D, doc, q_lens, dtype=dtype, seed=len(name) * 7, shuffle_tail=shuffle,
                        a_lens=None if ans is None else [ans] * P, name=name)
    out = _run(case)
    assert_close(out[: case.seq_len], _ref(case), what=name)


def test_prefill_is_deterministic():
    case = prefill_case(4, 128, 1200, _rng_lens(5, 11, 4, 40), seed=5, name="determinism")
    a = _run(case)
    b = _run(case)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_prefill_foreign_ids():
    # ids outside the streams: each such slot sees the document and the slots
    # carrying its own id, like a stream
    case = prefill_case(2, 128, 200, _rng_lens(9, 5, 3, 20), seed=9, shuffle_tail=True, name="foreign")
    sid = case.stream_id.clone()
    rng = np.random.default_rng(9)
    pick = rng.choice(np.arange(200, case.seq_len), 12, replace=False)
    sid[pick] = torch.from_numpy(rng.choice([-3, 77], 12).astype(np.int32))
    case.stream_id = sid
    out = _run(case)
    assert_close(out[: case.seq_len], _ref(case), what="foreign ids")


def test_prefill_full_size_sampled():
    case = prefill_doc16k_p256()
    T, doc = case.seq_len, case.doc_len
    out = _run(case)
    ids = case.stream_id.numpy()
    rng = np.random.default_rng(1)
    rows = {0, 1, 63, 64, 255, 256, 257, 4095, 4096, doc - 257, doc - 256, doc - 1, doc, doc + 1, T - 1}
    rows |= set(rng.choice(doc, 6, replace=False).tolist()) | set(rng.choice(np.arange(doc, T), 8, replace=False).tolist())
    for s in (0, 127, 255):  # first and last question slot of a few streams
        own = np.flatnonzero(ids == s + 1)
        rows |= {int(own[0]), int(own[-1])}
    rows = sorted(rows)
    say(f"  checking {len(rows)} rows of {T}")
    ref = _ref(case, rows=rows)
    assert_close(out[rows], ref[rows], what="prefill 16k document, 256 questions")


@pytest.mark.parametrize("first_id", [0, 1])
def test_prefill_single_slot(first_id):
    case = prefill_case(2, 64, 1 if first_id == 0 else 0, [] if first_id == 0 else [1], seed=2, name="one slot")
    assert case.seq_len == 1
    out = _run(case)
    # one visible key (itself): the output is its value
    assert torch.equal(out.cpu(), case.v)


@pytest.mark.parametrize("Hq,Hkv,D,dtype", [(8, 2, 128, torch.bfloat16), (7, 1, 64, torch.bfloat16),
                                          (4, 2, 64, torch.float32)])
def test_prefill_grouped_heads(Hq, Hkv, D, dtype):
    case = prefill_case(Hq, D, 650, _rng_lens(Hq, 9, 1, 40), dtype=dtype, seed=Hq * 3, shuffle_tail=True,
                        name=f"gqa{Hq}x{Hkv}", Hkv=Hkv)
    out = _run(case)
    assert_close(out[: case.seq_len], _ref(case), what=f"prefill {Hq}/{Hkv} heads")


def test_prefill_grouped_heads_full_size_sampled():
    # the 16k-token document with 256 questions, 28 query heads sharing 4
    case = prefill_case(28, 128, 16384, _rng_lens(1, 256, 8, 48), seed=1009, name="qwen_shape_prefill", Hkv=4)
    T, doc = case.seq_len, case.doc_len
    out = _run(case)
    rows = sorted({0, 255, 256, doc - 1, doc, doc + 1, (doc + T) // 2, T - 1} |
                  set(np.random.default_rng(2).choice(T, 8, replace=False).tolist()))
    ref = _ref(case, rows=rows)
    assert_close(out[rows], ref[rows], what="prefill 28/4 heads, 16k document")

