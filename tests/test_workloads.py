"""The seeded input generators: determinism, layout and encoding (CPU only)."""
import numpy as np
import torch

from workloads import (canonical_layout, decode_loop_layout, decode_loop_step_inputs, make_case,
                       permute_tail, ragged_case)


def test_layout_questions_contiguous_answers_interleaved():
    ids, own = canonical_layout(3, [2, 1, 3], [2, 0, 1])
    assert ids.tolist() == [0, 0, 0, 1, 1, 2, 3, 3, 3, 1, 3, 1]
    assert [o.tolist() for o in own] == [[3, 4, 9, 11], [5], [6, 7, 8, 10]]


def test_same_seed_same_bytes():
    a = make_case(2, 64, 10, [2, 3], [1, 1], seed=5)
    b = make_case(2, 64, 10, [2, 3], [1, 1], seed=5)
    c = make_case(2, 64, 10, [2, 3], [1, 1], seed=6)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert not torch.equal(a.k.view(torch.int16), c.k.view(torch.int16))


def test_bf16_is_round_to_nearest_even():
    c = make_case(1, 64, 4, [1], [0], seed=1)
    rng = np.random.Generator(np.random.PCG64(1))
    q32 = rng.standard_normal((1, 1, 64), dtype=np.float32)
    bits = q32.view(np.uint32).astype(np.uint64)
    rne = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(c.q.view(torch.int16).numpy().view(np.uint16), rne)


def test_outlier_rate_about_one_percent():
    c = ragged_case(4097, 7, seed=3, H=4, D=64)
    big = (c.k[: c.seq_len].float().abs() > 8).float().mean().item()
    assert 0.006 < big < 0.014


def test_extra_capacity_is_poisoned():
    c = make_case(2, 64, 4, [1, 1], [1, 1], seed=2, extra_capacity=5)
    assert c.k.shape[0] == c.seq_len + 5
    assert torch.isnan(c.k[c.seq_len:].float()).all()
    assert (c.stream_id[c.seq_len:] < 0).all()


def test_permute_tail_keeps_owner_rows():
    c = make_case(2, 64, 6, [3, 2], [2, 3], dtype=torch.float32, seed=4)
    p = permute_tail(c, 9)
    assert torch.equal(p.k[: c.doc_len], c.k[: c.doc_len])
    for s in range(c.P):
        assert sorted(p.stream_id[p.own_slots[s]].tolist()) == [s + 1] * len(c.own_slots[s])
        a = c.k[torch.from_numpy(c.own_slots[s])]
        b = p.k[torch.from_numpy(p.own_slots[s])]
        assert sorted(map(tuple, a.reshape(len(a), -1).tolist())) == sorted(map(tuple, b.reshape(len(b), -1).tolist()))


def test_decode_loop_inputs_regenerate_independently():
    ids, q_lens, base = decode_loop_layout(100, 4, 3, seed=1)
    assert len(ids) == base + 4 * 3
    a = decode_loop_step_inputs(2, 64, 4, len(ids), layer=1, step=2, seed=1)
    b = decode_loop_step_inputs(2, 64, 4, len(ids), layer=1, step=2, seed=1)
    assert torch.equal(a["q"].view(torch.int16), b["q"].view(torch.int16))
    assert "k0" not in a
