"""Pins of the prefill oracle to facts other than itself (CPU only), and a
check that plausible mistakes planted in a copy of its source fail them."""
import json
import os
import types

import numpy as np
import pytest
import torch

from oracle import oracle_decode, oracle_prefill, prefill_visible
from workloads import canonical_layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "pp_prefill_oracle.py")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _sdpa_causal(q, k, v, scale):
    """torch's causal scaled_dot_product_attention in float64, [T, H, d]."""
    t = [torch.from_numpy(np.asarray(x, dtype=np.float64)).permute(1, 0, 2).unsqueeze(0) for x in (q, k, v)]
    o = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True, scale=scale)
    return o.squeeze(0).permute(1, 0, 2).numpy()


def _rand(rng, T, H, d):
    return (rng.standard_normal((T, H, d)) for _ in range(3))


def test_golden_prefill_mask_figure(mod=None):
    m = mod or types.SimpleNamespace(prefill_visible=prefill_visible)
    g = _load("prefill_mask_figure_doc3_p3.json")
    ids = np.array(g["stream_id"])
    for i, want in enumerate(g["visible"]):
        assert m.prefill_visible(ids, i).tolist() == want, i


@pytest.mark.parametrize("T", [1, 7, 40])
def test_document_only_is_causal_attention(T):
    rng = np.random.default_rng(T)
    q, k, v = _rand(rng, T, 3, 8)
    got = oracle_prefill(q, k, v, np.zeros(T, dtype=np.int32), T, 0.4)
    np.testing.assert_allclose(got, _sdpa_causal(q, k, v, 0.4), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_each_question_prefilled_alone(seed):
    # the page's claim, at prefill: a stream's rows equal the causal
    # attention of the sequence "document, then this stream alone"
    rng = np.random.default_rng(20 + seed)
    P = int(rng.integers(1, 6))
    ids, _ = canonical_layout(int(rng.integers(0, 12)), rng.integers(1, 6, P).tolist(), rng.integers(0, 4, P).tolist())
    if seed == 2:  # streams' slots shuffled past the document, one late document slot
        d0 = int(np.count_nonzero(np.cumprod(ids == 0)))
        tail = np.concatenate([ids[d0:], [0]])
        rng.shuffle(tail)
        ids = np.concatenate([ids[:d0], tail]).astype(np.int32)
    T = len(ids)
    q, k, v = _rand(rng, T, 2, 8)
    got = oracle_prefill(q, k, v, ids, T, 0.35)
    for s in range(P):
        mine = np.flatnonzero((ids == 0) | (ids == s + 1))
        alone = _sdpa_causal(q[mine], k[mine], v[mine], 0.35)
        own = np.flatnonzero(ids[mine] == s + 1)
        np.testing.assert_allclose(got[mine[own]], alone[own], rtol=1e-12, atol=1e-12)


def test_last_slot_of_each_stream_is_its_decode_step():
    rng = np.random.default_rng(4)
    ids, _ = canonical_layout(9, [3, 2, 4], [2, 1, 0])
    T = len(ids)
    q, k, v = _rand(rng, T, 2, 8)
    got = oracle_prefill(q, k, v, ids, T, 0.5)
    for s in range(3):
        i = int(np.flatnonzero(ids == s + 1)[-1])
        dec = oracle_decode(np.stack([q[i]] * 3), k, v, ids, i + 1, 0.5, streams=[s])
        np.testing.assert_allclose(got[i], dec[s], rtol=1e-12, atol=1e-12)


def _owners_layout(rng, P):
    own = [-1] * int(rng.integers(1, 5))
    tail = [s for s in range(P) for _ in range(int(rng.integers(1, 4)))]
    rng.shuffle(tail)
    late = [-1] * int(rng.integers(0, 2))
    return own + tail + late


@pytest.mark.parametrize("seed", range(20))
def test_bruteforce_dense_mask(seed):
    rng = np.random.default_rng(300 + seed)
    P = int(rng.integers(1, 4))
    owners = _owners_layout(rng, P)
    T = len(owners)
    ids = np.array([0 if o < 0 else o + 1 for o in owners], dtype=np.int32)
    q, k, v = _rand(rng, T, 2, 4)
    mask = np.array([[j <= i and (owners[j] == -1 or owners[j] == owners[i]) for j in range(T)] for i in range(T)])
    x = np.einsum("ihd,jhd->hij", q, k) * 0.7
    x = np.where(mask[None], x, -np.inf)
    w = np.exp(x - x.max(-1, keepdims=True))
    w /= w.sum(-1, keepdims=True)
    want = np.einsum("hij,jhd->ihd", w, v)
    np.testing.assert_allclose(oracle_prefill(q, k, v, ids, T, 0.7), want, rtol=1e-12, atol=1e-12)


def test_foreign_ids_see_the_document_and_their_own_id():
    ids = np.array([0, 0, 7, 1, 7, 0, 1], dtype=np.int32)
    assert prefill_visible(ids, 4).tolist() == [0, 1, 2, 4]
    assert prefill_visible(ids, 5).tolist() == [0, 1, 5]
    assert prefill_visible(ids, 6).tolist() == [0, 1, 3, 5, 6]


@pytest.mark.parametrize("Hq,Hkv", [(6, 2), (7, 1)])
def test_grouped_heads_document_only_is_grouped_causal_sdpa(Hq, Hkv):
    rng = np.random.default_rng(Hq)
    T = 19
    q = rng.standard_normal((T, Hq, 8))
    k = rng.standard_normal((T, Hkv, 8))
    v = rng.standard_normal((T, Hkv, 8))
    got = oracle_prefill(q, k, v, np.zeros(T, dtype=np.int32), T, 0.6)
    t = [torch.from_numpy(x).permute(1, 0, 2).unsqueeze(0) for x in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True, scale=0.6, enable_gqa=True)
    np.testing.assert_allclose(got, ref.squeeze(0).permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_grouped_heads_equal_repeated_heads_in_prefill():
    rng = np.random.default_rng(3)
    ids, _ = canonical_layout(6, [3, 2], [1, 2])
    T = len(ids)
    q, k, v = rng.standard_normal((T, 4, 8)), rng.standard_normal((T, 2, 8)), rng.standard_normal((T, 2, 8))
    a = oracle_prefill(q, k, v, ids, T, 0.5)
    b = oracle_prefill(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), ids, T, 0.5)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------- mutants ---

MUTANTS = {
    "self excluded": ("ids = np.asarray(stream_id)[: i + 1]", "ids = np.asarray(stream_id)[: i]"),
    "document dropped": ("(ids == 0) | (ids == ids[i])", "(ids == ids[i])"),
    "other streams seen": ("(ids == 0) | (ids == ids[i])", "(ids == 0) | (ids >= 0)"),
    "not causal": ("ids = np.asarray(stream_id)[: i + 1]", "ids = np.asarray(stream_id)"),
    "grouped heads read the wrong key head": ("attend(qf[i, h], kf[h // G], vf[h // G], idx, scale)",
                                              "attend(qf[i, h], kf[h % kf.shape[0]], vf[h % kf.shape[0]], idx, scale)"),
}


def _mutant(name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1
    src = src.replace("from .pp_oracle import", "from oracle.pp_oracle import").replace(old, new)
    mod = types.ModuleType("prefill_mutant")
    exec(compile(src, "prefill_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod) -> bool:
    try:
        test_golden_prefill_mask_figure(mod)
    except (AssertionError, IndexError):
        return False
    rng = np.random.default_rng(5)
    T = 12
    q, k, v = _rand(rng, T, 2, 4)
    ids = np.array([0, 0, 0, 1, 1, 2, 2, 3, 3, 1, 2, 3], dtype=np.int32)
    owners = [-1, -1, -1, 0, 0, 1, 1, 2, 2, 0, 1, 2]
    mask = np.array([[j <= i and (owners[j] == -1 or owners[j] == owners[i]) for j in range(T)] for i in range(T)])
    x = np.where(mask[None], np.einsum("ihd,jhd->hij", q, k), -np.inf)
    w = np.exp(x - x.max(-1, keepdims=True))
    w /= w.sum(-1, keepdims=True)
    try:
        got = mod.oracle_prefill(q, k, v, ids, T, 1.0)
        qg, kg = rng.standard_normal((7, 4, 8)), rng.standard_normal((7, 2, 8))
        gqa = mod.oracle_prefill(qg, kg, kg, np.zeros(7, dtype=np.int32), 7, 0.5)
    except Exception:
        return False
    t = [torch.from_numpy(x).permute(1, 0, 2).unsqueeze(0) for x in (qg, kg, kg)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=True, scale=0.5, enable_gqa=True)
    ok_gqa = np.allclose(gqa, ref.squeeze(0).permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    return bool(np.allclose(got, np.einsum("hij,jhd->ihd", w, v), rtol=0, atol=1e-12)) and bool(ok_gqa)


def test_unmutated_copy_passes():
    mod = types.ModuleType("prefill_copy")
    exec(compile(open(SRC).read().replace("from .pp_oracle import", "from oracle.pp_oracle import"), "prefill_copy",
                 "exec"), mod.__dict__)
    assert _pins_pass(mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert not _pins_pass(_mutant(name)), name
