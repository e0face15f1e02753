"""Pins of the fp64 oracle to facts other than itself (CPU only).

Each test states what fixes the expected value: a hand-derived closed form,
an independent formulation (dense mask built from the layout, not from the
ids), a library routine (torch's scaled_dot_product_attention in fp64), or
an invariant of softmax attention.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import doc_prefix_len, oracle_decode, tail_lists, visible_slots
from workloads import canonical_layout, make_case, permute_tail

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- golden ---

def test_golden_closed_form_two_streams():
    g = _load("closed_form_two_streams.json")
    ev = {"0": 0.0, "5": 5.0, "7": 7.0, "ln2": math.log(2), "ln3": math.log(3), "ln5": math.log(5)}
    k = np.array([[[ev[x] for x in row] for row in slot] for slot in g["k_exprs"]])
    q = np.array(g["q"])
    v = np.array(g["v"])
    ids = np.array(g["stream_id"], dtype=np.int32)
    out, W = oracle_decode(q, k, v, ids, len(ids), g["scale"], return_weights=True)
    np.testing.assert_allclose(out, np.array(g["expected_out"]), rtol=0, atol=g["tolerance"])
    for s, w in g["expected_weights"].items():
        np.testing.assert_allclose(W[(int(s), 0)][1], w, rtol=0, atol=g["tolerance"])


def test_golden_mask_figure():
    g = _load("mask_figure_doc3_p3.json")
    ids = np.array(g["stream_id"], dtype=np.int32)
    T = len(ids)
    assert doc_prefix_len(ids, T) == g["doc_prefix_len"]
    for s in range(g["P"]):
        assert visible_slots(ids, T, s).tolist() == g["visible"][str(s)]
    d, lists = tail_lists(ids, T, g["P"])
    assert d == g["doc_prefix_len"]
    for s in range(g["P"]):
        assert lists[s].tolist() == [j for j in g["visible"][str(s)] if j >= d]


# ----------------------------------------------------- brute force (dense) ---

def _random_layout(rng, P, max_doc=4, max_own=4, extras=True):
    """Owners per slot: -1 = document, s = stream s, -2 = junk (foreign id)."""
    owners = [-1] * int(rng.integers(0, max_doc + 1))
    tail = []
    for s in range(P):
        tail += [s] * int(rng.integers(0, max_own + 1))
    if extras:
        tail += [-1] * int(rng.integers(0, 3))  # document slots after the prefix
        tail += [-2] * int(rng.integers(0, 3))
    rng.shuffle(tail)
    return owners + tail


def _ids_from_owners(rng, owners, P):
    ids = []
    for o in owners:
        if o == -1:
            ids.append(0)
        elif o == -2:
            ids.append(int(rng.choice([-5, -1, P + 1, P + 9, 2**31 - 1])))
        else:
            ids.append(o + 1)
    return np.array(ids, dtype=np.int32)


def _dense_reference(q, k, v, owners, scale):
    """Masked softmax over a dense [P, T] mask built from slot owners (not
    from ids), with torch fp64 ops."""
    P, H, d = q.shape
    T = len(owners)
    own = torch.tensor(owners)
    mask = torch.zeros(P, T, dtype=torch.bool)
    for s in range(P):
        mask[s] = (own == -1) | (own == s)
    qt, kt, vt = (torch.from_numpy(x).double() for x in (q, k, v))
    scores = torch.einsum("phd,thd->pht", qt, kt) * scale  # [P,H,T]
    m = mask[:, None, :].expand(P, H, T)
    scores = scores.masked_fill(~m, float("-inf"))
    w = torch.softmax(scores, dim=-1)
    w = torch.where(m.any(-1, keepdim=True), w, torch.zeros_like(w))
    return torch.einsum("pht,thd->phd", w, vt).numpy()


@pytest.mark.parametrize("seed", range(60))
def test_bruteforce_dense_mask(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.integers(1, 5))
    H = int(rng.integers(1, 3))
    d = int(rng.choice([4, 8]))
    owners = _random_layout(rng, P)
    if not owners:
        owners = [-1]
    ids = _ids_from_owners(rng, owners, P)
    T = len(owners)
    scale = float(rng.uniform(0.2, 2.0))
    q = rng.standard_normal((P, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    out = oracle_decode(q, k, v, ids, T, scale)
    ref = _dense_reference(q, k, v, owners, scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_bruteforce_page_figure_shape():
    """3-token document, 3 streams (the project page's mask figure)."""
    g = _load("mask_figure_doc3_p3.json")
    ids = np.array(g["stream_id"], dtype=np.int32)
    owners = [-1 if i == 0 else i - 1 for i in ids]
    rng = np.random.default_rng(7)
    q = rng.standard_normal((3, 2, 8))
    k = rng.standard_normal((len(ids), 2, 8))
    v = rng.standard_normal((len(ids), 2, 8))
    out = oracle_decode(q, k, v, ids, len(ids), 0.35)
    np.testing.assert_allclose(out, _dense_reference(q, k, v, owners, 0.35), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------- library routines ---

def _sdpa_last_row(q_row, K, V, scale, causal):
    """torch fp64 scaled_dot_product_attention; q_row [H,d], K,V [n,H,d]."""
    n, H, d = K.shape
    Kt = torch.from_numpy(K).double().permute(1, 0, 2)[None]  # [1,H,n,d]
    Vt = torch.from_numpy(V).double().permute(1, 0, 2)[None]
    if causal:
        # full causal attention over the sequence whose last query is q_row;
        # earlier queries are arbitrary, only the last row is used
        Q = torch.zeros(1, H, n, d, dtype=torch.float64)
        Q[0, :, -1] = torch.from_numpy(q_row).double()
        o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, is_causal=True, scale=scale)
        return o[0, :, -1].numpy()
    Q = torch.from_numpy(q_row).double()[None, :, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, scale=scale)
    return o[0, :, 0].numpy()


@pytest.mark.parametrize("seed", range(5))
def test_p1_equals_causal_attention(seed):
    """With one stream and its own token appended last, the step is the last
    row of plain causal attention over document | question | answer | self."""
    rng = np.random.default_rng(100 + seed)
    doc, ql, al = int(rng.integers(1, 40)), int(rng.integers(0, 10)), int(rng.integers(0, 10))
    H, d = 3, 16
    ids, _ = canonical_layout(doc, [ql], [al + 1])  # +1: the current token's own K/V
    T = len(ids)
    q = rng.standard_normal((1, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    out = oracle_decode(q, k, v, ids, T, 1 / math.sqrt(d))
    ref = _sdpa_last_row(q[0], k, v, 1 / math.sqrt(d), causal=True)
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_each_stream_equals_decoding_alone(seed):
    """Each answer is the same as decoding its question alone: plain (unmasked)
    attention over the document followed by the stream's own slots, with the
    compacted sequence built from the layout, not from the ids."""
    rng = np.random.default_rng(200 + seed)
    P, H, d = 5, 2, 16
    q_lens = rng.integers(1, 6, P).tolist()
    a_lens = rng.integers(0, 6, P).tolist()
    case = make_case(H, d, int(rng.integers(1, 30)), q_lens, a_lens, dtype=torch.float32, seed=seed)
    case = permute_tail(case, seed)
    k, v = case.k.double().numpy(), case.v.double().numpy()
    q = case.q.double().numpy()
    out = oracle_decode(q, k, v, case.stream_id.numpy(), case.seq_len, case.scale)
    for s in range(P):
        sel = np.concatenate([np.arange(case.doc_len), case.own_slots[s]]).astype(np.int64)
        ref = _sdpa_last_row(q[s], k[sel], v[sel], case.scale, causal=False)
        np.testing.assert_allclose(out[s], ref, rtol=1e-12, atol=1e-12)


# -------------------------------------------------------------- invariants ---

def _small_case(seed=0, P=4, H=2, d=8, doc=6):
    rng = np.random.default_rng(seed)
    return make_case(H, d, doc, rng.integers(1, 5, P).tolist(), rng.integers(0, 5, P).tolist(),
                     dtype=torch.float32, seed=seed)


@pytest.mark.parametrize("bad", [1.5, np.inf, -np.inf, np.nan])
def test_isolation_bit_identical(bad):
    c = _small_case(3)
    q, k, v = c.q.double().numpy(), c.k.double().numpy(), c.v.double().numpy()
    ids = c.stream_id.numpy()
    base = oracle_decode(q, k, v, ids, c.seq_len, c.scale)
    for s in range(c.P):
        k2, v2 = k.copy(), v.copy()
        for o in range(c.P):
            if o != s:
                k2[c.own_slots[o]] = bad * (1 + k2[c.own_slots[o]] ** 2)
                v2[c.own_slots[o]] = bad
        out = oracle_decode(q, k2, v2, ids, c.seq_len, c.scale, streams=[s])
        assert np.array_equal(out[s], base[s])


def test_single_visible_key_returns_its_value():
    rng = np.random.default_rng(4)
    P, H, d = 3, 2, 8
    ids = np.array([0, 1 + 1, 2 + 1, 2 + 1], dtype=np.int32)  # stream 0 sees only slot 0
    q = rng.standard_normal((P, H, d)) * 10
    k = rng.standard_normal((4, H, d)) * 10
    v = rng.standard_normal((4, H, d))
    out = oracle_decode(q, k, v, ids, 4, 0.7)
    assert np.array_equal(out[0], v[0])


def test_weights_sum_to_one():
    c = _small_case(5, P=6, doc=40)
    _, W = oracle_decode(c.q, c.k, c.v, c.stream_id.numpy(), c.seq_len, c.scale, return_weights=True)
    for (s, h), (idx, w) in W.items():
        assert abs(w.sum() - 1.0) <= 1e-12
        assert len(idx) == c.doc_len + len(c.own_slots[s])
        assert np.all(w > 0)


def test_zero_keys_give_mean_of_visible_values():
    c = _small_case(6, P=4, doc=9)
    q, v = c.q.double().numpy(), c.v.double().numpy()
    k = np.zeros_like(v)
    out = oracle_decode(q, k, v, c.stream_id.numpy(), c.seq_len, c.scale)
    for s in range(c.P):
        sel = np.concatenate([np.arange(c.doc_len), c.own_slots[s]]).astype(np.int64)
        np.testing.assert_allclose(out[s], v[sel].mean(axis=0), rtol=0, atol=1e-14)


@pytest.mark.parametrize("scale", [0.0, -0.0])
def test_zero_scale_gives_mean_of_visible_values(scale):
    # every visible logit is 0 whatever the keys: the uniform softmax over V_s
    c = _small_case(16, P=5, doc=23)
    v = c.v.double().numpy()
    out = oracle_decode(c.q, c.k, v, c.stream_id.numpy(), c.seq_len, scale)
    for s in range(c.P):
        sel = np.concatenate([np.arange(c.doc_len), c.own_slots[s]]).astype(np.int64)
        np.testing.assert_allclose(out[s], v[sel].mean(axis=0), rtol=0, atol=1e-14)


def test_constant_values_give_that_constant():
    c = _small_case(7)
    v = np.broadcast_to(np.array([0.25 * i - 1 for i in range(c.D)]), c.v.shape).copy()
    out = oracle_decode(c.q, c.k, v, c.stream_id.numpy(), c.seq_len, c.scale)
    np.testing.assert_allclose(out, np.broadcast_to(v[0], out.shape), rtol=0, atol=1e-14)


@pytest.mark.parametrize("mag", [1.0, 1e3])
def test_shift_invariance(mag):
    """k_j += u for every slot shifts all of a query's scores by the same
    amount; softmax ignores it.  mag=1e3 overflows exp() unless the maximum is
    subtracted first."""
    c = _small_case(8)
    q, k, v = c.q.double().numpy(), c.k.double().numpy(), c.v.double().numpy()
    ids = c.stream_id.numpy()
    base = oracle_decode(q, k, v, ids, c.seq_len, c.scale)
    rng = np.random.default_rng(9)
    u = rng.standard_normal((c.H, c.D)) * mag
    out = oracle_decode(q, k + u[None], v, ids, c.seq_len, c.scale)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, base, rtol=1e-9 if mag > 1 else 1e-12, atol=1e-9 if mag > 1 else 1e-12)


def test_permutation_invariance():
    c = _small_case(10, P=5, doc=12)
    pc = permute_tail(c, 11)
    a = oracle_decode(c.q, c.k, c.v, c.stream_id.numpy(), c.seq_len, c.scale)
    b = oracle_decode(pc.q, pc.k, pc.v, pc.stream_id.numpy(), pc.seq_len, pc.scale)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_empty_visible_set_gives_zeros():
    ids = np.array([2, 2, 3], dtype=np.int32)  # stream 0 (id 1) has nothing visible
    rng = np.random.default_rng(12)
    out = oracle_decode(rng.standard_normal((3, 1, 4)), rng.standard_normal((3, 1, 4)),
                        rng.standard_normal((3, 1, 4)), ids, 3, 1.0)
    assert np.array_equal(out[0], np.zeros((1, 4)))
    assert np.all(np.isfinite(out[1])) and np.all(np.isfinite(out[2]))


def test_only_first_seq_len_slots_are_read():
    c = make_case(2, 8, 5, [2, 3], [1, 2], dtype=torch.float32, seed=13, extra_capacity=7)
    out = oracle_decode(c.q, c.k, c.v, c.stream_id.numpy(), c.seq_len, c.scale)
    assert np.all(np.isfinite(out))


# ---------------------------------------------- grouped key/value heads ---

@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (28, 4), (6, 6)])
def test_grouped_heads_match_sdpa(Hq, Hkv):
    # each stream against torch's grouped-query SDPA over its own visible
    # slots (fp64, CPU): an independent implementation of the head sharing
    rng = np.random.default_rng(Hq * 10 + Hkv)
    P, d = 4, 16
    ids, own = canonical_layout(9, [2, 3, 1, 4], [1, 2, 0, 1])
    T = len(ids)
    q = rng.standard_normal((P, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    got = oracle_decode(q, k, v, ids, T, 0.3)
    for s in range(P):
        idx = visible_slots(ids, T, s)
        qt = torch.from_numpy(q[s][:, None, :]).unsqueeze(0)              # [1, Hq, 1, d]
        kt = torch.from_numpy(k[idx].transpose(1, 0, 2).copy()).unsqueeze(0)  # [1, Hkv, n, d]
        vt = torch.from_numpy(v[idx].transpose(1, 0, 2).copy()).unsqueeze(0)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=0.3, enable_gqa=True)
        np.testing.assert_allclose(got[s], ref[0, :, 0, :].numpy(), rtol=1e-12, atol=1e-12)


def test_grouped_heads_equal_repeated_heads():
    # sharing a key/value head among G query heads = giving each query head
    # its own copy of it
    rng = np.random.default_rng(77)
    ids, _ = canonical_layout(5, [2, 2], [1, 1])
    T = len(ids)
    q = rng.standard_normal((2, 6, 8))
    k = rng.standard_normal((T, 2, 8))
    v = rng.standard_normal((T, 2, 8))
    a = oracle_decode(q, k, v, ids, T, 0.5)
    b = oracle_decode(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), ids, T, 0.5)
    np.testing.assert_array_equal(a, b)
    with pytest.raises(ValueError):
        oracle_decode(q, k[:, :1].repeat(4, axis=1), v[:, :1].repeat(4, axis=1), ids, T, 0.5)
