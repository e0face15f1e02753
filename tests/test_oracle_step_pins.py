"""Pins of the step oracle (shared positions, rotary embedding, bf16
rounding, the appending step) to facts other than itself (CPU only), and a
check that plausible mistakes planted in a copy of its source fail them."""
import json
import math
import os
import types

import numpy as np
import pytest
import torch

from oracle import oracle_append_step, oracle_decode, rope, round_bf16, shared_positions, visible_slots
from workloads import canonical_layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "pp_step_oracle.py")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------ bf16 rounding ---

def test_round_bf16_matches_torch_on_fp32_values():
    # torch's fp32 -> bf16 cast rounds to nearest even; on fp32-representable
    # inputs that is one rounding of the exact value, the same as ours
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(200000), rng.standard_normal(20000) * 1e30,
                        rng.standard_normal(20000) * 1e-37]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even 1;
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: goes to 1 + 2^-6
    assert round_bf16(1 + 2.0 ** -8) == 1.0
    assert round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert round_bf16(-(1 + 2.0 ** -8 + 2.0 ** -30)) == -(1 + 2.0 ** -7)
    assert round_bf16(0.0) == 0.0 and math.isnan(float(round_bf16(np.nan)))
    assert np.isinf(round_bf16(3.5e38))


# --------------------------------------------------------- shared positions ---

def test_golden_positions_on_the_mask_figure():
    g = _load("shared_positions_figure_doc3_p3.json")
    ids = np.array(g["stream_id"], dtype=np.int32)
    assert shared_positions(ids, len(ids)).tolist() == g["positions"]


def test_one_stream_has_plain_positions():
    ids, _ = canonical_layout(37, [5], [4])
    assert shared_positions(ids, len(ids)).tolist() == list(range(len(ids)))


@pytest.mark.parametrize("seed", range(4))
def test_every_stream_sees_positions_of_its_own_sequence(seed):
    # "as if its question were the only one": listing the slots stream s sees
    # (document, then its own, ascending) gives positions 0, 1, 2, ...
    rng = np.random.default_rng(seed)
    P = int(rng.integers(1, 9))
    ids, _ = canonical_layout(int(rng.integers(0, 40)), rng.integers(1, 9, P).tolist(), rng.integers(0, 6, P).tolist())
    pos = shared_positions(ids, len(ids))
    for s in range(P):
        own = visible_slots(ids, len(ids), s)
        assert pos[own].tolist() == list(range(len(own)))


def test_positions_brute_force_with_late_document_and_foreign_ids():
    rng = np.random.default_rng(11)
    ids = rng.choice([0, 0, 1, 2, 3, 9, -4], size=60)
    pos = shared_positions(ids, 60)
    for j in range(60):
        want = sum(1 for i in range(j) if ids[i] == 0 or ids[i] == ids[j])
        assert pos[j] == want, j


# ----------------------------------------------------------------- rotary ---

def test_golden_rope_hand_example():
    g = _load("rope_d4_base100.json")
    for case in g["cases"]:
        np.testing.assert_allclose(rope(np.array(g["x"]), case["pos"], g["base"]), case["expected"], rtol=0,
                                   atol=g["tolerance"])


@pytest.mark.parametrize("d", [64, 128])
def test_rope_equals_complex_rotation(d):
    # the pair (x_i, x_{i+d/2}) as the complex number x_i + i x_{i+d/2},
    # multiplied by exp(i * pos * base^(-2i/d))
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, d))
    pos = np.array([0, 1, 17, 4095, 31824])
    for base in (1e4, 1e6):
        z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * np.outer(pos, np.power(base, -np.arange(0, d, 2) / d)))
        np.testing.assert_allclose(rope(x, pos, base), np.concatenate([z.real, z.imag], axis=1), rtol=0, atol=1e-9)


def test_rope_invariants():
    rng = np.random.default_rng(5)
    d = 128
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    # position 0 is the identity; base <= 0 switches the rotation off
    np.testing.assert_array_equal(rope(q, 0, 1e4), q)
    np.testing.assert_array_equal(rope(q, 123, 0.0), q)
    # rotations preserve the norm of every pair
    r = rope(q, 977, 1e4)
    np.testing.assert_allclose(np.hypot(r[:64], r[64:]), np.hypot(q[:64], q[64:]), rtol=1e-13)
    # scores depend on the distance between positions only
    a = rope(q, 900, 1e4) @ rope(k, 300, 1e4)
    b = rope(q, 600, 1e4) @ rope(k, 0, 1e4)
    assert abs(a - b) < 1e-10
    # rotations compose
    np.testing.assert_allclose(rope(rope(q, 40, 1e4), 2, 1e4), rope(q, 42, 1e4), atol=1e-12)
    # the first pair turns by exactly pos radians, for any base
    e0 = np.zeros(d)
    e0[0] = 1.0
    r = rope(e0, 2.5, 1e6)
    assert abs(r[0] - math.cos(2.5)) < 1e-15 and abs(r[64] - math.sin(2.5)) < 1e-15


# ------------------------------------------------------------- whole step ---

def _alone(ids, s):
    return visible_slots(ids, len(ids), s)


@pytest.mark.parametrize("seed", range(3))
def test_step_answers_equal_decoding_each_question_alone(seed):
    # the page's claim for both changes together: with shared positions, a
    # stream's answer is the same as decoding its question alone (a one-stream
    # request of the document and its own tokens, with plain positions)
    rng = np.random.default_rng(100 + seed)
    P, H, d, doc = int(rng.integers(2, 6)), 2, 16, int(rng.integers(1, 30))
    ids, _ = canonical_layout(doc, rng.integers(1, 6, P).tolist(), rng.integers(0, 4, P).tolist())
    T0 = len(ids)
    raw_k = rng.standard_normal((T0, H, d))  # keys before rotation
    v = rng.standard_normal((T0 + P, H, d))
    pos = shared_positions(ids, T0)
    k = np.zeros((T0 + P, H, d))
    k[:T0] = rope(raw_k, pos[:, None], 1e4)
    q, kn, vn = rng.standard_normal((P, H, d)), rng.standard_normal((P, H, d)), rng.standard_normal((P, H, d))
    sid = np.concatenate([ids, np.full(P, -7)]).astype(np.int32)
    r = oracle_append_step(q, kn, vn, k, v, sid, T0, 0.3, 1e4, store_bf16=False)
    for s in range(P):
        mine = _alone(ids, s)
        n = len(mine)
        k1 = np.concatenate([rope(raw_k[mine], np.arange(n)[:, None], 1e4), rope(kn[s:s + 1], np.array([[n]]), 1e4)])
        v1 = np.concatenate([v[mine], vn[s:s + 1]])
        o1 = oracle_decode(rope(q[s:s + 1], np.array([[n]]), 1e4), k1, v1, np.zeros(n + 1, dtype=np.int32), n + 1, 0.3)
        np.testing.assert_allclose(r["out"][s], o1[0], rtol=1e-12, atol=1e-12)


def test_step_without_rotation_is_an_append_then_the_decode():
    rng = np.random.default_rng(8)
    P, H, d = 3, 2, 8
    ids, _ = canonical_layout(6, [2, 3, 1], [1, 0, 2])
    T0 = len(ids)
    k, v = rng.standard_normal((T0 + P, H, d)), rng.standard_normal((T0 + P, H, d))
    q, kn, vn = rng.standard_normal((P, H, d)), rng.standard_normal((P, H, d)), rng.standard_normal((P, H, d))
    sid = np.concatenate([ids, np.zeros(P)]).astype(np.int32)
    r = oracle_append_step(q, kn, vn, k, v, sid, T0, 0.5, 0.0, store_bf16=False)
    k2, v2 = k.copy(), v.copy()
    k2[T0:], v2[T0:] = kn, vn
    sid2 = np.concatenate([ids, np.arange(1, P + 1)]).astype(np.int32)
    np.testing.assert_array_equal(r["stream_id"], sid2)
    np.testing.assert_allclose(r["out"], oracle_decode(q, k2, v2, sid2, T0 + P, 0.5), rtol=0, atol=0)
    assert r["pos"].tolist() == [6 + 2 + 1, 6 + 3 + 0, 6 + 1 + 2]


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (6, 1)])
def test_grouped_step_equals_the_step_with_heads_repeated(Hq, Hkv):
    # query head h reads key/value head h // (Hq / Hkv): the grouped step is
    # the plain step on caches and new keys with each key/value head repeated
    # for its group of query heads (the rotation acts per head, so repeating
    # before or after it is the same)
    rng = np.random.default_rng(Hq * 10 + Hkv)
    P, d = 3, 8
    G = Hq // Hkv
    ids, _ = canonical_layout(5, [2, 1, 3], [1, 2, 0])
    T0 = len(ids)
    k, v = rng.standard_normal((T0 + P, Hkv, d)), rng.standard_normal((T0 + P, Hkv, d))
    q, kn, vn = rng.standard_normal((P, Hq, d)), rng.standard_normal((P, Hkv, d)), rng.standard_normal((P, Hkv, d))
    sid = np.concatenate([ids, np.zeros(P)]).astype(np.int32)
    r = oracle_append_step(q, kn, vn, k, v, sid, T0, 0.4, 1e4, store_bf16=False)
    rep = lambda a: np.repeat(a, G, axis=1)  # noqa: E731
    full = oracle_append_step(q, rep(kn), rep(vn), rep(k), rep(v), sid, T0, 0.4, 1e4, store_bf16=False)
    np.testing.assert_allclose(r["out"], full["out"], rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(rep(r["k_rot"]), full["k_rot"])
    assert r["k_cache"].shape == (T0 + P, Hkv, d)


def test_step_rounds_to_bf16_when_asked():
    rng = np.random.default_rng(9)
    P, H, d = 2, 1, 8
    ids, _ = canonical_layout(3, [1, 1], [0, 0])
    k, v = rng.standard_normal((7, H, d)), rng.standard_normal((7, H, d))
    q, kn, vn = rng.standard_normal((P, H, d)), rng.standard_normal((P, H, d)), rng.standard_normal((P, H, d))
    sid = np.concatenate([ids, np.zeros(2)]).astype(np.int32)
    r = oracle_append_step(q, kn, vn, k, v, sid, 5, 0.5, 1e4)
    t = torch.from_numpy(r["k_rot"]).float()
    np.testing.assert_array_equal(t.to(torch.bfloat16).double().numpy(), r["k_rot"])  # already bf16 values
    np.testing.assert_array_equal(r["v_cache"][5:], round_bf16(vn))


# ---------------------------------------------------------------- mutants ---

MUTANTS = {
    "pairs interleaved": ("lo, hi = x[..., :half], x[..., half:]", "lo, hi = x[..., 0::2], x[..., 1::2]"),
    "rotation sign": ("[lo * c - hi * s, hi * c + lo * s]", "[lo * c + hi * s, hi * c - lo * s]"),
    "angle exponent halved": ("theta = float(base) ** (-2.0 * np.arange(half) / d)",
                              "theta = float(base) ** (-1.0 * np.arange(half) / d)"),
    "positions count every slot": ("pos[j] = n_doc + c", "pos[j] = j"),
    "positions skip the document": ("pos[j] = n_doc + c", "pos[j] = c"),
    "positions start at one": ("pos[j] = n_doc + c", "pos[j] = n_doc + c + 1"),
    "round toward zero": ("r = np.rint(x / q) * q", "r = np.trunc(x / q) * q"),
    "one significant bit short": ("q = np.ldexp(1.0, e - 8)", "q = np.ldexp(1.0, e - 7)"),
    "new slot id off by one": ("ids[base_len:seq_len] = np.arange(1, P + 1)", "ids[base_len:seq_len] = np.arange(P)"),
    "value rotated too": ("V[base_len:seq_len] = rnd(vn)", "V[base_len:seq_len] = rnd(rope(vn, pos[:, None], rope_base))"),
}


def _mutant(name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name!r} not unique"
    src = src.replace("from .pp_oracle import", "from oracle.pp_oracle import").replace(old, new)
    mod = types.ModuleType("step_oracle_mutant")
    exec(compile(src, "step_oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod) -> bool:
    checks = []
    g = _load("rope_d4_base100.json")
    for case in g["cases"]:
        checks.append(np.allclose(mod.rope(np.array(g["x"]), case["pos"], g["base"]), case["expected"], rtol=0,
                                  atol=1e-12))
    f = _load("shared_positions_figure_doc3_p3.json")
    checks.append(mod.shared_positions(np.array(f["stream_id"]), len(f["stream_id"])).tolist() == f["positions"])
    x = np.random.default_rng(3).standard_normal(5000).astype(np.float32)
    checks.append(np.array_equal(mod.round_bf16(x.astype(np.float64)),
                                 torch.from_numpy(x).to(torch.bfloat16).double().numpy()))
    rng = np.random.default_rng(8)
    P, H, d = 3, 2, 8
    ids, _ = canonical_layout(6, [2, 3, 1], [1, 0, 2])
    T0 = len(ids)
    k, v = rng.standard_normal((T0 + P, H, d)), rng.standard_normal((T0 + P, H, d))
    q, kn, vn = rng.standard_normal((P, H, d)), rng.standard_normal((P, H, d)), rng.standard_normal((P, H, d))
    sid = np.concatenate([ids, np.zeros(P)]).astype(np.int32)
    r = mod.oracle_append_step(q, kn, vn, k, v, sid, T0, 0.5, 1e4, store_bf16=False)
    k2, v2 = k.copy(), v.copy()
    k2[T0:], v2[T0:] = rope(kn, np.array([[9], [9], [9]]), 1e4), vn
    sid2 = np.concatenate([ids, np.arange(1, P + 1)]).astype(np.int32)
    want = oracle_decode(rope(q, np.array([[9], [9], [9]]), 1e4), k2, v2, sid2, T0 + P, 0.5)
    checks.append(np.allclose(r["out"], want, rtol=0, atol=1e-12))
    return all(checks)


def test_unmutated_copy_passes():
    mod = types.ModuleType("step_oracle_copy")
    src = open(SRC).read().replace("from .pp_oracle import", "from oracle.pp_oracle import")
    exec(compile(src, "step_oracle_copy", "exec"), mod.__dict__)
    assert _pins_pass(mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert not _pins_pass(_mutant(name)), name
