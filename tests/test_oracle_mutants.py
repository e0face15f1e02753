"""Plant plausible mistakes in a copy of the oracle's source (CPU only) and
check that the pins reject every one of them.  The real oracle is untouched:
each mutant is compiled from edited text into a throwaway module."""
import math
import os
import types

import numpy as np
import pytest
import torch

import tests.test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "pp_oracle.py")

MUTANTS = {
    "stream index off by one": ("(ids == s + 1)", "(ids == s)"),
    "document dropped": ("(ids == 0) | (ids == s + 1)", "(ids == s + 1)"),
    "scale divides": ("x *= scale", "x /= scale"),
    "max not subtracted": ("m = np.max(x)", "m = 0.0"),
    "not normalised": ("w = e / np.sum(e)", "w = e"),
    "keys used as values": ("o += w[r:] @ V[idx[r:]]", "o += w[r:] @ K[idx[r:]]"),
    "gather off by one": ("x[r:] = K[idx[r:]] @ qv", "x[r:] = K[idx[r:] - 1] @ qv"),
    "prefix run too long": ("r = int(np.searchsorted(idx - np.arange(idx.size), 1))",
                            "r = int(np.searchsorted(idx - np.arange(idx.size), 2))"),
    "head transposed": ("out[s, h] = o", "out[s, (h + 1) % H] = o"),
    "grouped heads read the wrong key head": ("attend(qf[s, h], kf[h // G], vf[h // G], idx, scale)\n",
                                              "attend(qf[s, h], kf[h % kf.shape[0]], vf[h % kf.shape[0]], idx, scale)\n"),
    "doc prefix stops late": ("return int(nz[0]) if nz.size else int(seq_len)",
                              "return int(nz[0]) + 1 if nz.size else int(seq_len)"),
}


def _mutant(name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name!r} not unique"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(mod) -> bool:
    """Run a selection of the pins against `mod`; True if all hold."""
    checks = []
    # golden closed form and figure
    g = pins._load("closed_form_two_streams.json")
    ev = {"0": 0.0, "5": 5.0, "7": 7.0, "ln2": math.log(2), "ln3": math.log(3), "ln5": math.log(5)}
    k = np.array([[[ev[x] for x in row] for row in slot] for slot in g["k_exprs"]])
    ids = np.array(g["stream_id"], dtype=np.int32)
    out = mod.oracle_decode(np.array(g["q"]), k, np.array(g["v"]), ids, 4, 1.0)
    checks.append(np.allclose(out, g["expected_out"], rtol=0, atol=1e-12))
    f = pins._load("mask_figure_doc3_p3.json")
    fid = np.array(f["stream_id"], dtype=np.int32)
    checks.append(mod.doc_prefix_len(fid, len(fid)) == f["doc_prefix_len"])
    # dense brute force
    for seed in range(12):
        rng = np.random.default_rng(seed)
        P, H, d = int(rng.integers(1, 5)), int(rng.integers(1, 3)), 8
        owners = pins._random_layout(rng, P) or [-1]
        sid = pins._ids_from_owners(rng, owners, P)
        T = len(owners)
        q, kk, v = (rng.standard_normal(s) for s in ((P, H, d), (T, H, d), (T, H, d)))
        o = mod.oracle_decode(q, kk, v, sid, T, 0.6)
        checks.append(np.allclose(o, pins._dense_reference(q, kk, v, owners, 0.6), rtol=1e-12, atol=1e-12))
    # large shift (exp overflow without max subtraction)
    c = pins._small_case(8)
    q, kk, v = c.q.double().numpy(), c.k.double().numpy(), c.v.double().numpy()
    sid = c.stream_id.numpy()
    base = mod.oracle_decode(q, kk, v, sid, c.seq_len, c.scale)
    u = np.random.default_rng(9).standard_normal((c.H, c.D)) * 1e3
    with np.errstate(all="ignore"):
        sh = mod.oracle_decode(q, kk + u[None], v, sid, c.seq_len, c.scale)
    checks.append(bool(np.all(np.isfinite(sh))) and np.allclose(sh, base, rtol=1e-9, atol=1e-9))
    # grouped key/value heads against torch's grouped-query SDPA
    rng = np.random.default_rng(12)
    ids = np.array([0, 0, 0, 1, 1, 2], dtype=np.int32)
    q, kk, v = rng.standard_normal((2, 6, 8)), rng.standard_normal((6, 2, 8)), rng.standard_normal((6, 2, 8))
    o = mod.oracle_decode(q, kk, v, ids, 6, 0.5)
    for s in range(2):
        idx = np.flatnonzero((ids == 0) | (ids == s + 1))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[s][None, :, None, :]), torch.from_numpy(kk[idx].transpose(1, 0, 2).copy())[None],
            torch.from_numpy(v[idx].transpose(1, 0, 2).copy())[None], scale=0.5, enable_gqa=True)
        checks.append(np.allclose(o[s], ref[0, :, 0, :].numpy(), rtol=1e-12, atol=1e-12))
    return all(bool(x) for x in checks)


def test_unmutated_copy_passes():
    src = open(SRC).read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(src, "oracle_copy", "exec"), mod.__dict__)
    assert _pins_pass(mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with np.errstate(all="ignore"):
        assert not _pins_pass(_mutant(name)), f"pins did not catch: {name}"
