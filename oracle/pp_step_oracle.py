"""fp64 CPU oracle for a whole decode step that appends one token per stream.

TEST INFRASTRUCTURE ONLY.  Nothing in the library calls this module; only the
tests, the smoke check and the benchmark's CPU-baseline leg use it.  It
imports nothing from the HIP path and shares no code with it; the attention
itself is the plain definition in `pp_oracle`.

What a step does, beyond the attention of one decode token per stream
(Parallel Prompting project page, "How it works"):

* every stream appends one slot per step, carrying its stream id (the
  paragraph after the two numbered items: a step appends one token per
  stream and keeps a fixed shape);
* positions are shared (item 2): every stream's positions start right after
  the document, as if its question were the only one.  Written out: the
  position of a slot is the number of earlier slots visible to the token in
  it,  pos(j) = |{ i < j : id[i] == 0  or  id[i] == id[j] }|.  A document
  slot counts the document slots before it; a slot of stream s counts the
  document slots and stream s's own slots before it, which is its index in
  the sequence "document, then stream s alone";
* the new token's query and key are rotated at that position (rotary
  position embedding, rotate-half pairing: dims i and i + d/2 form a pair
  turned by the angle pos * base^(-2i/d), i < d/2; the pages name no
  variant, this is the pairing of the Llama family the pages' CodeLlama
  model belongs to), stored in the cache's element type, and the value is
  stored unrotated; base <= 0 means no rotation.

All arithmetic is float64; results stored in bf16 are rounded to nearest
even by `round_bf16`, written from the bf16 format's definition.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .pp_oracle import oracle_decode, to_f64

__all__ = ["round_bf16", "shared_positions", "rope", "oracle_append_step"]


def round_bf16(x) -> np.ndarray:
    """Nearest bf16 value of each float64 element, ties to even.

    bf16 keeps 8 significant bits (1 implicit + 7 stored) and the exponent
    range of fp32, so for a normal value x = m * 2^e with m in [0.5, 1) the
    representable neighbours are multiples of 2^(e-8); below the smallest
    normal (2^-126) the spacing stays 2^-133.  Overflow past the largest
    finite bf16 gives inf.  NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)  # subnormal range: fixed quantum 2^-133
    q = np.ldexp(1.0, e - 8)
    r = np.rint(x / q) * q  # np.rint rounds half to even; x / q is exact
    big = np.abs(r) > np.ldexp(255.0, 127 - 7)  # largest finite bf16 = (2 - 2^-7) * 2^127
    return np.where(big, np.copysign(np.inf, x), r)


def shared_positions(stream_id, seq_len: int) -> np.ndarray:
    """Position of every slot j < seq_len under the shared-positions rule
    (project page, "How it works", item 2): the number of earlier slots the
    token in slot j sees -- document slots (id 0), plus, for a stream's slot,
    that stream's earlier slots.  Counted with running tallies per id."""
    ids = np.asarray(stream_id)[:seq_len].astype(np.int64)
    pos = np.empty(seq_len, dtype=np.int64)
    n_doc = 0
    n_own: Dict[int, int] = {}
    for j, a in enumerate(ids.tolist()):
        if a == 0:
            pos[j] = n_doc
            n_doc += 1
        else:
            c = n_own.get(a, 0)
            pos[j] = n_doc + c
            n_own[a] = c + 1
    return pos


def rope(x, pos, base: float) -> np.ndarray:
    """Rotary position embedding of x [..., d] at position(s) pos
    (broadcast against x[..., 0]), rotate-half pairing: for i < d/2 the pair
    (x_i, x_{i+d/2}) is turned by the angle pos * base^(-2i/d).  base <= 0
    returns x unchanged."""
    x = np.asarray(x, dtype=np.float64)
    if base <= 0:
        return x.copy()
    d = x.shape[-1]
    half = d // 2
    theta = float(base) ** (-2.0 * np.arange(half) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def oracle_append_step(q, k_new, v_new, k_cache, v_cache, stream_id, base_len: int, scale: float,
                       rope_base: float, store_bf16: bool = True, streams=None) -> Dict[str, np.ndarray]:
    """One decode step that appends: stream s's new slot is base_len + s
    (id s + 1); its query and key are rotated at the slot's shared position,
    the key and the value are stored in the cache, and every stream attends
    over the first base_len + P slots.

    q: [P, Hq, d]; k_new, v_new: [P, Hkv, d]; k_cache, v_cache: [T >=
    base_len + P, Hkv, d], Hq a multiple of Hkv, query head h reading
    key/value head h // (Hq // Hkv) (the first base_len slots hold earlier,
    already rotated keys); stream_id:
    [T] (slots >= base_len are overwritten).  With store_bf16 the rotated
    query and key and the stored value are rounded to bf16 (the caches'
    element type), else kept in float64.
    Returns {out, q_rot, k_rot, pos, k_cache, v_cache, stream_id, seq_len}."""
    qf, kn, vn = to_f64(q), to_f64(k_new), to_f64(v_new)
    P = qf.shape[0]
    seq_len = base_len + P
    ids = np.array(stream_id.cpu().numpy() if hasattr(stream_id, "cpu") else stream_id, dtype=np.int64)
    ids[base_len:seq_len] = np.arange(1, P + 1)
    pos = shared_positions(ids, seq_len)[base_len:seq_len]
    rnd = round_bf16 if store_bf16 else (lambda a: a)
    q_rot = rnd(rope(qf, pos[:, None], rope_base))
    k_rot = rnd(rope(kn, pos[:, None], rope_base))
    K = to_f64(k_cache[:seq_len]).copy()
    V = to_f64(v_cache[:seq_len]).copy()
    K[base_len:seq_len] = k_rot
    V[base_len:seq_len] = rnd(vn)
    out = oracle_decode(q_rot, K, V, ids, seq_len, scale, streams=streams)
    return {"out": out, "q_rot": q_rot, "k_rot": k_rot, "pos": pos, "k_cache": K, "v_cache": V,
            "stream_id": ids, "seq_len": np.int64(seq_len)}
