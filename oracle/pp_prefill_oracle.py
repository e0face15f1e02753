"""fp64 CPU oracle for the prefill of a packed Parallel Prompting request.

TEST INFRASTRUCTURE ONLY.  Nothing in the library calls this module; only the
tests and the benchmark's CPU-baseline leg use it.  It shares no code with the
HIP path; the attention of one query is `pp_oracle.attend`.

What it computes (Parallel Prompting project page, "How it works": the
document and all the questions go into one request, every KV slot carries a
stream id, and the stream rule is added to the causal mask): every slot i of
the packed sequence is a query and attends to

    V(i) = { j <= i : id[j] == 0  or  id[j] == id[i] }   (ascending)

-- a document slot to the document up to itself, a stream's slot to the
whole document before it and to its own stream's slots up to itself.  Each
row is computed on its own, over only its visible slots.  With grouped
key/value heads (fewer in k and v than in q), query head h reads key/value
head h // (Hq / Hkv), as in the decode oracle.
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

from .pp_oracle import attend, to_f64

__all__ = ["prefill_visible", "oracle_prefill"]


def prefill_visible(stream_id, i: int) -> np.ndarray:
    """Ascending slots that query slot i sees in the prefill: slots j <= i
    holding the document (id 0) or i's own id."""
    ids = np.asarray(stream_id)[: i + 1]
    return np.flatnonzero((ids == 0) | (ids == ids[i]))


def oracle_prefill(q, k, v, stream_id, seq_len: int, scale: float, rows: Optional[Iterable[int]] = None,
                   heads: Optional[Iterable[int]] = None) -> np.ndarray:
    """Reference prefill output [seq_len, H, d] (float64; rows not in `rows`
    are NaN).  q: [T >= seq_len, H, d], k, v: [T >= seq_len, Hkv, d] with H a
    multiple of Hkv, of any float dtype, cast exactly to float64; stream_id:
    [T] integers."""
    qf = to_f64(q[:seq_len])
    ids = np.asarray(stream_id.cpu().numpy() if hasattr(stream_id, "cpu") else stream_id).astype(np.int64)[:seq_len]
    kf = np.ascontiguousarray(to_f64(k[:seq_len]).transpose(1, 0, 2))
    vf = np.ascontiguousarray(to_f64(v[:seq_len]).transpose(1, 0, 2))
    T, H, d = qf.shape
    if H % kf.shape[0] != 0:
        raise ValueError(f"{H} query heads cannot share {kf.shape[0]} key/value heads evenly")
    G = H // kf.shape[0]
    rows = range(T) if rows is None else list(rows)
    heads = range(H) if heads is None else list(heads)
    out = np.full((T, H, d), np.nan)
    for i in rows:
        idx = prefill_visible(ids, i)
        for h in heads:
            out[i, h] = attend(qf[i, h], kf[h // G], vf[h // G], idx, scale)
    return out
