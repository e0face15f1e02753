"""fp64 CPU oracle for one decode step of Parallel Prompting attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the library calls this module; only the
tests, the smoke check and the benchmark's CPU-baseline leg use it, to check
and to time against the HIP path.  It imports nothing from that path and
shares no code with it.

What it computes (Parallel Prompting project page, "How it works", item 1,
the stream mask; arXiv abstract): every KV slot carries a stream id.  A
decode-step query of stream s attends to the shared document and to stream
s's own slots, and to nothing else.  The project page states that each answer
is then the same as decoding its question alone, so the result has a plain
definition, written out here stream by stream:

  for each stream s in [0, P) and head h in [0, H):
    V_s  = { j < seq_len : id[j] == 0  or  id[j] == s + 1 }  (ascending)
    x_j  = scale * <q[s,h,:], k[j,h,:]>                      for j in V_s
    w_j  = exp(x_j - max_j x_j) / sum_j exp(x_j - max_j x_j)
    out[s,h,:] = sum_j w_j * v[j,h,:]          (zeros when V_s is empty)

Id encoding: the page writes -1 for the document and numbers streams from
0; this library uses 0 for the document and s+1 for stream s (the same mask
shifted by one).  Ids outside {0, ..., P} are visible to no stream.  No
position test is made: in a decode step every cached slot precedes the query,
and whether the query's own K/V is already in the cache is the caller's
choice.  Positions only act upstream (rotary embedding), so they do not
enter here.

Each stream is computed independently over only its visible slots; the
shared document is never contracted once for all streams (that reuse is the
method under test, not part of its definition).  Inputs are cast exactly to
float64 before any arithmetic.

Grouped key/value heads (the pages' real-benchmark model shares each
key/value head among several query heads; the pages give no head counts):
with Hq query heads and Hkv key/value heads, query head h reads key/value
head h // (Hq / Hkv).  Hkv = Hq is the one-head-per-key case.
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Tuple

import numpy as np

__all__ = [
    "to_f64",
    "visible_slots",
    "doc_prefix_len",
    "tail_lists",
    "attend",
    "oracle_decode",
]


def to_f64(t) -> np.ndarray:
    """Exact cast of a torch tensor (bf16 / fp32, any device) or array to float64."""
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").double().numpy()


def visible_slots(stream_id: np.ndarray, seq_len: int, s: int) -> np.ndarray:
    """Ascending slots j < seq_len that stream s attends to: the document
    (id 0) and stream s's own slots (id s+1)  [project page, "How it works",
    item 1].  Any other id is invisible to stream s."""
    ids = np.asarray(stream_id)[:seq_len]
    return np.flatnonzero((ids == 0) | (ids == s + 1))


def doc_prefix_len(stream_id: np.ndarray, seq_len: int) -> int:
    """Length of the leading run of document slots (id 0): the shared prefix
    that is packed first in the request  [project page, illustration:
    document and questions in one sequence]."""
    ids = np.asarray(stream_id)[:seq_len]
    nz = np.flatnonzero(ids != 0)
    return int(nz[0]) if nz.size else int(seq_len)


def tail_lists(stream_id: np.ndarray, seq_len: int, P: int) -> Tuple[int, List[np.ndarray]]:
    """The integer visibility plan: the document prefix length, and for each
    stream the ascending slots past that prefix that it attends to (its own
    slots and any later document slots)."""
    d = doc_prefix_len(stream_id, seq_len)
    out = []
    for s in range(P):
        idx = visible_slots(stream_id, seq_len, s)
        out.append(idx[idx >= d])
    return d, out


def attend(qv: np.ndarray, K: np.ndarray, V: np.ndarray, idx: np.ndarray, scale: float,
           return_weights: bool = False):
    """Softmax attention of one query vector over the slots `idx` of one head.

    K, V: [T, d] float64 for this head.  The leading part of `idx` that is the
    contiguous run 0, 1, ..., r-1 is read through a view instead of a copy;
    that changes storage only, the sum is still over exactly `idx`.
    """
    d = qv.shape[0]
    if idx.size == 0:
        return (np.zeros(d), np.zeros(0)) if return_weights else np.zeros(d)
    r = int(np.searchsorted(idx - np.arange(idx.size), 1))  # idx[i] == i for i < r
    x = np.empty(idx.size)
    if r:
        x[:r] = K[:r] @ qv
    if r < idx.size:
        x[r:] = K[idx[r:]] @ qv
    x *= scale
    m = np.max(x)
    e = np.exp(x - m)
    w = e / np.sum(e)
    o = np.zeros(d)
    if r:
        o += w[:r] @ V[:r]
    if r < idx.size:
        o += w[r:] @ V[idx[r:]]
    return (o, w) if return_weights else o


def oracle_decode(q, k, v, stream_id, seq_len: int, scale: float,
                  streams: Optional[Iterable[int]] = None,
                  heads: Optional[Iterable[int]] = None,
                  return_weights: bool = False):
    """Reference output of one decode step.

    q: [P, H, d]; k, v: [T >= seq_len, Hkv, d] with H a multiple of Hkv
    (torch tensors or arrays of any float dtype, cast exactly to float64);
    stream_id: [T] integers.
    Returns out [P, H, d] float64 (rows of streams not in `streams` are NaN),
    and with `return_weights` also a dict {(s, h): (idx, w)}.
    """
    qf = to_f64(q)
    P, H, d = qf.shape
    ids = np.asarray(stream_id.cpu().numpy() if hasattr(stream_id, "cpu") else stream_id)
    ids = ids.astype(np.int64)
    # per-head contiguous float64 copies [H, T, d] of the first seq_len slots
    kf = np.ascontiguousarray(to_f64(k[:seq_len]).transpose(1, 0, 2))
    vf = np.ascontiguousarray(to_f64(v[:seq_len]).transpose(1, 0, 2))
    if H % kf.shape[0] != 0:
        raise ValueError(f"{H} query heads cannot share {kf.shape[0]} key/value heads evenly")
    G = H // kf.shape[0]  # query heads per key/value head
    streams = range(P) if streams is None else list(streams)
    heads = range(H) if heads is None else list(heads)
    out = np.full((P, H, d), np.nan)
    weights = {}
    for s in streams:
        idx = visible_slots(ids, seq_len, s)
        for h in heads:
            if return_weights:
                o, w = attend(qf[s, h], kf[h // G], vf[h // G], idx, scale, return_weights=True)
                weights[(s, h)] = (idx, w)
            else:
                o = attend(qf[s, h], kf[h // G], vf[h // G], idx, scale)
            out[s, h] = o
    return (out, weights) if return_weights else out
