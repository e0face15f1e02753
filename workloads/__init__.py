"""Seeded synthetic inputs for one decode step of Parallel Prompting attention.

This module only draws random numbers and lays slots out; it computes nothing
of the attention itself.  Both the fp64 oracle's tests and the HIP path's
tests / benchmark take their inputs from here, so the two sides see the same
bytes while sharing no arithmetic.

Layout of one request (Parallel Prompting project page, illustration
"the document and all questions go into one sequence" and "How it works"):

    [ document | question of stream 0 | ... | question of stream P-1 | answers ]

* document slots carry stream id 0 (the page writes -1; this library shifts
  every id by +1 so ids fit an unsigned-looking int32 range: 0 = document,
  s+1 = stream s);
* each stream's question is one contiguous run, streams in order;
* answer tokens are interleaved by decode step: for step t = 0, 1, ... every
  stream whose answer is longer than t appends one slot, streams in order
  (each decode step appends one token per stream, "How it works").

All values are N(0, 1) from numpy's PCG64 generator, drawn in float32 and
rounded to bfloat16 with round-to-nearest-even by torch's CPU cast.  Integer
lengths "uniform a-b" are inclusive.  Outliers (ragged sweep) multiply each K
element independently, with probability `outlier_frac`, by `outlier_mult`
before rounding.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

__all__ = [
    "Case",
    "make_case",
    "canonical_layout",
    "permute_tail",
    "named_workload",
    "WORKLOADS",
    "decode_loop_step_inputs",
    "long_answer_case",
    "PrefillCase",
    "prefill_case",
    "prefill_doc16k_p256",
    "MultiCase",
    "multi_case",
    "ServingPool",
    "serving_pool",
]


@dataclasses.dataclass
class Case:
    """One decode step's inputs (torch CPU tensors) plus the layout it came from."""

    q: torch.Tensor  # [P, H, D]
    k: torch.Tensor  # [capacity, H, D]
    v: torch.Tensor  # [capacity, H, D]
    stream_id: torch.Tensor  # [capacity] int32
    seq_len: int
    P: int
    H: int
    D: int
    scale: float
    doc_len: int
    q_lens: List[int]
    a_lens: List[int]
    # slot indices owned by each stream, as laid out (ascending), for tests
    # that build expectations from the layout rather than from the ids
    own_slots: List[np.ndarray]
    name: str = ""

    @property
    def dtype(self) -> torch.dtype:
        return self.q.dtype

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes of one step: the document once, and each
        stream's own slots once (read by their owner only)."""
        per_tok = 2 * self.H * self.D * self.q.element_size()
        return per_tok * (self.doc_len + sum(len(o) for o in self.own_slots))


def canonical_layout(doc_len: int, q_lens: Sequence[int], a_lens: Sequence[int]):
    """Return (stream_id[int32], own_slots list) for doc | questions | answers
    interleaved by step."""
    P = len(q_lens)
    assert len(a_lens) == P
    ids: List[int] = [0] * doc_len
    own: List[List[int]] = [[] for _ in range(P)]
    for s, ql in enumerate(q_lens):
        for _ in range(ql):
            own[s].append(len(ids))
            ids.append(s + 1)
    max_a = max(a_lens) if P else 0
    for t in range(max_a):
        for s in range(P):
            if a_lens[s] > t:
                own[s].append(len(ids))
                ids.append(s + 1)
    return np.asarray(ids, dtype=np.int32), [np.asarray(o, dtype=np.int64) for o in own]


def _round(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dtype) if dtype != torch.float32 else t.clone()


def make_case(
    H: int,
    D: int,
    doc_len: int,
    q_lens: Sequence[int],
    a_lens: Sequence[int],
    dtype: torch.dtype = torch.bfloat16,
    seed: int = 0,
    outlier_frac: float = 0.0,
    outlier_mult: float = 50.0,
    extra_capacity: int = 0,
    name: str = "",
) -> Case:
    """Draw Q/K/V ~ N(0,1) for the canonical layout.  Slots past seq_len
    (`extra_capacity`) are filled with NaN: nothing may read them."""
    ids, own = canonical_layout(doc_len, q_lens, a_lens)
    P = len(q_lens)
    T = int(ids.shape[0])
    cap = T + int(extra_capacity)
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((P, H, D), dtype=np.float32)
    k = rng.standard_normal((cap, H, D), dtype=np.float32)
    v = rng.standard_normal((cap, H, D), dtype=np.float32)
    if outlier_frac > 0:
        mask = rng.random((cap, H, D), dtype=np.float32) < outlier_frac
        k[mask] *= np.float32(outlier_mult)
    if extra_capacity:
        k[T:] = np.nan
        v[T:] = np.nan
    sid = np.full(cap, -7, dtype=np.int32)  # junk past seq_len
    sid[:T] = ids
    return Case(
        q=_round(q, dtype),
        k=_round(k, dtype),
        v=_round(v, dtype),
        stream_id=torch.from_numpy(sid),
        seq_len=T,
        P=P,
        H=H,
        D=D,
        scale=1.0 / math.sqrt(D),
        doc_len=doc_len,
        q_lens=list(map(int, q_lens)),
        a_lens=list(map(int, a_lens)),
        own_slots=own,
        name=name,
    )


def permute_tail(case: Case, seed: int) -> Case:
    """Randomly permute the slots after the document, moving each slot's id
    and K/V rows together (visibility depends on ids, not on positions)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T, d0 = case.seq_len, case.doc_len
    perm = np.arange(T)
    perm[d0:] = d0 + rng.permutation(T - d0)
    # new slot i holds old slot perm[i]
    inv = np.empty_like(perm)
    inv[perm] = np.arange(T)
    k = case.k.clone()
    v = case.v.clone()
    sid = case.stream_id.clone()
    k[:T] = case.k[torch.from_numpy(perm)]
    v[:T] = case.v[torch.from_numpy(perm)]
    sid[:T] = case.stream_id[torch.from_numpy(perm)]
    own = [np.sort(inv[o]) for o in case.own_slots]
    return dataclasses.replace(case, k=k, v=v, stream_id=sid, own_slots=own, name=case.name + "+perm")


def _uniform_ints(rng: np.random.Generator, lo: int, hi: int, n: int) -> List[int]:
    return [int(x) for x in rng.integers(lo, hi + 1, size=n)]


# --------------------------------------------------------------------------
# Named workloads.  The model shape is CodeLlama-7B's attention (32 heads of
# 128 dims, multi-head), the document/question/answer sizes follow the
# project page's speedup and demo settings (8k-16k-token documents, 64-256
# questions, a 12000-token document with 256 questions and 32-token answers).
# --------------------------------------------------------------------------

def _tiny_f32(seed: int) -> Case:
    return make_case(4, 64, 256, [8] * 4, [4] * 4, dtype=torch.float32, seed=seed,
                     name="tiny_f32_h4_d64_doc256_p4")


def _doc8k_p64(seed: int) -> Case:
    rng = np.random.Generator(np.random.PCG64(seed ^ 0x5EED))
    return make_case(32, 128, 8192, _uniform_ints(rng, 16, 32, 64), [16] * 64,
                     dtype=torch.bfloat16, seed=seed, name="codellama7b_doc8k_p64")


def _doc16k_p256(seed: int) -> Case:
    rng = np.random.Generator(np.random.PCG64(seed ^ 0x5EED))
    return make_case(32, 128, 16384, _uniform_ints(rng, 8, 48, 256), [31] * 256,
                     dtype=torch.bfloat16, seed=seed, name="codellama7b_doc16k_p256")


def ragged_case(doc_len: int, P: int, seed: int, H: int = 32, D: int = 128) -> Case:
    """Ragged stress sweep member: questions uniform 1-128, answers uniform
    0-64, 1% of K elements multiplied by 50."""
    rng = np.random.Generator(np.random.PCG64(seed ^ 0xA11CE))
    return make_case(H, D, doc_len, _uniform_ints(rng, 1, 128, P), _uniform_ints(rng, 0, 64, P),
                     dtype=torch.bfloat16, seed=seed, outlier_frac=0.01, outlier_mult=50.0,
                     name=f"ragged_doc{doc_len}_p{P}")


def long_answer_case(answer_len: int, seed: int, doc_len: int = 8192, P: int = 128, H: int = 32,
                     D: int = 128) -> Case:
    """Long-answer sweep member: an 8k-token document with 128 questions
    (uniform 16-32 tokens) and `answer_len` answer tokens already decoded per
    stream (the pages sweep answers up to 1,024 tokens at this shape)."""
    rng = np.random.Generator(np.random.PCG64(seed ^ 0x10A6))
    return make_case(H, D, doc_len, _uniform_ints(rng, 16, 32, P), [answer_len] * P, dtype=torch.bfloat16,
                     seed=seed, name=f"codellama7b_doc{doc_len // 1024}k_p{P}_answers{answer_len}")


@dataclasses.dataclass
class MultiCase:
    q: torch.Tensor          # [B, P, Hq, D]
    k: torch.Tensor          # [B, T, Hkv, D]
    v: torch.Tensor
    stream_id: torch.Tensor  # [B, T] int32
    seq_lens: List[int]      # per request
    doc_lens: List[int]
    P: int
    Hq: int
    Hkv: int
    D: int
    scale: float
    name: str


def multi_case(Hq: int, Hkv: int, D: int, P: int, doc_lens: Sequence[int], q_range=(8, 48), a_len: int = 31,
               dtype: torch.dtype = torch.bfloat16, seed: int = 0, name: str = "") -> MultiCase:
    """B = len(doc_lens) independent requests, each its own document and P
    streams (questions uniform in q_range, a_len prior answer tokens), laid
    out one after another with room for the longest; rows past a request's
    length hold NaN (nothing may read them) and junk ids."""
    rng = np.random.Generator(np.random.PCG64(seed))
    layouts = []
    for dl in doc_lens:
        ids, _ = canonical_layout(int(dl), _uniform_ints(rng, q_range[0], q_range[1], P), [a_len] * P)
        layouts.append(ids)
    T = max(len(x) for x in layouts)
    B = len(doc_lens)
    sid = np.full((B, T), -5, dtype=np.int32)
    for b, ids in enumerate(layouts):
        sid[b, : len(ids)] = ids
    q = rng.standard_normal((B, P, Hq, D), dtype=np.float32)
    k = rng.standard_normal((B, T, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((B, T, Hkv, D), dtype=np.float32)
    for b, ids in enumerate(layouts):
        k[b, len(ids):] = np.nan
        v[b, len(ids):] = np.nan
    return MultiCase(q=_round(q, dtype), k=_round(k, dtype), v=_round(v, dtype), stream_id=torch.from_numpy(sid),
                     seq_lens=[len(x) for x in layouts], doc_lens=[int(x) for x in doc_lens], P=P, Hq=Hq, Hkv=Hkv,
                     D=D, scale=1.0 / math.sqrt(D), name=name)


@dataclasses.dataclass
class ServingPool:
    """Requests waiting to be decoded, each with its own document, P streams
    and answer length (every stream of a request answers that many tokens);
    caches hold the document, the questions and all the answers' K/V in the
    canonical layout, so the cache at a request's step t is its first
    base + (t + 1) * P slots."""
    ids: List[np.ndarray]           # per request [T_r] int32
    k: List[torch.Tensor]           # per request [T_r, Hkv, D]
    v: List[torch.Tensor]
    base: List[int]                 # document + questions, per request
    answer_lens: List[int]
    P: int
    Hq: int
    Hkv: int
    D: int
    seed: int

    def queries(self, r: int, t: int, dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
        """The P queries [P, Hq, D] of request r at its answer step t."""
        rng = np.random.Generator(np.random.PCG64([self.seed, r, t]))
        return _round(rng.standard_normal((self.P, self.Hq, self.D), dtype=np.float32), dtype)


def serving_pool(answer_lens: Sequence[int], P: int, Hq: int, Hkv: int, D: int, doc_range=(64, 256),
                 q_range=(2, 12), dtype: torch.dtype = torch.bfloat16, seed: int = 0) -> ServingPool:
    rng = np.random.Generator(np.random.PCG64(seed))
    ids_l, k_l, v_l, base = [], [], [], []
    for a in answer_lens:
        doc = int(rng.integers(doc_range[0], doc_range[1] + 1))
        q_lens = _uniform_ints(rng, q_range[0], q_range[1], P)
        ids, _ = canonical_layout(doc, q_lens, [int(a)] * P)
        T = len(ids)
        ids_l.append(ids)
        k_l.append(_round(rng.standard_normal((T, Hkv, D), dtype=np.float32), dtype))
        v_l.append(_round(rng.standard_normal((T, Hkv, D), dtype=np.float32), dtype))
        base.append(doc + sum(q_lens))
    return ServingPool(ids=ids_l, k=k_l, v=v_l, base=base, answer_lens=[int(a) for a in answer_lens], P=P, Hq=Hq,
                       Hkv=Hkv, D=D, seed=seed)


@dataclasses.dataclass
class PrefillCase:
    q: torch.Tensor          # [T, H, D]: one query per slot
    k: torch.Tensor
    v: torch.Tensor
    stream_id: torch.Tensor  # [T] int32
    seq_len: int
    doc_len: int
    H: int
    D: int
    scale: float
    name: str


def prefill_case(H: int, D: int, doc_len: int, q_lens: Sequence[int], dtype: torch.dtype = torch.bfloat16,
                 seed: int = 0, a_lens: Optional[Sequence[int]] = None, shuffle_tail: bool = False,
                 name: str = "", Hkv: Optional[int] = None) -> PrefillCase:
    """The packed request before decoding: the document, then each stream's
    question (and, if given, answer tokens), Q/K/V ~ N(0,1) for every slot
    (H query heads; K/V with Hkv heads, default H).  shuffle_tail permutes
    the slots after the document (ids with them)."""
    a = [0] * len(q_lens) if a_lens is None else a_lens
    ids, _ = canonical_layout(doc_len, q_lens, a)
    rng = np.random.Generator(np.random.PCG64(seed))
    if shuffle_tail:
        tail = ids[doc_len:].copy()
        rng.shuffle(tail)
        ids = np.concatenate([ids[:doc_len], tail]).astype(np.int32)
    T = int(ids.shape[0])
    hk = H if Hkv is None else Hkv
    q = rng.standard_normal((T, H, D), dtype=np.float32)
    k = rng.standard_normal((T, hk, D), dtype=np.float32)
    v = rng.standard_normal((T, hk, D), dtype=np.float32)
    return PrefillCase(q=_round(q, dtype), k=_round(k, dtype), v=_round(v, dtype), stream_id=torch.from_numpy(ids),
                       seq_len=T, doc_len=doc_len, H=H, D=D, scale=1.0 / math.sqrt(D), name=name)


def prefill_doc16k_p256(seed: int = 1006) -> PrefillCase:
    """Prefill of the 16k-token document with 256 questions of 8-48 tokens."""
    rng = np.random.Generator(np.random.PCG64(seed ^ 0x5EED))
    return prefill_case(32, 128, 16384, _uniform_ints(rng, 8, 48, 256), seed=seed,
                        name="codellama7b_prefill_doc16k_p256")


WORKLOADS: Dict[str, object] = {
    "tiny_f32_h4_d64_doc256_p4": _tiny_f32,
    "codellama7b_doc8k_p64": _doc8k_p64,
    "codellama7b_doc16k_p256": _doc16k_p256,
}


def named_workload(name: str, seed: int = 1000) -> Case:
    return WORKLOADS[name](seed)  # type: ignore[operator]


# --------------------------------------------------------------------------
# Multi-step decode loop (attention only): a 12000-token document, 256
# streams, 32 answer steps, 32 independent layers.  Question lengths uniform
# 8-48.  At each step every stream appends one K/V slot (its id s+1), then
# attends, so the step's own token is visible to it.
# --------------------------------------------------------------------------

def decode_loop_layout(doc_len: int, P: int, steps: int, seed: int, q_lo: int = 8, q_hi: int = 48):
    """Return (stream_id for the whole loop's capacity, q_lens, base_len).
    Slots [base_len + t*P, base_len + (t+1)*P) are step t's appended tokens."""
    rng = np.random.Generator(np.random.PCG64(seed ^ 0x5EED))
    q_lens = _uniform_ints(rng, q_lo, q_hi, P)
    ids, _ = canonical_layout(doc_len, q_lens, [steps] * P)
    base = doc_len + sum(q_lens)
    return ids, q_lens, base


def decode_loop_step_inputs(H: int, D: int, P: int, capacity: int, layer: int, step: int,
                            seed: int, dtype=torch.bfloat16, base_len: Optional[int] = None,
                            Hkv: Optional[int] = None):
    """Fresh N(0,1) values for one (layer, step): the step's queries [P,H,D],
    and, at step 0, the layer's initial cache [base_len,Hkv,D] (K and V);
    at every step the P appended K/V rows [P,Hkv,D] (Hkv defaults to H).
    Each (layer, step) has its own PCG64 stream, so any sample can be
    regenerated without the others."""
    Hkv = H if Hkv is None else Hkv
    rng = np.random.Generator(np.random.PCG64([seed, layer, step]))
    q = rng.standard_normal((P, H, D), dtype=np.float32)
    k_new = rng.standard_normal((P, Hkv, D), dtype=np.float32)
    v_new = rng.standard_normal((P, Hkv, D), dtype=np.float32)
    out = {"q": _round(q, dtype), "k_new": _round(k_new, dtype), "v_new": _round(v_new, dtype)}
    if step == 0:
        assert base_len is not None
        rng0 = np.random.Generator(np.random.PCG64([seed, layer, 1 << 20]))
        k0 = rng0.standard_normal((base_len, Hkv, D), dtype=np.float32)
        v0 = rng0.standard_normal((base_len, Hkv, D), dtype=np.float32)
        out["k0"] = _round(k0, dtype)
        out["v0"] = _round(v0, dtype)
    return out
