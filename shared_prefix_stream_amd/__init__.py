"""Parallel Prompting decode-step attention on AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libppattn.so`` (declared in
``include/ppattn.h``).  It only marshals arguments: every step of the
computation runs in the library's HIP kernels.  PyTorch provides device
memory (output and workspace tensors) and the current HIP stream.

    out = pp_attn_decode(q, k_cache, v_cache, stream_id, seq_len)

q [P, H, d]; k_cache, v_cache [T >= seq_len, H, d] (bf16 or fp32, on the GPU,
contiguous); stream_id [T] int32 with 0 = document, s+1 = stream s.  See
the header for the exact definition and contract.

The same kernels also serve: pp_attn_decode_batched (the per-question
baseline), pp_attn_plan / pp_attn_decode_planned (one plan per step for all
layers), pp_step_plan / pp_attn_decode_append (a step that appends one token
per stream, rotary embedding at shared positions, graph-replayable),
pp_attn_prefill (the packed request prefilled under the stream mask) and
pp_attn_decode_multi (several requests per launch, grouped key/value heads,
retired streams).  Schedules for refilling request slots are in
``shared_prefix_stream_amd.batching``.

If the library has not been built (``python -m shared_prefix_stream_amd.build``)
every entry point raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

__all__ = [
    "PPError",
    "library_path",
    "abi_version",
    "workspace_bytes",
    "pp_attn_decode",
    "pp_attn_decode_batched",
    "pp_attn_decode_noalloc",
    "pp_attn_plan",
    "pp_attn_decode_profiled",
    "PROFILE_STAGES",
    "pp_attn_decode_planned",
    "pp_step_plan",
    "pp_step_plan_multi",
    "pp_attn_decode_append_multi",
    "pp_attn_decode_append",
    "prefill_workspace_bytes",
    "pp_attn_prefill",
    "multi_workspace_bytes",
    "pp_attn_decode_multi",
    "stream_read",
    "PP_OK",
    "PP_ERR_INVALID_ARG",
    "PP_ERR_UNSUPPORTED",
    "PP_ERR_WORKSPACE",
    "PP_ERR_HIP",
    "PP_BF16",
    "PP_F32",
]

PP_OK, PP_ERR_INVALID_ARG, PP_ERR_UNSUPPORTED, PP_ERR_WORKSPACE, PP_ERR_HIP = 0, 1, 2, 3, 4
PP_PLAN_WORKSPACE_BYTES = 512
PP_BF16, PP_F32 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libppattn.so"
_lib = None


class PPError(RuntimeError):
    """A non-OK pp_status_t from the library."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    """The in-tree libppattn.so, or the library PP_ATTN_LIBRARY names (for
    instance an AddressSanitizer build of the host code)."""
    return os.environ.get("PP_ATTN_LIBRARY") or os.path.join(_HERE, _LIB_NAME)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m shared_prefix_stream_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    lib.pp_abi_version.restype = ctypes.c_int
    lib.pp_abi_version.argtypes = []
    lib.pp_status_string.restype = ctypes.c_char_p
    lib.pp_status_string.argtypes = [ctypes.c_int]
    lib.pp_last_error_message.restype = ctypes.c_char_p
    lib.pp_last_error_message.argtypes = []
    lib.pp_attn_workspace_bytes.restype = sz
    lib.pp_attn_workspace_bytes.argtypes = [i64, i32, i32, i32, ctypes.c_int]
    for name in ("pp_attn_decode", "pp_attn_decode_batched"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, f32, vp, ctypes.c_int, vp, sz, vp]
    lib.pp_attn_decode_profiled.restype = ctypes.c_int
    lib.pp_attn_decode_profiled.argtypes = [i32, vp, vp, vp, vp, i64, i32, i32, i32, f32, vp, ctypes.c_int, vp, sz, vp,
                                            ctypes.POINTER(vp), i32]
    lib.pp_attn_plan.restype = ctypes.c_int
    lib.pp_attn_plan.argtypes = [vp, i64, i32, vp, vp, vp, i64, vp, sz, vp]
    lib.pp_attn_decode_planned.restype = ctypes.c_int
    lib.pp_attn_decode_planned.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, f32, vp, ctypes.c_int, vp, vp, vp, i64,
                                           vp, sz, vp]
    lib.pp_step_plan.restype = ctypes.c_int
    lib.pp_step_plan.argtypes = [vp, vp, i64, i32, vp, vp, vp, i64, vp]
    lib.pp_attn_decode_append.restype = ctypes.c_int
    lib.pp_attn_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, f32, ctypes.c_double, vp,
                                          vp, vp, i64, vp, ctypes.c_int, vp, sz, vp]
    lib.pp_step_plan_multi.restype = ctypes.c_int
    lib.pp_step_plan_multi.argtypes = [vp, vp, vp, i64, i32, i32, vp, vp, vp, i64, vp]
    lib.pp_attn_decode_append_multi.restype = ctypes.c_int
    lib.pp_attn_decode_append_multi.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, f32,
                                                ctypes.c_double, vp, vp, vp, i64, vp, ctypes.c_int, vp, sz, vp]
    lib.pp_attn_prefill_workspace_bytes.restype = sz
    lib.pp_attn_prefill_workspace_bytes.argtypes = [i64, i32, i32, ctypes.c_int]
    lib.pp_attn_prefill.restype = ctypes.c_int
    lib.pp_attn_prefill.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, f32, vp, ctypes.c_int, vp, sz, vp]
    lib.pp_attn_multi_workspace_bytes.restype = sz
    lib.pp_attn_multi_workspace_bytes.argtypes = [i64, i32, i32, i32, i32, i32, ctypes.c_int]
    for name in ("pp_attn_decode_multi", "pp_attn_decode_multi_batched"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, i32, f32, vp, ctypes.c_int, vp, sz, vp]
    lib.pp_attn_decode_noalloc.restype = ctypes.c_int
    lib.pp_attn_decode_noalloc.argtypes = [vp, vp, vp, vp, i64, i32, i32, i32, f32, vp, ctypes.c_int, vp]
    lib.pp_attn_plan_workspace_bytes.restype = sz
    lib.pp_attn_plan_workspace_bytes.argtypes = [i64, i32]
    lib.pp_stream_read.restype = ctypes.c_int
    lib.pp_stream_read.argtypes = [vp, sz, vp, i32, vp]
    _lib = lib
    return lib


def raw():
    """The loaded ctypes library (for tests of the C ABI itself)."""
    return _load()


def _check(status: int) -> None:
    if status != PP_OK:
        lib = _load()
        msg = (lib.pp_last_error_message() or b"").decode()
        base = (lib.pp_status_string(status) or b"").decode()
        text = f"{base}: {msg}" if msg else base
        if status in (PP_ERR_INVALID_ARG, PP_ERR_UNSUPPORTED, PP_ERR_WORKSPACE):
            err = PPError(status, text)
            raise ValueError(text) from err
        raise PPError(status, text)


def abi_version() -> int:
    return int(_load().pp_abi_version())


def _dtype_code(dtype) -> int:
    import torch

    if dtype == torch.bfloat16:
        return PP_BF16
    if dtype == torch.float32:
        return PP_F32
    raise ValueError(f"unsupported dtype {dtype} (bfloat16 or float32)")


def workspace_bytes(seq_len: int, P: int, H: int, d: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    n = int(_load().pp_attn_workspace_bytes(int(seq_len), int(P), int(H), int(d), code))
    if n == 0:
        raise ValueError(f"invalid shape seq_len={seq_len} P={P} H={H} d={d}")
    return n


def _stream_handle(device) -> int:
    import torch

    return int(torch.cuda.current_stream(device).cuda_stream)


def _prepare(q, k_cache, v_cache, stream_id, seq_len, scale, out, workspace):
    import torch

    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("stream_id", stream_id)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 3 or k_cache.dim() != 3 or v_cache.dim() != 3:
        raise ValueError("q, k_cache, v_cache must be [P,H,d], [T,H,d], [T,H,d]")
    P, H, d = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[1:] != (H, d):
        raise ValueError(f"k_cache/v_cache shape {tuple(k_cache.shape)} does not match q {tuple(q.shape)}")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, k_cache and v_cache must share one dtype")
    if stream_id.dtype != torch.int32 or stream_id.dim() != 1:
        raise ValueError("stream_id must be a 1-D int32 tensor")
    T = k_cache.shape[0]
    if seq_len is None:
        seq_len = T
    if not (1 <= seq_len <= T) or stream_id.shape[0] < seq_len:
        raise ValueError(f"seq_len={seq_len} must be in [1, {T}] and <= len(stream_id)")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _dtype_code(q.dtype)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous GPU tensor shaped and typed like q")
    if workspace is None:  # (a caller's workspace is checked by the library itself)
        workspace = torch.empty(workspace_bytes(seq_len, P, H, d, code), dtype=torch.uint8, device=q.device)
    return P, H, d, int(seq_len), float(scale), code, out, workspace


def _decode(fn_name, q, k_cache, v_cache, stream_id, seq_len=None, scale=None, out=None, workspace=None):
    P, H, d, seq_len, scale, code, out, workspace = _prepare(q, k_cache, v_cache, stream_id, seq_len, scale, out,
                                                             workspace)
    fn = getattr(_load(), fn_name)
    st = fn(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), stream_id.data_ptr(), seq_len, P, H, d, scale,
            out.data_ptr(), code, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            _stream_handle(q.device))
    _check(st)
    return out


def pp_attn_decode(q, k_cache, v_cache, stream_id, seq_len: Optional[int] = None, scale: Optional[float] = None,
                   out=None, workspace=None):
    """One decode step; the document is read once for all P streams.
    Enqueued on torch's current stream; returns `out` without synchronising."""
    return _decode("pp_attn_decode", q, k_cache, v_cache, stream_id, seq_len, scale, out, workspace)


def pp_attn_decode_batched(q, k_cache, v_cache, stream_id, seq_len: Optional[int] = None,
                           scale: Optional[float] = None, out=None, workspace=None):
    """The same step as P independent per-question requests (the baseline)."""
    return _decode("pp_attn_decode_batched", q, k_cache, v_cache, stream_id, seq_len, scale, out, workspace)


PP_NOALLOC_SCRATCH_BYTES = 64 << 20


def pp_attn_decode_noalloc(q, k_cache, v_cache, stream_id, seq_len: Optional[int] = None,
                           scale: Optional[float] = None, out=None):
    """pp_attn_decode with the library's fixed per-GPU scratch array as its
    workspace (no allocation in the call; calls overlapping on one GPU race)."""
    import torch

    if out is None:
        out = torch.empty_like(q)
    P, H, d, seq_len, scale, code, out, _ = _prepare(q, k_cache, v_cache, stream_id, seq_len, scale, out,
                                                     torch.empty(0, dtype=torch.uint8, device=q.device))
    st = _load().pp_attn_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), stream_id.data_ptr(),
                                        seq_len, P, H, d, scale, out.data_ptr(), code, _stream_handle(q.device))
    _check(st)
    return out


def pp_attn_decode_planned(q, k_cache, v_cache, stream_id, plan, seq_len: Optional[int] = None,
                           scale: Optional[float] = None, out=None, workspace=None):
    """pp_attn_decode with a plan `(doc_len, counts, slots)` returned by
    pp_attn_plan for the same stream_id and seq_len (one plan per step serves
    every layer).  `slots` is [P, capacity] (capacity may be 0)."""
    import torch

    P, H, d, seq_len, scale, code, out, workspace = _prepare(q, k_cache, v_cache, stream_id, seq_len, scale, out,
                                                             workspace)
    doc_len, counts, slots = plan
    for name, t in (("doc_len", doc_len), ("counts", counts), ("slots", slots)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.int32:
            raise ValueError(f"plan {name} must be an int32 GPU tensor")
    if doc_len.numel() < 1 or counts.shape != (P,) or slots.dim() != 2 or slots.shape[0] != P:
        raise ValueError("plan must be (doc_len [1], counts [P], slots [P, capacity])")
    cap = int(slots.shape[1])
    if cap > 0 and not slots.is_contiguous():
        raise ValueError("plan slots must be contiguous")
    st = _load().pp_attn_decode_planned(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), stream_id.data_ptr(), seq_len, P, H, d, scale,
        out.data_ptr(), code, doc_len.data_ptr(), counts.data_ptr(), slots.data_ptr() if cap > 0 else None, cap,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_handle(q.device))
    _check(st)
    return out


PP_PROFILE_EVENTS = 6
PROFILE_STAGES = ("plan", "document", "own_slots_merge")


def pp_attn_decode_profiled(events, q, k_cache, v_cache, stream_id, seq_len: Optional[int] = None,
                            scale: Optional[float] = None, out=None, workspace=None, batched: bool = False):
    """pp_attn_decode (or the batched baseline) with raw hipEvent_t handles
    bound to the start and end of each kernel: events[2i], events[2i + 1]
    bracket the i-th of (plan, document, own-slot gather + merge)."""
    P, H, d, seq_len, scale, code, out, workspace = _prepare(q, k_cache, v_cache, stream_id, seq_len, scale, out,
                                                             workspace)
    arr = (ctypes.c_void_p * len(events))(*events)
    st = _load().pp_attn_decode_profiled(
        1 if batched else 0, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), stream_id.data_ptr(), seq_len, P,
        H, d, scale, out.data_ptr(), code, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream_handle(q.device), arr, len(events))
    _check(st)
    return out


def pp_attn_plan(stream_id, seq_len: int, P: int, tail_capacity: int = 0) -> Tuple:
    """The device-side integer visibility plan: (doc_len [1], tail counts [P],
    tail slots [P, tail_capacity]) as int32 GPU tensors."""
    import torch

    if not isinstance(stream_id, torch.Tensor) or not stream_id.is_cuda or stream_id.dtype != torch.int32:
        raise ValueError("stream_id must be an int32 GPU tensor")
    dev = stream_id.device
    doc_len = torch.empty(1, dtype=torch.int32, device=dev)
    counts = torch.empty(P, dtype=torch.int32, device=dev)
    slots = torch.full((P, max(tail_capacity, 1)), -1, dtype=torch.int32, device=dev)
    ws = torch.empty(int(_load().pp_attn_plan_workspace_bytes(int(seq_len), int(P))), dtype=torch.uint8, device=dev)
    st = _load().pp_attn_plan(stream_id.data_ptr(), int(seq_len), int(P), doc_len.data_ptr(), counts.data_ptr(),
                              slots.data_ptr(), int(tail_capacity), ws.data_ptr(), ws.numel(), _stream_handle(dev))
    _check(st)
    return doc_len, counts, slots[:, :tail_capacity]


def _gpu_int32(name, t):
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 GPU tensor")


def pp_step_plan(stream_id, base_len, P: int, max_seq_len: Optional[int] = None,
                 tail_capacity: Optional[int] = None, plan=None) -> Tuple:
    """Start a decode step that appends one slot per stream at base_len[0] + s
    (base_len: int32 GPU tensor [1], advanced by the caller between steps).
    Writes the new ids into stream_id and returns the step's plan
    (head [2] = {doc_len, seq_len}, counts [P], slots [P, capacity]),
    written into `plan` when given (e.g. buffers reused by a captured graph)."""
    import torch

    _gpu_int32("stream_id", stream_id)
    _gpu_int32("base_len", base_len)
    if max_seq_len is None:
        max_seq_len = stream_id.numel()
    if not (1 <= max_seq_len <= stream_id.numel()):
        raise ValueError(f"max_seq_len={max_seq_len} must be in [1, len(stream_id)]")
    dev = stream_id.device
    if plan is None:
        if tail_capacity is None:
            tail_capacity = (min(int(max_seq_len), 2048) + 3) // 4 * 4
        head = torch.zeros(2, dtype=torch.int32, device=dev)
        counts = torch.zeros(P, dtype=torch.int32, device=dev)
        slots = torch.full((P, max(tail_capacity, 1)), -1, dtype=torch.int32, device=dev)[:, :tail_capacity]
    else:
        head, counts, slots = plan
        for name, t in (("head", head), ("counts", counts)):
            _gpu_int32(f"plan {name}", t)
        if head.numel() < 2 or counts.shape != (P,) or slots.dim() != 2 or slots.shape[0] != P:
            raise ValueError("plan must be (head [2], counts [P], slots [P, capacity])")
        tail_capacity = int(slots.shape[1])
        if tail_capacity > 0:
            _gpu_int32("plan slots", slots)
    _check(_load().pp_step_plan(stream_id.data_ptr(), base_len.data_ptr(), int(max_seq_len), int(P), head.data_ptr(),
                                counts.data_ptr(), slots.data_ptr() if tail_capacity > 0 else None,
                                int(tail_capacity), _stream_handle(dev)))
    return head, counts, slots


def pp_attn_decode_append(q, k_new, v_new, k_cache, v_cache, stream_id, plan, scale: Optional[float] = None,
                          rope_base: float = 10000.0, out=None, workspace=None, max_seq_len: Optional[int] = None):
    """One layer of a step started by pp_step_plan: the new keys and values
    go into the caches (keys and queries rotated at the streams' shared
    positions; rope_base <= 0 switches the rotation off), then the decode
    attention over the step's seq_len.  q [P, Hq, d]; k_new, v_new [P, Hkv,
    d]; k_cache, v_cache [T, Hkv, d] (Hq a multiple of Hkv).  Returns `out`
    [P, Hq, d] without synchronising."""
    import torch

    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("stream_id", stream_id)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if q.dim() != 3 or k_cache.dim() != 3 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [P, Hq, d] and k_cache, v_cache [T, Hkv, d]")
    P, H, d = q.shape
    T, Hkv, dk = k_cache.shape
    if dk != d:
        raise ValueError(f"k_cache {tuple(k_cache.shape)} does not match q {tuple(q.shape)}")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (P, Hkv, d):
            raise ValueError(f"{name} must be [P, Hkv, d] = {(P, Hkv, d)}, got {tuple(t.shape)}")
    if not (q.dtype == k_new.dtype == v_new.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, k_new, v_new, k_cache and v_cache must share one dtype")
    if stream_id.dtype != torch.int32 or stream_id.dim() != 1:
        raise ValueError("stream_id must be a 1-D int32 tensor")
    if max_seq_len is None:
        max_seq_len = min(T, stream_id.numel())
    max_seq_len = int(max_seq_len)
    if not (1 <= max_seq_len <= T) or stream_id.numel() < max_seq_len:
        raise ValueError(f"max_seq_len={max_seq_len} must be in [1, {T}] and <= len(stream_id)")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q.dtype)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous GPU tensor shaped and typed like q")
    if workspace is None:
        workspace = torch.empty(multi_workspace_bytes(max_seq_len, 1, P, H, Hkv, d, code), dtype=torch.uint8,
                                device=q.device)
    head, counts, slots = plan
    for name, t in (("head", head), ("counts", counts), ("slots", slots)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.int32:
            raise ValueError(f"plan {name} must be an int32 GPU tensor")
    if head.numel() < 2 or counts.shape != (P,) or slots.dim() != 2 or slots.shape[0] != P:
        raise ValueError("plan must be (head [2], counts [P], slots [P, capacity]) from pp_step_plan")
    cap = int(slots.shape[1])
    if cap > 0 and not slots.is_contiguous():
        raise ValueError("plan slots must be contiguous")
    st = _load().pp_attn_decode_append(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        stream_id.data_ptr(), max_seq_len, P, H, Hkv, d, scale, float(rope_base), head.data_ptr(), counts.data_ptr(),
        slots.data_ptr() if cap > 0 else None, cap, out.data_ptr(), code, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(q.device))
    _check(st)
    return out


def pp_step_plan_multi(stream_id, base_len, P: int, active=None, tail_capacity: Optional[int] = None, plan=None):
    """Start an appending step for B request slots: stream_id [B, T] and
    base_len [B] (request b's new slots at base_len[b] + s; a value outside
    [0, T - P] idles the slot), optional active [B, P] (0 retires a stream),
    all int32 on the GPU.  Returns the plan (head [2B] = doc lengths then
    step lengths, counts [B, P], slots [B, P, capacity]), written into `plan`
    when given."""
    import torch

    _gpu_int32("stream_id", stream_id)
    _gpu_int32("base_len", base_len)
    if stream_id.dim() != 2 or base_len.shape != (stream_id.shape[0],):
        raise ValueError("stream_id must be [B, T] and base_len [B]")
    B, T = stream_id.shape
    if active is not None:
        _gpu_int32("active", active)
        if tuple(active.shape) != (B, P):
            raise ValueError(f"active must be [B, P] = {(B, P)}")
    dev = stream_id.device
    if plan is None:
        if tail_capacity is None:
            tail_capacity = (min(int(T), 2048) + 3) // 4 * 4
        head = torch.zeros(2 * B, dtype=torch.int32, device=dev)
        counts = torch.zeros(B, P, dtype=torch.int32, device=dev)
        slots = torch.full((B, P, max(tail_capacity, 1)), -1, dtype=torch.int32, device=dev)[:, :, :tail_capacity]
    else:
        head, counts, slots = plan
        for name, t in (("head", head), ("counts", counts)):
            _gpu_int32(f"plan {name}", t)
        if head.numel() < 2 * B or tuple(counts.shape) != (B, P) or slots.dim() != 3 or slots.shape[:2] != (B, P):
            raise ValueError("plan must be (head [2B], counts [B, P], slots [B, P, capacity])")
    tail_capacity = int(slots.shape[2])
    if tail_capacity > 0:
        _gpu_int32("plan slots", slots)
    _check(_load().pp_step_plan_multi(stream_id.data_ptr(), base_len.data_ptr(),
                                      None if active is None else active.data_ptr(), int(T), int(B), int(P),
                                      head.data_ptr(), counts.data_ptr(),
                                      slots.data_ptr() if tail_capacity > 0 else None, tail_capacity,
                                      _stream_handle(dev)))
    return head, counts, slots


def pp_attn_decode_append_multi(q, k_new, v_new, k_cache, v_cache, stream_id, plan, active=None,
                                scale: Optional[float] = None, rope_base: float = 10000.0, out=None, workspace=None):
    """One layer of an appending step of B request slots started by
    pp_step_plan_multi: q [B, P, Hq, d], k_new, v_new [B, P, Hkv, d],
    k_cache, v_cache [B, T, Hkv, d], stream_id [B, T], optional active
    [B, P].  Returns out [B, P, Hq, d] (zeros for idle slots and retired
    streams) without synchronising."""
    import torch

    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("stream_id", stream_id)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if q.dim() != 4 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B, P, Hq, d] and k_cache, v_cache [B, T, Hkv, d]")
    B, P, H, d = q.shape
    _, T, Hkv, dk = k_cache.shape
    if k_cache.shape[0] != B or dk != d:
        raise ValueError(f"k_cache {tuple(k_cache.shape)} does not match q {tuple(q.shape)}")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (B, P, Hkv, d):
            raise ValueError(f"{name} must be [B, P, Hkv, d] = {(B, P, Hkv, d)}")
    if not (q.dtype == k_new.dtype == v_new.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, k_new, v_new, k_cache and v_cache must share one dtype")
    if stream_id.dtype != torch.int32 or tuple(stream_id.shape) != (B, T):
        raise ValueError("stream_id must be an int32 [B, T] tensor")
    if active is not None:
        _gpu_int32("active", active)
        if tuple(active.shape) != (B, P) or not active.is_contiguous():
            raise ValueError(f"active must be a contiguous [B, P] = {(B, P)} tensor")
    head, counts, slots = plan
    for name, t in (("head", head), ("counts", counts), ("slots", slots)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.int32:
            raise ValueError(f"plan {name} must be an int32 GPU tensor")
    if head.numel() < 2 * B or tuple(counts.shape) != (B, P) or slots.dim() != 3 or slots.shape[:2] != (B, P):
        raise ValueError("plan must be (head [2B], counts [B, P], slots [B, P, capacity]) from pp_step_plan_multi")
    cap = int(slots.shape[2])
    if cap > 0 and not slots.is_contiguous():
        raise ValueError("plan slots must be contiguous")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q.dtype)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous GPU tensor shaped and typed like q")
    if workspace is None:
        workspace = torch.empty(multi_workspace_bytes(T, B, P, H, Hkv, d, code), dtype=torch.uint8, device=q.device)
    _check(_load().pp_attn_decode_append_multi(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        stream_id.data_ptr(), None if active is None else active.data_ptr(), int(T), int(B), int(P), int(H),
        int(Hkv), int(d), scale, float(rope_base), head.data_ptr(), counts.data_ptr(),
        slots.data_ptr() if cap > 0 else None, cap, out.data_ptr(), code, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(q.device)))
    return out


def prefill_workspace_bytes(seq_len: int, H: int, d: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    n = int(_load().pp_attn_prefill_workspace_bytes(int(seq_len), int(H), int(d), code))
    if n == 0:
        raise ValueError(f"invalid prefill shape seq_len={seq_len} H={H} d={d}")
    return n


def pp_attn_prefill(q, k, v, stream_id, seq_len: Optional[int] = None, scale: Optional[float] = None, out=None,
                    workspace=None):
    """Prefill of the packed request: every slot i < seq_len attends to the
    slots j <= i holding the document (id 0) or its own id.  q [T >= seq_len,
    Hq, d], k, v [T, Hkv, d] (Hq a multiple of Hkv) on the GPU; returns out
    [T, Hq, d] (rows >= seq_len untouched) without synchronising."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("stream_id", stream_id)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2]:
        raise ValueError("q must be [T, Hq, d] and k, v [T, Hkv, d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share one dtype")
    if stream_id.dtype != torch.int32 or stream_id.dim() != 1:
        raise ValueError("stream_id must be a 1-D int32 tensor")
    T, H, d = q.shape
    seq_len = T if seq_len is None else int(seq_len)
    if not (1 <= seq_len <= T) or stream_id.shape[0] < seq_len:
        raise ValueError(f"seq_len={seq_len} must be in [1, {T}] and <= len(stream_id)")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q.dtype)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous GPU tensor shaped and typed like q")
    if workspace is None:
        workspace = torch.empty(prefill_workspace_bytes(seq_len, H, d, code), dtype=torch.uint8, device=q.device)
    _check(_load().pp_attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), stream_id.data_ptr(), seq_len, H,
                                   int(k.shape[1]), d, scale, out.data_ptr(), code, workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream_handle(q.device)))
    return out


def multi_workspace_bytes(max_seq_len: int, B: int, P: int, Hq: int, Hkv: int, d: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    n = int(_load().pp_attn_multi_workspace_bytes(int(max_seq_len), int(B), int(P), int(Hq), int(Hkv), int(d), code))
    if n == 0:
        raise ValueError(f"invalid shape max_seq_len={max_seq_len} B={B} P={P} Hq={Hq} Hkv={Hkv} d={d}")
    return n


def pp_attn_decode_multi(q, k_cache, v_cache, stream_id, seq_lens, scale: Optional[float] = None, out=None,
                         workspace=None, batched: bool = False, active=None):
    """B requests in one launch, grouped key/value heads: q [B, P, Hq, d],
    k_cache/v_cache [B, T, Hkv, d], stream_id [B, T] int32, seq_lens [B]
    int32, optional active [B, P] int32 (0 retires a stream), all on the GPU.
    batched=True runs the per-question baseline.  Returns out [B, P, Hq, d]
    without synchronising."""
    import torch

    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("stream_id", stream_id),
                    ("seq_lens", seq_lens)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if q.dim() != 4 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [B, P, Hq, d] and k_cache, v_cache [B, T, Hkv, d]")
    B, P, Hq, d = q.shape
    _, T, Hkv, dk = k_cache.shape
    if k_cache.shape[0] != B or dk != d:
        raise ValueError(f"k_cache {tuple(k_cache.shape)} does not match q {tuple(q.shape)}")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, k_cache and v_cache must share one dtype")
    if stream_id.dtype != torch.int32 or tuple(stream_id.shape) != (B, T):
        raise ValueError("stream_id must be an int32 [B, T] tensor")
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,):
        raise ValueError("seq_lens must be an int32 [B] tensor")
    if active is not None:
        if (not isinstance(active, torch.Tensor) or not active.is_cuda or not active.is_contiguous()
                or active.dtype != torch.int32 or tuple(active.shape) != (B, P)):
            raise ValueError("active must be a contiguous int32 [B, P] GPU tensor")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q.dtype)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous GPU tensor shaped and typed like q")
    if workspace is None:
        workspace = torch.empty(multi_workspace_bytes(T, B, P, Hq, Hkv, d, code), dtype=torch.uint8, device=q.device)
    fn = _load().pp_attn_decode_multi_batched if batched else _load().pp_attn_decode_multi
    _check(fn(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), stream_id.data_ptr(), seq_lens.data_ptr(),
              None if active is None else active.data_ptr(), T, B, P,
              Hq, Hkv, d, scale, out.data_ptr(), code, workspace.data_ptr(),
              workspace.numel() * workspace.element_size(), _stream_handle(q.device)))
    return out


def stream_read(buf, sink, blocks_per_cu: int = 8) -> None:
    """Read every byte of the contiguous GPU tensor `buf` once on the current
    stream (measurement aid, include/ppmeasure.h); `sink` is a GPU int32 or
    uint32 tensor of at least one element."""
    if not buf.is_cuda or not sink.is_cuda:
        raise ValueError("stream_read needs GPU tensors")
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    _check(_load().pp_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), int(blocks_per_cu),
                                  _stream_handle(buf.device)))
