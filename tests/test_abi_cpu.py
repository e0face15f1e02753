"""The C ABI on a machine without a GPU: the library loads, exports every
symbol the headers under include/ declare, and rejects bad arguments on the host
before any HIP call (only fake, never-dereferenced pointers are passed)."""
import ctypes
import math
import os
import re

import pytest

import shared_prefix_stream_amd as pp

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
HEADER = os.path.join(INCLUDE, "ppattn.h")

# fake device addresses, 16-byte aligned and far apart
Q, K, V, SID, OUT, WS = (0x10000000 * i for i in range(1, 7))


def _declared_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = open(os.path.join(INCLUDE, h)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(pp_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = pp.raw()
    names = _declared_functions()
    assert set(names) >= {"pp_attn_decode", "pp_attn_decode_batched", "pp_attn_workspace_bytes", "pp_attn_plan",
                          "pp_attn_decode_planned", "pp_step_plan", "pp_attn_decode_append",
                          "pp_attn_prefill", "pp_attn_prefill_workspace_bytes", "pp_attn_decode_multi",
                          "pp_attn_decode_multi_batched", "pp_attn_multi_workspace_bytes", "pp_abi_version", "pp_status_string", "pp_last_error_message"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_abi_version_and_status_strings():
    lib = pp.raw()
    assert pp.abi_version() == 2
    for code in range(5):
        assert lib.pp_status_string(code).decode().startswith("PP_")
    assert b"unknown" in lib.pp_status_string(99)


def _decode(fn="pp_attn_decode", q=Q, k=K, v=V, sid=SID, seq_len=1000, P=8, H=4, d=128, scale=0.088, out=OUT,
            dtype=pp.PP_BF16, ws=WS, ws_bytes=None, stream=None):
    lib = pp.raw()
    if ws_bytes is None:
        ws_bytes = lib.pp_attn_workspace_bytes(seq_len, P, H, d, dtype) if d in (64, 128) and dtype in (0, 1) else 1 << 20
    return getattr(lib, fn)(q, k, v, sid, seq_len, P, H, d, scale, out, dtype, ws, ws_bytes, stream)


@pytest.mark.parametrize("fn", ["pp_attn_decode", "pp_attn_decode_batched"])
@pytest.mark.parametrize("kw,status", [
    (dict(P=0), pp.PP_ERR_INVALID_ARG),
    (dict(P=70000), pp.PP_ERR_INVALID_ARG),
    (dict(H=0), pp.PP_ERR_INVALID_ARG),
    (dict(seq_len=0), pp.PP_ERR_INVALID_ARG),
    (dict(seq_len=(1 << 30) + 1), pp.PP_ERR_INVALID_ARG),
    (dict(q=None), pp.PP_ERR_INVALID_ARG),
    (dict(k=None), pp.PP_ERR_INVALID_ARG),
    (dict(v=None), pp.PP_ERR_INVALID_ARG),
    (dict(sid=None), pp.PP_ERR_INVALID_ARG),
    (dict(out=None), pp.PP_ERR_INVALID_ARG),
    (dict(scale=math.inf), pp.PP_ERR_INVALID_ARG),
    (dict(scale=math.nan), pp.PP_ERR_INVALID_ARG),
    (dict(q=Q + 8), pp.PP_ERR_INVALID_ARG),
    (dict(sid=SID + 4), pp.PP_ERR_INVALID_ARG),
    (dict(out=Q + 64), pp.PP_ERR_INVALID_ARG),       # out overlaps q
    (dict(out=K + 4096), pp.PP_ERR_INVALID_ARG),     # out overlaps k_cache
    (dict(out=WS + 256), pp.PP_ERR_INVALID_ARG),     # out overlaps workspace
    (dict(ws=V + 256), pp.PP_ERR_INVALID_ARG),       # workspace overlaps v_cache
    (dict(d=96), pp.PP_ERR_UNSUPPORTED),
    (dict(d=256), pp.PP_ERR_UNSUPPORTED),
    (dict(dtype=7), pp.PP_ERR_UNSUPPORTED),
    (dict(ws=None), pp.PP_ERR_WORKSPACE),
    (dict(ws_bytes=1024), pp.PP_ERR_WORKSPACE),
])
def test_host_validation(fn, kw, status):
    assert _decode(fn, **kw) == status
    assert pp.raw().pp_last_error_message().decode() != ""


def test_workspace_bytes():
    lib = pp.raw()
    assert lib.pp_attn_workspace_bytes(0, 8, 4, 128, pp.PP_BF16) == 0
    assert lib.pp_attn_workspace_bytes(100, 8, 4, 96, pp.PP_BF16) == 0
    assert lib.pp_attn_workspace_bytes(100, 8, 4, 128, 5) == 0
    # at least one split of partial states (m, l, d floats) per (stream, head)
    for (T, P, H, d) in [(304, 4, 4, 64), (31488, 256, 32, 128), (82000, 512, 32, 128), (1, 1, 1, 64)]:
        n = lib.pp_attn_workspace_bytes(T, P, H, d, pp.PP_BF16)
        assert n >= P * H * (d + 2) * 4 + 256
    assert lib.pp_last_error_message() == b""


def test_profiled_validation():
    lib = pp.raw()
    ev = (ctypes.c_void_p * pp.PP_PROFILE_EVENTS)(*[0x1000 * (i + 1) for i in range(pp.PP_PROFILE_EVENTS)])
    ws_bytes = lib.pp_attn_workspace_bytes(1000, 8, 4, 128, pp.PP_BF16)

    def call(events, n_events, P=8):
        return lib.pp_attn_decode_profiled(0, Q, K, V, SID, 1000, P, 4, 128, 0.088, OUT, pp.PP_BF16, WS, ws_bytes,
                                           None, events, n_events)

    assert call(None, pp.PP_PROFILE_EVENTS) == pp.PP_ERR_INVALID_ARG
    assert call(ev, pp.PP_PROFILE_EVENTS - 1) == pp.PP_ERR_INVALID_ARG
    with_null = (ctypes.c_void_p * pp.PP_PROFILE_EVENTS)(*([0x1000] * (pp.PP_PROFILE_EVENTS - 1) + [None]))
    assert call(with_null, pp.PP_PROFILE_EVENTS) == pp.PP_ERR_INVALID_ARG
    # the decode arguments are still checked
    assert call(ev, pp.PP_PROFILE_EVENTS, P=0) == pp.PP_ERR_INVALID_ARG
    assert 2 * len(pp.PROFILE_STAGES) == pp.PP_PROFILE_EVENTS
    text = open(HEADER).read()
    assert re.search(r"#define PP_PROFILE_EVENTS %d\b" % pp.PP_PROFILE_EVENTS, text)


def test_plan_validation():
    lib = pp.raw()
    n = pp.PP_PLAN_WORKSPACE_BYTES
    assert lib.pp_attn_plan(None, 10, 2, OUT, WS, K, 4, V, n, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_attn_plan(SID, 0, 2, OUT, WS, K, 4, V, n, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_attn_plan(SID, 10, 0, OUT, WS, K, 4, V, n, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_attn_plan(SID, 10, 2, None, WS, K, 4, V, n, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_attn_plan(SID, 10, 2, OUT, None, K, 4, V, n, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_attn_plan(SID, 10, 2, OUT, WS, None, 4, V, n, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_attn_plan(SID, 10, 2, OUT, WS, K, -1, V, n, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_attn_plan(SID + 4, 10, 2, OUT, WS, K, 4, V, n, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_attn_plan(SID, 10, 2, OUT, WS, K, 4, None, n, None) == pp.PP_ERR_WORKSPACE
    assert lib.pp_attn_plan(SID, 10, 2, OUT, WS, K, 4, V, 100, None) == pp.PP_ERR_WORKSPACE


def test_planned_validation():
    lib = pp.raw()
    PD, PC, PS = 0x70000000, 0x80000000, 0x90000000  # fake plan buffers
    ws_bytes = lib.pp_attn_workspace_bytes(1000, 8, 4, 128, pp.PP_BF16)

    def call(pd=PD, pc=PC, ps=PS, cap=16, P=8, out=OUT, ws=WS, wsb=ws_bytes):
        return lib.pp_attn_decode_planned(Q, K, V, SID, 1000, P, 4, 128, 0.088, out, pp.PP_BF16, pd, pc, ps, cap, ws,
                                          wsb, None)

    assert call(pd=None) == pp.PP_ERR_INVALID_ARG
    assert call(pc=None) == pp.PP_ERR_INVALID_ARG
    assert call(cap=-1) == pp.PP_ERR_INVALID_ARG
    assert call(ps=None) == pp.PP_ERR_INVALID_ARG
    assert call(out=PC + 16) == pp.PP_ERR_INVALID_ARG     # out overlaps the counts
    assert call(ps=WS + 512) == pp.PP_ERR_INVALID_ARG     # slots overlap the workspace
    assert call(P=0) == pp.PP_ERR_INVALID_ARG             # the decode arguments are still checked
    assert call(wsb=1024) == pp.PP_ERR_WORKSPACE
    assert lib.pp_last_error_message().decode() != ""


def test_step_plan_validation():
    lib = pp.raw()
    BASE, HEAD, CNT, SL = 0x60000000, 0x70000000, 0x80000000, 0x90000000

    def call(sid=SID, base=BASE, max_len=1000, P=8, head=HEAD, cnt=CNT, sl=SL, cap=16):
        return lib.pp_step_plan(sid, base, max_len, P, head, cnt, sl, cap, None)

    assert call(sid=None) == pp.PP_ERR_INVALID_ARG
    assert call(base=None) == pp.PP_ERR_INVALID_ARG
    assert call(head=None) == pp.PP_ERR_INVALID_ARG
    assert call(cnt=None) == pp.PP_ERR_INVALID_ARG
    assert call(sl=None) == pp.PP_ERR_INVALID_ARG             # capacity > 0 needs slots
    assert call(cap=-1) == pp.PP_ERR_INVALID_ARG
    assert call(P=0) == pp.PP_ERR_INVALID_ARG
    assert call(max_len=7) == pp.PP_ERR_INVALID_ARG            # P > max_seq_len
    assert call(max_len=0) == pp.PP_ERR_INVALID_ARG
    assert call(sid=SID + 4) == pp.PP_ERR_INVALID_ARG          # misaligned ids
    assert call(head=SID + 400) == pp.PP_ERR_INVALID_ARG       # written over the ids
    assert call(base=SID + 3996) == pp.PP_ERR_INVALID_ARG      # base inside the ids
    assert call(cnt=SL + 64) == pp.PP_ERR_INVALID_ARG          # plan buffers overlap
    assert lib.pp_last_error_message().decode() != ""


def test_decode_append_validation():
    lib = pp.raw()
    KN, VN, HEAD, CNT, SL = 0x70000000, 0x78000000, 0x80000000, 0x90000000, 0xA0000000
    ws_bytes = lib.pp_attn_workspace_bytes(1000, 8, 4, 128, pp.PP_BF16)

    def call(q=Q, kn=KN, vn=VN, k=K, v=V, max_len=1000, P=8, rope=1e4, out=OUT, head=HEAD, ws=WS, wsb=ws_bytes,
             Hq=4, Hkv=4):
        return lib.pp_attn_decode_append(q, kn, vn, k, v, SID, max_len, P, Hq, Hkv, 128, 0.088, rope, head, CNT, SL,
                                         16, out, pp.PP_BF16, ws, wsb, None)

    assert call(kn=None) == pp.PP_ERR_INVALID_ARG
    assert call(vn=VN + 8) == pp.PP_ERR_INVALID_ARG            # misaligned
    assert call(rope=float("inf")) == pp.PP_ERR_INVALID_ARG
    assert call(head=None) == pp.PP_ERR_INVALID_ARG
    assert call(q=K + 4096) == pp.PP_ERR_INVALID_ARG           # the written cache holds q
    assert call(kn=V + 1024) == pp.PP_ERR_INVALID_ARG          # ... or a new key
    assert call(v=K + 1000 * 4 * 128 * 2 - 256) == pp.PP_ERR_INVALID_ARG  # the caches overlap
    assert call(head=K + 64) == pp.PP_ERR_INVALID_ARG          # the plan lives in a cache
    assert call(head=OUT + 4) == pp.PP_ERR_INVALID_ARG         # plan head (8 bytes) overlaps out
    assert call(kn=OUT) == pp.PP_ERR_INVALID_ARG
    assert call(vn=WS + 4096) == pp.PP_ERR_INVALID_ARG
    assert call(P=0) == pp.PP_ERR_INVALID_ARG
    assert call(max_len=6, wsb=1 << 30) == pp.PP_ERR_INVALID_ARG  # P > max_seq_len
    assert call(wsb=1024) == pp.PP_ERR_WORKSPACE
    assert call(Hkv=3) == pp.PP_ERR_INVALID_ARG                # 4 query heads are not a multiple of 3
    assert call(Hkv=0) == pp.PP_ERR_INVALID_ARG
    # grouped heads: the caches and the new keys hold Hkv = 1 row per slot,
    # and the workspace is the grouped one
    gq_bytes = lib.pp_attn_multi_workspace_bytes(1000, 1, 8, 4, 1, 128, pp.PP_BF16)
    assert gq_bytes > 0
    assert call(v=K + 1000 * 128 * 2, Hkv=1, wsb=gq_bytes - 1) == pp.PP_ERR_WORKSPACE
    assert call(v=K + 1000 * 128 * 2 - 256, Hkv=1, wsb=gq_bytes) == pp.PP_ERR_INVALID_ARG  # caches overlap
    assert call(kn=OUT - 8 * 128 * 2 + 16, Hkv=1, wsb=gq_bytes) == pp.PP_ERR_INVALID_ARG  # one-row key ends in out
    assert lib.pp_last_error_message().decode() != ""


def test_step_plan_multi_validation():
    lib = pp.raw()
    BASE, ACT, HEAD, CNT, SL = 0x60000000, 0x68000000, 0x70000000, 0x80000000, 0x90000000

    def call(sid=SID, base=BASE, act=ACT, max_len=1000, B=3, P=8, head=HEAD, cnt=CNT, sl=SL, cap=16):
        return lib.pp_step_plan_multi(sid, base, act, max_len, B, P, head, cnt, sl, cap, None)

    assert call(B=0) == pp.PP_ERR_INVALID_ARG
    assert call(B=70000) == pp.PP_ERR_INVALID_ARG
    assert call(P=1001) == pp.PP_ERR_INVALID_ARG
    assert call(base=None) == pp.PP_ERR_INVALID_ARG
    assert call(sid=SID + 4) == pp.PP_ERR_INVALID_ARG                  # misaligned ids
    assert call(head=SID + 3 * 1000 * 4 - 8) == pp.PP_ERR_INVALID_ARG  # head over request 2's ids
    assert call(act=SID + 2 * 1000 * 4) == pp.PP_ERR_INVALID_ARG        # active inside the ids
    assert call(head=ACT + 3 * 8 * 4 - 4) == pp.PP_ERR_INVALID_ARG      # head over the active flags
    assert call(cnt=HEAD + 20) == pp.PP_ERR_INVALID_ARG                 # counts over the 2B-entry head
    assert call(sl=CNT + 3 * 8 * 4 - 4) == pp.PP_ERR_INVALID_ARG        # lists over the B*P counts
    assert lib.pp_last_error_message().decode() != ""


def test_decode_append_multi_validation():
    lib = pp.raw()
    KN, VN, ACT, HEAD, CNT, SL = 0x70000000, 0x78000000, 0x7C000000, 0x80000000, 0x90000000, 0xA0000000
    B, P, Hq, Hkv, T = 3, 8, 8, 2, 1000
    ws_bytes = lib.pp_attn_multi_workspace_bytes(T, B, P, Hq, Hkv, 128, pp.PP_BF16)
    assert ws_bytes > lib.pp_attn_multi_workspace_bytes(T, 1, P, Hq, Hkv, 128, pp.PP_BF16)

    def call(q=Q, kn=KN, vn=VN, k=K, v=V, act=ACT, B=B, Hq=Hq, Hkv=Hkv, head=HEAD, out=OUT, ws=WS, wsb=ws_bytes):
        return lib.pp_attn_decode_append_multi(q, kn, vn, k, v, SID, act, T, B, P, Hq, Hkv, 128, 0.088, 1e4, head, CNT,
                                               SL, 16, out, pp.PP_BF16, ws, wsb, None)

    assert call(B=0) == pp.PP_ERR_INVALID_ARG
    assert call(Hkv=3) == pp.PP_ERR_INVALID_ARG
    assert call(head=None) == pp.PP_ERR_INVALID_ARG
    assert call(kn=None) == pp.PP_ERR_INVALID_ARG
    assert call(v=K + B * T * Hkv * 128 * 2 - 256) == pp.PP_ERR_INVALID_ARG  # the B caches overlap
    assert call(kn=OUT + B * P * Hq * 128 * 2 - 16) == pp.PP_ERR_INVALID_ARG  # new keys end inside out
    assert call(head=OUT + B * P * Hq * 128 * 2 - 8) == pp.PP_ERR_INVALID_ARG  # 2B-entry head overlaps out
    assert call(wsb=ws_bytes - 1) == pp.PP_ERR_WORKSPACE
    assert lib.pp_last_error_message().decode() != ""


def test_prefill_validation():
    lib = pp.raw()
    assert lib.pp_attn_prefill_workspace_bytes(0, 4, 128, pp.PP_BF16) == 0
    assert lib.pp_attn_prefill_workspace_bytes(100, 4, 96, pp.PP_BF16) == 0
    assert lib.pp_attn_prefill_workspace_bytes(65535 * 256 + 1, 4, 128, pp.PP_BF16) == 0
    n = lib.pp_attn_prefill_workspace_bytes(1000, 4, 128, pp.PP_BF16)
    assert n >= 1000 * 4 * (128 + 2) * 4  # one fp32 partial state per (slot, head)

    def call(q=Q, k=K, v=V, sid=SID, T=1000, out=OUT, ws=WS, wsb=n, scale=0.088, d=128, hkv=4):
        return lib.pp_attn_prefill(q, k, v, sid, T, 4, hkv, d, scale, out, pp.PP_BF16, ws, wsb, None)

    assert call(q=None) == pp.PP_ERR_INVALID_ARG
    assert call(sid=None) == pp.PP_ERR_INVALID_ARG
    assert call(T=0) == pp.PP_ERR_INVALID_ARG
    assert call(d=96) == pp.PP_ERR_UNSUPPORTED
    assert call(hkv=3) == pp.PP_ERR_INVALID_ARG               # 4 query heads cannot share 3
    assert call(hkv=0) == pp.PP_ERR_INVALID_ARG
    assert call(scale=float("nan")) == pp.PP_ERR_INVALID_ARG
    assert call(k=K + 2) == pp.PP_ERR_INVALID_ARG             # misaligned
    assert call(out=V + 1024) == pp.PP_ERR_INVALID_ARG        # out overlaps an input
    assert call(ws=Q + 4096) == pp.PP_ERR_INVALID_ARG         # workspace overlaps q
    assert call(wsb=n - 1) == pp.PP_ERR_WORKSPACE
    assert call(ws=None) == pp.PP_ERR_WORKSPACE
    assert lib.pp_last_error_message().decode() != ""


def test_multi_validation():
    lib = pp.raw()
    LENS = 0x70000000
    assert lib.pp_attn_multi_workspace_bytes(1000, 3, 8, 8, 3, 128, pp.PP_BF16) == 0  # 8 % 3 != 0
    assert lib.pp_attn_multi_workspace_bytes(1000, 0, 8, 8, 2, 128, pp.PP_BF16) == 0
    n = lib.pp_attn_multi_workspace_bytes(1000, 3, 8, 8, 2, 128, pp.PP_BF16)
    assert n >= 3 * 8 * 8 * (128 + 2) * 4
    assert n > lib.pp_attn_multi_workspace_bytes(1000, 1, 8, 8, 2, 128, pp.PP_BF16)

    def call(B=3, Hq=8, Hkv=2, lens=LENS, out=OUT, wsb=n, batched=False, active=None):
        fn = lib.pp_attn_decode_multi_batched if batched else lib.pp_attn_decode_multi
        return fn(Q, K, V, SID, lens, active, 1000, B, 8, Hq, Hkv, 128, 0.088, out, pp.PP_BF16, WS, wsb, None)

    assert call(B=0) == pp.PP_ERR_INVALID_ARG
    assert call(Hkv=3) == pp.PP_ERR_INVALID_ARG
    assert call(Hkv=0) == pp.PP_ERR_INVALID_ARG
    assert call(lens=None) == pp.PP_ERR_INVALID_ARG
    assert call(lens=OUT + 64) == pp.PP_ERR_INVALID_ARG        # lengths inside out
    assert call(out=K + 3 * 1000 * 2 * 128 * 2 - 64) == pp.PP_ERR_INVALID_ARG  # out overlaps the last request's keys
    assert call(wsb=n - 1) == pp.PP_ERR_WORKSPACE
    assert call(wsb=n - 1, batched=True) == pp.PP_ERR_WORKSPACE
    assert call(active=WS + 256) == pp.PP_ERR_INVALID_ARG      # stream flags inside the workspace
    assert lib.pp_last_error_message().decode() != ""


def test_python_binding_rejects_cpu_tensors():
    import torch

    q = torch.zeros(2, 1, 64)
    with pytest.raises(ValueError):
        pp.pp_attn_decode(q, q, q, torch.zeros(2, dtype=torch.int32))


def test_python_bindings_of_the_extensions_reject_host_tensors():
    # every binding checks its tensors before calling the library: host
    # tensors (there is no GPU here) are refused with ValueError
    import torch

    q = torch.zeros(2, 1, 64, dtype=torch.bfloat16)
    sid = torch.zeros(8, dtype=torch.int32)
    with pytest.raises(ValueError):
        pp.pp_attn_decode_batched(q, q, q, sid)
    with pytest.raises(ValueError):
        pp.pp_attn_decode_planned(q, q, q, sid, (sid[:1], sid[:2], sid[:2].view(2, 1)))
    with pytest.raises(ValueError):
        pp.pp_attn_plan(sid, 8, 2)
    with pytest.raises(ValueError):
        pp.pp_step_plan(sid, torch.zeros(1, dtype=torch.int32), 2)
    with pytest.raises(ValueError):
        pp.pp_attn_decode_append(q, q, q, q, q, sid, (sid[:2], sid[:2], sid[:2].view(2, 1)))
    with pytest.raises(ValueError):
        pp.pp_attn_prefill(q, q, q, sid[:2])
    with pytest.raises(ValueError):
        pp.pp_step_plan_multi(sid.view(1, 8), torch.zeros(1, dtype=torch.int32), 2)
    with pytest.raises(ValueError):
        pp.pp_attn_decode_append_multi(q.view(1, *q.shape), q.view(1, *q.shape), q.view(1, *q.shape),
                                       q.view(1, *q.shape), q.view(1, *q.shape), sid.view(1, 8),
                                       (sid[:2], sid[:2].view(1, 2), sid[:2].view(1, 2, 1)))
    q4 = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pp.pp_attn_decode_multi(q4, q4, q4, sid.view(1, 8), torch.ones(1, dtype=torch.int32))


def test_bench_refuses_several_gpus():
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(__file__))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=root, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_stream_read_validation():
    lib = pp.raw()
    # null, misaligned, empty or ragged sizes, blocks per CU out of range: rejected before any HIP call
    assert lib.pp_stream_read(None, 1024, OUT, 8, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_stream_read(Q + 8, 1024, OUT, 8, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_stream_read(Q, 0, OUT, 8, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_stream_read(Q, 1000, OUT, 8, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_stream_read(Q, 1024, None, 8, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_stream_read(Q, 1024, OUT, 0, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_stream_read(Q, 1024, OUT, 65, None) == pp.PP_ERR_INVALID_ARG


def test_plan_workspace_bytes():
    lib = pp.raw()
    # chunk rows of the two-pass plan: at most 64 chunks of P + 4 ints, never below the fixed minimum
    assert lib.pp_attn_plan_workspace_bytes(10, 2) == pp.PP_PLAN_WORKSPACE_BYTES
    n = lib.pp_attn_plan_workspace_bytes(31825, 256)
    assert n >= 32 * (256 + 4) * 4 and n < 64 * (256 + 4) * 4 + 1024
    assert lib.pp_attn_plan_workspace_bytes(1 << 20, 1024) >= 64 * (1024 + 4) * 4
    assert lib.pp_attn_plan_workspace_bytes(1000, 5000) == pp.PP_PLAN_WORKSPACE_BYTES  # one pass per stream
    assert lib.pp_attn_plan_workspace_bytes(0, 2) == 0 and lib.pp_attn_plan_workspace_bytes(10, 0) == 0
    # a workspace below the size for the shape is rejected
    big = lib.pp_attn_plan_workspace_bytes(31825, 256)
    assert lib.pp_attn_plan(SID, 31825, 256, OUT, WS, K, 4, V, big - 1, None) == pp.PP_ERR_WORKSPACE
    # a workspace over the ids is rejected
    assert lib.pp_attn_plan(SID, 31825, 256, OUT, WS, K, 4, SID, big, None) == pp.PP_ERR_INVALID_ARG


def test_noalloc_rejects_shapes_beyond_its_scratch_on_the_host():
    lib = pp.raw()
    T, P, H, d = 40000, 1024, 64, 128
    assert lib.pp_attn_workspace_bytes(T, P, H, d, pp.PP_BF16) > pp.PP_NOALLOC_SCRATCH_BYTES
    assert lib.pp_attn_decode_noalloc(Q, K, V, SID, T, P, H, d, 0.088, OUT, pp.PP_BF16, None) == pp.PP_ERR_WORKSPACE
    assert b"fixed scratch" in lib.pp_last_error_message()
    # an invalid shape gets the decode step's own status
    assert lib.pp_attn_decode_noalloc(Q, K, V, SID, 0, 8, 4, 128, 0.088, OUT, pp.PP_BF16, None) == pp.PP_ERR_INVALID_ARG
    assert lib.pp_attn_decode_noalloc(Q, K, V, SID, 100, 8, 4, 96, 0.088, OUT, pp.PP_BF16, None) == pp.PP_ERR_UNSUPPORTED
    text = open(HEADER).read()
    assert re.search(r"#define PP_NOALLOC_SCRATCH_BYTES \(\(size_t\)64 << 20\)", text)
    assert pp.PP_NOALLOC_SCRATCH_BYTES == 64 << 20
