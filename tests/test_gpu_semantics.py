"""GPU tests of the method's properties, through the C ABI:
isolation between streams (bit-identical), run-to-run determinism, the
integer visibility plan (bit-exact vs the oracle), layouts the canonical
generator does not produce, degenerate cases, and stream semantics."""
import dataclasses

import numpy as np
import pytest
import torch

import shared_prefix_stream_amd as pp
from oracle import tail_lists
from tests.gpu_helpers import assert_close, reference, run, say, to_gpu
from workloads import make_case, permute_tail

pytestmark = pytest.mark.gpu


def _case(seed, P=6, H=4, D=128, doc=700, dtype=torch.bfloat16, qmax=12, amax=8, **kw):
    rng = np.random.default_rng(seed)
    return make_case(H, D, doc, rng.integers(1, qmax + 1, P).tolist(), rng.integers(0, amax + 1, P).tolist(),
                     dtype=dtype, seed=seed, name=f"sem_p{P}_doc{doc}_s{seed}", **kw)


# ---------------------------------------------------------------- isolation ---

@pytest.mark.parametrize("entry", ["decode", "batched"])
@pytest.mark.parametrize("bad", ["finite", "inf", "nan"])
def test_other_streams_cannot_reach_a_stream(entry, bad):
    case = _case(1, P=5)
    base = run(case, entry).cpu()
    for s in range(case.P):
        k, v = case.k.clone(), case.v.clone()
        for o in range(case.P):
            if o == s:
                continue
            idx = torch.from_numpy(case.own_slots[o])
            if bad == "finite":
                k[idx] = (k[idx].float() * 3 + 1).to(k.dtype)
                v[idx] = (v[idx].float() - 2).to(v.dtype)
            else:
                val = float("inf") if bad == "inf" else float("nan")
                k[idx] = val
                v[idx] = val
        args = [case.q.cuda(), k.cuda(), v.cuda(), case.stream_id.cuda()]
        out = run(case, entry, gpu_args=args).cpu()
        assert torch.equal(out[s].view(torch.int16), base[s].view(torch.int16)), f"stream {s} changed"


# ------------------------------------------------------------- determinism ---

@pytest.mark.parametrize("entry", ["decode", "batched"])
def test_bitwise_reproducible(entry):
    case = _case(2, P=40, H=8, doc=3000)
    args = to_gpu(case)
    first = run(case, entry, gpu_args=args).clone()
    for _ in range(4):
        again = run(case, entry, gpu_args=args)
        assert torch.equal(first.view(torch.int16), again.view(torch.int16))


# ---------------------------------------------- concurrency and scheduling ---

def test_profiled_equals_decode():
    # the profiling variant binds events to the same kernels: same bits
    case = _case(21, P=70, H=8, doc=4100, qmax=40, amax=20)
    q, k, v, sid = to_gpu(case)
    say("  gpu: decode vs profiled")
    a = pp.pp_attn_decode(q, k, v, sid, seq_len=case.seq_len, scale=case.scale)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(pp.PP_PROFILE_EVENTS)]
    for e in evs:
        e.record()  # torch creates the underlying hipEvent_t on first record
    torch.cuda.synchronize()
    b = pp.pp_attn_decode_profiled([e.cuda_event for e in evs], q, k, v, sid, seq_len=case.seq_len,
                                   scale=case.scale)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for i in range(0, pp.PP_PROFILE_EVENTS, 2):  # each stage's kernel: start -> end
        assert evs[i].elapsed_time(evs[i + 1]) > 0.0
    assert_close(a, reference(case), what="decode")


def test_two_caller_streams():
    # calls enqueued from two streams, each with its own workspace
    c1, c2 = _case(22, P=9, doc=2000), _case(23, P=13, H=8, doc=900)
    g1, g2 = to_gpu(c1), to_gpu(c2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    say("  gpu: two caller streams")
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            o1 = pp.pp_attn_decode(*g1, seq_len=c1.seq_len, scale=c1.scale)
        with torch.cuda.stream(s2):
            o2 = pp.pp_attn_decode(*g2, seq_len=c2.seq_len, scale=c2.scale)
        outs.append((o1, o2))
    torch.cuda.synchronize()
    r1, r2 = reference(c1), reference(c2)
    for o1, o2 in outs:
        assert_close(o1, r1, what="stream 1")
        assert_close(o2, r2, what="stream 2")
        assert torch.equal(o1.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(o2.view(torch.int16), outs[0][1].view(torch.int16))


def test_graph_capture_replays():
    # a captured step replayed several times, with
    # eager work and synchronisations between replays; every replay must
    # equal the eager result
    case = _case(24, P=33, H=8, doc=3000, qmax=30, amax=20)
    q, k, v, sid = to_gpu(case)
    ws = torch.empty(pp.workspace_bytes(case.seq_len, case.P, case.H, case.D, q.dtype), dtype=torch.uint8,
                     device=q.device)
    eager = pp.pp_attn_decode(q, k, v, sid, seq_len=case.seq_len, scale=case.scale, workspace=ws).clone()
    out = torch.zeros_like(q)
    torch.cuda.synchronize()
    say("  gpu: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pp.pp_attn_decode(q, k, v, sid, seq_len=case.seq_len, scale=case.scale, out=out, workspace=ws)
    torch.cuda.synchronize()
    for i in range(4):
        say(f"  gpu: replay {i}")
        out.zero_()
        ws.fill_(0xFF)  # stale partial states must not matter
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"
        junk = pp.pp_attn_decode_batched(q, k, v, sid, seq_len=case.seq_len, scale=case.scale)
        torch.cuda.synchronize()
        del junk


# -------------------------------------------------------- integer plan (a1) ---

def _plan_check(ids_np, seq_len, P, cap=8192):
    sid = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).cuda()
    say(f"  gpu: pp_attn_plan T={seq_len} P={P}")
    doc_len, counts, slots = pp.pp_attn_plan(sid, seq_len, P, cap)
    torch.cuda.synchronize()
    d_ref, lists = tail_lists(ids_np, seq_len, P)
    assert int(doc_len.item()) == d_ref
    counts = counts.cpu().numpy()
    slots = slots.cpu().numpy()
    for s in range(P):
        assert counts[s] == len(lists[s]), f"stream {s}"
        n = min(len(lists[s]), cap)
        assert np.array_equal(slots[s, :n], lists[s][:n]), f"stream {s}"


def test_plan_canonical_and_permuted():
    case = _case(3, P=37, doc=5000, qmax=40, amax=30)
    _plan_check(case.stream_id.numpy(), case.seq_len, case.P)
    pc = permute_tail(case, 4)
    _plan_check(pc.stream_id.numpy(), pc.seq_len, pc.P)


def test_plan_junk_ids_late_document_and_no_document():
    rng = np.random.default_rng(5)
    P = 9
    ids = np.concatenate([np.zeros(300), rng.integers(-3, P + 4, 7000)]).astype(np.int32)
    ids[rng.integers(300, 7300, 50)] = 0  # document slots after the prefix
    _plan_check(ids, len(ids), P)
    _plan_check(ids, 4000, P)  # seq_len inside the buffer (not a multiple of 4 away from anything)
    _plan_check(ids[300:].copy(), 5001, P)  # first slot not a document slot: doc_len 0


def test_plan_all_document_and_many_own_slots():
    _plan_check(np.zeros(10001, dtype=np.int32), 10001, 3)
    # one stream owning more slots than one 4096-slot compaction chunk holds
    ids = np.concatenate([np.zeros(17), np.ones(9000), np.full(3, 2)]).astype(np.int32)
    _plan_check(ids, len(ids), 2, cap=10000)


def test_plan_headline_shape_canonical_and_permuted():
    # doc 16k, 256 streams: chunks past the document, questions and interleaved answers
    from workloads import named_workload

    case = named_workload("codellama7b_doc16k_p256", seed=1002)
    _plan_check(case.stream_id.numpy(), case.seq_len, case.P, cap=2048)
    pc = permute_tail(case, 9)
    _plan_check(pc.stream_id.numpy(), pc.seq_len, pc.P, cap=2048)


@pytest.mark.parametrize("doc", [0, 1, 255, 256, 257, 2047, 2048, 2049, 32767, 32768, 32769])
def test_plan_prefix_and_end_at_row_and_wave_edges(doc):
    # the plan reads ids in rows of 256 slots, 2048 per wave and 32768 per
    # round, and skips rows outside [doc_len, seq_len): the prefix end and the
    # sequence end on and around those edges, with late document slots and
    # foreign ids in the tail
    rng = np.random.default_rng(doc + 17)
    P = 5
    n = 4100
    ids = np.concatenate([np.zeros(doc), rng.integers(1, P + 1, n)]).astype(np.int32)
    ids[doc + rng.integers(1, n, 6)] = 0
    ids[doc + rng.integers(1, n, 6)] = P + 3
    T = len(ids)
    for seq_len in sorted({T, doc + 1, doc + 255, doc + 256, doc + 257, doc + 2048, doc + 2049, T - 1}):
        if 1 <= seq_len <= T:
            _plan_check(ids, seq_len, P)


@pytest.mark.parametrize("P", [1, 1023, 1024, 1025])
def test_plan_stream_counts_around_the_two_pass_limit(P):
    # up to 1024 streams the plan takes two passes over chunks of the ids, past that one pass per stream
    rng = np.random.default_rng(P)
    n = 40000
    ids = np.concatenate([np.zeros(3000), rng.integers(1, P + 1, n)]).astype(np.int32)
    _plan_check(ids, len(ids), P, cap=256)
    ids[rng.integers(3000, 3000 + n, 20)] = 0  # late document slots in a few chunks
    ids[rng.integers(3000, 3000 + n, 20)] = P + 7  # foreign ids
    _plan_check(ids, len(ids), P, cap=256)


def test_plan_long_sequence_multi_slot_chunks():
    # more than 64 chunks' worth of slots: chunks of several 1024-slot sub-chunks
    rng = np.random.default_rng(11)
    P = 300
    ids = np.concatenate([np.zeros(70001), rng.integers(0, P + 2, 90000)]).astype(np.int32)
    _plan_check(ids, len(ids), P, cap=512)
    ids2 = ids.copy()
    ids2[70001:] = rng.integers(1, P + 1, 90000)  # no late document slots: every chunk on the ranked path
    _plan_check(ids2, len(ids2), P, cap=512)
    _plan_check(ids2, 150003, P, cap=512)


# ---------------------------------------------------------- layout variants ---

@pytest.mark.parametrize("entry", ["decode", "batched"])
def test_permuted_tail_layout(entry):
    case = permute_tail(_case(6, P=11, doc=900), 7)
    assert_close(run(case, entry), reference(case), what=case.name)


@pytest.mark.parametrize("entry", ["decode", "batched"])
def test_late_document_slots_and_foreign_ids(entry):
    case = _case(8, P=6, doc=400)
    rng = np.random.default_rng(9)
    sid = case.stream_id.clone()
    tail = np.arange(case.doc_len, case.seq_len)
    pick = rng.choice(tail, 12, replace=False)
    sid[torch.from_numpy(pick[:6])] = 0            # visible to every stream
    sid[torch.from_numpy(pick[6:9])] = -1          # the page's document id: not this encoding's
    sid[torch.from_numpy(pick[9:])] = case.P + 3   # no such stream
    case.stream_id = sid
    assert_close(run(case, entry), reference(case), what="late-doc/foreign ids")


@pytest.mark.parametrize("entry", ["decode", "batched"])
def test_stream_with_more_slots_than_the_plan_lists(entry):
    # stream 0 sees more slots past the prefix than the plan keeps per stream
    # (2048): its workgroups compact the list themselves; stream 1 uses the
    # plan's list; later document slots are in both
    case = make_case(4, 128, 600, [2500, 10], [600, 12], seed=17, name="long-own-list")
    rng = np.random.default_rng(18)
    sid = case.stream_id.clone()
    pick = rng.choice(np.arange(case.doc_len, case.seq_len), 40, replace=False)
    sid[torch.from_numpy(pick)] = 0
    case.stream_id = sid
    assert_close(run(case, entry), reference(case), what="long own list")


@pytest.mark.parametrize("entry", ["decode", "batched"])
def test_only_first_seq_len_slots_read(entry):
    case = _case(10, P=4, doc=500, extra_capacity=333)  # slots past seq_len hold NaN
    assert_close(run(case, entry), reference(case), what="extra capacity")


# ------------------------------------------------------------ degenerate ---

@pytest.mark.parametrize("entry", ["decode", "batched"])
def test_empty_visible_set_gives_zeros(entry):
    # no document at all; stream 1 owns nothing
    case = make_case(2, 128, 0, [3, 0, 2], [1, 0, 2], seed=11, name="no-doc")
    out = run(case, entry).cpu()
    assert torch.equal(out[1], torch.zeros_like(out[1]))
    assert_close(out, reference(case), what="no-doc")


@pytest.mark.parametrize("entry", ["decode", "batched"])
def test_single_visible_key_returns_its_value(entry):
    case = make_case(4, 128, 1, [0, 0, 0], [0, 0, 0], seed=12, name="doc1")
    out = run(case, entry).cpu()
    for s in range(3):
        assert torch.equal(out[s].view(torch.int16), case.v[0].view(torch.int16))


@pytest.mark.parametrize("entry", ["decode", "batched"])
def test_p1_is_causal_attention(entry):
    # one stream, its current token's K/V appended last: plain causal attention
    case = make_case(4, 128, 2000, [30], [9], seed=13, name="p1")
    assert_close(run(case, entry), reference(case), what="P=1")


@pytest.mark.parametrize("entry", ["decode", "batched"])
def test_peaked_softmax_outliers(entry):
    case = _case(14, P=8, doc=2000, outlier_frac=0.01, outlier_mult=50.0)
    assert_close(run(case, entry), reference(case), what="outliers")


@pytest.mark.parametrize("entry", ["decode", "batched"])
@pytest.mark.parametrize("kind", ["large_scale", "negative_scale", "all_scores_very_negative", "mixed_splits"])
def test_extreme_score_ranges(entry, kind):
    # score ranges whose softmax sums leave [2^-64, 2^64] without a running
    # maximum: exp2 of the scaled scores overflows, or every term underflows
    case = _case(16, P=5, doc=3000)
    if kind == "large_scale":
        case = dataclasses.replace(case, scale=3.0)
    elif kind == "negative_scale":
        case = dataclasses.replace(case, scale=-3.0)
    elif kind == "all_scores_very_negative":
        case = dataclasses.replace(case, q=case.q.abs(), k=-case.k.abs(), scale=1.0)
    else:  # only the document's second half has huge scores (some splits normal, some not)
        k = case.k.clone()
        k[1500:case.doc_len] *= 8
        case = dataclasses.replace(case, k=k, scale=0.4)
    assert_close(run(case, entry), reference(case), what=kind)


@pytest.mark.parametrize("capacity", ["full", "short", "zero"])
def test_planned_decode_reuses_one_plan_across_layers(capacity):
    # one plan for the step's ids, three "layers" with their own q/k/v: the
    # planned entry gives what pp_attn_decode gives (bitwise), also when the
    # plan's lists are cut short and completed on the device
    rng = np.random.default_rng(18)
    q_lens, a_lens = rng.integers(1, 13, 9).tolist(), rng.integers(0, 9, 9).tolist()
    layers = [make_case(4, 128, 1300, q_lens, a_lens, seed=18 + i, name=f"layer{i}") for i in range(3)]
    sid = layers[0].stream_id.to("cuda:0")
    T, P = layers[0].seq_len, layers[0].P
    cap = {"full": T, "short": 3, "zero": 0}[capacity]
    plan = pp.pp_attn_plan(sid, T, P, tail_capacity=cap)
    torch.cuda.synchronize()
    if capacity == "short":
        assert int(plan[1].max()) > cap  # the device-side completion is exercised
    for case in layers:
        q, k, v, _ = to_gpu(case)
        a = pp.pp_attn_decode(q, k, v, sid, seq_len=T, scale=case.scale)
        b = pp.pp_attn_decode_planned(q, k, v, sid, plan, seq_len=T, scale=case.scale)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), case.name
        assert_close(b, reference(case), what=case.name)


# -------------------------------------------------------------- streams ---

def test_runs_on_a_side_stream_without_host_sync():
    case = _case(15, P=12, doc=1200)
    args = to_gpu(case)
    side = torch.cuda.Stream()
    say("  gpu: decode on a side stream")
    with torch.cuda.stream(side):
        out = pp.pp_attn_decode(*args, seq_len=case.seq_len, scale=case.scale)
        out2 = pp.pp_attn_decode_batched(*args, seq_len=case.seq_len, scale=case.scale)
    side.synchronize()
    ref = reference(case)
    assert_close(out, ref, what="side stream")
    assert_close(out2, ref, what="side stream batched")


def test_decode_and_batched_agree():
    case = _case(16, P=33, H=8, doc=4100)
    a = run(case, "decode").double().cpu().numpy()
    b = run(case, "batched").double().cpu().numpy()
    assert np.abs(a - b).max() <= 2e-2
