"""GPU parity of the appending decode step: ids and plan written by
pp_step_plan, keys and queries rotated at the shared positions and appended
by pp_attn_decode_append, then the attention; a multi-step, multi-layer loop
captured once as a HIP graph and replayed step after step.  Expected values
come from the step oracle, which runs its own loop from the same seeded
inputs."""
import numpy as np
import pytest
import torch

import shared_prefix_stream_amd as pp
from oracle import oracle_append_step, tail_lists
from tests.gpu_helpers import assert_close, say
from workloads import canonical_layout, decode_loop_layout, decode_loop_step_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _bf16_ulp(x):
    _, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def _rot_bound(want, x):
    """Largest difference allowed between a rotated element rounded once from
    an fp32 rotation and the exact rotation rounded once: one bf16 unit of the
    result, plus the fp32 rounding of the pair's products (which decides the
    rounding when the two products nearly cancel)."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    mag = np.abs(x[..., :h]) + np.abs(x[..., h:])
    mag = np.concatenate([mag, mag], axis=-1)
    return _bf16_ulp(want) * 1.0001 + mag * 2.0 ** -21


# ------------------------------------------------------------ step plan ---

@pytest.mark.parametrize("shape", ["ragged", "doc_only_before", "empty_cache", "short_lists"])
def test_step_plan_writes_ids_and_the_plan(shape):
    rng = np.random.default_rng(31)
    P = 37
    if shape == "empty_cache":
        ids0 = np.zeros(0, dtype=np.int32)
    elif shape == "doc_only_before":
        ids0 = np.zeros(1500, dtype=np.int32)
    else:
        ids0, _ = canonical_layout(1300, rng.integers(1, 30, P).tolist(), rng.integers(0, 9, P).tolist())
    T0 = len(ids0)
    cap_total = T0 + P + 77
    ids = np.concatenate([ids0, np.zeros(cap_total - T0, dtype=np.int32)])  # stale document-looking ids
    sid = _i32(ids)
    base = _i32([T0])
    tail_cap = 4 if shape == "short_lists" else 2048
    say(f"  gpu: pp_step_plan {shape} T0={T0} P={P}")
    head, counts, slots = pp.pp_step_plan(sid, base, P, max_seq_len=cap_total, tail_capacity=tail_cap)
    torch.cuda.synchronize()
    want = ids.copy()
    want[T0:T0 + P] = np.arange(1, P + 1)
    np.testing.assert_array_equal(sid.cpu().numpy(), want)  # only the new slots changed
    d_ref, lists = tail_lists(want, T0 + P, P)
    assert head.cpu().tolist() == [d_ref, T0 + P]
    c = counts.cpu().numpy()
    sl = slots.cpu().numpy()
    for s in range(P):
        assert c[s] == len(lists[s]), s
        n = min(len(lists[s]), tail_cap)
        np.testing.assert_array_equal(sl[s, :n], lists[s][:n])


@pytest.mark.parametrize("T0", [255, 256, 2047, 2048, 2049, 32767, 32768])
def test_step_plan_new_slots_at_row_and_wave_edges(T0):
    # the step's new slots start on and around the edges of the plan kernel's
    # rows (256 slots), waves (2048) and rounds (32768), behind stale ids
    rng = np.random.default_rng(T0)
    P = 300
    ids0 = np.zeros(T0, dtype=np.int32)
    ids0[T0 // 2:] = rng.integers(1, P + 1, T0 - T0 // 2)
    cap_total = T0 + P + 300
    ids = np.concatenate([ids0, rng.integers(0, P + 5, cap_total - T0).astype(np.int32)])
    sid = _i32(ids)
    say(f"  gpu: pp_step_plan T0={T0} P={P}")
    head, counts, slots = pp.pp_step_plan(sid, _i32([T0]), P, max_seq_len=cap_total, tail_capacity=2048)
    torch.cuda.synchronize()
    want = ids.copy()
    want[T0:T0 + P] = np.arange(1, P + 1)
    np.testing.assert_array_equal(sid.cpu().numpy(), want)
    d_ref, lists = tail_lists(want, T0 + P, P)
    assert head.cpu().tolist() == [d_ref, T0 + P]
    c = counts.cpu().numpy()
    sl = slots.cpu().numpy()
    for s in range(P):
        assert c[s] == len(lists[s]), s
        n = min(len(lists[s]), 2048)
        np.testing.assert_array_equal(sl[s, :n], lists[s][:n])


@pytest.mark.parametrize("base", [-1, 60])
def test_step_plan_out_of_range_base_is_an_empty_step(base):
    P, T = 8, 64
    ids = np.arange(T, dtype=np.int32) % 3
    sid = _i32(ids)
    head, counts, _ = pp.pp_step_plan(sid, _i32([base]), P, max_seq_len=T)
    torch.cuda.synchronize()
    assert head.cpu().tolist() == [0, 0]
    assert counts.cpu().tolist() == [0] * P
    np.testing.assert_array_equal(sid.cpu().numpy(), ids)
    # a layer of such a step writes nothing to the caches and zeros to out
    q = torch.randn(P, 2, 64, device=DEV).to(torch.bfloat16)
    k = torch.randn(T, 2, 64, device=DEV).to(torch.bfloat16)
    v = torch.randn(T, 2, 64, device=DEV).to(torch.bfloat16)
    k0, v0 = k.clone(), v.clone()
    out = pp.pp_attn_decode_append(q, q, q, k, v, sid, (head, counts, _), rope_base=1e4)
    torch.cuda.synchronize()
    assert torch.equal(k, k0) and torch.equal(v, v0)
    assert torch.count_nonzero(out).item() == 0


# ------------------------------------------------- append + rotate + attend ---

def _step_case(seed, P, H, D, doc, dtype, Hkv=None):
    Hkv = H if Hkv is None else Hkv
    rng = np.random.default_rng(seed)
    ids0, _ = canonical_layout(doc, rng.integers(1, 40, P).tolist(), rng.integers(0, 12, P).tolist())
    T0 = len(ids0)
    cap = T0 + P + 5
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(cap, Hkv, D, generator=g).to(dtype)
    v = torch.randn(cap, Hkv, D, generator=g).to(dtype)
    q = torch.randn(P, H, D, generator=g).to(dtype)
    kn, vn = (torch.randn(P, Hkv, D, generator=g).to(dtype) for _ in range(2))
    ids = np.concatenate([ids0, np.full(cap - T0, 0, dtype=np.int32)])
    return ids, T0, cap, k, v, q, kn, vn


@pytest.mark.parametrize("rope_base", [0.0, 1e4, 1e6])
@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 64)])
def test_decode_append_matches_the_oracle(rope_base, dtype, D):
    P, H = 13, 4
    ids, T0, cap, k, v, q, kn, vn = _step_case(41 + D, P, H, D, doc=700, dtype=dtype)
    scale = 1.0 / np.sqrt(D)
    kg, vg, sid = k.to(DEV), v.to(DEV), _i32(ids)
    say(f"  gpu: pp_attn_decode_append {dtype} D={D} base={rope_base} T0={T0} P={P}")
    plan = pp.pp_step_plan(sid, _i32([T0]), P, max_seq_len=cap)
    out = pp.pp_attn_decode_append(q.to(DEV), kn.to(DEV), vn.to(DEV), kg, vg, sid, plan, scale=scale,
                                   rope_base=rope_base)
    torch.cuda.synchronize()
    bf = dtype == torch.bfloat16
    r = oracle_append_step(q, kn, vn, k, v, ids, T0, scale, rope_base, store_bf16=bf)
    assert_close(out, r["out"], what=f"{dtype} D={D} base={rope_base}")
    kw = kg.double().cpu().numpy()
    vw = vg.double().cpu().numpy()
    # rows outside the step's new slots are untouched; values are copied as is
    np.testing.assert_array_equal(kw[:T0], k[:T0].double().numpy())
    np.testing.assert_array_equal(kw[T0 + P:], k[T0 + P:].double().numpy())
    np.testing.assert_array_equal(vw[T0:T0 + P], vn.double().numpy())
    # the rotated keys: one rounding of an fp32 rotation against the oracle's
    # rounding of the exact one -- equal, or one unit in the last place apart
    got, want = kw[T0:T0 + P], r["k_rot"]
    if rope_base <= 0:
        np.testing.assert_array_equal(got, kn.double().numpy())
    elif bf:
        diff = np.abs(got - want)
        assert (diff <= _rot_bound(want, kn.double().numpy())).all(), diff.max()
        assert (diff == 0).mean() > 0.99
    else:
        np.testing.assert_allclose(got, want, rtol=2e-6, atol=2e-6)


def test_decode_append_without_rotation_equals_append_then_decode():
    P, H, D = 21, 8, 128
    ids, T0, cap, k, v, q, kn, vn = _step_case(57, P, H, D, doc=2100, dtype=torch.bfloat16)
    kg, vg, sid = k.to(DEV), v.to(DEV), _i32(ids)
    plan = pp.pp_step_plan(sid, _i32([T0]), P, max_seq_len=cap)
    out = pp.pp_attn_decode_append(q.to(DEV), kn.to(DEV), vn.to(DEV), kg, vg, sid, plan, rope_base=0.0)
    k2, v2 = k.clone(), v.clone()
    k2[T0:T0 + P], v2[T0:T0 + P] = kn, vn
    ids2 = ids.copy()
    ids2[T0:T0 + P] = np.arange(1, P + 1)
    ref = pp.pp_attn_decode(q.to(DEV), k2.to(DEV), v2.to(DEV), _i32(ids2), seq_len=T0 + P)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


# ------------------------------------------- graph of a multi-layer step ---

def _loop(doc, P, steps, layers, H, D, seed, rope_base, check_oracle, use_graph, Hkv=None):
    """32-step style loop: at every step each stream appends one slot and
    every layer attends.  Returns the per-(step, layer) outputs on the host
    and, with check_oracle, compares each with the step oracle's own loop."""
    ids_full, _, base0 = decode_loop_layout(doc, P, steps, seed)
    cap = len(ids_full)
    scale = 1.0 / np.sqrt(D)
    ids = ids_full.copy()
    ids[base0:] = 0  # the appended region holds stale ids until a step writes them
    sid = _i32(ids)
    Hkv = H if Hkv is None else Hkv
    K = [torch.empty(cap, Hkv, D, dtype=torch.bfloat16, device=DEV) for _ in layers]
    V = [torch.empty_like(K[0]) for _ in layers]
    oK, oV = [], []
    for i, layer in enumerate(layers):
        inp = decode_loop_step_inputs(H, D, P, cap, layer, 0, seed, base_len=base0, Hkv=Hkv)
        K[i][:base0] = inp["k0"].to(DEV)
        V[i][:base0] = inp["v0"].to(DEV)
        if check_oracle:
            oK.append(np.zeros((cap, Hkv, D)))
            oV.append(np.zeros((cap, Hkv, D)))
            oK[i][:base0] = inp["k0"].double().numpy()
            oV[i][:base0] = inp["v0"].double().numpy()
    o_ids = ids.copy()
    base = _i32([base0])
    plan = (torch.zeros(2, dtype=torch.int32, device=DEV), torch.zeros(P, dtype=torch.int32, device=DEV),
            torch.zeros(P, 256, dtype=torch.int32, device=DEV))
    ws = torch.empty(pp.multi_workspace_bytes(cap, 1, P, H, Hkv, D, torch.bfloat16), dtype=torch.uint8, device=DEV)
    qin = [torch.empty(P, h, D, dtype=torch.bfloat16, device=DEV) for _ in layers for h in (H, Hkv, Hkv)]
    outs = [torch.empty(P, H, D, dtype=torch.bfloat16, device=DEV) for _ in layers]

    def step():
        pp.pp_step_plan(sid, base, P, max_seq_len=cap, plan=plan)
        for i in range(len(layers)):
            pp.pp_attn_decode_append(qin[3 * i], qin[3 * i + 1], qin[3 * i + 2], K[i], V[i], sid, plan, scale=scale,
                                     rope_base=rope_base, out=outs[i], workspace=ws, max_seq_len=cap)
        base.add_(P)

    graph = None
    if use_graph:
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        say("  gpu: capture")
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        base.fill_(base0)  # capture does not run the work
    results = []
    for t in range(steps):
        inps = [decode_loop_step_inputs(H, D, P, cap, layer, t, seed, base_len=base0, Hkv=Hkv) for layer in layers]
        for i, inp in enumerate(inps):
            qin[3 * i].copy_(inp["q"])
            qin[3 * i + 1].copy_(inp["k_new"])
            qin[3 * i + 2].copy_(inp["v_new"])
        if graph is not None:
            graph.replay()
        else:
            step()
        torch.cuda.synchronize()
        results.append([o.clone() for o in outs])
        assert int(base.item()) == base0 + (t + 1) * P
        if check_oracle:
            b = base0 + t * P
            for i, inp in enumerate(inps):
                r = oracle_append_step(inp["q"], inp["k_new"], inp["v_new"], oK[i], oV[i], o_ids, b, scale, rope_base)
                oK[i][b:b + P] = r["k_cache"][b:b + P]
                oV[i][b:b + P] = r["v_cache"][b:b + P]
                assert_close(outs[i], r["out"], what=f"step {t} layer {layers[i]}")
            o_ids[b:b + P] = np.arange(1, P + 1)
            if t % 8 == 0:
                say(f"  checked step {t}")
    np.testing.assert_array_equal(sid.cpu().numpy()[:base0 + steps * P], ids_full[:base0 + steps * P])
    return results


def test_graph_of_the_step_replays_every_step():
    # one capture of (plan + 4 layers + advance), replayed 32 times: every
    # step matches the oracle's own loop and the eager calls bit for bit
    args = dict(doc=512, P=16, steps=32, layers=[0, 1, 2, 3], H=32, D=128, seed=91, rope_base=1e6)
    g = _loop(**args, check_oracle=True, use_graph=True)
    e = _loop(**args, check_oracle=False, use_graph=False)
    for t in range(len(g)):
        for i in range(len(g[t])):
            assert torch.equal(g[t][i].view(torch.int16), e[t][i].view(torch.int16)), (t, i)


def test_full_size_appending_step_sampled():
    # the 12000-token document with 256 streams, at its last answer step
    # (31 answers already in the cache), one layer with rotation
    doc, P, steps, H, D, seed = 12000, 256, 32, 32, 128, 1003
    ids_full, _, base0 = decode_loop_layout(doc, P, steps, seed)
    cap = len(ids_full)
    t = steps - 1
    b = base0 + t * P
    k = torch.empty(cap, H, D, dtype=torch.bfloat16)
    v = torch.empty_like(k)
    inp0 = decode_loop_step_inputs(H, D, P, cap, 5, 0, seed, base_len=base0)
    k[:base0], v[:base0] = inp0["k0"], inp0["v0"]
    for u in range(t):  # earlier answers, as already-rotated cache rows
        inp = decode_loop_step_inputs(H, D, P, cap, 5, u, seed, base_len=base0)
        k[base0 + u * P: base0 + (u + 1) * P] = inp["k_new"]
        v[base0 + u * P: base0 + (u + 1) * P] = inp["v_new"]
    ids = ids_full.copy()
    ids[b:] = 0
    step_inp = decode_loop_step_inputs(H, D, P, cap, 5, t, seed)
    sid = _i32(ids)
    kg, vg = k.to(DEV), v.to(DEV)
    say(f"  gpu: full-size appending step T={b + P} P={P}")
    plan = pp.pp_step_plan(sid, _i32([b]), P, max_seq_len=cap)
    out = pp.pp_attn_decode_append(step_inp["q"].to(DEV), step_inp["k_new"].to(DEV), step_inp["v_new"].to(DEV), kg,
                                   vg, sid, plan, rope_base=1e6)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    streams = sorted({0, P - 1} | set(rng.choice(P, 6, replace=False).tolist()))
    r = oracle_append_step(step_inp["q"], step_inp["k_new"], step_inp["v_new"], k, v, ids, b, 1.0 / np.sqrt(D), 1e6,
                           streams=streams)
    assert_close(out, r["out"], streams, what="full-size appending step")
    got = kg[b:b + P].double().cpu().numpy()
    diff = np.abs(got - r["k_rot"])
    assert (diff <= _rot_bound(r["k_rot"], step_inp["k_new"].double().numpy())).all()
    assert (diff == 0).mean() > 0.99, (diff == 0).mean()
    assert r["pos"].tolist() == (doc + np.array([np.count_nonzero(ids_full[:b] == s + 1) for s in range(P)])).tolist()


@pytest.mark.parametrize("P", [1, 300])
def test_decode_append_stream_counts(P):
    H, D = 2, 128
    ids, T0, cap, k, v, q, kn, vn = _step_case(70 + P, P, H, D, doc=333, dtype=torch.bfloat16)
    kg, vg, sid = k.to(DEV), v.to(DEV), _i32(ids)
    say(f"  gpu: appending step P={P} T0={T0}")
    plan = pp.pp_step_plan(sid, _i32([T0]), P, max_seq_len=cap)
    out = pp.pp_attn_decode_append(q.to(DEV), kn.to(DEV), vn.to(DEV), kg, vg, sid, plan, rope_base=1e4)
    torch.cuda.synchronize()
    r = oracle_append_step(q, kn, vn, k, v, ids, T0, 1.0 / np.sqrt(D), 1e4)
    assert_close(out, r["out"], what=f"appending step P={P}")


# ----------------------------------------------- grouped key/value heads ---

@pytest.mark.parametrize("Hq,Hkv,D,dtype,rope_base", [(8, 2, 128, torch.bfloat16, 1e4),
                                                     (28, 4, 128, torch.bfloat16, 1e6),
                                                     (7, 1, 64, torch.bfloat16, 1e4),
                                                     (4, 2, 64, torch.float32, 1e4),
                                                     (6, 3, 128, torch.bfloat16, 0.0)])
def test_decode_append_grouped_heads(Hq, Hkv, D, dtype, rope_base):
    P = 19
    ids, T0, cap, k, v, q, kn, vn = _step_case(Hq * 13 + Hkv, P, Hq, D, doc=900, dtype=dtype, Hkv=Hkv)
    kg, vg, sid = k.to(DEV), v.to(DEV), _i32(ids)
    say(f"  gpu: pp_attn_decode_append grouped Hq={Hq} Hkv={Hkv} {dtype} D={D} base={rope_base} T0={T0} P={P}")
    plan = pp.pp_step_plan(sid, _i32([T0]), P, max_seq_len=cap)
    out = pp.pp_attn_decode_append(q.to(DEV), kn.to(DEV), vn.to(DEV), kg, vg, sid, plan, rope_base=rope_base)
    torch.cuda.synchronize()
    bf = dtype == torch.bfloat16
    r = oracle_append_step(q, kn, vn, k, v, ids, T0, 1.0 / np.sqrt(D), rope_base, store_bf16=bf)
    assert_close(out, r["out"], what=f"grouped {Hq}/{Hkv} {dtype} D={D} base={rope_base}")
    kw, vw = kg.double().cpu().numpy(), vg.double().cpu().numpy()
    np.testing.assert_array_equal(kw[:T0], k[:T0].double().numpy())
    np.testing.assert_array_equal(kw[T0 + P:], k[T0 + P:].double().numpy())
    np.testing.assert_array_equal(vw[T0:T0 + P], vn.double().numpy())
    got, want = kw[T0:T0 + P], r["k_rot"]
    if rope_base <= 0:
        np.testing.assert_array_equal(got, kn.double().numpy())
    elif bf:
        diff = np.abs(got - want)
        assert (diff <= _rot_bound(want, kn.double().numpy())).all(), diff.max()
        assert (diff == 0).mean() > 0.99
    else:
        np.testing.assert_allclose(got, want, rtol=2e-6, atol=2e-6)


def test_full_size_grouped_appending_step_sampled():
    # the 12000-token document with 256 streams at its last answer step, 28
    # query heads sharing 4 key/value heads (the grouped decode loop's shape)
    doc, P, steps, H, Hkv, D, seed = 12000, 256, 32, 28, 4, 128, 1011
    ids_full, _, base0 = decode_loop_layout(doc, P, steps, seed)
    cap = len(ids_full)
    t = steps - 1
    b = base0 + t * P
    k = torch.empty(cap, Hkv, D, dtype=torch.bfloat16)
    v = torch.empty_like(k)
    inp0 = decode_loop_step_inputs(H, D, P, cap, 3, 0, seed, base_len=base0, Hkv=Hkv)
    k[:base0], v[:base0] = inp0["k0"], inp0["v0"]
    for u in range(t):  # earlier answers, as already-rotated cache rows
        inp = decode_loop_step_inputs(H, D, P, cap, 3, u, seed, base_len=base0, Hkv=Hkv)
        k[base0 + u * P: base0 + (u + 1) * P] = inp["k_new"]
        v[base0 + u * P: base0 + (u + 1) * P] = inp["v_new"]
    ids = ids_full.copy()
    ids[b:] = 0
    step_inp = decode_loop_step_inputs(H, D, P, cap, 3, t, seed, Hkv=Hkv)
    sid = _i32(ids)
    kg, vg = k.to(DEV), v.to(DEV)
    say(f"  gpu: full-size grouped appending step T={b + P} P={P} Hq={H} Hkv={Hkv}")
    plan = pp.pp_step_plan(sid, _i32([b]), P, max_seq_len=cap)
    out = pp.pp_attn_decode_append(step_inp["q"].to(DEV), step_inp["k_new"].to(DEV), step_inp["v_new"].to(DEV), kg,
                                   vg, sid, plan, rope_base=1e6)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    streams = sorted({0, P - 1} | set(rng.choice(P, 6, replace=False).tolist()))
    r = oracle_append_step(step_inp["q"], step_inp["k_new"], step_inp["v_new"], k, v, ids, b, 1.0 / np.sqrt(D), 1e6,
                           streams=streams)
    assert_close(out, r["out"], streams, what="full-size grouped appending step")
    got = kg[b:b + P].double().cpu().numpy()
    diff = np.abs(got - r["k_rot"])
    assert (diff <= _rot_bound(r["k_rot"], step_inp["k_new"].double().numpy())).all()
    np.testing.assert_array_equal(vg[b:b + P].view(torch.int16).cpu().numpy(),
                                  step_inp["v_new"].view(torch.int16).numpy())


def test_graph_of_the_grouped_step_replays_every_step():
    # 28 query heads sharing 4 key/value heads: one capture of (plan + 2
    # layers + advance), replayed 12 times, against the oracle's own loop
    args = dict(doc=700, P=24, steps=12, layers=[0, 1], H=28, Hkv=4, D=128, seed=97, rope_base=1e6)
    g = _loop(**args, check_oracle=True, use_graph=True)
    e = _loop(**args, check_oracle=False, use_graph=False)
    for t in range(len(g)):
        for i in range(len(g[t])):
            assert torch.equal(g[t][i].view(torch.int16), e[t][i].view(torch.int16)), (t, i)
