"""GPU parity of the appending step over several request slots
(pp_step_plan_multi + pp_attn_decode_append_multi) against the step oracle,
request by request: idle slots, retired streams, grouped heads, and a
continuous-batching loop in which finished slots take new requests."""
import numpy as np
import pytest
import torch

import shared_prefix_stream_amd as pp
from oracle import oracle_append_step
from shared_prefix_stream_amd.batching import continuous_schedule
from tests.gpu_helpers import assert_close, say
from workloads import canonical_layout

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _i32(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32)).to(DEV)


def _request(seed, doc, P, Hkv, D, dtype):
    """A request's ids and caches before its first answer step."""
    rng = np.random.default_rng(seed)
    ids, _ = canonical_layout(doc, rng.integers(1, 20, P).tolist(), rng.integers(0, 4, P).tolist())
    g = torch.Generator().manual_seed(seed)
    k0 = torch.randn(len(ids), Hkv, D, generator=g).to(dtype)
    v0 = torch.randn(len(ids), Hkv, D, generator=g).to(dtype)
    return ids, k0, v0


def _step_inputs(seed, t, P, Hq, Hkv, D, dtype):
    g = torch.Generator().manual_seed(seed * 1000 + t)
    return (torch.randn(P, Hq, D, generator=g).to(dtype), torch.randn(P, Hkv, D, generator=g).to(dtype),
            torch.randn(P, Hkv, D, generator=g).to(dtype))


@pytest.mark.parametrize("Hq,Hkv,D,dtype", [(8, 2, 128, torch.bfloat16), (4, 2, 64, torch.float32),
                                          (4, 4, 128, torch.bfloat16)])
def test_multi_append_matches_the_oracle(Hq, Hkv, D, dtype):
    # three slots: two busy requests with different documents, one idle slot
    # (base_len -1); stream 2 of the last request is retired
    B, P, T = 3, 11, 2400
    docs = [700, None, 1500]
    reqs = [None if doc is None else _request(40 + b, doc, P, Hkv, D, dtype) for b, doc in enumerate(docs)]
    ids = np.zeros((B, T), dtype=np.int32)
    k = torch.zeros(B, T, Hkv, D, dtype=dtype)
    v = torch.zeros_like(k)
    base = []
    for b, r in enumerate(reqs):
        if r is None:
            base.append(-1)
            ids[b] = 7  # an idle slot's rows are left as they are
            continue
        n = len(r[0])
        ids[b, :n], k[b, :n], v[b, :n] = r
        base.append(n)
    active = np.ones((B, P), dtype=np.int32)
    active[2, 2] = 0
    q, kn, vn = (torch.stack(x) for x in zip(*[_step_inputs(b + 1, 0, P, Hq, Hkv, D, dtype) for b in range(B)]))
    sid, kg, vg = _i32(ids), k.to(DEV), v.to(DEV)
    say(f"  gpu: multi append B={B} P={P} Hq={Hq} Hkv={Hkv} D={D} {dtype} base={base}")
    plan = pp.pp_step_plan_multi(sid, _i32(base), P, active=_i32(active))
    out = pp.pp_attn_decode_append_multi(q.to(DEV), kn.to(DEV), vn.to(DEV), kg, vg, sid, plan, active=_i32(active),
                                         rope_base=1e4)
    torch.cuda.synchronize()
    head = plan[0].cpu().numpy()
    bf = dtype == torch.bfloat16
    for b, r in enumerate(reqs):
        if r is None:
            assert head[b] == 0 and head[B + b] == 0
            assert torch.count_nonzero(out[b]).item() == 0
            np.testing.assert_array_equal(sid[b].cpu().numpy(), ids[b])
            assert torch.count_nonzero(kg[b]).item() == 0
            continue
        n = base[b]
        streams = [s for s in range(P) if active[b, s]]
        ref = oracle_append_step(q[b], kn[b], vn[b], k[b], v[b], ids[b], n, 1.0 / np.sqrt(D), 1e4, store_bf16=bf,
                                 streams=streams)
        assert head[B + b] == n + P
        assert_close(out[b], ref["out"], streams, what=f"request {b}")
        for s in range(P):
            if not active[b, s]:
                assert torch.count_nonzero(out[b, s]).item() == 0
        np.testing.assert_array_equal(sid[b, :n + P].cpu().numpy(), ref["stream_id"][:n + P])
        # a retired stream's new slot keeps its old key and value (zeros here)
        live = active[b].astype(bool)
        assert torch.count_nonzero(kg[b, n:n + P][~torch.from_numpy(live)]).item() == 0
        assert torch.count_nonzero(vg[b, n:n + P][~torch.from_numpy(live)]).item() == 0
        np.testing.assert_array_equal(vg[b, n:n + P].cpu().double().numpy()[live], vn[b].double().numpy()[live])
        kw = kg[b, n:n + P].cpu().double().numpy()[live]
        if bf:
            assert (kw == ref["k_rot"][live]).mean() > 0.99
        else:
            np.testing.assert_allclose(kw, ref["k_rot"][live], rtol=2e-6, atol=2e-6)


def test_one_request_equals_the_single_request_step():
    P, Hq, Hkv, D, dtype = 17, 8, 2, 128, torch.bfloat16
    ids, k0, v0 = _request(5, 1300, P, Hkv, D, dtype)
    n = len(ids)
    T = n + P + 3
    outs = []
    for multi in (False, True):
        sid = torch.zeros(T, dtype=torch.int32, device=DEV)
        sid[:n] = _i32(ids)
        k = torch.zeros(T, Hkv, D, dtype=dtype, device=DEV)
        v = torch.zeros_like(k)
        k[:n], v[:n] = k0.to(DEV), v0.to(DEV)
        q, kn, vn = (x.to(DEV) for x in _step_inputs(5, 0, P, Hq, Hkv, D, dtype))
        if multi:
            plan = pp.pp_step_plan_multi(sid.view(1, T), _i32([n]), P)
            o = pp.pp_attn_decode_append_multi(q[None], kn[None], vn[None], k[None], v[None], sid.view(1, T), plan)[0]
        else:
            plan = pp.pp_step_plan(sid, _i32([n]), P)
            o = pp.pp_attn_decode_append(q, kn, vn, k, v, sid, plan)
        outs.append((o, k, v, sid))
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_continuous_batching_loop_of_appending_steps():
    # 5 requests through 2 slots, answers of 2-5 tokens: every step plans all
    # slots at once, idle slots carry base_len -1, and each busy slot's output
    # is checked against the oracle's own loop for its request
    B, P, Hq, Hkv, D, dtype = 2, 6, 4, 2, 64, torch.bfloat16
    ans = [3, 2, 5, 2, 4]
    docs = [300, 520, 130, 410, 260]
    T = 900
    reqs = [_request(70 + r, docs[r], P, Hkv, D, dtype) for r in range(len(ans))]
    sid = torch.zeros(B, T, dtype=torch.int32, device=DEV)
    K = torch.zeros(B, T, Hkv, D, dtype=dtype, device=DEV)
    V = torch.zeros_like(K)
    state = {}  # request -> (ids, K, V) of the oracle's own loop
    owner = [None] * B
    for step in continuous_schedule(ans, B):
        base = []
        for b, x in enumerate(step):
            if x is None:
                base.append(-1)
                continue
            r, t = x
            ids0, k0, v0 = reqs[r]
            n0 = len(ids0)
            if owner[b] != r:  # the slot takes a new request: its prefilled rows
                owner[b] = r
                sid[b].zero_()
                sid[b, :n0] = _i32(ids0)
                K[b, :n0], V[b, :n0] = k0.to(DEV), v0.to(DEV)
                ids = np.zeros(T, dtype=np.int32)
                ids[:n0] = ids0
                ko = np.zeros((T, Hkv, D))
                vo = np.zeros((T, Hkv, D))
                ko[:n0], vo[:n0] = k0.double().numpy(), v0.double().numpy()
                state[r] = (ids, ko, vo)
            base.append(n0 + t * P)
        inp = [_step_inputs(100 + (x[0] if x else 0), x[1] if x else 0, P, Hq, Hkv, D, dtype) for x in step]
        q, kn, vn = (torch.stack(c).to(DEV) for c in zip(*inp))
        plan = pp.pp_step_plan_multi(sid, _i32(base), P)
        out = pp.pp_attn_decode_append_multi(q, kn, vn, K, V, sid, plan, rope_base=1e4)
        torch.cuda.synchronize()
        for b, x in enumerate(step):
            if x is None:
                assert torch.count_nonzero(out[b]).item() == 0
                continue
            r, t = x
            ids, ko, vo = state[r]
            n = base[b]
            ref = oracle_append_step(inp[b][0], inp[b][1], inp[b][2], ko, vo, ids, n, 1.0 / np.sqrt(D), 1e4)
            assert_close(out[b], ref["out"], what=f"request {r} step {t} slot {b}")
            ko[n:n + P], vo[n:n + P] = ref["k_cache"][n:n + P], ref["v_cache"][n:n + P]
            ids[n:n + P] = np.arange(1, P + 1)
    say(f"  checked {len(continuous_schedule(ans, B))} steps of {len(ans)} requests in {B} slots")


def test_multi_append_lists_past_the_plan_capacity():
    # a plan capacity of 4 slots: the streams whose lists overflow are
    # compacted by the gather kernel itself, up to their request's step length
    B, P, Hq, Hkv, D, dtype, T = 2, 9, 8, 2, 128, torch.bfloat16, 1600
    reqs = [_request(90 + b, doc, P, Hkv, D, dtype) for b, doc in enumerate([400, 1100])]
    ids = np.zeros((B, T), dtype=np.int32)
    k = torch.zeros(B, T, Hkv, D, dtype=dtype)
    v = torch.zeros_like(k)
    base = []
    for b, (i0, k0, v0) in enumerate(reqs):
        ids[b, :len(i0)], k[b, :len(i0)], v[b, :len(i0)] = i0, k0, v0
        base.append(len(i0))
    q, kn, vn = (torch.stack(x) for x in zip(*[_step_inputs(b + 7, 0, P, Hq, Hkv, D, dtype) for b in range(B)]))
    sid, kg, vg = _i32(ids), k.to(DEV), v.to(DEV)
    say(f"  gpu: multi append, capacity 4, base={base}")
    plan = pp.pp_step_plan_multi(sid, _i32(base), P, tail_capacity=4)
    out = pp.pp_attn_decode_append_multi(q.to(DEV), kn.to(DEV), vn.to(DEV), kg, vg, sid, plan, rope_base=1e4)
    torch.cuda.synchronize()
    counts = plan[1].cpu().numpy()
    assert (counts > 4).sum() >= P, counts  # most lists overflow (short questions may not)
    for b in range(B):
        ref = oracle_append_step(q[b], kn[b], vn[b], k[b], v[b], ids[b], base[b], 1.0 / np.sqrt(D), 1e4)
        assert_close(out[b], ref["out"], what=f"request {b}, lists past the capacity")


def test_graph_of_the_multi_step_replays_every_step():
    # one capture of (plan of all slots + 2 layers + advance of the busy
    # slots), replayed 5 times; slot 1 idles throughout (base -1)
    B, P, Hq, Hkv, D, dtype, T, L, steps = 3, 6, 4, 2, 64, torch.bfloat16, 1400, 2, 5
    reqs = {0: _request(11, 500, P, Hkv, D, dtype), 2: _request(12, 800, P, Hkv, D, dtype)}

    def setup():
        sid = torch.zeros(B, T, dtype=torch.int32, device=DEV)
        K = torch.zeros(L, B, T, Hkv, D, dtype=dtype, device=DEV)
        V = torch.zeros_like(K)
        base = torch.full((B,), -1, dtype=torch.int32, device=DEV)
        for b, (i0, k0, v0) in reqs.items():
            n = len(i0)
            sid[b, :n] = _i32(i0)
            K[:, b, :n], V[:, b, :n] = k0.to(DEV), v0.to(DEV)
            base[b] = n
        return sid, K, V, base

    busy = _i32([1, 0, 1]) * P
    g = torch.Generator().manual_seed(3)
    qs = torch.randn(L, B, P, Hq, D, generator=g).to(dtype).to(DEV)
    kvn = torch.randn(L, 2, B, P, Hkv, D, generator=g).to(dtype).to(DEV)
    ws = torch.empty(pp.multi_workspace_bytes(T, B, P, Hq, Hkv, D, dtype), dtype=torch.uint8, device=DEV)
    plan = (torch.zeros(2 * B, dtype=torch.int32, device=DEV), torch.zeros(B, P, dtype=torch.int32, device=DEV),
            torch.zeros(B, P, 64, dtype=torch.int32, device=DEV))
    outs = torch.empty(L, B, P, Hq, D, dtype=dtype, device=DEV)
    results = {}
    for use_graph in (False, True):
        sid, K, V, base = setup()
        base0 = base.clone()

        def step():
            pp.pp_step_plan_multi(sid, base, P, plan=plan)
            for i in range(L):
                pp.pp_attn_decode_append_multi(qs[i], kvn[i, 0], kvn[i, 1], K[i], V[i], sid, plan, rope_base=1e6,
                                               out=outs[i], workspace=ws)
            base.add_(busy)

        graph = None
        if use_graph:
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            say("  gpu: capture of the multi-request step")
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
            base.copy_(base0)  # capture does not run the work; the captured buffers start again
        res = []
        for t in range(steps):
            if graph is not None:
                graph.replay()
            else:
                step()
            torch.cuda.synchronize()
            res.append(outs.clone())
        results[use_graph] = res
        if graph is not None:
            assert base.cpu().tolist() == [reqs[0][0].size + steps * P, -1, reqs[2][0].size + steps * P]
    for t in range(steps):
        assert torch.equal(results[True][t].view(torch.int16), results[False][t].view(torch.int16)), t
        assert torch.count_nonzero(results[True][t][:, 1]).item() == 0
