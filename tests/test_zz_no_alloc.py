"""The decode step with the library's fixed scratch array as its workspace
(pp_attn_decode_noalloc), through the C ABI: the same kernels as
pp_attn_decode, so the same bits; two calls in a row, the second smaller
(the array keeps the first call's contents); a shape too large for the
array is rejected."""
import ctypes

import numpy as np
import pytest
import torch

import shared_prefix_stream_amd as pp
from tests.gpu_helpers import assert_close, reference, say
from workloads import make_case, named_workload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _call_noalloc(case, out):
    """pp_attn_decode_noalloc through the raw C ABI (no Python-side workspace)."""
    q, k, v, sid = (t.to(DEV) for t in (case.q, case.k, case.v, case.stream_id))
    code = pp.PP_BF16 if case.q.dtype == torch.bfloat16 else pp.PP_F32
    stream = torch.cuda.current_stream().cuda_stream
    st = pp.raw().pp_attn_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), sid.data_ptr(), case.seq_len,
                                         case.P, case.H, case.D, case.scale, out.data_ptr(), code, stream)
    return st, (q, k, v, sid)


def test_noalloc_equals_decode_on_two_calls_in_a_row():
    big = named_workload("codellama7b_doc8k_p64", seed=1001)
    rng = np.random.default_rng(3)
    small = make_case(4, 128, 700, rng.integers(1, 20, 7).tolist(), rng.integers(0, 9, 7).tolist(),
                      dtype=torch.bfloat16, seed=3, name="small_p7_h4")
    for case in (big, small):
        say(f"  gpu: pp_attn_decode_noalloc {case.name} T={case.seq_len} P={case.P} H={case.H}")
        out = torch.full_like(case.q, float("nan"), device=DEV)
        st, (q, k, v, sid) = _call_noalloc(case, out)
        assert st == pp.PP_OK, pp.raw().pp_last_error_message()
        ref = pp.pp_attn_decode(q, k, v, sid, seq_len=case.seq_len, scale=case.scale)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), case.name
        if case is small:
            assert_close(out, reference(case), what=case.name)


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    lib = pp.raw()
    T, P, H, d = 40000, 1024, 64, 128
    assert lib.pp_attn_workspace_bytes(T, P, H, d, pp.PP_BF16) > pp.PP_NOALLOC_SCRATCH_BYTES
    fake = 0x10000000  # never dereferenced: the size check comes first
    st = lib.pp_attn_decode_noalloc(fake, fake * 2, fake * 3, fake * 4, T, P, H, d, 0.088, fake * 5, pp.PP_BF16,
                                    None)
    assert st == pp.PP_ERR_WORKSPACE
    assert b"fixed scratch" in lib.pp_last_error_message()
