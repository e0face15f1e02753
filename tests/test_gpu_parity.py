"""GPU parity of both entry points against the fp64 oracle, through the C ABI.

Tolerance: max |gpu - oracle| <= 2e-2 over all elements and, per (stream,
head) row, max |gpu - oracle| / max |oracle| <= 1e-2 (bf16 inputs, fp32
accumulation).  Small shapes are checked on every stream; the full-size
headline workload (doc 16k, P = 256) on every stream as well."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import assert_close, reference, run, say, to_gpu
from workloads import make_case, named_workload, permute_tail, ragged_case

pytestmark = pytest.mark.gpu


def _rng_case(seed, P, H, D, doc, qmax=20, amax=10, dtype=torch.bfloat16, **kw):
    rng = np.random.default_rng(seed)
    return make_case(H, D, doc, rng.integers(1, qmax + 1, P).tolist(), rng.integers(0, amax + 1, P).tolist(),
                     dtype=dtype, seed=seed, name=f"rand_p{P}_h{H}_d{D}_doc{doc}", **kw)


@pytest.mark.parametrize("entry", ["decode", "batched"])
def test_tiny_f32_workload(entry):
    case = named_workload("tiny_f32_h4_d64_doc256_p4", seed=1000)
    assert_close(run(case, entry), reference(case), what=case.name)


SMALL = [
    # (P, H, D, doc): query tiles of 16/64/128/256 per workgroup, several
    # document tiles with a ragged last one, P past one 256-query tile
    (1, 4, 128, 1000), (5, 4, 128, 777), (17, 2, 128, 1500), (64, 3, 128, 640),
    (100, 2, 128, 1025), (130, 2, 128, 300), (256, 2, 128, 2049), (300, 1, 128, 513),
    (7, 4, 64, 999), (70, 2, 64, 1100), (200, 2, 64, 700),
]


@pytest.mark.parametrize("entry", ["decode", "batched"])
@pytest.mark.parametrize("P,H,D,doc", SMALL)
def test_small_bf16_all_streams(entry, P, H, D, doc):
    case = _rng_case(10 + P + doc, P, H, D, doc)
    assert_close(run(case, entry), reference(case), what=case.name)


@pytest.mark.parametrize("entry", ["decode", "batched"])
@pytest.mark.parametrize("P,H,D,doc", [(9, 4, 64, 300), (40, 2, 128, 700)])
def test_small_f32_all_streams(entry, P, H, D, doc):
    case = _rng_case(20 + P, P, H, D, doc, dtype=torch.float32)
    assert_close(run(case, entry), reference(case), what=case.name)


@pytest.mark.parametrize("entry", ["decode", "batched"])
def test_doc8k_p64_all_streams(entry):
    case = named_workload("codellama7b_doc8k_p64", seed=1001)
    assert_close(run(case, entry), reference(case), what=case.name)


@pytest.mark.parametrize("entry", ["decode", "batched"])
def test_doc16k_p256_all_streams(entry):
    case = named_workload("codellama7b_doc16k_p256", seed=1002)
    assert_close(run(case, entry), reference(case), what=case.name)
