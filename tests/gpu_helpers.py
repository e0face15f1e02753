"""Shared helpers of the GPU tests: run a case through the HIP library and
compare with the fp64 oracle at the agreed tolerance."""
import numpy as np
import torch

import shared_prefix_stream_amd as pp
from oracle import oracle_decode

ATOL = 2e-2      # max |gpu - oracle| over all elements
ROW_RTOL = 1e-2  # per (stream, head) row: max |gpu - oracle| / max |oracle|

ENTRY_POINTS = {"decode": pp.pp_attn_decode, "batched": pp.pp_attn_decode_batched}


def say(msg):
    print(msg, flush=True)


def to_gpu(case, dev="cuda:0"):
    return [t.to(dev) for t in (case.q, case.k, case.v, case.stream_id)]


def run(case, entry="decode", gpu_args=None, stream=None):
    args = gpu_args if gpu_args is not None else to_gpu(case)
    say(f"  gpu: {entry} {case.name} P={case.P} H={case.H} D={case.D} T={case.seq_len} doc={case.doc_len}")
    out = ENTRY_POINTS[entry](*args, seq_len=case.seq_len, scale=case.scale)
    torch.cuda.synchronize()
    return out


def reference(case, streams=None):
    return oracle_decode(case.q, case.k, case.v, case.stream_id.numpy(), case.seq_len, case.scale, streams=streams)


def assert_close(got, ref, streams=None, what=""):
    g = got.double().cpu().numpy() if isinstance(got, torch.Tensor) else got
    # every element the call wrote must be finite, also in rows not compared
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    if streams is not None:
        g, ref = g[streams], ref[streams]
    err = np.abs(g - ref)
    rowmax = np.abs(ref).max(axis=-1)
    rel = err.max(axis=-1) / np.maximum(rowmax, 1e-6)
    assert err.max() <= ATOL, f"{what}: max |err| {err.max():.3e} > {ATOL}"
    assert rel.max() <= ROW_RTOL, f"{what}: max row-relative err {rel.max():.3e} > {ROW_RTOL}"
    return float(err.max()), float(rel.max())
