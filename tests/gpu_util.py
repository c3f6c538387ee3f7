"""Helpers shared by the GPU parity tests: upload seeded inputs, compare with
the oracle.  Tolerances (norm-wise relative error max|g-o| / max|o|): 1e-4 on
fp32 paths, 2e-2 on bf16 paths with fp32 accumulation; slot indices and
untouched cache rows bit-exact."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle.mtla as om
import synth

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def needs_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")


def relerr(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def tdtype(storage):
    return torch.bfloat16 if storage == "bf16" else torch.float32


def code(storage):
    from kv_cache_compressed_amd import MTLA_BF16, MTLA_F32
    return MTLA_BF16 if storage == "bf16" else MTLA_F32


def dev(x, storage):
    return torch.from_numpy(np.ascontiguousarray(x)).to(tdtype(storage)).cuda().contiguous()


def host(t):
    return t.detach().to(torch.float64).cpu().numpy()


def layer(dims, seed, storage, pe_rows):
    """(weights dict, oracle weights with P table, GPU layer) for one layer."""
    from kv_cache_compressed_amd import MTLALayer
    w = synth.make_weights(dims, seed, storage, pe_rows=pe_rows)
    W = om.with_position_table(w, pe_rows)
    L = MTLALayer.from_arrays(dims, w, code(storage))
    return w, W, L
