"""GPU parity of mtla_merge_append and mtla_gate_pos_table against the oracle."""
import numpy as np
import pytest
import torch

import oracle.mtla as om
import synth
from synth import Dims
from gpu_util import TOL, dev, host, layer, needs_gpu, relerr, say

pytestmark = pytest.mark.gpu


def test_gate_pos_table_matches_oracle():
    needs_gpu()
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=2)
    w, W, L = layer(dims, 11, "bf16", pe_rows=300)
    got = L.gate_pos.cpu().numpy().astype(np.float64)
    e = relerr(got, W["P"])
    say("gate table relerr", e)
    assert e < 1e-4


@pytest.mark.parametrize("storage,s,B", [("f32", 2, 3), ("bf16", 2, 32), ("bf16", 4, 17),
                                         ("bf16", 1, 5), ("bf16", 3, 40)])
def test_merge_append_matches_oracle(storage, s, B):
    needs_gpu()
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=s)
    say("merge_append", storage, s, B)
    rng = np.random.default_rng(5000 + s * 100 + B)
    pos = rng.integers(0, 200, size=B).astype(np.int32)
    pos[0] = 0                      # opens slot 0
    pos[-1] = 199                   # the largest position
    max_slots = 199 // s + 4
    w, W, L = layer(dims, 21 + s, storage, pe_rows=max_slots)
    state = synth.make_decode_state(dims, pos, max_slots, seed=31 + B, storage=storage)
    step = synth.make_step(dims, w, pos, seed=41 + B, storage=storage)
    cache = dev(np.concatenate([state["lat"], state["rope"]], axis=-1), storage)
    before = host(cache)
    L.merge_append(cache, dev(step["x"], storage), dev(step["KR"], storage),
                   torch.from_numpy(pos).cuda(), int(pos.max()))
    torch.cuda.synchronize()
    after = host(cache)
    for b in range(B):
        lat, rk = state["lat"][b].copy(), state["rope"][b].copy()
        j = om.merge_append(lat, rk, int(pos[b]), step["x"][b], step["KR"][b], W, s)
        assert j == pos[b] // s
        # only row j changed, bit for bit elsewhere (NaN poison included)
        other = np.ones(max_slots, bool)
        other[j] = False
        assert np.array_equal(after[b][other], before[b][other], equal_nan=True), b
        assert relerr(after[b, j, :dims.r], lat[j]) < TOL[storage], (b, relerr(after[b, j, :dims.r], lat[j]))
        assert np.array_equal(after[b, j, dims.r:], rk[j])


def test_gate_content_map_matches_product():
    """W_gate = W_hc W_dkv, the content branch folded into the latent map:
    W_gate x = W_hc (W_dkv x) by associativity."""
    needs_gpu()
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=2)
    w, W, L = layer(dims, 12, "bf16", pe_rows=8)
    got = host(L.W_gate)
    ref = w["W_hc"] @ w["W_dkv"]
    e = relerr(got, ref)
    say("gate content map relerr", e)
    assert e < 1e-2      # one bf16 rounding of each entry
