"""GPU checks of the decode path's guards and of what it must never read:
positions outside [0, max_pos] are dropped on the device and counted in the
workspace's status word; a workspace filled with NaN before a call changes
nothing; the hyper-network gate folded into the latent map at the LLM-scale
dimensions against the pages' form Linear(c) = W_hc c + b_hc."""
import numpy as np
import pytest
import torch

import oracle.mtla as om
import synth
from synth import Dims
from gpu_util import TOL, dev, host, layer, needs_gpu, relerr, say

pytestmark = pytest.mark.gpu


def _guard_case(dims, pos, max_pos, ms, seed):
    """Decode step where some positions break the max_pos contract while
    their slot still lies inside the allocated cache (so even an unguarded
    kernel would stay in bounds).  Valid sequences match the oracle; dropped
    ones leave every cache row bit-identical (NaN poison included), get a
    zero output row, and are counted."""
    pos = np.asarray(pos, dtype=np.int32)
    B = len(pos)
    assert (ms - 1) * dims.s >= pos.max()          # every slot index inside the cache
    w, W, L = layer(dims, seed, "bf16", pe_rows=ms)
    state = synth.make_decode_state(dims, np.maximum(pos, 0), ms, seed=seed + 1)
    step = synth.make_step(dims, w, np.maximum(pos, 0), seed=seed + 2)
    cache = dev(np.concatenate([state["lat"], state["rope"]], axis=-1), "bf16")
    before = host(cache)
    Y = L.decode_step(cache, dev(step["x"], "bf16"), dev(step["QR"], "bf16"),
                      dev(step["KR"], "bf16"), torch.from_numpy(pos).cuda(), max_pos)
    torch.cuda.synchronize()
    Yg, after = host(Y), host(cache)
    dropped = [b for b in range(B) if pos[b] < 0 or pos[b] > max_pos]
    assert L.dropped_frames() == len(dropped)
    for b in range(B):
        if b in dropped:
            assert np.array_equal(after[b], before[b], equal_nan=True), b
            assert np.all(Yg[b] == 0.0), b
            continue
        lat, rk = state["lat"][b].copy(), state["rope"][b].copy()
        y, _ = om.decode_step(lat, rk, int(pos[b]), step["x"][b], step["QR"][b], step["KR"][b], W,
                              dims.s, dims.scale)
        j = pos[b] // dims.s
        other = np.ones(ms, bool)
        other[j] = False
        assert np.array_equal(after[b][other], before[b][other], equal_nan=True), b
        e = relerr(Yg[b], y)
        assert e < TOL["bf16"], (b, e)
    return L


def test_decode_position_guard_balanced_work_list():
    needs_gpu()
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=2)
    say("decode guard, balanced work list")
    L = _guard_case(dims, [10, 301, 799, -1, 0, 300, -7, 1500], max_pos=300, ms=760, seed=9100)
    # the next call on the same workspace counts afresh
    dims1 = dims
    w, W, L2 = layer(dims1, 9101, "bf16", pe_rows=40)
    pos = np.array([3, 5], dtype=np.int32)
    state = synth.make_decode_state(dims1, pos, 40, seed=9102)
    step = synth.make_step(dims1, w, pos, seed=9103)
    cache = dev(np.concatenate([state["lat"], state["rope"]], axis=-1), "bf16")
    L2.decode_step(cache, dev(step["x"], "bf16"), dev(step["QR"], "bf16"), dev(step["KR"], "bf16"),
                   torch.from_numpy(pos).cuda(), 5)
    assert L2.dropped_frames() == 0


def test_decode_position_guard_uniform_splits():
    """More than 256 sequences: splits sized from max_pos on the host."""
    needs_gpu()
    dims = Dims(d=256, H=8, d_h=64, r=256, d_hR=32, s=3)
    rng = np.random.default_rng(9200)
    pos = rng.integers(0, 400, size=272).astype(np.int32)
    pos[[5, 77, 271]] = [401, -2, 1000]
    say("decode guard, uniform splits, B=272")
    _guard_case(dims, pos, max_pos=400, ms=400, seed=9200)


def test_merge_append_position_guard():
    needs_gpu()
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=2)
    pos = np.array([4, 201, -1, 200, 7], dtype=np.int32)
    max_pos, ms = 200, 150
    w, W, L = layer(dims, 9300, "bf16", pe_rows=ms)
    state = synth.make_decode_state(dims, np.maximum(pos, 0), ms, seed=9301)
    step = synth.make_step(dims, w, np.maximum(pos, 0), seed=9302)
    cache = dev(np.concatenate([state["lat"], state["rope"]], axis=-1), "bf16")
    before = host(cache)
    L.merge_append(cache, dev(step["x"], "bf16"), dev(step["KR"], "bf16"),
                   torch.from_numpy(pos).cuda(), max_pos)
    torch.cuda.synchronize()
    after = host(cache)
    from kv_cache_compressed_amd import OP_MERGE
    assert L.dropped_frames(OP_MERGE) == 2
    for b in range(len(pos)):
        if pos[b] < 0 or pos[b] > max_pos:
            assert np.array_equal(after[b], before[b], equal_nan=True), b
            continue
        lat, rk = state["lat"][b].copy(), state["rope"][b].copy()
        j = om.merge_append(lat, rk, int(pos[b]), step["x"][b], step["KR"][b], W, dims.s)
        assert relerr(after[b, j, :dims.r], lat[j]) < TOL["bf16"]


def test_decode_poisoned_workspace():
    """Filling the decode workspace with NaN bytes before a step changes no
    bit of the result or the cache: nothing stale is read."""
    needs_gpu()
    for cfg, B in ((2, 32), (3, 64)):
        name, dims, ex = synth.config(cfg)
        rng = np.random.default_rng(9400 + cfg)
        if "ctx" in ex:
            pos = np.full(B, ex["ctx"] - 1, dtype=np.int32)
        else:
            pos = (rng.integers(ex["ctx_lo"], ex["ctx_hi"] + 1, size=B) - 1).astype(np.int32)
        ms = int(pos.max()) // dims.s + 2
        w, W, L = layer(dims, 9400 + cfg, "bf16", pe_rows=ms)
        state = synth.make_decode_state(dims, pos, ms, seed=9410 + cfg)
        step = synth.make_step(dims, w, pos, seed=9420 + cfg)
        args = (dev(step["x"], "bf16"), dev(step["QR"], "bf16"), dev(step["KR"], "bf16"),
                torch.from_numpy(pos).cuda(), int(pos.max()))
        outs = []
        for fill in (0x00, 0xFF):
            cache = dev(np.concatenate([state["lat"], state["rope"]], axis=-1), "bf16")
            from kv_cache_compressed_amd import OP_DECODE
            L.workspace(OP_DECODE, B, int(pos.max())).fill_(fill)
            Y = L.decode_step(cache, *args)
            outs.append((Y.clone(), cache.clone()))
        torch.cuda.synchronize()
        say("poisoned decode workspace", name)
        assert torch.isfinite(outs[1][0].float()).all()
        assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
        assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))


def test_prefill_poisoned_workspace():
    needs_gpu()
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=2)
    B, T = 3, 333
    w, W, L = layer(dims, 9500, "bf16", pe_rows=om.n_slots(T, dims.s))
    seq = synth.make_sequence(dims, w, B, T, 9501, "bf16")
    X, QR, KR = dev(seq["X"], "bf16"), dev(seq["QR"], "bf16"), dev(seq["KR"], "bf16")
    from kv_cache_compressed_amd import OP_PREFILL
    outs = []
    for fill in (0x00, 0xFF):
        L.workspace(OP_PREFILL, B, T).fill_(fill)
        outs.append(L.prefill(X, QR, KR).clone())
    torch.cuda.synchronize()
    say("poisoned prefill workspace")
    assert torch.isfinite(outs[1].float()).all()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_gate_fold_at_llm_dims():
    """The library takes the content branch folded into the latent map
    (W_gate = W_hc W_dkv, one bf16 rounding of each entry).  At the LLM-scale
    dimensions (d = 4096, r = 512), the merged slot of one step -- opened
    afresh (t mod s == 0) or accumulated -- against the oracle's pages' form
    sigmoid((W_hc c + b_hc) * P_j) * c: within the path's bf16 bound 2e-2
    (norm-wise).  Against the oracle fed the library's own rounded W_gate the
    difference is the slot's own bf16 rounding (bound 4e-3)."""
    needs_gpu()
    _, dims, _ = synth.config(5)
    pos = np.array([0, 2, 7, 9, 12, 13], dtype=np.int32)
    ms = 8
    w, W, L = layer(dims, 9600, "bf16", pe_rows=ms)
    state = synth.make_decode_state(dims, pos, ms, seed=9601)
    step = synth.make_step(dims, w, pos, seed=9602)
    cache = dev(np.concatenate([state["lat"], state["rope"]], axis=-1), "bf16")
    L.merge_append(cache, dev(step["x"], "bf16"), dev(step["KR"], "bf16"),
                   torch.from_numpy(pos).cuda(), int(pos.max()))
    torch.cuda.synchronize()
    after = host(cache)
    Wg = host(L.W_gate)                       # the folded map as the library holds it
    for b, t in enumerate(pos):
        j = t // dims.s
        lat = state["lat"][b].copy()
        om.merge_append(lat, state["rope"][b].copy(), int(t), step["x"][b], step["KR"][b], W,
                        dims.s)
        e_pages = relerr(after[b, j, :dims.r], lat[j])
        # the same step with the folded map: gate pre-activation W_gate x + b_hc
        x = step["x"][b]
        c = W["W_dkv"] @ x
        g = (Wg @ x + W["b_hc"]) * W["P"][j]
        u = om.sigmoid(g) * c
        ref = u if t % dims.s == 0 else state["lat"][b][j] + u
        e_fold = relerr(after[b, j, :dims.r], ref)
        say(f"  t={t} vs pages' form {e_pages:.3g}, vs folded map {e_fold:.3g}")
        assert e_pages < TOL["bf16"]
        assert e_fold < 4e-3
