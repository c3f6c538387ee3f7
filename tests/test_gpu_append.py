"""GPU parity of mtla_append_chunk (chunked merge-append) against the oracle,
and the prefill -> chunk -> decode hand-off of a serving sequence."""
import numpy as np
import pytest
import torch

import oracle.mtla as om
import synth
from synth import Dims
from gpu_util import TOL, dev, host, layer, needs_gpu, relerr, say

pytestmark = pytest.mark.gpu


def _check_chunk(dims, storage, B, Lc, pos0, lens, seed, pe_extra=3):
    """One chunk per sequence over a synthetic cache standing at pos0[b];
    compares every touched slot and every written C' row with the oracle and
    requires everything else to be bit-identical (NaN poison included)."""
    s = dims.s
    n = np.full(B, Lc) if lens is None else np.clip(lens, 0, Lc)
    last = pos0 + np.maximum(n, 1) - 1
    max_slots = int(last.max()) // s + pe_extra
    w, W, Lyr = layer(dims, seed, storage, pe_rows=max_slots)
    state = synth.make_decode_state(dims, pos0, max_slots, seed=seed + 1, storage=storage)
    ch = synth.make_chunk(dims, w, pos0, Lc, seed=seed + 2, storage=storage)
    cache = dev(np.concatenate([state["lat"], state["rope"]], axis=-1), storage)
    before = host(cache)
    cprime = dev(np.full((B, Lc, dims.r), np.nan), storage)
    lens_t = torch.from_numpy(lens.astype(np.int32)).cuda() if lens is not None else None
    Lyr.append_chunk(cache, dev(ch["X"], storage), dev(ch["KR"], storage),
                     torch.from_numpy(pos0.astype(np.int32)).cuda(), int(last.max()),
                     lens=lens_t, Cprime=cprime)
    torch.cuda.synchronize()
    after, cp = host(cache), host(cprime)
    worst = 0.0
    for b in range(B):
        t0, nb = int(pos0[b]), int(n[b])
        lat, rk = state["lat"][b].copy(), state["rope"][b].copy()
        ref_cp = om.merge_chunk(lat, rk, t0, ch["X"][b, :nb], ch["KR"][b, :nb], W, s)
        touched = np.zeros(max_slots, bool)
        if nb:
            touched[t0 // s: (t0 + nb - 1) // s + 1] = True
        assert np.array_equal(after[b][~touched], before[b][~touched], equal_nan=True), b
        for j in np.nonzero(touched)[0]:
            e = relerr(after[b, j, :dims.r], lat[j])
            worst = max(worst, e)
            assert e < TOL[storage], (b, j, e)
            assert np.array_equal(after[b, j, dims.r:], rk[j]), (b, j)
        if nb:
            e = relerr(cp[b, :nb], ref_cp)
            worst = max(worst, e)
            assert e < TOL[storage], (b, e)
        assert np.all(np.isnan(cp[b, nb:])), b
    say(f"  worst relerr {worst:.3g}")


@pytest.mark.parametrize("storage,s,B,Lc", [("f32", 2, 3, 7), ("bf16", 2, 8, 33),
                                            ("bf16", 4, 5, 64), ("bf16", 1, 4, 9),
                                            ("bf16", 3, 6, 1), ("f32", 5, 2, 130)])
def test_append_chunk_matches_oracle(storage, s, B, Lc):
    needs_gpu()
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=s)
    say("append_chunk", storage, s, B, Lc)
    rng = np.random.default_rng(7000 + 10 * s + B)
    pos0 = rng.integers(0, 300, size=B)
    pos0[0] = 0                                  # opens slot 0
    if B > 1:
        pos0[1] = s * 37 + (s - 1 if s > 1 else 0)   # enters a group at its last frame
    _check_chunk(dims, storage, B, Lc, pos0, None, seed=7100 + s)


def test_append_chunk_ragged_lengths():
    """Per-sequence lengths: empty, one frame, mid-group ends, full chunk."""
    needs_gpu()
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=3)
    pos0 = np.array([0, 5, 7, 9, 100, 31, 2, 64])
    lens = np.array([0, 1, 2, 40, 17, 40, 3, 39])
    _check_chunk(dims, "bf16", len(pos0), 40, pos0, lens, seed=7300)


def test_append_chunk_wide_latent():
    needs_gpu()
    dims = Dims(d=1024, H=16, d_h=128, r=512, d_hR=64, s=2)
    _check_chunk(dims, "bf16", 4, 21, np.array([3, 0, 50, 11]), None, seed=7400)


def test_append_chunk_serving_shape():
    """32 sequences, chunks of 512 frames at positions spread over 0..2047."""
    needs_gpu()
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=2)
    rng = np.random.default_rng(7500)
    pos0 = rng.integers(0, 2048, size=32)
    _check_chunk(dims, "bf16", 32, 512, pos0, None, seed=7500)


def test_append_chunk_empty_changes_nothing():
    needs_gpu()
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=2)
    w, W, Lyr = layer(dims, 7600, "bf16", pe_rows=8)
    cache = Lyr.new_cache(2, 8, fill=1.5)
    X = torch.empty(2, 0, dims.d, dtype=torch.bfloat16, device="cuda")
    KR = torch.empty(2, 0, dims.d_hR, dtype=torch.bfloat16, device="cuda")
    Lyr.append_chunk(cache, X, KR, torch.zeros(2, dtype=torch.int32, device="cuda"), 0)
    torch.cuda.synchronize()
    assert bool((cache == 1.5).all())


@pytest.mark.parametrize("storage", ["f32", "bf16"])
def test_chunks_rebuild_the_prefill_cache(storage):
    """Chunks with boundaries inside and on groups, from an empty cache, give
    the cache and intermediate states of the parallel form."""
    needs_gpu()
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=4)
    T, B = 97, 2
    ms = om.n_slots(T, dims.s) + 1
    w, W, Lyr = layer(dims, 7700, storage, pe_rows=ms)
    seq = synth.make_sequence(dims, w, B, T, 7701, storage)
    X, KR = dev(seq["X"], storage), dev(seq["KR"], storage)
    cache = Lyr.new_cache(B, ms, fill=float("nan"))
    cuts = [0, 1, 6, 8, 30, 31, 64, 96, T]
    cps = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        cp = torch.full((B, b - a, dims.r), float("nan"), dtype=X.dtype, device="cuda")
        pos0 = torch.full((B,), a, dtype=torch.int32, device="cuda")
        Lyr.append_chunk(cache, X[:, a:b].contiguous(), KR[:, a:b].contiguous(), pos0, b - 1,
                         Cprime=cp)
        cps.append(cp)
    torch.cuda.synchronize()
    got_cp = host(torch.cat(cps, dim=1))
    got = host(cache)
    n = om.n_slots(T, dims.s)
    for b in range(B):
        pf = om.prefill(seq["X"][b], seq["QR"][b], seq["KR"][b], W, dims.s, dims.scale)
        e1 = relerr(got_cp[b], pf["Cp"])
        e2 = relerr(got[b, :n, :dims.r], pf["cache_lat"])
        say(f"  b={b} C' relerr {e1:.3g} cache relerr {e2:.3g}")
        assert e1 < TOL[storage] and e2 < TOL[storage]
        assert np.array_equal(got[b, :n, dims.r:], pf["cache_rope"])
        assert np.all(np.isnan(got[b, n:]))


def test_prefill_chunk_decode_handoff():
    """Serving hand-off: a prefill that ends inside a group, a chunk that
    finishes that group and ends inside another, then decoding steps; every
    output equals decoding the whole sequence frame by frame."""
    needs_gpu()
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=4)
    T0, T1, T = 37, 58, 66
    B = 2
    ms = om.n_slots(T, dims.s) + 2
    w, W, Lyr = layer(dims, 7800, "bf16", pe_rows=ms)
    seq = synth.make_sequence(dims, w, B, T, 7801, "bf16")
    X, QR, KR = dev(seq["X"], "bf16"), dev(seq["QR"], "bf16"), dev(seq["KR"], "bf16")
    cache = Lyr.new_cache(B, ms, fill=float("nan"))
    Lyr.prefill(X[:, :T0].contiguous(), QR[:, :T0].contiguous(), KR[:, :T0].contiguous(),
                cache=cache)
    pos0 = torch.full((B,), T0, dtype=torch.int32, device="cuda")
    Lyr.append_chunk(cache, X[:, T0:T1].contiguous(), KR[:, T0:T1].contiguous(), pos0, T1 - 1)
    ys = []
    for t in range(T1, T):
        pos = torch.full((B,), t, dtype=torch.int32, device="cuda")
        ys.append(Lyr.decode_step(cache, X[:, t].contiguous(), QR[:, t].contiguous(),
                                  KR[:, t].contiguous(), pos, t).clone())
    torch.cuda.synchronize()
    got_cache = host(cache)
    for b in range(B):
        ref = om.decode_sequence(seq["X"][b], seq["QR"][b], seq["KR"][b], W, dims.s, dims.scale)
        got = np.stack([host(y)[b] for y in ys])
        e = relerr(got, ref["Y"][T1:])
        n = om.n_slots(T, dims.s)
        e2 = relerr(got_cache[b, :n, :dims.r], ref["cache_lat"])
        say(f"  b={b} decode-after-chunk relerr {e:.3g} cache relerr {e2:.3g}")
        assert e < TOL["bf16"] and e2 < TOL["bf16"]
