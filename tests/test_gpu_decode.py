"""GPU parity of mtla_decode_step against the oracle's incremental decoding."""
import numpy as np
import pytest
import torch

import oracle.mtla as om
import synth
from synth import Dims
from gpu_util import TOL, dev, host, layer, needs_gpu, relerr, say

pytestmark = pytest.mark.gpu


def test_tiny_fp32_full_sequence():
    """All 64 incremental steps of the tiny fp32 layer from an empty cache,
    against the oracle step by step, and the final cache."""
    needs_gpu()
    name, dims, ex = synth.config(1)
    T = ex["T"]
    say("decode", name)
    w, W, L = layer(dims, synth.seed_for(1), "f32", pe_rows=T // dims.s + 1)
    seq = synth.make_sequence(dims, w, 1, T, synth.seed_for(1) + 1, "f32")
    ref = om.decode_sequence(seq["X"][0], seq["QR"][0], seq["KR"][0], W, dims.s, dims.scale)
    cache = L.new_cache(1, T // dims.s + 2, fill=float("nan"))
    X, QR, KR = dev(seq["X"], "f32"), dev(seq["QR"], "f32"), dev(seq["KR"], "f32")
    ys = []
    for t in range(T):
        pos = torch.tensor([t], dtype=torch.int32, device="cuda")
        ys.append(L.decode_step(cache, X[:, t].contiguous(), QR[:, t].contiguous(),
                                KR[:, t].contiguous(), pos, t).clone())
    torch.cuda.synchronize()
    Y = np.stack([host(y)[0] for y in ys])
    errs = [relerr(Y[t], ref["Y"][t]) for t in range(T)]
    say("max step relerr", max(errs))
    assert max(errs) < TOL["f32"], int(np.argmax(errs))
    n = om.n_slots(T, dims.s)
    got = host(cache)[0]
    assert relerr(got[:n, :dims.r], ref["cache_lat"]) < TOL["f32"]
    assert relerr(got[:n, dims.r:], ref["cache_rope"]) < TOL["f32"]
    assert np.all(np.isnan(got[n:]))          # rows past the live slots untouched


def _decode_case(dims, pos, storage, seed, max_slots=None, check=None, Lw=None):
    pos = np.asarray(pos, dtype=np.int32)
    B = len(pos)
    max_pos = int(pos.max())
    ms = max_slots or (max_pos // dims.s + 5)
    w, W, L = Lw or layer(dims, seed, storage, pe_rows=ms)
    state = synth.make_decode_state(dims, pos, ms, seed=seed + 1, storage=storage)
    step = synth.make_step(dims, w, pos, seed=seed + 2, storage=storage)
    cache = dev(np.concatenate([state["lat"], state["rope"]], axis=-1), storage)
    before = host(cache)
    Y = L.decode_step(cache, dev(step["x"], storage), dev(step["QR"], storage),
                      dev(step["KR"], storage), torch.from_numpy(pos).cuda(), max_pos)
    torch.cuda.synchronize()
    Yg, after = host(Y), host(cache)
    check = range(B) if check is None else check
    Yref = []
    for b in check:
        lat, rk = state["lat"][b].copy(), state["rope"][b].copy()
        y, _ = om.decode_step(lat, rk, int(pos[b]), step["x"][b], step["QR"][b], step["KR"][b], W,
                              dims.s, dims.scale)
        Yref.append(y)
        j = pos[b] // dims.s
        other = np.ones(ms, bool)
        other[j] = False
        assert np.array_equal(after[b][other], before[b][other], equal_nan=True), b
        assert relerr(after[b, j, :dims.r], lat[j]) < TOL[storage]
    e = relerr(Yg[list(check)], np.stack(Yref))
    say("decode relerr", e)
    assert e < TOL[storage]
    return Yg


def test_speech_decoder_step_b32_ctx2048():
    needs_gpu()
    name, dims, ex = synth.config(2)
    say("decode", name)
    _decode_case(dims, [ex["ctx"] - 1] * ex["B"], "bf16", synth.seed_for(2))


def test_ragged_long_decode_b64_s4():
    needs_gpu()
    name, dims, ex = synth.config(3)
    rng = np.random.default_rng(synth.seed_for(3))
    L_b = rng.integers(ex["ctx_lo"], ex["ctx_hi"] + 1, size=ex["B"])
    say("decode", name, "partial newest slots:", int(np.sum(L_b % dims.s != 0)))
    _decode_case(dims, L_b - 1, "bf16", synth.seed_for(3))


@pytest.mark.parametrize("s,pos", [
    (1, [0, 1, 2, 300]),                 # plain latent attention, every slot final
    (2, [0, 1, 64, 127, 128, 129]),      # split boundaries at 128 slots
    (3, [2, 3, 4, 383, 385, 1000]),
    (4, [0, 4, 8191, 8190, 5, 4095]),
    (7, [6, 7, 13, 14, 2000]),
])
def test_decode_edge_positions(s, pos):
    needs_gpu()
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=s)
    say("decode edge", s, pos)
    _decode_case(dims, pos, "bf16", 7000 + s)


@pytest.mark.parametrize("H", [1, 4, 16, 20, 32])
def test_decode_head_counts(H):
    needs_gpu()
    dims = Dims(d=256, H=H, d_h=64, r=256, d_hR=32, s=2)
    say("decode heads", H)
    _decode_case(dims, [5, 700, 1999], "bf16", 7100 + H)


def test_decode_batch_above_128():
    """More than 128 sequences: the projections take the tiled path and the
    split counters are cleared by their own kernel."""
    needs_gpu()
    dims = Dims(d=256, H=8, d_h=64, r=256, d_hR=32, s=2)
    rng = np.random.default_rng(7300)
    pos = rng.integers(0, 600, size=136)
    say("decode B=136")
    _decode_case(dims, pos, "bf16", 7300, check=[0, 1, 67, 135])


@pytest.mark.parametrize("storage", ["bf16", "f32"])
def test_decode_batch_between_64_and_128(storage):
    """65..128 sequences: both projections take the tiled path -- the output
    projection with K split over workgroups and combined by the last split of
    each tile -- with the split counters cleared by their own kernel."""
    needs_gpu()
    dims = Dims(d=256, H=8, d_h=64, r=256, d_hR=32, s=3)
    rng = np.random.default_rng(7350)
    pos = rng.integers(0, 900, size=100)
    say("decode B=100", storage)
    _decode_case(dims, pos, storage, 7350, check=[0, 1, 50, 99])


@pytest.mark.parametrize("B,d,H,r,dR", [
    (128, 1024, 32, 512, 64),   # input: 1088 column groups, 4 or 5 per workgroup, 16 stages
                                # through a 15-slot ring; output: 16 tiles x 8 splits (XCD-placed)
    (65, 1024, 32, 512, 64),    # 65 rows: the last wave's rows mostly padding
    (97, 224, 8, 256, 32),      # output: 14 groups in 4 tiles of 3 or 4, 8 splits
    (80, 5120, 4, 256, 32),     # output: 80 tiles x 3 splits, the last one shorter
])
def test_decode_weight_streaming_projections(B, d, H, r, dR):
    """65..128 sequences in bf16: the projections stream the weights (the
    workgroup's columns through an LDS ring, its rows of X in registers);
    every branch of the work split against the oracle."""
    needs_gpu()
    dims = Dims(d=d, H=H, d_h=64, r=r, d_hR=dR, s=2)
    rng = np.random.default_rng(7600 + B + d)
    pos = rng.integers(0, 600, size=B)
    say("decode weight streaming", B, d, H, r)
    _decode_case(dims, pos, "bf16", 7600 + B, check=[0, 1, B // 2, B - 1])


def test_decode_wide_latent_fp32():
    needs_gpu()
    dims = Dims(d=256, H=4, d_h=128, r=512, d_hR=64, s=2)
    say("decode r=512 fp32")
    _decode_case(dims, [0, 3, 300], "f32", 7200)


@pytest.mark.parametrize("H,r,dR,storage,s", [
    (8, 256, 32, "bf16", 1),     # 64-row stages, 9 loads per wave: register-staged stream
    (32, 256, 32, "bf16", 1),    # 32-row stages, 5 loads per wave, 8-slot ring
    (48, 256, 32, "bf16", 1),    # 16-row stages, padding load blocks
    (4, 512, 64, "f32", 2),      # 147 KB stages: one-slot ring, one stage per split
    (8, 256, 32, "f32", 2),      # 72 KB stages: a two-slot ring cannot refill, one stage per split
])
def test_decode_long_splits(H, r, dR, storage, s):
    """Contexts long enough that each split streams many stages (beyond the
    LDS ring: the later ones pass through registers), with ragged ends."""
    needs_gpu()
    dims = Dims(d=256, H=H, d_h=max(r // 4, 64), r=r, d_hR=dR, s=s)
    rng = np.random.default_rng(7400 + H)
    pos = rng.integers(8000 * s, 16000 * s, size=8)
    say("decode long splits", H, r, storage, s)
    _decode_case(dims, pos, storage, 7400 + H, check=[0, 3, 7])


def test_decode_is_deterministic():
    needs_gpu()
    _, dims, ex = synth.config(2)
    pos = np.full(8, 1999, dtype=np.int32)
    w, W, L = layer(dims, 77, "bf16", pe_rows=1100)
    state = synth.make_decode_state(dims, pos, 1100, seed=78)
    step = synth.make_step(dims, w, pos, seed=79)
    outs = []
    for _ in range(2):
        cache = dev(np.concatenate([state["lat"], state["rope"]], axis=-1), "bf16")
        Y = L.decode_step(cache, dev(step["x"], "bf16"), dev(step["QR"], "bf16"),
                          dev(step["KR"], "bf16"), torch.from_numpy(pos).cuda(), 1999)
        outs.append((Y.clone(), cache.clone()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))


def test_llm_dims_ragged_decode():
    """The LLM-scale model dims (d = 4096, H = 32, d_h = 128, r = 512,
    bf16) with ragged positions: the first frame, open and live partial
    newest slots, and sequences of up to 8192 slots spread over several
    stages and splits of the balanced work list; every sequence against the
    oracle."""
    needs_gpu()
    dims = Dims(d=4096, H=32, d_h=128, r=512, d_hR=64, s=2)
    pos = [0, 1, 2, 63, 64, 1023, 2048, 4095, 7777, 12000, 16382, 16383]
    say("decode LLM dims, ragged", pos)
    _decode_case(dims, pos, "bf16", 7700)


def test_llm_scale_decode_sampled():
    """Full-size LLM-scale step (B=128, H=32, r=512, 16384 slots, the
    benchmark's launch configuration); the cache is seeded random bf16 made
    on the GPU; the oracle checks seven sampled sequences."""
    needs_gpu()
    name, dims, ex = synth.config(5)
    B, ctx = ex["B"], ex["ctx"]
    say("decode", name, "building weights")
    ms = ctx // dims.s + 8
    w, W, L = layer(dims, synth.seed_for(5), "bf16", pe_rows=ms)
    pos = np.full(B, ctx - 1, dtype=np.int32)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(synth.seed_for(5))
    cache = torch.empty(B, ms, dims.r + dims.d_hR, dtype=torch.bfloat16, device="cuda")
    cache[..., :dims.r].normal_(0.0, 0.7, generator=gen)
    cache[..., dims.r:].normal_(0.0, 1.0, generator=gen)
    cache[:, ctx // dims.s:] = float("nan")
    # Both ends of the batch and of each half (the work list gives every
    # sequence two splits of 8192 slots here), plus an interior sequence.
    sample = [0, 1, 63, 64, 77, 126, 127]
    before = {b: host(cache[b]) for b in sample}
    step = synth.make_step(dims, w, pos, seed=synth.seed_for(5) + 2)
    say("decode", name, "running")
    Y = L.decode_step(cache, dev(step["x"], "bf16"), dev(step["QR"], "bf16"),
                      dev(step["KR"], "bf16"), torch.from_numpy(pos).cuda(), ctx - 1)
    torch.cuda.synchronize()
    Yg = host(Y)
    for b in sample:
        lat, rk = before[b][:, :dims.r].copy(), before[b][:, dims.r:].copy()
        y, _ = om.decode_step(lat, rk, ctx - 1, step["x"][b], step["QR"][b], step["KR"][b], W,
                              dims.s, dims.scale)
        e = relerr(Yg[b], y)
        say("  seq", b, "relerr", e)
        assert e < TOL["bf16"]
        after = host(cache[b])
        j = (ctx - 1) // dims.s
        assert relerr(after[j, :dims.r], lat[j]) < TOL["bf16"]
