"""GPU parity of mtla_prefill_strided against the oracle's masked parallel
form, and prefill -> decode hand-off."""
import numpy as np
import pytest
import torch

import oracle.mtla as om
import synth
from synth import Dims
from gpu_util import TOL, dev, host, layer, needs_gpu, relerr, say

pytestmark = pytest.mark.gpu


def _prefill_case(dims, B, T, storage, seed, with_cache=True):
    ms = om.n_slots(T, dims.s) + 3
    w, W, L = layer(dims, seed, storage, pe_rows=ms)
    seq = synth.make_sequence(dims, w, B, T, seed + 1, storage)
    cache = L.new_cache(B, ms, fill=float("nan")) if with_cache else None
    Cp = torch.empty(B, T, dims.r, dtype=L.dtype, device="cuda")
    Y = L.prefill(dev(seq["X"], storage), dev(seq["QR"], storage), dev(seq["KR"], storage),
                  cache=cache, Cprime=Cp)
    torch.cuda.synchronize()
    Yg, Cpg = host(Y), host(Cp)
    cg = host(cache) if with_cache else None
    n = om.n_slots(T, dims.s)
    for b in range(B):
        ref = om.prefill(seq["X"][b], seq["QR"][b], seq["KR"][b], W, dims.s, dims.scale)
        ey, ec = relerr(Yg[b], ref["Y"]), relerr(Cpg[b], ref["Cp"])
        say(f"  b={b} Y relerr {ey:.3g}  C' relerr {ec:.3g}")
        assert ey < TOL[storage], (b, ey)
        assert ec < TOL[storage], (b, ec)
        if with_cache:
            assert relerr(cg[b, :n, :dims.r], ref["cache_lat"]) < TOL[storage]
            assert np.array_equal(cg[b, :n, dims.r:], ref["cache_rope"])
            assert np.all(np.isnan(cg[b, n:]))
            # the cache rows are the group-final states, bit for bit
            e = np.minimum(np.arange(n) * dims.s + dims.s - 1, T - 1)
            assert np.array_equal(cg[b, :n, :dims.r], Cpg[b, e])
    return Yg


def test_tiny_fp32():
    needs_gpu()
    name, dims, ex = synth.config(1)
    say("prefill", name)
    _prefill_case(dims, ex["B"], ex["T"], "f32", synth.seed_for(1))


@pytest.mark.parametrize("s,T", [(1, 40), (2, 1), (2, 129), (3, 67), (4, 5), (5, 200), (80, 64)])
def test_fp32_strides_and_ragged_lengths(s, T):
    needs_gpu()
    dims = Dims(d=256, H=4, d_h=64, r=256, d_hR=32, s=s)
    say("prefill fp32", s, T)
    _prefill_case(dims, 2, T, "f32", 8000 + s * 7 + T)


@pytest.mark.parametrize("s,T,H", [(2, 300, 8), (3, 250, 8), (2, 97, 16), (4, 160, 32), (2, 64, 3),
                                     (1, 130, 8), (2, 1, 8), (80, 64, 4), (2, 520, 2),
                                     (2, 333, 5), (3, 211, 6)])
def test_bf16_multi_sequence(s, T, H):
    needs_gpu()
    dims = Dims(d=512, H=H, d_h=64, r=256, d_hR=32, s=s)
    say("prefill bf16", s, T, H)
    _prefill_case(dims, 3, T, "bf16", 8100 + s + T + H)


def test_bf16_wide_latent():
    needs_gpu()
    dims = Dims(d=256, H=8, d_h=128, r=512, d_hR=64, s=2)
    say("prefill r=512")
    _prefill_case(dims, 2, 150, "bf16", 8200)


def test_full_size_prefill_sampled():
    """The benchmark's prefill launch (B=16, T=4096, s=2): intermediate states
    and cache of all sixteen sequences in full, outputs of three sequences on
    sampled rows computed one by one from the oracle's visible sets, and every
    output row of one sequence against the oracle's dense masked form."""
    needs_gpu()
    name, dims, ex = synth.config(4)
    B, T = ex["B"], ex["T"]
    say("prefill", name, "inputs")
    ms = om.n_slots(T, dims.s)
    w, W, L = layer(dims, synth.seed_for(4), "bf16", pe_rows=ms)
    seq = synth.make_sequence(dims, w, B, T, synth.seed_for(4) + 1, "bf16")
    cache = L.new_cache(B, ms)
    Cp = torch.empty(B, T, dims.r, dtype=torch.bfloat16, device="cuda")
    say("prefill", name, "running")
    Y = L.prefill(dev(seq["X"], "bf16"), dev(seq["QR"], "bf16"), dev(seq["KR"], "bf16"),
                  cache=cache, Cprime=Cp)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    Cprs = {}
    for b in range(B):
        # Intermediate states and cache of every sequence, in full.
        _, U = om.gated_latents(seq["X"][b], W, dims.s)
        Cpr = Cprs[b] = om.intermediate_states(U, dims.s)
        lat, rk, _ = om.compressed_cache(Cpr, seq["KR"][b], dims.s)
        assert relerr(host(Cp[b]), Cpr) < TOL["bf16"], b
        cg = host(cache[b])
        assert relerr(cg[:, :dims.r], lat) < TOL["bf16"], b
        assert np.array_equal(cg[:, dims.r:], rk), b
    for b in (0, 9, 15):
        X, QR, KR = seq["X"][b], seq["QR"][b], seq["KR"][b]
        Cpr = Cprs[b]
        rows = sorted(set([0, 1, 2, 3, T - 2, T - 1] + list(rng.integers(0, T, size=40))))
        Yg = host(Y[b, rows])
        Yr = []
        for m in rows:
            vis = [n for n in range(m + 1) if om.visible(m, n, dims.s)]
            qt = W["A"] @ X[m]
            o = om.attend_cache(qt, QR[m], Cpr[vis], KR[vis], dims.scale)
            Yr.append(om.output_projection(o, W["Bvo"]))
        e = relerr(Yg, np.stack(Yr))
        say(f"  b={b} sampled-row relerr {e:.3g}")
        assert e < TOL["bf16"]
    # One whole sequence, every row and head, against the oracle's dense
    # masked form (fp64).
    b = 9
    ref = om.prefill(seq["X"][b], seq["QR"][b], seq["KR"][b], W, dims.s, dims.scale)
    e = relerr(host(Y[b]), ref["Y"])
    say(f"  b={b} all {T} rows relerr {e:.3g}")
    assert e < TOL["bf16"]


def test_prefill_then_decode_resumes():
    """Prefill ends inside a group (T mod s != 0); decoding continues from the
    partial slot and matches decoding every frame from the start."""
    needs_gpu()
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=4)
    T0, T = 37, 46
    ms = om.n_slots(T, dims.s) + 2
    w, W, L = layer(dims, 8300, "bf16", pe_rows=ms)
    seq = synth.make_sequence(dims, w, 2, T, 8301, "bf16")
    X, QR, KR = dev(seq["X"], "bf16"), dev(seq["QR"], "bf16"), dev(seq["KR"], "bf16")
    cache = L.new_cache(2, ms, fill=float("nan"))
    L.prefill(X[:, :T0].contiguous(), QR[:, :T0].contiguous(), KR[:, :T0].contiguous(), cache=cache)
    ys = []
    for t in range(T0, T):
        pos = torch.full((2,), t, dtype=torch.int32, device="cuda")
        ys.append(L.decode_step(cache, X[:, t].contiguous(), QR[:, t].contiguous(),
                                KR[:, t].contiguous(), pos, t).clone())
    torch.cuda.synchronize()
    for b in range(2):
        ref = om.decode_sequence(seq["X"][b], seq["QR"][b], seq["KR"][b], W, dims.s, dims.scale)
        got = np.stack([host(y)[b] for y in ys])
        e = relerr(got, ref["Y"][T0:])
        say(f"  b={b} resumed relerr {e:.3g}")
        assert e < TOL["bf16"]


def test_large_tile_product_ragged_edges():
    """The output projection of a long batch takes the 256 x 256-tile product
    (K = H r = 2048): here with 32,769 rows (the last row tile holds one row)
    and d = 320 columns (the second column tile holds 64), checked on sampled
    rows that include the last one, all columns."""
    needs_gpu()
    dims = Dims(d=320, H=8, d_h=64, r=256, d_hR=32, s=2)
    B, T = 9, 3641
    assert B * T == 32769
    ms = om.n_slots(T, dims.s)
    w, W, L = layer(dims, 4100, "bf16", pe_rows=ms)
    seq = synth.make_sequence(dims, w, B, T, 4101, "bf16")
    say("prefill ragged large-tile product", B, T, dims.d)
    Y = L.prefill(dev(seq["X"], "bf16"), dev(seq["QR"], "bf16"), dev(seq["KR"], "bf16"))
    torch.cuda.synchronize()
    rng = np.random.default_rng(4102)
    for b in (0, 4, B - 1):
        X, QR, KR = seq["X"][b], seq["QR"][b], seq["KR"][b]
        _, U = om.gated_latents(X, W, dims.s)
        Cpr = om.intermediate_states(U, dims.s)
        rows = sorted(set([0, 1, 255, 256, T - 2, T - 1] + list(rng.integers(0, T, size=16))))
        Yg = host(Y[b, rows])
        Yr = []
        for m in rows:
            vis = [n for n in range(m + 1) if om.visible(m, n, dims.s)]
            o = om.attend_cache(W["A"] @ X[m], QR[m], Cpr[vis], KR[vis], dims.scale)
            Yr.append(om.output_projection(o, W["Bvo"]))
        e = relerr(Yg, np.stack(Yr))
        say(f"  b={b} sampled-row relerr {e:.3g}")
        assert e < TOL["bf16"]


def test_large_tile_input_projection():
    """The input projection (latent, gate pre-activation and absorbed
    queries: N = 2r + H r = 2560 columns, K = d) on the 256 x 256-tile product
    at d = 1024, a K twice the one the other prefill tests use, with 6,600 rows
    (the last row tile partly filled): the intermediate states in full, outputs
    on sampled rows."""
    needs_gpu()
    dims = Dims(d=1024, H=8, d_h=64, r=256, d_hR=32, s=2)
    B, T = 2, 3300
    ms = om.n_slots(T, dims.s)
    w, W, L = layer(dims, 4200, "bf16", pe_rows=ms)
    seq = synth.make_sequence(dims, w, B, T, 4201, "bf16")
    say("prefill large-tile input projection", B, T, dims.d)
    Cp = torch.empty(B, T, dims.r, dtype=torch.bfloat16, device="cuda")
    Y = L.prefill(dev(seq["X"], "bf16"), dev(seq["QR"], "bf16"), dev(seq["KR"], "bf16"), Cprime=Cp)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4202)
    for b in range(B):
        X, QR, KR = seq["X"][b], seq["QR"][b], seq["KR"][b]
        _, U = om.gated_latents(X, W, dims.s)
        Cpr = om.intermediate_states(U, dims.s)
        ec = relerr(host(Cp[b]), Cpr)
        rows = sorted(set([0, 1, 255, 256, T - 2, T - 1] + list(rng.integers(0, T, size=16))))
        Yg = host(Y[b, rows])
        Yr = []
        for m in rows:
            vis = [n for n in range(m + 1) if om.visible(m, n, dims.s)]
            o = om.attend_cache(W["A"] @ X[m], QR[m], Cpr[vis], KR[vis], dims.scale)
            Yr.append(om.output_projection(o, W["Bvo"]))
        e = relerr(Yg, np.stack(Yr))
        say(f"  b={b} C' relerr {ec:.3g}  sampled-row relerr {e:.3g}")
        assert ec < TOL["bf16"]
        assert e < TOL["bf16"]
