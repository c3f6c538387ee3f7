"""GPU parity of mtla_prefill_unabsorbed_backward (the backward of the
per-head parallel form) against the oracle's chain-rule backward."""
import numpy as np
import pytest
import torch

import oracle.mtla as om
import synth
from synth import Dims
from gpu_util import TOL, dev, host, needs_gpu, relerr, say

pytestmark = pytest.mark.gpu


def _layer(dims, seed, pe_rows, storage="bf16"):
    from kv_cache_compressed_amd import MTLALayer, MTLA_BF16, MTLA_F32
    w = synth.make_weights(dims, seed, storage, pe_rows=pe_rows)
    W = om.with_position_table(w, pe_rows)
    L = MTLALayer.from_arrays(dims, {**w, **synth.head_maps(w)},
                              MTLA_F32 if storage == "f32" else MTLA_BF16)
    return w, W, L


def _oracle_abi(gr, dims):
    """Oracle gradients in the library's layouts."""
    H, d, dh, r = dims.H, dims.d, dims.d_h, dims.r
    return dict(dW_dkv=gr["dW_dkv"], dW_hc=gr["dW_hc"], db_hc=gr["db_hc"], dgate_pos=gr["dP"],
                dW_Q=np.transpose(gr["dW_Q"], (0, 2, 1)).reshape(H * dh, d),
                dW_K=np.transpose(gr["dW_K"], (0, 2, 1)).reshape(H * dh, r),
                dW_V=np.transpose(gr["dW_V"], (0, 2, 1)).reshape(H * dh, r),
                dW_O=np.transpose(gr["dW_O"], (2, 0, 1)).reshape(d, H * dh))


def _check(dims, B, T, seed, T0=None, rows=None, storage="bf16"):
    """Backward at [B, T]; dY is nonzero only on sequences `rows` and frames
    < T0 (defaults: all), so the oracle runs on those prefixes only (frames
    before T0 do not depend on later ones) and the rest must be exact zeros."""
    T0 = T if T0 is None else T0
    rows = list(range(B)) if rows is None else rows
    ms = om.n_slots(T, dims.s) + 1
    w, W, L = _layer(dims, seed, ms, storage)
    seq = synth.make_sequence(dims, w, B, T, seed + 1, storage)
    rng = np.random.default_rng(seed + 2)
    dY = np.zeros((B, T, dims.d))
    for b in rows:
        dY[b, :T0] = synth.round_to(rng.normal(size=(T0, dims.d)), storage)
    X, QR, KR = dev(seq["X"], storage), dev(seq["QR"], storage), dev(seq["KR"], storage)
    dX, dQR, dKR, grads = L.backward_unabsorbed(X, QR, KR, dev(dY, storage))
    torch.cuda.synchronize()
    gX, gQR, gKR = host(dX), host(dQR), host(dKR)
    ref_w = None
    worst = 0.0
    for b in rows:
        x, qr, kr = seq["X"][b, :T0], seq["QR"][b, :T0], seq["KR"][b, :T0]
        gr = om.prefill_unabsorbed_backward(x, qr, kr, W, dims.s, dims.scale, dY[b, :T0])
        for name, got in (("dX", gX[b, :T0]), ("dQR", gQR[b, :T0]), ("dKR", gKR[b, :T0])):
            e = relerr(got, gr[name])
            worst = max(worst, e)
            assert e < TOL[storage], (b, name, e)
        ab = _oracle_abi(gr, dims)
        ref_w = ab if ref_w is None else {k: ref_w[k] + ab[k] for k in ref_w}
    # frames and sequences without a loss gradient get exactly zero
    assert not np.any(gX[:, T0:]) and not np.any(gQR[:, T0:]) and not np.any(gKR[:, T0:])
    for b in set(range(B)) - set(rows):
        assert not np.any(gX[b]) and not np.any(gQR[b]) and not np.any(gKR[b])
    for k, ref in ref_w.items():
        e = relerr(host(grads[k]), ref)
        worst = max(worst, e)
        assert e < TOL[storage], (k, e)
    say(f"  worst relerr {worst:.3g}")


@pytest.mark.parametrize("s,T,H,B", [(2, 1, 8, 1), (2, 130, 8, 2), (3, 257, 4, 1),
                                       (1, 64, 2, 2), (4, 300, 8, 1), (80, 100, 2, 1),
                                       (5, 96, 3, 2), (2, 513, 8, 1)])
def test_backward_matches_oracle(s, T, H, B):
    needs_gpu()
    dims = Dims(d=512, H=H, d_h=64, r=256, d_hR=32, s=s)
    say("backward per-head", s, T, H, B)
    _check(dims, B, T, 9500 + 7 * s + T + H)


@pytest.mark.parametrize("s,T,H,B", [(2, 1, 4, 1), (2, 130, 4, 2), (3, 257, 4, 1),
                                       (1, 64, 2, 2), (4, 300, 4, 1), (80, 100, 2, 1),
                                       (5, 96, 3, 2)])
def test_backward_llm_head_width(s, T, H, B):
    """The backward at the LLM-scale head widths (d_h = 128, d_hR = 64,
    r = 512): one 16-row tile per wave in both attention passes."""
    needs_gpu()
    dims = Dims(d=512, H=H, d_h=128, r=512, d_hR=64, s=s)
    say("backward per-head d_h=128", s, T, H, B)
    _check(dims, B, T, 9600 + 7 * s + T + H)


@pytest.mark.parametrize("d_h,r,dR", [(64, 256, 32), (128, 512, 64)])
@pytest.mark.parametrize("s,T,H,B", [(2, 1, 4, 1), (2, 130, 4, 2), (3, 257, 2, 1), (1, 64, 2, 2),
                                       (80, 100, 2, 1), (5, 96, 3, 2)])
def test_backward_fp32(s, T, H, B, d_h, r, dR):
    """The backward with fp32 storage at both head widths, every input and
    weight gradient against the oracle at 1e-4."""
    needs_gpu()
    dims = Dims(d=256, H=H, d_h=d_h, r=r, d_hR=dR, s=s)
    say("backward per-head fp32", d_h, s, T, H, B)
    _check(dims, B, T, 9900 + 7 * s + T + H + d_h, storage="f32")


def test_backward_full_size_prefix():
    """The benchmark's backward launch (B=16, T=4096, s=2) with the loss on
    the first 320 frames of two sequences: those gradients against the
    oracle, everything else exactly zero."""
    needs_gpu()
    name, dims, ex = synth.config(4)
    say("backward full size", name)
    _check(dims, ex["B"], ex["T"], 9600, T0=320, rows=[0, ex["B"] - 1])


def test_backward_llm_head_width_full_size_prefix():
    """The benchmark's backward launch at the LLM-scale head widths (8
    sequences of 4096 frames, d = 1024, H = 8, d_h = 128, r = 512) with the
    loss on the first 256 frames of two sequences: those gradients against
    the oracle, everything else exactly zero."""
    needs_gpu()
    dims = Dims(d=1024, H=8, d_h=128, r=512, d_hR=64, s=2)
    say("backward full size, d_h = 128")
    _check(dims, 8, 4096, 9650, T0=256, rows=[0, 7])


@pytest.mark.parametrize("storage", ["bf16", "f32"])
@pytest.mark.parametrize("d_h,r,dR", [(64, 256, 32), (128, 512, 64)])
def test_backward_is_deterministic(d_h, r, dR, storage):
    """Two calls on the same inputs give the same bits in every output:
    the input gradients and every reduction across workgroups (weight
    gradients, bias and position-table gradients) add their partials in a
    fixed order."""
    needs_gpu()
    dims = Dims(d=512, H=4, d_h=d_h, r=r, d_hR=dR, s=3)
    B, T = 2, 700
    ms = om.n_slots(T, dims.s) + 1
    w, W, L = _layer(dims, 9700 + d_h, ms, storage)
    seq = synth.make_sequence(dims, w, B, T, 9701, storage)
    rng = np.random.default_rng(9702)
    dY = dev(synth.round_to(rng.normal(size=(B, T, dims.d)), storage), storage)
    X, QR, KR = dev(seq["X"], storage), dev(seq["QR"], storage), dev(seq["KR"], storage)
    outs = []
    for _ in range(2):
        dX, dQR, dKR, grads = L.backward_unabsorbed(X, QR, KR, dY)
        outs.append([dX.clone(), dQR.clone(), dKR.clone()] + [grads[k].clone() for k in sorted(grads)])
    torch.cuda.synchronize()
    say("backward determinism", d_h, storage)
    names = ["dX", "dQR", "dKR"] + sorted(grads)
    for n, a, b in zip(names, outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), n
