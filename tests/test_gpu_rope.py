"""GPU parity of mtla_rope_inputs (the decoupled-RoPE query and key parts of
each frame) against the oracle's rotary definition, and a prefill fed with
them."""
import numpy as np
import pytest
import torch

import oracle.mtla as om
import synth
from synth import Dims
from gpu_util import TOL, dev, host, layer, needs_gpu, relerr, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("storage,H,dR,d", [("f32", 4, 32, 256), ("bf16", 8, 32, 512),
                                            ("bf16", 32, 64, 1024), ("f32", 3, 64, 128)])
def test_rope_inputs_match_oracle(storage, H, dR, d):
    needs_gpu()
    from kv_cache_compressed_amd import MTLA_BF16, MTLA_F32, make_dims, mtla_rope_inputs
    dims = make_dims(d, H, 2 * dR, 8 * dR, dR, 2, MTLA_BF16 if storage == "bf16" else MTLA_F32)
    rng = np.random.default_rng(9700 + H + dR)
    M = 301
    X = synth.round_to(rng.normal(size=(M, d)), storage)
    W_QR = synth.round_to(rng.normal(0, 1 / np.sqrt(d), size=(H, dR, d)), storage)
    W_KR = synth.round_to(rng.normal(0, 1 / np.sqrt(d), size=(dR, d)), storage)
    pos = rng.integers(0, 40000, size=M).astype(np.int32)
    pos[:3] = [0, 1, 32767]
    say("rope", storage, H, dR, d)
    QR, KR = mtla_rope_inputs(dims, dev(W_QR.reshape(H * dR, d), storage), dev(W_KR, storage),
                              dev(X, storage), torch.from_numpy(pos).cuda())
    torch.cuda.synchronize()
    rq, rk = om.rope_inputs(X, W_QR, W_KR, pos)
    eq, ek = relerr(host(QR), rq), relerr(host(KR), rk)
    say(f"  QR relerr {eq:.3g}  KR relerr {ek:.3g}")
    assert eq < TOL[storage] and ek < TOL[storage]


def test_prefill_on_library_rope_inputs():
    """Frames -> the library's rotary parts -> strided prefill, against the
    oracle doing both steps."""
    needs_gpu()
    from kv_cache_compressed_amd import mtla_rope_inputs
    dims = Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=2)
    T, B = 200, 2
    ms = om.n_slots(T, dims.s)
    w, W, L = layer(dims, 9800, "bf16", pe_rows=ms)
    rng = np.random.default_rng(9801)
    X = synth.round_to(rng.normal(size=(B, T, dims.d)), "bf16")
    W_QR = synth.round_to(w["W_QR"], "bf16")
    W_KR = synth.round_to(w["W_KR"], "bf16")
    pos = np.tile(np.arange(T, dtype=np.int32), (B, 1))
    Xd = dev(X, "bf16")
    QR, KR = mtla_rope_inputs(L.dims, dev(W_QR.reshape(-1, dims.d), "bf16"), dev(W_KR, "bf16"), Xd,
                              torch.from_numpy(pos).cuda())
    Y = L.prefill(Xd, QR, KR)
    torch.cuda.synchronize()
    for b in range(B):
        rq, rk = om.rope_inputs(X[b], W_QR, W_KR, pos[b])
        ref = om.prefill(X[b], rq, rk, W, dims.s, dims.scale)
        e = relerr(host(Y[b]), ref["Y"])
        say(f"  b={b} Y relerr {e:.3g}")
        assert e < TOL["bf16"]
