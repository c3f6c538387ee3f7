"""GPU check of mtla_decode_step_noalloc, the decode step on the library's
per-GPU scratch (no workspace, no allocation), through the C ABI: two calls
in a row -- the second with a smaller batch, context and a different stride --
each against mtla_decode_step on the same inputs (identical bits: the same
kernels in the same launch configuration) and against the oracle (bf16 bound
2e-2); and an oversized shape refused before anything is launched."""
import numpy as np
import pytest
import torch

import oracle.mtla as om
import synth
from synth import Dims
from gpu_util import TOL, dev, host, layer, needs_gpu, relerr, say

pytestmark = pytest.mark.gpu


def _case(dims, pos, seed, check):
    pos = np.asarray(pos, dtype=np.int32)
    B, max_pos = len(pos), int(pos.max())
    ms = max_pos // dims.s + 3
    w, W, L = layer(dims, seed, "bf16", pe_rows=ms)
    state = synth.make_decode_state(dims, pos, ms, seed=seed + 1)
    step = synth.make_step(dims, w, pos, seed=seed + 2)
    args = (dev(step["x"], "bf16"), dev(step["QR"], "bf16"), dev(step["KR"], "bf16"),
            torch.from_numpy(pos).cuda(), max_pos)
    rows = np.concatenate([state["lat"], state["rope"]], axis=-1)
    cache_ref, cache_na = dev(rows, "bf16"), dev(rows, "bf16")
    Y_ref = L.decode_step(cache_ref, *args)
    Y_na = torch.empty_like(Y_ref)
    L.decode_step_noalloc(cache_na, *args, Y_na)
    torch.cuda.synchronize()
    assert torch.equal(Y_na.view(torch.int16), Y_ref.view(torch.int16))
    assert torch.equal(cache_na.view(torch.int16), cache_ref.view(torch.int16))
    Yg = host(Y_na)
    for b in check:
        lat, rk = state["lat"][b].copy(), state["rope"][b].copy()
        y, _ = om.decode_step(lat, rk, int(pos[b]), step["x"][b], step["QR"][b], step["KR"][b], W,
                              dims.s, dims.scale)
        e = relerr(Yg[b], y)
        assert e < TOL["bf16"], (b, e)
    say("  noalloc == decode_step, oracle ok:", B, max_pos)


def test_noalloc_decode_two_calls():
    needs_gpu()
    name, dims, ex = synth.config(2)
    say("noalloc decode", name)
    _case(dims, [ex["ctx"] - 1] * ex["B"], 9700, check=[0, 17, 31])
    dims2 = Dims(d=256, H=4, d_h=64, r=256, d_hR=32, s=3)
    _case(dims2, [0, 5, 301, 640, 2], 9710, check=range(5))


def test_noalloc_refuses_oversized_shape():
    needs_gpu()
    from kv_cache_compressed_amd import MtlaError
    from kv_cache_compressed_amd import _lib as Lb
    _, dims, _ = synth.config(5)
    w, W, L = layer(Dims(d=dims.d, H=dims.H, d_h=dims.d_h, r=dims.r, d_hR=dims.d_hR, s=2), 9720,
                    "bf16", pe_rows=8)
    B, max_pos = 1024, 32767
    need = Lb.mtla_workspace_bytes(L.dims, Lb.OP_DECODE, B, max_pos)
    assert need > 64 << 20
    x = torch.zeros(B, dims.d, dtype=torch.bfloat16, device="cuda")
    qr = torch.zeros(B, dims.H, dims.d_hR, dtype=torch.bfloat16, device="cuda")
    kr = torch.zeros(B, dims.d_hR, dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(B, dtype=torch.int32, device="cuda")
    cache = torch.zeros(B, 1, dims.r + dims.d_hR, dtype=torch.bfloat16, device="cuda")
    Y = torch.zeros(B, dims.d, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(MtlaError) as ei:
        L.decode_step_noalloc(cache, x, qr, kr, pos, max_pos, Y)
    assert ei.value.status == Lb.MTLA_ERR_CAPACITY
