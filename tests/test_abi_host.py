"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments before touching
the GPU.  No kernel is launched here (no GPU needed): every call below fails
validation, which runs before any HIP call, and the pointers passed are never
dereferenced."""
import ctypes
import os
import re

import pytest

import kv_cache_compressed_amd as K
from kv_cache_compressed_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mtla.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mtla_[a-z_]+)\s*\(", text)))


def test_header_declares_the_three_hot_path_calls():
    syms = declared_symbols()
    for s in ("mtla_merge_append", "mtla_decode_step", "mtla_prefill_strided"):
        assert s in syms


def test_library_exports_every_declared_symbol():
    lib = K.load_library()
    for s in declared_symbols():
        assert hasattr(lib, s), s
    assert sorted(L.EXPORTED) == declared_symbols()


def test_status_strings():
    for code in range(5):
        assert K.mtla_status_string(code)
    assert "capacity" in K.mtla_status_string(L.MTLA_ERR_CAPACITY)


def _dims(**kw):
    base = dict(d=512, H=8, d_h=64, r=256, d_hR=32, s=2, dtype=L.MTLA_BF16)
    base.update(kw)
    return K.make_dims(**base)


def test_workspace_sizes():
    d = _dims()
    merge = K.mtla_workspace_bytes(d, L.OP_MERGE, 32, 2047)
    dec = K.mtla_workspace_bytes(d, L.OP_DECODE, 32, 2047)
    pre = K.mtla_workspace_bytes(d, L.OP_PREFILL, 16, 4096)
    assert 0 < merge < dec
    # prefill holds at least the absorbed queries and the attention output
    assert pre >= 2 * 16 * 4096 * 8 * 256 * 2
    assert K.mtla_workspace_bytes(_dims(s=0), L.OP_DECODE, 32, 2047) == 0
    assert K.mtla_workspace_bytes(_dims(r=128, d_hR=16), L.OP_DECODE, 32, 2047) == 0
    assert K.mtla_workspace_bytes(d, 7, 32, 2047) == 0
    # fp32 storage doubles the element size of the cache-typed buffers
    assert K.mtla_workspace_bytes(_dims(dtype=L.MTLA_F32), L.OP_PREFILL, 1, 64) > \
        K.mtla_workspace_bytes(_dims(), L.OP_PREFILL, 1, 64)


FAKE = 0x100000  # aligned, never dereferenced: every call below fails validation first


def _weights(rows=1024, A=FAKE, misalign=0):
    return L.Weights(FAKE + misalign, FAKE, FAKE, FAKE, rows, A, FAKE)


def _decode(dims, w, cache, B=32, max_pos=2047, ws_bytes=1 << 30, pos=FAKE):
    lib = K.load_library()
    return lib.mtla_decode_step(ctypes.byref(dims) if dims is not None else None, ctypes.byref(w),
                                ctypes.byref(cache), FAKE, FAKE, FAKE, pos, B, max_pos, FAKE, FAKE,
                                ws_bytes, None)


def _cache(max_slots=1024, stride=None):
    return L.Cache(FAKE, stride if stride is not None else max_slots * 288, max_slots)


@pytest.mark.parametrize("case,expect", [
    ("null_dims", L.MTLA_ERR_ARG),
    ("s_zero", L.MTLA_ERR_ARG),
    ("negative_r", L.MTLA_ERR_ARG),
    ("bad_dtype", L.MTLA_ERR_ARG),
    ("unsupported_r", L.MTLA_ERR_UNSUPPORTED),
    ("d_not_multiple_of_32", L.MTLA_ERR_UNSUPPORTED),
    ("too_many_heads", L.MTLA_ERR_UNSUPPORTED),
    ("misaligned_weight", L.MTLA_ERR_ARG),
    ("null_pos", L.MTLA_ERR_ARG),
    ("null_A", L.MTLA_ERR_ARG),
    ("short_batch_stride", L.MTLA_ERR_ARG),
    ("capacity_slots", L.MTLA_ERR_CAPACITY),
    ("capacity_gate_table", L.MTLA_ERR_CAPACITY),
    ("small_workspace", L.MTLA_ERR_ARG),
    ("zero_batch", L.MTLA_ERR_ARG),
])
def test_decode_rejects(case, expect):
    dims, w, cache = _dims(), _weights(), _cache()
    kw = {}
    if case == "null_dims":
        dims = None
    elif case == "s_zero":
        dims = _dims(s=0)
    elif case == "negative_r":
        dims = _dims(r=-1)
    elif case == "bad_dtype":
        dims = _dims(dtype=9)
    elif case == "unsupported_r":
        dims = _dims(r=128, d_hR=16)
    elif case == "d_not_multiple_of_32":
        dims = _dims(d=500)
    elif case == "too_many_heads":
        dims = _dims(H=65)
    elif case == "misaligned_weight":
        w = _weights(misalign=2)
    elif case == "null_pos":
        kw["pos"] = None
    elif case == "null_A":
        w = _weights(A=None)
    elif case == "short_batch_stride":
        cache = _cache(stride=1024 * 288 - 8)
    elif case == "capacity_slots":
        kw["max_pos"] = 2 * 1024        # slot 1024 == max_slots
    elif case == "capacity_gate_table":
        w = _weights(rows=100)
    elif case == "small_workspace":
        kw["ws_bytes"] = 1024
    elif case == "zero_batch":
        kw["B"] = 0
    st = _decode(dims, w, cache, **kw)
    assert st == expect, (case, st, K.load_library().mtla_last_error_detail())
    assert K.load_library().mtla_last_error_detail()


def test_prefill_and_merge_reject_before_launch():
    lib = K.load_library()
    d, w = _dims(), _weights(rows=8)
    # T = 64 frames need slot 31 < gate_pos_rows = 8: capacity error
    st = lib.mtla_prefill_strided(ctypes.byref(d), ctypes.byref(w), FAKE, FAKE, FAKE, 1, 64, FAKE,
                                  None, None, FAKE, 1 << 30, None)
    assert st == L.MTLA_ERR_CAPACITY
    st = lib.mtla_prefill_strided(ctypes.byref(d), ctypes.byref(_weights()), FAKE, FAKE, FAKE, 1,
                                  0, FAKE, None, None, FAKE, 1 << 30, None)
    assert st == L.MTLA_ERR_ARG
    small = _cache(max_slots=16)
    st = lib.mtla_prefill_strided(ctypes.byref(d), ctypes.byref(_weights()), FAKE, FAKE, FAKE, 1,
                                  64, FAKE, ctypes.byref(small), None, FAKE, 1 << 30, None)
    assert st == L.MTLA_ERR_CAPACITY
    st = lib.mtla_merge_append(ctypes.byref(_dims(s=0)), ctypes.byref(_weights()),
                               ctypes.byref(_cache()), FAKE, FAKE, FAKE, 4, 10, FAKE, 1 << 20, None)
    assert st == L.MTLA_ERR_ARG
    st = lib.mtla_gate_pos_table(ctypes.byref(d), FAKE, 16, 500, FAKE, FAKE, FAKE, None)
    assert st == L.MTLA_ERR_UNSUPPORTED


def _chunk(dims=None, w=None, cache=None, B=4, Lc=16, max_pos=100, ws_bytes=1 << 30, pos0=FAKE,
           lens=None, cprime=None, ws=FAKE):
    lib = K.load_library()
    dims = dims if dims is not None else _dims()
    w = w if w is not None else _weights()
    cache = cache if cache is not None else _cache()
    return lib.mtla_append_chunk(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(cache), FAKE,
                                 FAKE, pos0, lens, B, Lc, max_pos, cprime, ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    ("negative_length", L.MTLA_ERR_ARG),
    ("null_pos0", L.MTLA_ERR_ARG),
    ("misaligned_lens", L.MTLA_ERR_ARG),
    ("misaligned_cprime", L.MTLA_ERR_ARG),
    ("zero_batch", L.MTLA_ERR_ARG),
    ("capacity_slots", L.MTLA_ERR_CAPACITY),
    ("capacity_gate_table", L.MTLA_ERR_CAPACITY),
    ("small_workspace", L.MTLA_ERR_ARG),
    ("unsupported_r", L.MTLA_ERR_UNSUPPORTED),
])
def test_append_chunk_rejects(case, expect):
    kw = {}
    if case == "negative_length":
        kw["Lc"] = -1
    elif case == "null_pos0":
        kw["pos0"] = None
    elif case == "misaligned_lens":
        kw["lens"] = FAKE + 4
    elif case == "misaligned_cprime":
        kw["cprime"] = FAKE + 2
    elif case == "zero_batch":
        kw["B"] = 0
    elif case == "capacity_slots":
        kw["max_pos"] = 2 * 1024
    elif case == "capacity_gate_table":
        kw["w"] = _weights(rows=50)
    elif case == "small_workspace":
        kw["ws_bytes"] = 4 * 16 * 2 * 256 * 4 - 1
    elif case == "unsupported_r":
        kw["dims"] = _dims(r=128, d_hR=16)
    st = _chunk(**kw)
    assert st == expect, (case, st, K.load_library().mtla_last_error_detail())


def test_append_chunk_empty_is_a_noop():
    """L = 0 returns OK before any launch (nothing to merge)."""
    assert _chunk(Lc=0, ws=None, ws_bytes=0) == L.MTLA_OK
    lib = K.load_library()
    d, w, c = _dims(), _weights(), _cache()
    assert lib.mtla_append_chunk(ctypes.byref(d), ctypes.byref(w), ctypes.byref(c), None, None,
                                 FAKE, None, 4, 0, 0, None, None, 0, None) == L.MTLA_OK


def test_append_chunk_workspace():
    d = _dims()
    assert K.mtla_workspace_bytes(d, L.OP_CHUNK, 4, 16) >= 4 * 16 * 2 * 256 * 4
    assert K.mtla_workspace_bytes(d, L.OP_CHUNK, 4, 16) < K.mtla_workspace_bytes(d, L.OP_CHUNK, 4, 17)


def test_rope_inputs_reject_before_launch():
    lib = K.load_library()
    d = _dims()
    args = lambda base, ws_bytes=1 << 20, M=4: (ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, M,
                                                 ctypes.c_float(base), FAKE, FAKE, FAKE,
                                                 ws_bytes, None)
    assert lib.mtla_rope_inputs(*args(1.0)) == L.MTLA_ERR_ARG
    assert lib.mtla_rope_inputs(*args(10000.0, M=0)) == L.MTLA_ERR_ARG
    assert lib.mtla_rope_inputs(*args(10000.0, ws_bytes=16)) == L.MTLA_ERR_ARG
    assert K.mtla_workspace_bytes(d, L.OP_ROPE, 4, 1) >= 4 * 9 * 32 * 4


def _uw(rows=1024, W_Q=FAKE):
    return L.UnabsorbedWeights(FAKE, FAKE, FAKE, FAKE, rows, W_Q, FAKE, FAKE, FAKE)


def _unabsorbed(dims, w, B=2, T=64, ws_bytes=1 << 30, X=FAKE):
    return K.load_library().mtla_prefill_unabsorbed(
        ctypes.byref(dims), ctypes.byref(w), X, FAKE, FAKE, B, T, FAKE, None, None, FAKE, ws_bytes,
        None)


def _unabsorbed_bwd(dims, w, B=2, T=64, ws_bytes=1 << 30, X=FAKE, W_hc=FAKE, grads=True):
    g = L.UnabsorbedGrads(*([FAKE] * 8))
    return K.load_library().mtla_prefill_unabsorbed_backward(
        ctypes.byref(dims), ctypes.byref(w), W_hc, X, FAKE, FAKE, B, T, FAKE, FAKE, FAKE, FAKE,
        ctypes.byref(g) if grads else None, FAKE, ws_bytes, None)


@pytest.mark.parametrize("dtype", [L.MTLA_F32, L.MTLA_BF16])
@pytest.mark.parametrize("call", ["forward", "backward"])
@pytest.mark.parametrize("case,expect", [
    ("head_width_32", L.MTLA_ERR_UNSUPPORTED),
    ("wide_head_narrow_rope", L.MTLA_ERR_UNSUPPORTED),
    ("bad_dtype", L.MTLA_ERR_ARG),
    ("null_W_Q", L.MTLA_ERR_ARG),
    ("misaligned_X", L.MTLA_ERR_ARG),
    ("zero_frames", L.MTLA_ERR_ARG),
    ("capacity_gate_table", L.MTLA_ERR_CAPACITY),
    ("small_workspace", L.MTLA_ERR_ARG),
])
def test_per_head_form_rejects(case, expect, call, dtype):
    """The per-head forward and its backward take both storage types at
    (d_h, d_hR) = (64, 32) and (128, 64); every bad argument fails validation
    (the last case, a one-byte workspace, is the final check before any
    launch: reaching it shows the shape and dtype were accepted)."""
    kw, dkw, w = {}, dict(dtype=dtype), _uw()
    if case == "head_width_32":
        dkw.update(d_h=32)
    elif case == "wide_head_narrow_rope":
        dkw.update(d_h=128)
    elif case == "bad_dtype":
        dkw.update(dtype=7)
    elif case == "null_W_Q":
        w = _uw(W_Q=None)
    elif case == "misaligned_X":
        kw["X"] = FAKE + 2
    elif case == "zero_frames":
        kw["T"] = 0
    elif case == "capacity_gate_table":
        w = _uw(rows=8)   # T = 64 frames at s = 2 need slot 31
    elif case == "small_workspace":
        kw["ws_bytes"] = 1
    dims = _dims(**dkw)
    st = (_unabsorbed if call == "forward" else _unabsorbed_bwd)(dims, w, **kw)
    detail = K.load_library().mtla_last_error_detail().decode()
    assert st == expect, (case, st, detail)
    if case == "small_workspace":
        assert "workspace" in detail, detail


@pytest.mark.parametrize("case", ["null_grads", "null_W_hc"])
def test_per_head_backward_rejects_missing_buffers(case):
    dims = _dims(dtype=L.MTLA_F32)
    kw = {"grads": False} if case == "null_grads" else {"W_hc": None}
    assert _unabsorbed_bwd(dims, _uw(), **kw) == L.MTLA_ERR_ARG
