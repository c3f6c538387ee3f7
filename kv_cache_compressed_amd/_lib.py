"""ctypes binding of libmtla.so -- argument marshalling only.

Every function here converts torch tensors to device pointers, passes the
current HIP stream, calls the C entry point of the same name and raises
``MtlaError`` on a non-OK status.  No arithmetic of the method happens here;
when the built library is missing the import fails loudly.
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmtla.so")

MTLA_OK, MTLA_ERR_ARG, MTLA_ERR_CAPACITY, MTLA_ERR_UNSUPPORTED, MTLA_ERR_HIP = range(5)
MTLA_F32, MTLA_BF16 = 0, 1
OP_MERGE, OP_DECODE, OP_PREFILL, OP_CHUNK, OP_UNABSORBED, OP_BACKWARD, OP_ROPE = 0, 1, 2, 3, 4, 5, 6

EXPORTED = ("mtla_gate_pos_table", "mtla_gate_content_map", "mtla_merge_append",
            "mtla_append_chunk", "mtla_decode_step", "mtla_prefill_strided",
            "mtla_decode_step_timed", "mtla_prefill_strided_timed", "mtla_prefill_unabsorbed",
            "mtla_prefill_unabsorbed_timed", "mtla_prefill_unabsorbed_backward",
            "mtla_rope_inputs", "mtla_workspace_bytes", "mtla_decode_step_noalloc",
            "mtla_status_string", "mtla_last_error_detail")


class MtlaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"MTLA status {status}: {detail}")
        self.status = status
        self.detail = detail


class Dims(ctypes.Structure):
    _fields_ = [("d", c_int32), ("H", c_int32), ("d_h", c_int32), ("r", c_int32),
                ("d_hR", c_int32), ("s", c_int32), ("scale", c_float), ("dtype", c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [("W_dkv", c_void_p), ("W_gate", c_void_p), ("b_hc", c_void_p),
                ("gate_pos", c_void_p), ("gate_pos_rows", c_int32), ("A", c_void_p),
                ("Bvo", c_void_p)]


class UnabsorbedWeights(ctypes.Structure):
    _fields_ = [("W_dkv", c_void_p), ("W_gate", c_void_p), ("b_hc", c_void_p),
                ("gate_pos", c_void_p), ("gate_pos_rows", c_int32), ("W_Q", c_void_p),
                ("W_K", c_void_p), ("W_V", c_void_p), ("W_O", c_void_p)]


class UnabsorbedGrads(ctypes.Structure):
    _fields_ = [("dW_dkv", c_void_p), ("dW_hc", c_void_p), ("db_hc", c_void_p),
                ("dgate_pos", c_void_p), ("dW_Q", c_void_p), ("dW_K", c_void_p),
                ("dW_V", c_void_p), ("dW_O", c_void_p)]


class Cache(ctypes.Structure):
    _fields_ = [("slots", c_void_p), ("batch_stride", c_int64), ("max_slots", c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmtla.so (built in-tree by ``kv_cache_compressed_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    P = POINTER
    lib.mtla_gate_pos_table.argtypes = [P(Dims), c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                        c_void_p, c_void_p]
    lib.mtla_gate_content_map.argtypes = [P(Dims), c_void_p, c_void_p, c_void_p, c_void_p]
    lib.mtla_merge_append.argtypes = [P(Dims), P(Weights), P(Cache), c_void_p, c_void_p, c_void_p,
                                      c_int32, c_int32, c_void_p, c_size_t, c_void_p]
    lib.mtla_append_chunk.argtypes = [P(Dims), P(Weights), P(Cache), c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                      c_size_t, c_void_p]
    lib.mtla_decode_step.argtypes = [P(Dims), P(Weights), P(Cache), c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_size_t,
                                     c_void_p]
    lib.mtla_prefill_strided.argtypes = [P(Dims), P(Weights), c_void_p, c_void_p, c_void_p,
                                         c_int32, c_int32, c_void_p, P(Cache), c_void_p, c_void_p,
                                         c_size_t, c_void_p]
    lib.mtla_prefill_unabsorbed.argtypes = [P(Dims), P(UnabsorbedWeights), c_void_p, c_void_p,
                                            c_void_p, c_int32, c_int32, c_void_p, P(Cache),
                                            c_void_p, c_void_p, c_size_t, c_void_p]
    lib.mtla_prefill_unabsorbed_timed.argtypes = lib.mtla_prefill_unabsorbed.argtypes + [c_void_p]
    lib.mtla_prefill_unabsorbed_backward.argtypes = [
        P(Dims), P(UnabsorbedWeights), c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32,
        c_void_p, c_void_p, c_void_p, c_void_p, P(UnabsorbedGrads), c_void_p, c_size_t, c_void_p]
    lib.mtla_rope_inputs.argtypes = [P(Dims), c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                     c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.mtla_decode_step_timed.argtypes = lib.mtla_decode_step.argtypes + [c_void_p]
    lib.mtla_decode_step_noalloc.argtypes = [P(Dims), P(Weights), P(Cache), c_void_p, c_void_p,
                                             c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                             c_void_p]
    lib.mtla_prefill_strided_timed.argtypes = lib.mtla_prefill_strided.argtypes + [c_void_p]
    for f in ("mtla_gate_pos_table", "mtla_gate_content_map", "mtla_merge_append",
              "mtla_append_chunk", "mtla_decode_step", "mtla_decode_step_noalloc",
              "mtla_prefill_strided", "mtla_decode_step_timed", "mtla_prefill_strided_timed",
              "mtla_prefill_unabsorbed", "mtla_prefill_unabsorbed_timed",
              "mtla_prefill_unabsorbed_backward", "mtla_rope_inputs"):
        getattr(lib, f).restype = c_int32
    lib.mtla_workspace_bytes.argtypes = [P(Dims), c_int32, c_int32, c_int32]
    lib.mtla_workspace_bytes.restype = c_size_t
    lib.mtla_status_string.argtypes = [c_int32]
    lib.mtla_status_string.restype = c_char_p
    lib.mtla_last_error_detail.argtypes = []
    lib.mtla_last_error_detail.restype = c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != MTLA_OK:
        lib = load_library()
        raise MtlaError(status, lib.mtla_status_string(status).decode() + ": "
                        + lib.mtla_last_error_detail().decode())


def _stream() -> c_void_p:
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t) -> c_void_p:
    if t is None:
        return c_void_p(None)
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return c_void_p(t.data_ptr())


def torch_dtype(code: int):
    return torch.bfloat16 if code == MTLA_BF16 else torch.float32


def make_dims(d, H, d_h, r, d_hR, s, dtype=MTLA_BF16, scale=0.0) -> Dims:
    return Dims(int(d), int(H), int(d_h), int(r), int(d_hR), int(s), float(scale), int(dtype))


def make_weights(W_dkv, W_gate, b_hc, gate_pos, A=None, Bvo=None) -> Weights:
    """Gather device weight tensors ([out, in] layouts) into the C struct.
    ``W_gate`` comes from mtla_gate_content_map.  The tensors must stay alive
    while the struct is used."""
    return Weights(_ptr(W_dkv), _ptr(W_gate), _ptr(b_hc), _ptr(gate_pos), int(gate_pos.shape[0]),
                   _ptr(A), _ptr(Bvo))


def make_unabsorbed_weights(W_dkv, W_gate, b_hc, gate_pos, W_Q, W_K, W_V, W_O) -> UnabsorbedWeights:
    """Per-head maps in the ABI layouts: W_Q [H*d_h, d], W_K and W_V
    [H*d_h, r], W_O [d, H*d_h].  The tensors must stay alive while the struct
    is used."""
    return UnabsorbedWeights(_ptr(W_dkv), _ptr(W_gate), _ptr(b_hc), _ptr(gate_pos),
                             int(gate_pos.shape[0]), _ptr(W_Q), _ptr(W_K), _ptr(W_V), _ptr(W_O))


def make_cache(slots: torch.Tensor) -> Cache:
    """Cache struct over a [B, max_slots, r + d_hR] tensor."""
    B, max_slots, row = slots.shape
    return Cache(_ptr(slots), int(max_slots * row), int(max_slots))


def mtla_workspace_bytes(dims: Dims, op: int, B: int, T_or_max_pos: int) -> int:
    return int(load_library().mtla_workspace_bytes(ctypes.byref(dims), op, B, T_or_max_pos))


def mtla_status_string(status: int) -> str:
    return load_library().mtla_status_string(status).decode()


def workspace(dims: Dims, op: int, B: int, T_or_max_pos: int, device="cuda") -> torch.Tensor:
    n = mtla_workspace_bytes(dims, op, B, T_or_max_pos)
    if n == 0:
        raise MtlaError(MTLA_ERR_ARG, "workspace size query rejected the arguments")
    return torch.empty(n, dtype=torch.uint8, device=device)


def dropped_frames(ws: torch.Tensor) -> int:
    """The status word of a merge-append or decode-step workspace: the number
    of sequences whose position lay outside [0, max_pos] in the last call on
    it (their frames were not merged).  Reading it synchronises with the
    device."""
    return int(ws[:4].view(torch.int32).item())


def mtla_gate_pos_table(dims: Dims, pe, W_hp, b_hp, table=None):
    rows, d_pe = pe.shape
    if table is None:
        table = torch.empty(rows, dims.r, dtype=torch.float32, device=pe.device)
    _check(load_library().mtla_gate_pos_table(ctypes.byref(dims), _ptr(pe), rows, d_pe, _ptr(W_hp),
                                              _ptr(b_hp), _ptr(table), _stream()))
    return table


def mtla_gate_content_map(dims: Dims, W_hc, W_dkv, W_gate=None):
    if W_gate is None:
        W_gate = torch.empty(dims.r, dims.d, dtype=W_dkv.dtype, device=W_dkv.device)
    _check(load_library().mtla_gate_content_map(ctypes.byref(dims), _ptr(W_hc), _ptr(W_dkv),
                                                _ptr(W_gate), _stream()))
    return W_gate


def mtla_merge_append(dims: Dims, w: Weights, cache: Cache, X_t, KR_t, pos, max_pos: int,
                      ws=None):
    B = X_t.shape[0]
    if ws is None:
        ws = workspace(dims, OP_MERGE, B, max_pos, X_t.device)
    _check(load_library().mtla_merge_append(ctypes.byref(dims), ctypes.byref(w),
                                            ctypes.byref(cache), _ptr(X_t), _ptr(KR_t), _ptr(pos),
                                            B, int(max_pos), _ptr(ws), ws.numel(), _stream()))


def mtla_append_chunk(dims: Dims, w: Weights, cache: Cache, X, KR, pos0, max_pos: int, lens=None,
                      Cprime=None, ws=None):
    """Merge frames pos0[b] .. pos0[b] + n_b - 1 of X [B, L, d] into the cache
    (n_b = lens[b] or L); ``max_pos`` bounds every sequence's last frame."""
    B, Lc = X.shape[0], X.shape[1]
    if ws is None and Lc > 0:
        ws = workspace(dims, OP_CHUNK, B, Lc, X.device)
    _check(load_library().mtla_append_chunk(ctypes.byref(dims), ctypes.byref(w),
                                            ctypes.byref(cache), _ptr(X), _ptr(KR), _ptr(pos0),
                                            _ptr(lens), B, Lc, int(max_pos), _ptr(Cprime),
                                            _ptr(ws), ws.numel() if ws is not None else 0,
                                            _stream()))


def _events(events):
    """Two events -> the C array of their raw hipEvent_t handles.  Accepts
    torch.cuda.Event objects or raw handles (ints / c_void_p)."""
    handles = []
    for e in events:
        if isinstance(e, torch.cuda.Event):
            if e.cuda_event == 0:      # torch creates the underlying event on first record
                e.record()
            handles.append(e.cuda_event)
        else:
            handles.append(e.value if isinstance(e, c_void_p) else int(e))
    return (c_void_p * 2)(*handles)


def mtla_decode_step(dims: Dims, w: Weights, cache: Cache, X_t, QR_t, KR_t, pos, max_pos: int,
                     Y=None, ws=None, events=None):
    """``events``: optional pair of torch.cuda.Event recorded around the
    split-K attention kernel (the profiling entry point is used then)."""
    B = X_t.shape[0]
    if Y is None:
        Y = torch.empty(B, dims.d, dtype=X_t.dtype, device=X_t.device)
    if ws is None:
        ws = workspace(dims, OP_DECODE, B, max_pos, X_t.device)
    lib = load_library()
    args = [ctypes.byref(dims), ctypes.byref(w), ctypes.byref(cache), _ptr(X_t), _ptr(QR_t),
            _ptr(KR_t), _ptr(pos), B, int(max_pos), _ptr(Y), _ptr(ws), ws.numel(), _stream()]
    if events is None:
        _check(lib.mtla_decode_step(*args))
    else:
        _check(lib.mtla_decode_step_timed(*args, _events(events)))
    return Y


def mtla_decode_step_noalloc(dims: Dims, w: Weights, cache: Cache, X_t, QR_t, KR_t, pos,
                             max_pos: int, Y=None):
    """mtla_decode_step without a workspace: the library's per-GPU scratch is
    used (``Y`` must be given when nothing may be allocated)."""
    B = X_t.shape[0]
    if Y is None:
        Y = torch.empty(B, dims.d, dtype=X_t.dtype, device=X_t.device)
    _check(load_library().mtla_decode_step_noalloc(
        ctypes.byref(dims), ctypes.byref(w), ctypes.byref(cache), _ptr(X_t), _ptr(QR_t),
        _ptr(KR_t), _ptr(pos), B, int(max_pos), _ptr(Y), _stream()))
    return Y


def mtla_prefill_strided(dims: Dims, w: Weights, X, QR, KR, Y=None, cache: Cache | None = None,
                         Cprime=None, ws=None, events=None):
    """``events``: optional pair of torch.cuda.Event recorded around the
    strided attention kernel (the profiling entry point is used then)."""
    B, T = X.shape[0], X.shape[1]
    if Y is None:
        Y = torch.empty(B, T, dims.d, dtype=X.dtype, device=X.device)
    if ws is None:
        ws = workspace(dims, OP_PREFILL, B, T, X.device)
    cptr = ctypes.byref(cache) if cache is not None else None
    lib = load_library()
    args = [ctypes.byref(dims), ctypes.byref(w), _ptr(X), _ptr(QR), _ptr(KR), B, T, _ptr(Y), cptr,
            _ptr(Cprime), _ptr(ws), ws.numel(), _stream()]
    if events is None:
        _check(lib.mtla_prefill_strided(*args))
    else:
        _check(lib.mtla_prefill_strided_timed(*args, _events(events)))
    return Y


def mtla_prefill_unabsorbed(dims: Dims, w: UnabsorbedWeights, X, QR, KR, Y=None,
                            cache: Cache | None = None, Cprime=None, ws=None, events=None):
    """``events``: optional pair of torch.cuda.Event recorded around the
    per-head attention kernel (the profiling entry point is used then)."""
    B, T = X.shape[0], X.shape[1]
    if Y is None:
        Y = torch.empty(B, T, dims.d, dtype=X.dtype, device=X.device)
    if ws is None:
        ws = workspace(dims, OP_UNABSORBED, B, T, X.device)
    cptr = ctypes.byref(cache) if cache is not None else None
    lib = load_library()
    args = [ctypes.byref(dims), ctypes.byref(w), _ptr(X), _ptr(QR), _ptr(KR), B, T, _ptr(Y), cptr,
            _ptr(Cprime), _ptr(ws), ws.numel(), _stream()]
    if events is None:
        _check(lib.mtla_prefill_unabsorbed(*args))
    else:
        _check(lib.mtla_prefill_unabsorbed_timed(*args, _events(events)))
    return Y


def mtla_rope_inputs(dims: Dims, W_QR, W_KR, X, pos, base: float = 10000.0, QR=None, KR=None,
                     ws=None):
    """Rotary query and key parts of the frames X [..., d] at positions pos
    (same leading shape, int32): returns (QR [..., H, d_hR], KR [..., d_hR])."""
    lead = tuple(X.shape[:-1])
    M = 1
    for n in lead:
        M *= int(n)
    if QR is None:
        QR = torch.empty(*lead, dims.H, dims.d_hR, dtype=X.dtype, device=X.device)
    if KR is None:
        KR = torch.empty(*lead, dims.d_hR, dtype=X.dtype, device=X.device)
    if ws is None:
        ws = workspace(dims, OP_ROPE, M, 1, X.device)
    _check(load_library().mtla_rope_inputs(ctypes.byref(dims), _ptr(W_QR), _ptr(W_KR), _ptr(X),
                                           _ptr(pos), M, float(base), _ptr(QR), _ptr(KR),
                                           _ptr(ws), ws.numel(), _stream()))
    return QR, KR


GRAD_NAMES = ("dW_dkv", "dW_hc", "db_hc", "dgate_pos", "dW_Q", "dW_K", "dW_V", "dW_O")


def mtla_prefill_unabsorbed_backward(dims: Dims, w: UnabsorbedWeights, W_hc, X, QR, KR, dY,
                                     grads: dict, dX=None, dQR=None, dKR=None, ws=None):
    """Gradients of <dY, Y> for the per-head forward: returns (dX, dQR, dKR);
    the FP32 weight gradients go into the tensors of ``grads`` (keys
    GRAD_NAMES, preallocated by the caller in the weights' layouts)."""
    B, T = X.shape[0], X.shape[1]
    if dX is None:
        dX = torch.empty_like(X)
    if dQR is None:
        dQR = torch.empty_like(QR)
    if dKR is None:
        dKR = torch.empty_like(KR)
    if ws is None:
        ws = workspace(dims, OP_BACKWARD, B, T, X.device)
    g = UnabsorbedGrads(*[_ptr(grads[k]) for k in GRAD_NAMES])
    _check(load_library().mtla_prefill_unabsorbed_backward(
        ctypes.byref(dims), ctypes.byref(w), _ptr(W_hc), _ptr(X), _ptr(QR), _ptr(KR), B, T,
        _ptr(dY), _ptr(dX), _ptr(dQR), _ptr(dKR), ctypes.byref(g), _ptr(ws), ws.numel(),
        _stream()))
    return dX, dQR, dKR


def n_slots(T: int, s: int) -> int:
    return math.ceil(T / s)
