"""Convenience container for one MTLA layer on the GPU.

Holds the device weights in the layouts the C ABI takes, the fp32
position-branch table and the folded content-branch map (built once on the
GPU by mtla_gate_pos_table and mtla_gate_content_map) and reusable
workspaces, and forwards to the hot-path entry points.  It
only marshals arguments; all arithmetic runs in libmtla.so.
"""
from __future__ import annotations

import torch

from . import _lib as L


class MTLALayer:
    WEIGHTS = ("W_dkv", "W_hc", "b_hc", "W_hp", "b_hp", "pe", "A", "Bvo")

    HEAD_MAPS = ("W_Qh", "W_Kh", "W_Vh", "W_Oh")

    def __init__(self, d, H, d_h, r, d_hR, s, dtype=L.MTLA_BF16, scale=0.0, *, W_dkv, W_hc, b_hc,
                 W_hp, b_hp, pe, A, Bvo, W_Qh=None, W_Kh=None, W_Vh=None, W_Oh=None):
        self.dims = L.make_dims(d, H, d_h, r, d_hR, s, dtype, scale)
        self.dtype = L.torch_dtype(dtype)
        self.t = dict(W_dkv=W_dkv, W_hc=W_hc, b_hc=b_hc, W_hp=W_hp, b_hp=b_hp, pe=pe, A=A, Bvo=Bvo)
        for k, v in self.t.items():
            if v.dtype != self.dtype or not v.is_cuda or not v.is_contiguous():
                raise ValueError(f"{k} must be a contiguous device tensor of {self.dtype}")
        self.gate_pos = L.mtla_gate_pos_table(self.dims, pe, W_hp, b_hp)
        self.W_gate = L.mtla_gate_content_map(self.dims, W_hc, W_dkv)
        self.w = L.make_weights(W_dkv, self.W_gate, b_hc, self.gate_pos, A, Bvo)
        # Optional per-head maps ([out, in] layouts) for the unabsorbed form.
        self.heads = dict(W_Qh=W_Qh, W_Kh=W_Kh, W_Vh=W_Vh, W_Oh=W_Oh)
        self.wu = None
        if all(v is not None for v in self.heads.values()):
            for k, v in self.heads.items():
                if v.dtype != self.dtype or not v.is_cuda or not v.is_contiguous():
                    raise ValueError(f"{k} must be a contiguous device tensor of {self.dtype}")
            self.wu = L.make_unabsorbed_weights(W_dkv, self.W_gate, b_hc, self.gate_pos, W_Qh,
                                                W_Kh, W_Vh, W_Oh)
        self._ws = {}
        self._retired = []

    @classmethod
    def from_arrays(cls, dims, arrays: dict, dtype=L.MTLA_BF16, device="cuda", scale=0.0):
        """Upload a dict of host arrays (numpy or torch) holding the weights in
        the ABI layouts.  ``dims`` has attributes d, H, d_h, r, d_hR, s."""
        td = L.torch_dtype(dtype)
        t = {k: torch.as_tensor(arrays[k]).to(td).to(device).contiguous() for k in cls.WEIGHTS}
        for k in cls.HEAD_MAPS:
            if k in arrays:
                t[k] = torch.as_tensor(arrays[k]).to(td).to(device).contiguous()
        return cls(dims.d, dims.H, dims.d_h, dims.r, dims.d_hR, dims.s, dtype, scale, **t)

    @property
    def row(self) -> int:
        return self.dims.r + self.dims.d_hR

    def new_cache(self, B: int, max_slots: int, fill: float = 0.0) -> torch.Tensor:
        return torch.full((B, max_slots, self.row), fill, dtype=self.dtype, device="cuda")

    def workspace(self, op: int, B: int, n: int) -> torch.Tensor:
        """The layer's workspace for entry point ``op``, grown when a call
        needs more.  A buffer that a larger one replaces is kept alive for the
        layer's lifetime: a graph captured earlier may still write to it."""
        need = L.mtla_workspace_bytes(self.dims, op, B, n)
        ws = self._ws.get(op)
        if ws is None or ws.numel() < need:
            if ws is not None:
                self._retired.append(ws)
            ws = L.workspace(self.dims, op, B, n)
            self._ws[op] = ws
        return ws

    def dropped_frames(self, op: int = L.OP_DECODE) -> int:
        """Sequences whose frame the last merge-append (op OP_MERGE) or decode
        step (OP_DECODE) dropped for a position outside [0, max_pos]."""
        return L.dropped_frames(self._ws[op])

    def merge_append(self, cache: torch.Tensor, X_t, KR_t, pos, max_pos: int):
        L.mtla_merge_append(self.dims, self.w, L.make_cache(cache), X_t, KR_t, pos, max_pos,
                            self.workspace(L.OP_MERGE, X_t.shape[0], max_pos))

    def append_chunk(self, cache: torch.Tensor, X, KR, pos0, max_pos: int, lens=None, Cprime=None):
        ws = self.workspace(L.OP_CHUNK, X.shape[0], X.shape[1]) if X.shape[1] > 0 else None
        L.mtla_append_chunk(self.dims, self.w, L.make_cache(cache), X, KR, pos0, max_pos, lens,
                            Cprime, ws)

    def decode_step(self, cache: torch.Tensor, X_t, QR_t, KR_t, pos, max_pos: int, Y=None,
                    events=None):
        return L.mtla_decode_step(self.dims, self.w, L.make_cache(cache), X_t, QR_t, KR_t, pos,
                                  max_pos, Y, self.workspace(L.OP_DECODE, X_t.shape[0], max_pos),
                                  events)

    def decode_step_noalloc(self, cache: torch.Tensor, X_t, QR_t, KR_t, pos, max_pos: int, Y):
        """decode_step on the library's per-GPU scratch (no workspace)."""
        return L.mtla_decode_step_noalloc(self.dims, self.w, L.make_cache(cache), X_t, QR_t, KR_t,
                                          pos, max_pos, Y)

    def prefill(self, X, QR, KR, Y=None, cache: torch.Tensor | None = None, Cprime=None,
                events=None):
        c = L.make_cache(cache) if cache is not None else None
        return L.mtla_prefill_strided(self.dims, self.w, X, QR, KR, Y, c, Cprime,
                                      self.workspace(L.OP_PREFILL, X.shape[0], X.shape[1]),
                                      events)

    def prefill_unabsorbed(self, X, QR, KR, Y=None, cache: torch.Tensor | None = None,
                           Cprime=None, events=None):
        if self.wu is None:
            raise ValueError("the layer was built without the per-head maps W_Qh, W_Kh, W_Vh, W_Oh")
        c = L.make_cache(cache) if cache is not None else None
        return L.mtla_prefill_unabsorbed(self.dims, self.wu, X, QR, KR, Y, c, Cprime,
                                         self.workspace(L.OP_UNABSORBED, X.shape[0], X.shape[1]),
                                         events)

    def backward_unabsorbed(self, X, QR, KR, dY):
        """Gradients of <dY, Y> for prefill_unabsorbed: (dX, dQR, dKR, grads)
        with grads a dict of FP32 weight gradients in the weights' layouts."""
        if self.wu is None:
            raise ValueError("the layer was built without the per-head maps W_Qh, W_Kh, W_Vh, W_Oh")
        d = self.dims
        HD = d.H * d.d_h
        shapes = dict(dW_dkv=(d.r, d.d), dW_hc=(d.r, d.r), db_hc=(d.r,),
                      dgate_pos=tuple(self.gate_pos.shape), dW_Q=(HD, d.d), dW_K=(HD, d.r),
                      dW_V=(HD, d.r), dW_O=(d.d, HD))
        grads = {k: torch.empty(v, dtype=torch.float32, device=X.device) for k, v in shapes.items()}
        dX, dQR, dKR = L.mtla_prefill_unabsorbed_backward(
            d, self.wu, self.t["W_hc"], X, QR, KR, dY, grads,
            ws=self.workspace(L.OP_BACKWARD, X.shape[0], X.shape[1]))
        return dX, dQR, dKR, grads
