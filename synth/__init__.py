"""Seeded synthetic inputs for the MTLA hot path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It draws random tensors, rounds them to a storage precision and
builds the inputs that sit *upstream* of the MTLA boundary (positional tables,
rotary-embedded query/key parts, random low-rank absorbed weights).  It holds
none of MTLA's own arithmetic: no latent projection, no hyper-network gate, no
temporal merge, no mask and no attention.

Workload shapes follow the five workloads the method is measured on here:

  tiny_fp32        B=1,  d=256,  H=4,  d_h=64,  r=256, d_hR=32, s=2, T=64, fp32
  decode_b32       B=32, d=512,  H=8,  d_h=64,  r=256, d_hR=32, s=2, context 2048, bf16
  ragged_b64_s4    B=64, d=512,  H=8,  d_h=64,  r=256, d_hR=32, s=4, context ~U{4096..8192}, bf16
  prefill_b16      B=16, d=512,  H=8,  d_h=64,  r=256, d_hR=32, s=2, T=4096, bf16
  llm_decode_b128  B=128, d=4096, H=32, d_h=128, r=512, d_hR=64, s=2, context 32768, bf16

Weight layouts are the ones the C-ABI takes: every linear map is stored as a
row-major [out, in] matrix (the layout ``torch.nn.Linear`` keeps), so
``y = x @ W.T``.

  W_dkv [r, d]         latent projection              C = X W_dkv^T
  W_hc  [r, r], b_hc   hyper-network content branch   Linear(c_i)
  W_hp  [r, d_pe], b_hp hyper-network position branch Linear(pe_j)
  A     [H, r, d]      A[h] = (W_Q^(h) W_K^(h)T)^T    q~_h = x A[h]^T
  Bvo   [d, H, r]      Bvo[:, h, :] = (W_V^(h) W_O^(h))^T
  pe    [rows, d_pe]   sinusoidal positional encodings, indexed by slot j

The unabsorbed per-head factors W_Q, W_K, W_V, W_O are returned as well so a
test can evaluate plain multi-head attention with explicit keys and values.
A and Bvo are drawn as products of those Gaussian factors (fp64), which is how
a random rank-d_h matrix is sampled.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, asdict

import numpy as np

__all__ = [
    "Dims", "CONFIGS", "config", "round_to", "make_weights", "make_sequence",
    "make_decode_state", "make_step", "sinusoidal_table", "rope", "seed_for",
]


@dataclass(frozen=True)
class Dims:
    d: int
    H: int
    d_h: int
    r: int
    d_hR: int
    s: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_h)

    def asdict(self):
        return asdict(self)


# name -> (dims, extra); extra holds batch and length information.
CONFIGS = {
    1: ("tiny_fp32", Dims(d=256, H=4, d_h=64, r=256, d_hR=32, s=2),
        dict(B=1, T=64, storage="f32")),
    2: ("decode_b32_ctx2048", Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=2),
        dict(B=32, ctx=2048, storage="bf16")),
    3: ("ragged_decode_b64_s4", Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=4),
        dict(B=64, ctx_lo=4096, ctx_hi=8192, storage="bf16")),
    4: ("prefill_b16_t4096", Dims(d=512, H=8, d_h=64, r=256, d_hR=32, s=2),
        dict(B=16, T=4096, storage="bf16")),
    5: ("llm_decode_b128_ctx32768", Dims(d=4096, H=32, d_h=128, r=512, d_hR=64, s=2),
        dict(B=128, ctx=32768, storage="bf16")),
}


def config(n: int):
    """Return (name, Dims, extra-dict) for workload ``n`` (1..5)."""
    name, dims, extra = CONFIGS[n]
    return name, dims, dict(extra)


def seed_for(n: int) -> int:
    return 1000 + n


def round_to(x, storage: str) -> np.ndarray:
    """Round an array to the storage precision and return it as fp64.

    'f64' leaves it unchanged, 'f32' rounds to float32, 'bf16' rounds to
    bfloat16 with round-to-nearest-even (through torch's CPU conversion).
    """
    x = np.asarray(x, dtype=np.float64)
    if storage == "f64":
        return x
    if storage == "f32":
        return x.astype(np.float32).astype(np.float64)
    if storage == "bf16":
        import torch
        t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
        return t.to(torch.float64).numpy()
    raise ValueError(storage)


def sinusoidal_table(rows: int, width: int) -> np.ndarray:
    """Standard sinusoidal positional encodings: even columns sin, odd cos."""
    pos = np.arange(rows, dtype=np.float64)[:, None]
    k = np.arange(0, width, 2, dtype=np.float64)[None, :]
    ang = pos / np.power(10000.0, k / width)
    out = np.zeros((rows, width), dtype=np.float64)
    out[:, 0::2] = np.sin(ang)
    out[:, 1::2] = np.cos(ang[:, : width // 2])
    return out


def rope(v: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Rotary embedding over adjacent pairs (2k, 2k+1), base 10000.

    ``v`` has shape [..., n, width] where axis -2 is indexed by ``positions``
    (or broadcastable to it)."""
    width = v.shape[-1]
    k = np.arange(width // 2, dtype=np.float64)
    theta = np.power(10000.0, -2.0 * k / width)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * theta
    cos, sin = np.cos(ang), np.sin(ang)
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = a * sin + b * cos
    return out


def make_weights(dims: Dims, seed: int, storage: str = "f64", pe_rows: int = 64) -> dict:
    """Draw all weights of one MTLA layer.  Every returned array is fp64
    holding values exactly representable in ``storage``."""
    d, H, d_h, r, dR = dims.d, dims.H, dims.d_h, dims.r, dims.d_hR
    rng = np.random.default_rng(seed)
    g = lambda shape, fan_in: rng.normal(0.0, 1.0 / math.sqrt(fan_in), size=shape)
    d_pe = d
    w = {}
    w["W_dkv"] = g((r, d), d)
    w["W_hc"] = g((r, r), r)
    w["b_hc"] = g((r,), r)
    w["W_hp"] = g((r, d_pe), d_pe)
    w["b_hp"] = g((r,), d_pe)
    w["W_Q"] = g((H, d, d_h), d)
    w["W_K"] = g((H, r, d_h), r)
    w["W_V"] = g((H, r, d_h), r)
    w["W_O"] = g((H, d_h, d), H * d_h)
    w["W_QR"] = g((H, dR, d), d)
    w["W_KR"] = g((dR, d), d)
    # Random rank-d_h matrices formed from the factors above.
    w["A"] = np.matmul(w["W_K"], np.transpose(w["W_Q"], (0, 2, 1)))          # [H, r, d]
    w["Bvo"] = np.transpose(np.matmul(w["W_V"], w["W_O"]), (2, 0, 1)).copy()  # [d, H, r]
    w["pe"] = sinusoidal_table(pe_rows, d_pe)
    # The per-head factors are rounded after A and Bvo are formed from them.
    for k in ("W_dkv", "W_hc", "b_hc", "W_hp", "b_hp", "A", "Bvo", "pe",
              "W_Q", "W_K", "W_V", "W_O"):
        w[k] = round_to(w[k], storage)
    return w


def head_maps(w: dict) -> dict:
    """The per-head maps of ``w`` in the library's [out, in] layouts, same
    values: W_Qh [H*d_h, d] (rows of head h map x to its query), W_Kh and
    W_Vh [H*d_h, r], W_Oh [d, H*d_h] (columns of head h)."""
    H, d, d_h = w["W_Q"].shape
    r = w["W_K"].shape[1]
    return dict(W_Qh=np.transpose(w["W_Q"], (0, 2, 1)).reshape(H * d_h, d).copy(),
                W_Kh=np.transpose(w["W_K"], (0, 2, 1)).reshape(H * d_h, r).copy(),
                W_Vh=np.transpose(w["W_V"], (0, 2, 1)).reshape(H * d_h, r).copy(),
                W_Oh=np.transpose(w["W_O"], (2, 0, 1)).reshape(d, H * d_h).copy())


def make_sequence(dims: Dims, w: dict, B: int, T: int, seed: int, storage: str = "f64",
                  start: int = 0) -> dict:
    """Frames X [B, T, d] ~ N(0, 1) plus their rotary query/key parts.

    QR [B, T, H, d_hR] and KR [B, T, d_hR] are rotary-embedded projections of
    X at absolute positions start..start+T-1, rounded to ``storage``."""
    rng = np.random.default_rng(seed)
    X = round_to(rng.normal(0.0, 1.0, size=(B, T, dims.d)), storage)
    pos = np.arange(start, start + T, dtype=np.float64)
    H, dR = dims.H, dims.d_hR
    qr = (X @ w["W_QR"].reshape(H * dR, dims.d).T).reshape(B, T, H, dR)
    qr = rope(np.transpose(qr, (0, 2, 1, 3)), pos)          # [B, H, T, dR]
    QR = np.transpose(qr, (0, 2, 1, 3)).copy()
    KR = rope(X @ w["W_KR"].T, pos)                          # [B, T, dR]
    return dict(X=X, QR=round_to(QR, storage), KR=round_to(KR, storage))


def make_decode_state(dims: Dims, pos: np.ndarray, max_slots: int, seed: int,
                      storage: str = "bf16", latent_std: float = 0.7) -> dict:
    """A synthetic compressed cache standing just before the decode step at
    0-based frame positions ``pos`` [B].

    Rows the step may legitimately read hold seeded N(0, latent_std^2) latent
    values and N(0, 1) rotary-key values.  Every row the step must not read --
    rows past the newest slot, and the newest slot itself when the step opens
    it afresh (pos % s == 0) -- is filled with NaN, so any stray read shows up
    in the output.  Returns dict(lat [B, max_slots, r], rope [B, max_slots, dR]).
    """
    s = dims.s
    B = len(pos)
    rng = np.random.default_rng(seed)
    lat = round_to(rng.normal(0.0, latent_std, size=(B, max_slots, dims.r)), storage)
    rk = round_to(rng.normal(0.0, 1.0, size=(B, max_slots, dims.d_hR)), storage)
    for b, t in enumerate(np.asarray(pos)):
        live = t // s + (0 if t % s == 0 else 1)   # rows holding valid content
        lat[b, live:] = np.nan
        rk[b, live:] = np.nan
        rk[b, t // s] = np.nan   # the step overwrites this rotary key before use
    return dict(lat=lat, rope=rk)


def make_step(dims: Dims, w: dict, pos: np.ndarray, seed: int, storage: str = "bf16") -> dict:
    """One new frame per sequence for a decode step at 0-based positions
    ``pos`` [B]: x [B, d] ~ N(0, 1), QR [B, H, d_hR] and KR [B, d_hR] rotated
    at each sequence's own position."""
    pos = np.asarray(pos)
    B = len(pos)
    H, dR = dims.H, dims.d_hR
    rng = np.random.default_rng(seed)
    x = round_to(rng.normal(0.0, 1.0, size=(B, dims.d)), storage)
    qr = (x @ w["W_QR"].reshape(H * dR, dims.d).T).reshape(B, H, dR)
    qr = rope(qr, pos[:, None].astype(np.float64))
    kr = rope(x @ w["W_KR"].T, pos.astype(np.float64))
    return dict(x=x, QR=round_to(qr, storage), KR=round_to(kr, storage))


def make_chunk(dims: Dims, w: dict, pos0: np.ndarray, L: int, seed: int,
               storage: str = "bf16") -> dict:
    """A chunk of L new frames per sequence starting at 0-based positions
    ``pos0`` [B]: X [B, L, d] ~ N(0, 1), and QR [B, L, H, d_hR], KR [B, L, d_hR]
    rotated at each frame's absolute position pos0[b] + i."""
    pos0 = np.asarray(pos0)
    B = len(pos0)
    H, dR = dims.H, dims.d_hR
    rng = np.random.default_rng(seed)
    X = round_to(rng.normal(0.0, 1.0, size=(B, L, dims.d)), storage)
    pos = (pos0[:, None] + np.arange(L)[None, :]).astype(np.float64)      # [B, L]
    qr = (X @ w["W_QR"].reshape(H * dR, dims.d).T).reshape(B, L, H, dR)
    QR = rope(qr, pos[:, :, None])
    KR = rope(X @ w["W_KR"].T, pos)
    return dict(X=X, QR=round_to(QR, storage), KR=round_to(KR, storage))
