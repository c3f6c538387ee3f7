"""Plain CPU oracle of the MTLA hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP kernels or their binding.

It follows the method as the pages describe it, in the pages' order and
notation, computing in the precision of its inputs (fp64 for parity; the
benchmark's CPU baseline feeds fp32 arrays through the same code).  Sources,
cited by page title and section:

  [Notes]  "Multi-head Temporal Latent Attention" -- paper notes (zhaoyang97
           Paper-Notes, NeurIPS 2025), section 方法详解 (method): 整体框架
           (overall framework), 关键设计 (key designs: hyper-network temporal
           merging, stride-aware causal mask, decoupled RoPE with temporal
           compression), and 损失函数/训练策略 (hyper-parameters, cache size).
  [Fig1]   "Multi-head Temporal Latent Attention" (sciencestack.ai), Figure 1
           caption: absorption of the latent-to-KV maps into the query/output
           projections.
  [Fig2]   same page, Figure 2 caption: (a) incremental inference with the
           temporary slot, (b) rejected pre-downsampling, (c) training under
           the stride-aware causal mask.
  [Modit]  modit3d.com article on MTLA: the s=2 walk-through (cache length 1
           after the first and after the second token) and the large-s limit.

Readings taken where the pages leave a step open (each one is listed with its
reason in the design notes of this repository):

  * Indices.  The pages count from 1 and call column n group-final when
    n mod s = 0.  Here frames are counted from 0: frame i belongs to slot
    j = floor(i/s), and frame n is group-final when n mod s = s-1.  The last
    slot may be partial (T not a multiple of s).
  * The gate is per channel: both Linear maps output r values and the product
    of the two is element-wise, so w_i is a vector in R^r.
  * pe_j is indexed by the slot j = floor(i/s); the hyper-network position
    branch Linear(pe_j) is evaluated into a table once.
  * Both hyper-network Linear maps carry a bias; the latent, query and output
    maps carry none.  The merge weights are not normalised.
  * The compressed RoPE key of a slot is the RoPE key of the newest frame
    merged into it (overwritten on every append); Q^R, K^R arrive rotated.
  * K^R is one vector per frame shared by all heads; Q^R is per head.
  * The softmax scale is 1/sqrt(d_h).
  * Heads are combined as y = sum_h o_h Bvo_h.

Parity unpinned: the exact gate parameterisation (what pe_j is, its width and
form, and the biases) -- the pages print no values for it.

Weight layouts ([out, in] row-major, so y = x @ W.T):
  W_dkv [r, d], W_hc [r, r], b_hc [r], W_hp [r, d_pe], b_hp [r],
  A [H, r, d] with A[h] = (W_Q^(h) W_K^(h)T)^T, Bvo [d, H, r] with
  Bvo[:, h, :] = (W_V^(h) W_O^(h))^T.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# index conventions ([Notes] 关键设计 / stride-aware causal mask; [Fig2] (a))
# ---------------------------------------------------------------------------


def slot_of(i: int, s: int) -> int:
    """Slot that frame i (0-based) is merged into: every s adjacent frames
    share one slot ([Notes] 整体框架 and hyper-network temporal merging)."""
    return i // s


def n_slots(T: int, s: int) -> int:
    """Compressed cache length after T frames: ceil(T/s) ([Notes] 整体框架
    and hyper-network temporal merging: T latents become ceil(T/s) slots)."""
    return -(-T // s)


def is_group_final(n: int, s: int) -> bool:
    """0-based form of the printed 'n mod s = 0' (1-based) test."""
    return n % s == s - 1


def visible(m: int, n: int, s: int) -> bool:
    """Stride-aware causal mask ([Notes] 关键设计 / stride-aware causal mask):
    query m may attend column n iff n = m, or n < m and n is group-final."""
    return n == m or (n < m and is_group_final(n, s))


def mask_matrix(T: int, s: int) -> np.ndarray:
    """Boolean [T, T] matrix of ``visible``."""
    m = np.arange(T)[:, None]
    n = np.arange(T)[None, :]
    return (n == m) | ((n < m) & (n % s == s - 1))


# ---------------------------------------------------------------------------
# per-frame quantities ([Notes] 整体框架; hyper-network temporal merging)
# ---------------------------------------------------------------------------


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def position_branch(pe, W_hp, b_hp):
    """Linear(pe_j) for every row j of the positional table: pe W_hp^T + b_hp."""
    return pe @ W_hp.T + b_hp


def latent(x_i, W_dkv):
    """c_i: the low-rank latent of frame x_i ([Notes] 整体框架, the MLA part)."""
    return W_dkv @ x_i


def merge_weight(c_i, j, W_hc, b_hc, P):
    """w_i = Sigmoid(Linear(c_i) * Linear(pe_j)), '*' element-wise
    ([Notes] 关键设计 / hyper-network temporal merging).  ``P`` holds
    Linear(pe_j) row by row."""
    return sigmoid((W_hc @ c_i + b_hc) * P[j])


def frame_update(x_i, i, W, s):
    """(c_i, w_i, w_i * c_i) for frame i.  Both the parallel and the
    incremental form call this one routine, row by row, so their group sums
    add identical numbers in identical order."""
    c = latent(x_i, W["W_dkv"])
    w = merge_weight(c, slot_of(i, s), W["W_hc"], W["b_hc"], W["P"])
    return c, w, w * c


def with_position_table(W, rows: int):
    """Copy of weight dict ``W`` with P = Linear(pe_j) evaluated for j < rows."""
    W = dict(W)
    W["P"] = position_branch(W["pe"][:rows], W["W_hp"], W["b_hp"])
    return W


# ---------------------------------------------------------------------------
# training form: intermediate states and the compressed cache
# ([Notes] 关键设计 / stride-aware causal mask; [Fig2] (c))
# ---------------------------------------------------------------------------


def gated_latents(X, W, s):
    """U [T, r] with U[i] = w_i * c_i, and C [T, r] with C[i] = c_i."""
    T = X.shape[0]
    C = np.empty((T, W["W_dkv"].shape[0]), dtype=X.dtype)
    U = np.empty_like(C)
    for i in range(T):
        C[i], _, U[i] = frame_update(X[i], i, W, s)
    return C, U


def intermediate_states(U, s):
    """C^' [T, r]: position i holds the merge of its group so far,
    sum_{i' = s*floor(i/s)}^{i} U[i'], added left to right.  The group-final
    rows are the fully merged slots; the others are the temporary versions
    c^'_j that incremental decoding attends to ([Fig2] (a), (c))."""
    Cp = np.empty_like(U)
    for i in range(U.shape[0]):
        if i % s == 0:
            Cp[i] = U[i]
        else:
            Cp[i] = Cp[i - 1] + U[i]
    return Cp


def compressed_cache(Cp, KR, s):
    """Compressed cache after T frames: ceil(T/s) slots.  Slot j holds the
    newest state of group j (row e(j) = min(s*j + s - 1, T - 1) of C^') and
    the RoPE key of that same newest frame ([Notes] 整体框架; decoupled RoPE
    with temporal compression)."""
    T = Cp.shape[0]
    e = np.array([min(s * j + s - 1, T - 1) for j in range(n_slots(T, s))], dtype=np.int64)
    return Cp[e].copy(), KR[e].copy(), e


# ---------------------------------------------------------------------------
# absorbed attention ([Notes] 关键设计 / decoupled RoPE: the Y formula; [Fig1])
# ---------------------------------------------------------------------------


def absorbed_queries(X, A):
    """q~ [T, H, r]: q~_{m,h} = x_m (W_Q^(h) W_K^(h)T) = x_m A[h]^T."""
    H, r, d = A.shape
    return (X @ A.reshape(H * r, d).T).reshape(X.shape[0], H, r)


def softmax_rows(z):
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def output_projection(O, Bvo):
    """y = sum_h o_h (W_V^(h) W_O^(h)) for O [..., H, r], Bvo [d, H, r]."""
    return np.einsum("...hr,dhr->...d", O, Bvo)


def prefill(X, QR, KR, W, s, scale):
    """Parallel (training-form) forward of one sequence under the
    stride-aware causal mask.

    X [T, d], QR [T, H, d_hR], KR [T, d_hR].  Every query m scores every
    column n of the intermediate-state sequence,
        z = (q~_{m,h} . C^'_n + Q^R_{m,h} . K^R_n) * scale,
    masked columns are excluded from the softmax, and o_{m,h} = sum_n p_n C^'_n.
    Training uses the uncompressed K^R ([Notes] decoupled RoPE).
    Returns dict(Y [T, d], O [T, H, r], Cp [T, r], cache_lat, cache_rope).
    """
    T = X.shape[0]
    H = W["A"].shape[0]
    _, U = gated_latents(X, W, s)
    Cp = intermediate_states(U, s)
    Qt = absorbed_queries(X, W["A"])
    M = mask_matrix(T, s)
    O = np.empty((T, H, Cp.shape[1]), dtype=X.dtype)
    for h in range(H):
        z = (Qt[:, h, :] @ Cp.T + QR[:, h, :] @ KR.T) * scale
        z = np.where(M, z, -np.inf)
        O[:, h, :] = softmax_rows(z) @ Cp
    lat, rk, _ = compressed_cache(Cp, KR, s)
    return dict(Y=output_projection(O, W["Bvo"]), O=O, Cp=Cp, cache_lat=lat, cache_rope=rk)


# ---------------------------------------------------------------------------
# incremental decoding ([Notes] stride-aware mask motivation; [Fig2] (a);
# [Modit] s = 2 walk-through)
# ---------------------------------------------------------------------------


def attend_cache(qt, qr, lat, rk, scale):
    """Absorbed attention of one query over n cache slots.
    qt [H, r], qr [H, d_hR], lat [n, r], rk [n, d_hR] -> o [H, r]."""
    z = (qt @ lat.T + qr @ rk.T) * scale
    return softmax_rows(z) @ lat


def merge_append(lat, rk, t, x_t, kr_t, W, s):
    """Fold frame t into the cache in place.  Slot j = floor(t/s) is opened
    afresh when t starts a group and accumulated otherwise; its RoPE key
    becomes K^R_t.  ``lat`` [max_slots, r], ``rk`` [max_slots, d_hR].
    Returns the slot index j."""
    _, _, u = frame_update(x_t, t, W, s)
    j = slot_of(t, s)
    if t % s == 0:
        lat[j] = u
    else:
        lat[j] = lat[j] + u
    rk[j] = kr_t
    return j


def decode_step(lat, rk, t, x_t, qr_t, kr_t, W, s, scale):
    """One incremental decoding step of one sequence at 0-based frame t:
    merge-append, then attention over slots 0..floor(t/s), the newest one
    possibly still temporary.  Returns (y_t [d], o_t [H, r])."""
    j = merge_append(lat, rk, t, x_t, kr_t, W, s)
    qt = W["A"] @ x_t                                   # [H, r]
    o = attend_cache(qt, qr_t, lat[: j + 1], rk[: j + 1], scale)
    return output_projection(o, W["Bvo"]), o


def decode_sequence(X, QR, KR, W, s, scale, max_slots=None):
    """Run decode_step for t = 0..T-1 from an empty cache.
    Returns dict(Y [T, d], O [T, H, r], cache_lat, cache_rope) with the cache
    trimmed to its ceil(T/s) live slots."""
    T, r = X.shape[0], W["W_dkv"].shape[0]
    ms = max_slots if max_slots is not None else n_slots(T, s)
    lat = np.zeros((ms, r), dtype=X.dtype)
    rk = np.zeros((ms, KR.shape[1]), dtype=X.dtype)
    Y, O = [], []
    for t in range(T):
        y, o = decode_step(lat, rk, t, X[t], QR[t], KR[t], W, s, scale)
        Y.append(y)
        O.append(o)
    n = n_slots(T, s)
    return dict(Y=np.stack(Y), O=np.stack(O), cache_lat=lat[:n].copy(), cache_rope=rk[:n].copy())


def merge_chunk(lat, rk, t0, Xc, KRc, W, s):
    """Merge-append of L consecutive frames t0 .. t0+L-1 (``Xc`` [L, d],
    ``KRc`` [L, d_hR]) into the cache in place: the incremental merge of
    [Fig2] (a), one frame after the other.  A chunk that starts inside a group
    (t0 mod s != 0) therefore continues that group's live temporary slot
    instead of opening a new one, and each slot it touches ends holding the
    newest state of its group and the RoPE key of the newest frame merged
    into it.  Returns C' [L, r]: row i is the state of frame t0+i's slot right
    after that frame was merged (the intermediate state of [Fig2] (c))."""
    Cp = np.empty((Xc.shape[0], lat.shape[1]), dtype=lat.dtype)
    for i in range(Xc.shape[0]):
        j = merge_append(lat, rk, t0 + i, Xc[i], KRc[i], W, s)
        Cp[i] = lat[j]
    return Cp


# ---------------------------------------------------------------------------
# the per-head (unabsorbed) form ([Fig1] before absorption; [Notes] decoupled
# RoPE: training may keep the RoPE keys uncompressed) -- also the pin of the
# absorbed form above
# ---------------------------------------------------------------------------


def mha_unabsorbed(X, QR, KR, Cp, W_Q, W_K, W_V, W_O, s, scale):
    """Multi-head attention with explicit per-head queries, keys and values
    ([Fig1] (b) before absorption): Q_h = X W_Q^(h), K_h = C^' W_K^(h),
    V_h = C^' W_V^(h), y = sum_h softmax(mask((Q_h K_h^T + Q^R_h K^R^T) scale))
    V_h W_O^(h).  W_Q [H, d, d_h], W_K, W_V [H, r, d_h], W_O [H, d_h, d]."""
    T = X.shape[0]
    M = mask_matrix(T, s)
    Y = np.zeros((T, W_O.shape[2]), dtype=X.dtype)
    for h in range(W_Q.shape[0]):
        Q = X @ W_Q[h]
        K = Cp @ W_K[h]
        V = Cp @ W_V[h]
        z = (Q @ K.T + QR[:, h, :] @ KR.T) * scale
        z = np.where(M, z, -np.inf)
        Y += softmax_rows(z) @ V @ W_O[h]
    return Y


def prefill_unabsorbed(X, QR, KR, W, s, scale):
    """Parallel forward in the per-head form: the gate and group sums of the
    strided prefill, then ``mha_unabsorbed``.  W holds the hyper-network
    (W_dkv, W_hc, b_hc, P) and the per-head maps W_Q [H, d, d_h],
    W_K, W_V [H, r, d_h], W_O [H, d_h, d].  Returns dict(Y, Cp)."""
    _, U = gated_latents(X, W, s)
    Cp = intermediate_states(U, s)
    Y = mha_unabsorbed(X, QR, KR, Cp, W["W_Q"], W["W_K"], W["W_V"], W["W_O"], s, scale)
    return dict(Y=Y, Cp=Cp)


# ---------------------------------------------------------------------------
# backward of the per-head parallel form (the gradients that training under
# the stride-aware mask needs: [Notes] stride-aware causal mask, the parallel
# training it enables; [Fig2] (c)), by the chain rule through the forward
# steps above, last step first
# ---------------------------------------------------------------------------


def prefill_unabsorbed_backward(X, QR, KR, W, s, scale, dY):
    """Gradients of <dY, Y> for Y = prefill_unabsorbed(X, QR, KR, W, s, scale).

    Returns dict with dX [T, d], dQR [T, H, d_hR], dKR [T, d_hR], and the
    weight gradients dW_dkv [r, d], dW_hc [r, r], db_hc [r], dP [rows, r]
    (rows of the position-branch table P = Linear(pe_j)), dW_Q [H, d, d_h],
    dW_K, dW_V [H, r, d_h], dW_O [H, d_h, d]."""
    T = X.shape[0]
    H = W["W_Q"].shape[0]
    C, U = gated_latents(X, W, s)
    Cp = intermediate_states(U, s)
    Mk = mask_matrix(T, s)
    g = {k: np.zeros_like(W[k]) for k in ("W_dkv", "W_hc", "b_hc", "P", "W_Q", "W_K", "W_V",
                                           "W_O")}
    dX = np.zeros_like(X)
    dQR = np.zeros_like(QR)
    dKR = np.zeros_like(KR)
    dCp = np.zeros_like(Cp)
    # attention, head by head: Y = sum_h softmax(Z_h) V_h W_O^(h)
    for h in range(H):
        Q = X @ W["W_Q"][h]
        K = Cp @ W["W_K"][h]
        V = Cp @ W["W_V"][h]
        Z = np.where(Mk, (Q @ K.T + QR[:, h, :] @ KR.T) * scale, -np.inf)
        Pm = softmax_rows(Z)
        O = Pm @ V
        g["W_O"][h] = O.T @ dY
        dO = dY @ W["W_O"][h].T
        dPm = dO @ V.T
        dV = Pm.T @ dO
        # softmax rows: dZ = P * (dP - <dP, P>_row); then the logit scale
        dZ = Pm * (dPm - np.sum(dPm * Pm, axis=1, keepdims=True)) * scale
        dQ = dZ @ K
        dK = dZ.T @ Q
        dQR[:, h, :] = dZ @ KR
        dKR += dZ.T @ QR[:, h, :]
        g["W_Q"][h] = X.T @ dQ
        dX += dQ @ W["W_Q"][h].T
        g["W_K"][h] = Cp.T @ dK
        g["W_V"][h] = Cp.T @ dV
        dCp += dK @ W["W_K"][h].T + dV @ W["W_V"][h].T
    # group sums: C'_i = sum of U over the frames of i's group up to i, so
    # dU_i = sum of dC' over the frames of i's group from i on
    dU = np.empty_like(dCp)
    for i in range(T - 1, -1, -1):
        if i % s == s - 1 or i == T - 1:
            dU[i] = dCp[i]
        else:
            dU[i] = dCp[i] + dU[i + 1]
    # gate, frame by frame: a = W_hc c + b_hc, w = Sigmoid(a * P_j), u = w * c
    for i in range(T):
        j = slot_of(i, s)
        c = C[i]
        a = W["W_hc"] @ c + W["b_hc"]
        w = sigmoid(a * W["P"][j])
        dw = dU[i] * c
        dgate = dw * w * (1.0 - w)
        da = dgate * W["P"][j]
        g["P"][j] += dgate * a
        g["b_hc"] += da
        g["W_hc"] += np.outer(da, c)
        dc = dU[i] * w + W["W_hc"].T @ da
        g["W_dkv"] += np.outer(dc, X[i])
        dX[i] += W["W_dkv"].T @ dc
    return dict(dX=dX, dQR=dQR, dKR=dKR, dW_dkv=g["W_dkv"], dW_hc=g["W_hc"], db_hc=g["b_hc"],
                dP=g["P"], dW_Q=g["W_Q"], dW_K=g["W_K"], dW_V=g["W_V"], dW_O=g["W_O"])


# ---------------------------------------------------------------------------
# decoupled RoPE inputs ([Notes] decoupled RoPE with temporal compression: the
# RoPE-carrying query and key parts Q^R, K^R).  The pages do not spell out
# the rotary form; the reading taken is the standard one: adjacent pairs
# (2k, 2k+1) of a width-w vector turn by pos * base^(-2k/w); Q^R per head from
# W_QR^(h) x, K^R shared by the heads from W_KR x.
# ---------------------------------------------------------------------------


def rope_rotate(v, pos, base=10000.0):
    """Rotate the adjacent pairs of the last axis of v [..., w] by the
    angles pos * base^(-2k/w), k = 0 .. w/2-1; ``pos`` broadcasts against
    v's leading axes."""
    w = v.shape[-1]
    theta = base ** (-2.0 * np.arange(w // 2) / w)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    cs, sn = np.cos(ang), np.sin(ang)
    out = np.empty_like(v)
    out[..., 0::2] = v[..., 0::2] * cs - v[..., 1::2] * sn
    out[..., 1::2] = v[..., 0::2] * sn + v[..., 1::2] * cs
    return out


def rope_inputs(X, W_QR, W_KR, positions, base=10000.0):
    """Q^R [T, H, d_hR] and K^R [T, d_hR] of frames X [T, d] at absolute
    positions [T]: W_QR [H, d_hR, d] ([out, in] per head), W_KR [d_hR, d]."""
    H, dR, d = W_QR.shape
    q = (X @ W_QR.reshape(H * dR, d).T).reshape(X.shape[0], H, dR)
    k = X @ W_KR.T
    pos = np.asarray(positions, dtype=np.float64)
    return rope_rotate(q, pos[:, None], base), rope_rotate(k, pos, base)


# ---------------------------------------------------------------------------
# reference forms used only to pin the ones above
# ---------------------------------------------------------------------------


def prefill_predownsampled(X, QR, KR, W, s, scale):
    """The rejected alternative of [Fig2] (b): merge every group fully first,
    then let query m attend slots 0..floor(m/s) with causal masking over slots.
    The slot holding m then already contains frames after m.  Used only as a
    negative control."""
    T = X.shape[0]
    _, U = gated_latents(X, W, s)
    Cp = intermediate_states(U, s)
    lat, rk, _ = compressed_cache(Cp, KR, s)
    Qt = absorbed_queries(X, W["A"])
    O = np.empty((T, W["A"].shape[0], lat.shape[1]), dtype=X.dtype)
    for m in range(T):
        j = slot_of(m, s)
        O[m] = attend_cache(Qt[m], QR[m], lat[: j + 1], rk[: j + 1], scale)
    return output_projection(O, W["Bvo"])
