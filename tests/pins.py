"""Pins of the CPU oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own formulas.

Each ``pin_*`` function raises AssertionError when the oracle disagrees.  They
are plain functions (not tests) so that the mutation tests can run every pin
against an oracle with a planted mistake and require that one of them fails.
All oracle calls go through the module object ``om`` so a monkeypatched
function is picked up.
"""
from __future__ import annotations

import math
import os

import numpy as np

import oracle.mtla as om
import synth
from synth import Dims

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TINY = Dims(d=256, H=4, d_h=64, r=256, d_hR=32, s=2)   # d == r on purpose:
# a transposed square operand is then shape-compatible and must be caught by
# value, not by a shape error.


def relerr(got, ref):
    """Norm-wise relative error max|got - ref| / max|ref|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def _layer(dims: Dims, seed: int, T: int, storage="f64"):
    W = synth.make_weights(dims, seed, storage, pe_rows=max(om.n_slots(T, dims.s) + 1, 8))
    W = om.with_position_table(W, W["pe"].shape[0])
    seq = synth.make_sequence(dims, W, 1, T, seed + 7, storage)
    return W, seq["X"][0], seq["QR"][0], seq["KR"][0]


# ---------------------------------------------------------------------------
# index conventions
# ---------------------------------------------------------------------------


def load_mask_fixture():
    rows = []
    with open(os.path.join(GOLDEN, "stride_mask.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            head, cols = line.split(":")
            s, T, m = (int(v) for v in head.split())
            rows.append((s, T, m, {int(v) for v in cols.split()}))
    return rows


def pin_mask_printed_rule():
    """The vectorised mask equals the hand-written table of the printed rule
    (1-based on the page, shifted to 0-based here)."""
    for s, T, m1, cols1 in load_mask_fixture():
        M = om.mask_matrix(T, s)
        got = {n + 1 for n in range(T) if M[m1 - 1, n]}
        assert got == cols1, (s, T, m1, got, cols1)
        for n in range(T):
            assert bool(M[m1 - 1, n]) == om.visible(m1 - 1, n, s)


def pin_mask_double_loop():
    """Mask from a brute-force double loop over the 1-based printed rule."""
    for s in (1, 2, 3, 4, 5):
        for T in (1, 2, 3, 7, 13):
            ref = np.zeros((T, T), dtype=bool)
            for m1 in range(1, T + 1):
                for n1 in range(1, T + 1):
                    ref[m1 - 1, n1 - 1] = (n1 == m1) or (n1 < m1 and n1 % s == 0)
            assert np.array_equal(om.mask_matrix(T, s), ref), (s, T)


def pin_slot_counts():
    """ceil(T/s) slots after T frames, both forms, bit-exact integers."""
    dims0 = Dims(d=8, H=1, d_h=4, r=16, d_hR=2, s=1)
    for s in (1, 2, 3, 4):
        dims = Dims(**{**dims0.asdict(), "s": s})
        for T in range(1, 3 * s + 2):
            assert om.n_slots(T, s) == math.ceil(T / s)
            W, X, QR, KR = _layer(dims, 11 + s, T)
            pf = om.prefill(X, QR, KR, W, s, dims.scale)
            dc = om.decode_sequence(X, QR, KR, W, s, dims.scale, max_slots=T + 1)
            assert pf["cache_lat"].shape[0] == math.ceil(T / s)
            assert dc["cache_lat"].shape[0] == math.ceil(T / s)
            # slot index of every frame and the group-final set
            for i in range(T):
                assert om.slot_of(i, s) == (i + 1 + s - 1) // s - 1


def pin_worked_example_s2():
    """The s = 2 walk-through: slot contents after each of 6 steps.

    With c_i = e_i (one-hot latents) and a hyper-network whose content branch
    is zero, every merge weight is Sigmoid(0) = 1/2 exactly, so each slot is
    one half times the indicator of the frames merged into it."""
    s, T, r, d = 2, 6, 8, 8
    W = dict(W_dkv=np.eye(r, d), W_hc=np.zeros((r, r)), b_hc=np.zeros(r),
             P=np.ones((4, r)))
    lat = np.full((4, r), np.nan)
    rk = np.full((4, 2), np.nan)
    expect = []
    with open(os.path.join(GOLDEN, "worked_example_s2.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            step, length, slots, temp = line.split()
            expect.append((int(step), int(length),
                           [sorted(int(v) for v in g.split(",")) for g in slots.split(";")],
                           temp == "yes"))
    X = np.eye(T, d)
    for t in range(T):
        j = om.merge_append(lat, rk, t, X[t], np.array([t, -t], float), W, s)
        step, length, slots, temp = expect[t]
        assert step == t + 1 and j + 1 == length, (t, j, length)
        for jj, members in enumerate(slots):
            got = [i + 1 for i in range(r) if lat[jj, i] != 0]
            assert got == members, (t, jj, got, members)
            assert np.all(lat[jj, [m - 1 for m in members]] == 0.5)
        # the newest slot is temporary exactly when the step does not end a group
        assert (not om.is_group_final(t, s)) == temp
        # RoPE key of the newest slot is the newest frame's
        assert np.array_equal(rk[j], [t, -t])


def pin_cache_size_law():
    """Elements per slot r + d_hR = 4.5 d_h; per token 9 d_h / (2 s)."""
    with open(os.path.join(GOLDEN, "cache_size.txt")) as f:
        rows = [tuple(int(v) for v in l.split()) for l in f if l.strip() and not l.startswith("#")]
    for d_h, s, per_token in rows:
        r, dR = 4 * d_h, d_h // 2
        T = 12 * s
        slots = om.n_slots(T, s)
        assert slots * (r + dR) == per_token * T, (d_h, s)


# ---------------------------------------------------------------------------
# structured inputs with exact answers: the gate and the latent map
# ---------------------------------------------------------------------------


def pin_latent_orientation():
    """W_dkv with a single nonzero entry (a, b) maps x to c with c_a = x_b."""
    r, d, a, b = 6, 5, 4, 1
    Wd = np.zeros((r, d))
    Wd[a, b] = 1.0
    x = np.arange(1.0, d + 1)
    c = om.latent(x, Wd)
    ref = np.zeros(r)
    ref[a] = x[b]
    assert np.array_equal(c, ref)


def pin_gate_structure():
    """Content branch with a single nonzero weight (a, b) and zero bias:
    Linear(c) has c_b at channel a and 0 elsewhere, so w_a = Sigmoid(c_b P_ja)
    and every other channel is Sigmoid(0) = 1/2.  The position branch is
    indexed by the slot floor(i/s)."""
    r, s, a, b = 6, 3, 2, 5
    Wh = np.zeros((r, r))
    Wh[a, b] = 1.0
    P = np.arange(1.0, 4 * r + 1).reshape(4, r) / 10.0   # distinct rows
    W = dict(W_dkv=np.eye(r), W_hc=Wh, b_hc=np.zeros(r), P=P)
    for i in range(9):
        c = np.linspace(-1, 1, r) + 0.1 * i
        cc, w, u = om.frame_update(c, i, W, s)
        assert np.array_equal(cc, c)
        j = i // s
        for ch in range(r):
            ref = 1.0 / (1.0 + math.exp(-(c[b] * P[j, a]))) if ch == a else 0.5
            assert abs(w[ch] - ref) < 1e-15, (i, ch)
        assert np.allclose(u, w * c, rtol=0, atol=0)


def pin_gate_bias_and_position():
    """Zero content weights and unit bias: Linear(c) = 1, so w_i is
    Sigmoid(Linear(pe_j)) with j = floor(i/s), and Linear(pe) = pe W_hp^T + b_hp
    for a W_hp with one nonzero entry."""
    r, dpe, s = 4, 3, 2
    Whp = np.zeros((r, dpe))
    Whp[1, 2] = 2.0
    bhp = np.array([0.5, -0.25, 0.0, 1.0])
    pe = np.arange(15.0).reshape(5, dpe)
    P = om.position_branch(pe, Whp, bhp)
    for j in range(5):
        ref = bhp.copy()
        ref[1] += 2.0 * pe[j, 2]
        assert np.array_equal(P[j], ref)
    W = dict(W_dkv=np.eye(r), W_hc=np.zeros((r, r)), b_hc=np.ones(r), P=P)
    for i in range(9):
        _, w, _ = om.frame_update(np.ones(r), i, W, s)
        ref = 1.0 / (1.0 + np.exp(-P[i // s]))
        assert np.max(np.abs(w - ref)) < 1e-15


# ---------------------------------------------------------------------------
# equivalences the pages state
# ---------------------------------------------------------------------------


def pin_absorbed_equals_unabsorbed():
    """Absorbed attention equals multi-head attention with explicit keys and
    values (associativity of the matrix products)."""
    for s, T in ((2, 64), (3, 17), (1, 9)):
        dims = Dims(**{**TINY.asdict(), "s": s})
        W, X, QR, KR = _layer(dims, 100 + s, T)
        pf = om.prefill(X, QR, KR, W, s, dims.scale)
        ref = om.mha_unabsorbed(X, QR, KR, pf["Cp"], W["W_Q"], W["W_K"], W["W_V"], W["W_O"],
                                s, dims.scale)
        assert relerr(pf["Y"], ref) < 1e-12, (s, T, relerr(pf["Y"], ref))


def pin_decode_equals_prefill():
    """Step-by-step decoding equals the masked parallel form at every
    position; the caches agree bit for bit."""
    for s, T in ((1, 9), (2, 64), (2, 13), (3, 16), (4, 18), (5, 7)):
        dims = Dims(**{**TINY.asdict(), "s": s})
        W, X, QR, KR = _layer(dims, 200 + s, T)
        pf = om.prefill(X, QR, KR, W, s, dims.scale)
        dc = om.decode_sequence(X, QR, KR, W, s, dims.scale)
        assert relerr(dc["Y"], pf["Y"]) < 1e-12, (s, T, relerr(dc["Y"], pf["Y"]))
        assert relerr(dc["O"], pf["O"]) < 1e-12
        assert np.array_equal(dc["cache_lat"], pf["cache_lat"]), (s, T)
        assert np.array_equal(dc["cache_rope"], pf["cache_rope"]), (s, T)


def pin_resume_from_partial_prefill():
    """A prefill that ends inside a group leaves that slot partial; decoding
    onward from it equals decoding every frame from the start."""
    s, T0, T = 3, 10, 17
    dims = Dims(**{**TINY.asdict(), "s": s})
    W, X, QR, KR = _layer(dims, 301, T)
    full = om.decode_sequence(X, QR, KR, W, s, dims.scale)
    pf = om.prefill(X[:T0], QR[:T0], KR[:T0], W, s, dims.scale)
    ms = om.n_slots(T, s)
    lat = np.zeros((ms, dims.r))
    rk = np.zeros((ms, dims.d_hR))
    lat[: pf["cache_lat"].shape[0]] = pf["cache_lat"]
    rk[: pf["cache_rope"].shape[0]] = pf["cache_rope"]
    for t in range(T0, T):
        y, _ = om.decode_step(lat, rk, t, X[t], QR[t], KR[t], W, s, dims.scale)
        assert relerr(y, full["Y"][t]) < 1e-12, t
    assert np.array_equal(lat, full["cache_lat"])


def _sdpa(qt, qr, keys_lat, keys_rope, mask, scale):
    import torch
    import torch.nn.functional as F
    H = qt.shape[1]
    q = torch.from_numpy(np.concatenate([qt, qr], axis=-1)).permute(1, 0, 2)      # [H, T, r+dR]
    k = torch.from_numpy(np.concatenate([keys_lat, keys_rope], axis=-1))[None].expand(H, -1, -1)
    v = torch.from_numpy(keys_lat)[None].expand(H, -1, -1)
    if mask is None:
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
    else:
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=torch.from_numpy(mask), scale=scale)
    return o.permute(1, 0, 2).numpy()


def pin_s1_is_causal_mla():
    """s = 1: every frame is group-final, the mask is the ordinary causal
    mask and MTLA is causal latent attention over the gated latents; compare
    with torch's scaled_dot_product_attention (CPU, fp64, is_causal)."""
    dims = Dims(**{**TINY.asdict(), "s": 1})
    T = 24
    W, X, QR, KR = _layer(dims, 401, T)
    pf = om.prefill(X, QR, KR, W, 1, dims.scale)
    _, U = om.gated_latents(X, W, 1)
    assert np.array_equal(pf["Cp"], U)
    O = _sdpa(om.absorbed_queries(X, W["A"]), QR, U, KR, None, dims.scale)
    assert relerr(pf["O"], O) < 1e-12


def pin_any_s_matches_sdpa():
    """Any s: the masked attention equals torch's SDPA with a boolean mask
    built by a double loop from the printed rule."""
    for s, T in ((2, 20), (3, 19), (4, 9)):
        dims = Dims(**{**TINY.asdict(), "s": s})
        W, X, QR, KR = _layer(dims, 500 + s, T)
        pf = om.prefill(X, QR, KR, W, s, dims.scale)
        mask = np.zeros((T, T), dtype=bool)
        for m1 in range(1, T + 1):
            for n1 in range(1, T + 1):
                mask[m1 - 1, n1 - 1] = (n1 == m1) or (n1 < m1 and n1 % s == 0)
        O = _sdpa(om.absorbed_queries(X, W["A"]), QR, pf["Cp"], KR, mask, dims.scale)
        assert relerr(pf["O"], O) < 1e-12, (s, relerr(pf["O"], O))


def pin_unabsorbed_matches_sdpa():
    """The per-head form: for every head, torch's SDPA over the explicit
    queries [X W_Q^(h) | Q^R_h], keys [C' W_K^(h) | K^R] and values C' W_V^(h)
    under the printed-rule mask, mapped through W_O^(h) and summed."""
    import torch
    import torch.nn.functional as F
    for s, T in ((2, 21), (3, 16), (1, 7)):
        dims = Dims(**{**TINY.asdict(), "s": s})
        W, X, QR, KR = _layer(dims, 520 + s, T)
        Cp = om.prefill(X, QR, KR, W, s, dims.scale)["Cp"]
        mask = np.zeros((T, T), dtype=bool)
        for m1 in range(1, T + 1):
            for n1 in range(1, T + 1):
                mask[m1 - 1, n1 - 1] = (n1 == m1) or (n1 < m1 and n1 % s == 0)
        Y = np.zeros((T, dims.d))
        for h in range(dims.H):
            q = torch.from_numpy(np.concatenate([X @ W["W_Q"][h], QR[:, h, :]], axis=-1))
            k = torch.from_numpy(np.concatenate([Cp @ W["W_K"][h], KR], axis=-1))
            v = torch.from_numpy(Cp @ W["W_V"][h])
            o = F.scaled_dot_product_attention(q[None], k[None], v[None],
                                               attn_mask=torch.from_numpy(mask)[None],
                                               scale=dims.scale)[0].numpy()
            Y += o @ W["W_O"][h]
        ref = om.mha_unabsorbed(X, QR, KR, Cp, W["W_Q"], W["W_K"], W["W_V"], W["W_O"], s,
                                dims.scale)
        assert relerr(ref, Y) < 1e-12, (s, T, relerr(ref, Y))


def pin_backward_matches_finite_differences():
    """Every gradient of the per-head parallel form against central finite
    differences of the (separately pinned) forward: for a random direction V
    of each input and weight, <grad, V> equals (L(+eps V) - L(-eps V)) / 2eps
    with L = <dY, Y>, in fp64.  Partial last groups (T mod s != 0) and s = 1
    included."""
    rng = np.random.default_rng(1301)
    for s, T in ((3, 10), (2, 9), (1, 6)):
        dims = Dims(d=16, H=2, d_h=4, r=8, d_hR=4, s=s)
        W = synth.make_weights(dims, 1300 + s, "f64", pe_rows=om.n_slots(T, s) + 1)
        W = om.with_position_table(W, W["pe"].shape[0])
        seq = synth.make_sequence(dims, W, 1, T, 1310 + s, "f64")
        inp = dict(X=seq["X"][0], QR=seq["QR"][0], KR=seq["KR"][0])
        dY = rng.normal(size=(T, dims.d))
        gr = om.prefill_unabsorbed_backward(inp["X"], inp["QR"], inp["KR"], W, s, dims.scale, dY)

        def loss(i, w):
            return float(np.sum(om.prefill_unabsorbed(i["X"], i["QR"], i["KR"], w, s,
                                                      dims.scale)["Y"] * dY))
        eps = 1e-5
        for name, key in (("dX", "X"), ("dQR", "QR"), ("dKR", "KR")):
            V = rng.normal(size=inp[key].shape)
            fd = (loss({**inp, key: inp[key] + eps * V}, W)
                  - loss({**inp, key: inp[key] - eps * V}, W)) / (2 * eps)
            an = float(np.sum(gr[name] * V))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (s, name, fd, an)
        for name, key in (("dW_dkv", "W_dkv"), ("dW_hc", "W_hc"), ("db_hc", "b_hc"), ("dP", "P"),
                          ("dW_Q", "W_Q"), ("dW_K", "W_K"), ("dW_V", "W_V"), ("dW_O", "W_O")):
            V = rng.normal(size=W[key].shape)
            fd = (loss(inp, {**W, key: W[key] + eps * V})
                  - loss(inp, {**W, key: W[key] - eps * V})) / (2 * eps)
            an = float(np.sum(gr[name] * V))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (s, name, fd, an)


def pin_rope_closed_form():
    """Rotary pairs by hand: width 4, base 16 -- pair 0 turns by pos, pair 1
    by pos / 4; unit vectors land on (cos, sin) and (-sin, cos); position 0
    is the identity; lengths of pairs are kept."""
    for p in (0.0, 1.0, 3.0, 1000.0):
        v = np.array([1.0, 0.0, 0.0, 1.0])
        got = om.rope_rotate(v, p, base=16.0)
        a0, a1 = p, p / 4.0
        ref = np.array([math.cos(a0), math.sin(a0), -math.sin(a1), math.cos(a1)])
        assert np.max(np.abs(got - ref)) < 1e-12, (p, got, ref)
    rng = np.random.default_rng(1401)
    v = rng.normal(size=(5, 32))
    r = om.rope_rotate(v, np.arange(5) * 7.0)
    assert np.array_equal(om.rope_rotate(v, 0.0), v)
    n0 = v[:, 0::2] ** 2 + v[:, 1::2] ** 2
    n1 = r[:, 0::2] ** 2 + r[:, 1::2] ** 2
    assert np.max(np.abs(n0 - n1)) < 1e-12


def pin_rope_relative_position():
    """The rotary score depends on the offset only: <R_m q, R_n k> =
    <R_(m-n) q, k> for any positions (rotations compose)."""
    rng = np.random.default_rng(1402)
    for w in (2, 8, 32):
        q, k = rng.normal(size=w), rng.normal(size=w)
        for m, n in ((5, 3), (0, 9), (4096, 4000), (12, 12)):
            lhs = om.rope_rotate(q, m) @ om.rope_rotate(k, n)
            rhs = om.rope_rotate(q, m - n) @ k
            assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(lhs)), (w, m, n, lhs, rhs)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------


def pin_half_gate_group_mean():
    """W_hc = 0, b_hc = 0: every w is Sigmoid(0) = 1/2 exactly, so at s = 2 a
    full slot is the mean of its two latents (bit-exact)."""
    dims = TINY
    T = 10
    W, X, QR, KR = _layer(dims, 601, T)
    W["W_hc"] = np.zeros_like(W["W_hc"])
    W["b_hc"] = np.zeros_like(W["b_hc"])
    pf = om.prefill(X, QR, KR, W, 2, dims.scale)
    C = X @ W["W_dkv"].T
    for i in range(T):
        assert np.max(np.abs(C[i] - om.latent(X[i], W["W_dkv"]))) < 1e-12
    Cr = np.stack([om.latent(X[i], W["W_dkv"]) for i in range(T)])
    assert np.array_equal(pf["cache_lat"], 0.5 * (Cr[0::2] + Cr[1::2]))


def pin_large_s_limit():
    """s >= T: a single slot, each query sees only its own position, so y_m
    is the current state C'_m through the output map, whatever the queries."""
    dims = Dims(**{**TINY.asdict(), "s": 16})
    T = 12
    W, X, QR, KR = _layer(dims, 701, T)
    pf = om.prefill(X, QR, KR, W, 16, dims.scale)
    assert pf["cache_lat"].shape[0] == 1
    assert np.array_equal(pf["O"], np.repeat(pf["Cp"][:, None, :], dims.H, axis=1))
    W2 = dict(W)
    W2["A"] = W["A"] * -3.0
    pf2 = om.prefill(X, QR * 5.0, KR, W2, 16, dims.scale)
    assert np.array_equal(pf["Y"], pf2["Y"])


def pin_uniform_softmax():
    """Zero absorbed query weights and zero Q^R: all scores are 0, the softmax
    is uniform over the visible set, and o_m is the plain mean of the visible
    states (computed here by an explicit loop over the printed rule)."""
    s, T = 3, 11
    dims = Dims(**{**TINY.asdict(), "s": s})
    W, X, QR, KR = _layer(dims, 801, T)
    W["A"] = np.zeros_like(W["A"])
    pf = om.prefill(X, np.zeros_like(QR), KR, W, s, dims.scale)
    for m1 in range(1, T + 1):
        vis = [n1 - 1 for n1 in range(1, T + 1) if n1 == m1 or (n1 < m1 and n1 % s == 0)]
        mean = sum(pf["Cp"][n] for n in vis) / len(vis)
        for h in range(dims.H):
            assert np.max(np.abs(pf["O"][m1 - 1, h] - mean)) < 1e-13


def pin_first_step():
    """t = 0: one slot holding w_0 c_0 is all the query can see, so the
    softmax weight is exactly 1 and o_0 = w_0 c_0 for every head."""
    dims = TINY
    W, X, QR, KR = _layer(dims, 901, 3)
    lat = np.zeros((2, dims.r))
    rk = np.zeros((2, dims.d_hR))
    _, o = om.decode_step(lat, rk, 0, X[0], QR[0], KR[0], W, 2, dims.scale)
    _, _, u0 = om.frame_update(X[0], 0, W, 2)
    for h in range(dims.H):
        assert np.array_equal(o[h], u0)


def pin_predownsampling_differs():
    """The rejected pre-downsampling variant agrees with decoding at
    group-final positions and differs at every other position, where its slot
    already holds later frames."""
    s, T = 2, 16
    dims = TINY
    W, X, QR, KR = _layer(dims, 1001, T)
    dc = om.decode_sequence(X, QR, KR, W, s, dims.scale)
    pd = om.prefill_predownsampled(X, QR, KR, W, s, dims.scale)
    for t in range(T):
        e = relerr(pd[t], dc["Y"][t])
        if om.is_group_final(t, s) or t == T - 1:
            assert e < 1e-12, (t, e)
        else:
            assert e > 1e-3, (t, e)


# ---------------------------------------------------------------------------
# chunked (multi-frame) merge-append
# ---------------------------------------------------------------------------


def pin_chunked_append_equals_prefill():
    """Merging a sequence chunk by chunk -- boundaries inside groups as well
    as on them, empty chunks included -- leaves exactly the cache of the
    parallel form, untouched rows stay untouched, and the chunks' states
    concatenate to the parallel form's C' (bit for bit: both add the same
    per-frame updates in the same order)."""
    rng = np.random.default_rng(1101)
    for s, T in ((1, 9), (2, 13), (3, 17), (4, 18), (5, 7)):
        dims = Dims(**{**TINY.asdict(), "s": s})
        W, X, QR, KR = _layer(dims, 1100 + s, T)
        pf = om.prefill(X, QR, KR, W, s, dims.scale)
        n = om.n_slots(T, s)
        lat = np.full((n + 2, dims.r), np.nan)
        rk = np.full((n + 2, dims.d_hR), np.nan)
        cuts = {0, 1, min(s + 1, T), T - 2, T} | set(rng.integers(1, T, size=3).tolist())
        cuts = sorted(c for c in cuts if 0 <= c <= T)
        states = []
        for a, b in zip(cuts[:-1] + [T], cuts[1:] + [T]):   # last pair is an empty chunk
            states.append(om.merge_chunk(lat, rk, a, X[a:b], KR[a:b], W, s))
        assert np.array_equal(np.concatenate(states), pf["Cp"]), (s, T)
        assert np.array_equal(lat[:n], pf["cache_lat"]), (s, T)
        assert np.array_equal(rk[:n], pf["cache_rope"]), (s, T)
        assert np.all(np.isnan(lat[n:])) and np.all(np.isnan(rk[n:]))


def pin_chunk_continues_live_slot():
    """Closed form of a chunk over a cache the oracle did not write: with a
    zero content branch every merge weight is 1/2, so a chunk starting inside
    group j0 adds half of each of its latents to whatever slot j0 holds, and
    a chunk starting on a group boundary discards it.  Latents are small
    integers, so every sum is exact."""
    r = d = 8
    for s, t0, L in ((2, 3, 6), (3, 4, 7), (4, 8, 5), (3, 6, 2), (1, 5, 4)):
        W = dict(W_dkv=np.eye(r, d), W_hc=np.zeros((r, r)), b_hc=np.zeros(r),
                 P=np.ones((16, r)))
        X = np.arange(1.0, L * d + 1.0).reshape(L, d) % 7.0 - 3.0
        KRc = np.stack([np.array([t0 + i, 100.0 + i]) for i in range(L)])
        j0 = t0 // s
        v = np.arange(r, dtype=np.float64) * 0.25 - 1.0     # prior content of slot j0
        lat = np.full((16, r), np.nan)
        rk = np.full((16, 2), np.nan)
        lat[j0] = v
        rk[j0] = [-1.0, -1.0]
        Cp = om.merge_chunk(lat, rk, t0, X, KRc, W, s)
        for i in range(L):
            f = t0 + i
            j = f // s
            first = max(t0, s * j)
            expect = (v if first > s * j else 0.0) + 0.5 * X[first - t0: i + 1].sum(axis=0)
            assert np.array_equal(Cp[i], expect), (s, t0, i)
        for j in range(j0, (t0 + L - 1) // s + 1):
            last = min(t0 + L - 1, s * j + s - 1)
            assert np.array_equal(lat[j], Cp[last - t0]), (s, t0, j)
            assert np.array_equal(rk[j], KRc[last - t0]), (s, t0, j)
        assert np.all(np.isnan(lat[(t0 + L - 1) // s + 1:]))


ALL_PINS = [
    pin_mask_printed_rule, pin_mask_double_loop, pin_slot_counts, pin_worked_example_s2,
    pin_cache_size_law, pin_latent_orientation, pin_gate_structure, pin_gate_bias_and_position,
    pin_absorbed_equals_unabsorbed, pin_decode_equals_prefill, pin_resume_from_partial_prefill,
    pin_s1_is_causal_mla, pin_any_s_matches_sdpa, pin_half_gate_group_mean, pin_large_s_limit,
    pin_uniform_softmax, pin_first_step, pin_predownsampling_differs,
    pin_chunked_append_equals_prefill, pin_chunk_continues_live_slot, pin_unabsorbed_matches_sdpa,
    pin_backward_matches_finite_differences, pin_rope_closed_form, pin_rope_relative_position,
]
