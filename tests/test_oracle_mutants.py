"""Plant plausible mistakes in the oracle (on the CPU, by monkeypatching) and
require that at least one pin catches each of them."""
import numpy as np
import pytest

import oracle.mtla as om
import pins


def _mut_group_final_zero(mp):
    mp.setattr(om, "is_group_final", lambda n, s: n % s == 0)

    def mask(T, s):
        m = np.arange(T)[:, None]
        n = np.arange(T)[None, :]
        return (n == m) | ((n < m) & (n % s == 0))
    mp.setattr(om, "mask_matrix", mask)

    def cache(Cp, KR, s):
        T = Cp.shape[0]
        e = np.array([min(s * j, T - 1) for j in range(om.n_slots(T, s))], dtype=np.int64)
        return Cp[e].copy(), KR[e].copy(), e
    mp.setattr(om, "compressed_cache", cache)


def _mut_drop_rope(mp):
    orig = om.prefill

    def prefill(X, QR, KR, W, s, scale):
        return orig(X, QR * 0.0, KR, W, s, scale)
    mp.setattr(om, "prefill", prefill)


def _mut_transpose_whc(mp):
    mp.setattr(om, "merge_weight",
               lambda c, j, W_hc, b_hc, P: om.sigmoid((W_hc.T @ c + b_hc) * P[j]))


def _mut_position_by_frame(mp):
    def fu(x_i, i, W, s):
        c = om.latent(x_i, W["W_dkv"])
        w = om.merge_weight(c, min(i, W["P"].shape[0] - 1), W["W_hc"], W["b_hc"], W["P"])
        return c, w, w * c
    mp.setattr(om, "frame_update", fu)


def _mut_additive_gate(mp):
    mp.setattr(om, "merge_weight",
               lambda c, j, W_hc, b_hc, P: om.sigmoid((W_hc @ c + b_hc) + P[j]))


def _mut_no_reset(mp):
    def ma(lat, rk, t, x_t, kr_t, W, s):
        _, _, u = om.frame_update(x_t, t, W, s)
        j = om.slot_of(t, s)
        lat[j] = lat[j] + u          # accumulates even when t opens a new group
        rk[j] = kr_t
        return j
    mp.setattr(om, "merge_append", ma)


def _mut_rope_key_first_frame(mp):
    orig = om.merge_append

    def ma(lat, rk, t, x_t, kr_t, W, s):
        keep = rk[om.slot_of(t, s)].copy()
        j = orig(lat, rk, t, x_t, kr_t, W, s)
        if t % s != 0:
            rk[j] = keep
        return j
    mp.setattr(om, "merge_append", ma)


def _mut_plain_prefix_sum(mp):
    mp.setattr(om, "intermediate_states", lambda U, s: np.cumsum(U, axis=0))


def _mut_bvo_transposed(mp):
    mp.setattr(om, "output_projection", lambda O, Bvo: np.einsum("...hr,rhd->...d", O, Bvo))


def _mut_a_transposed(mp):
    # reads A[h] as if it were stored [d, r] (shape-compatible since d == r)
    mp.setattr(om, "absorbed_queries", lambda X, A: np.einsum("td,hdr->thr", X, A))


def _mut_latent_transposed(mp):
    mp.setattr(om, "latent", lambda x, W: W.T @ x)


def _mut_scale_with_rope_width(mp):
    orig = om.prefill

    def prefill(X, QR, KR, W, s, scale):
        return orig(X, QR, KR, W, s, 1.0 / np.sqrt(1.0 / scale ** 2 + KR.shape[1]))
    mp.setattr(om, "prefill", prefill)


def _mut_sigmoid_sign(mp):
    mp.setattr(om, "sigmoid", lambda x: 1.0 / (1.0 + np.exp(x)))


def _mut_decode_excludes_newest(mp):
    def ds(lat, rk, t, x_t, qr_t, kr_t, W, s, scale):
        j = om.merge_append(lat, rk, t, x_t, kr_t, W, s)
        qt = W["A"] @ x_t
        n = j + 1 if (t % s == s - 1 or j == 0) else j
        o = om.attend_cache(qt, qr_t, lat[:n], rk[:n], scale)
        return om.output_projection(o, W["Bvo"]), o
    mp.setattr(om, "decode_step", ds)


def _mut_chunk_opens_fresh(mp):
    orig = om.merge_chunk

    def mc(lat, rk, t0, Xc, KRc, W, s):
        if Xc.shape[0] and t0 % s:
            lat[om.slot_of(t0, s)] = 0.0     # forgets the live partial slot
        return orig(lat, rk, t0, Xc, KRc, W, s)
    mp.setattr(om, "merge_chunk", mc)


def _mut_chunk_relative_positions(mp):
    def mc(lat, rk, t0, Xc, KRc, W, s):
        Cp = np.empty((Xc.shape[0], lat.shape[1]))
        for i in range(Xc.shape[0]):
            j = om.merge_append(lat, rk, i, Xc[i], KRc[i], W, s) + om.slot_of(t0, s)
            Cp[i] = lat[j]
        return Cp
    mp.setattr(om, "merge_chunk", mc)


def _mut_chunk_state_before_merge(mp):
    def mc(lat, rk, t0, Xc, KRc, W, s):
        Cp = np.empty((Xc.shape[0], lat.shape[1]))
        for i in range(Xc.shape[0]):
            j = om.slot_of(t0 + i, s)
            Cp[i] = lat[j] if (t0 + i) % s else 0.0
            om.merge_append(lat, rk, t0 + i, Xc[i], KRc[i], W, s)
        return Cp
    mp.setattr(om, "merge_chunk", mc)


def _mut_unabsorbed_values_from_keys(mp):
    orig = om.mha_unabsorbed

    def mha(X, QR, KR, Cp, W_Q, W_K, W_V, W_O, s, scale):
        return orig(X, QR, KR, Cp, W_Q, W_K, W_K, W_O, s, scale)
    mp.setattr(om, "mha_unabsorbed", mha)


def _mut_unabsorbed_causal_mask(mp):
    orig = om.mha_unabsorbed

    def mha(X, QR, KR, Cp, W_Q, W_K, W_V, W_O, s, scale):
        return orig(X, QR, KR, Cp, W_Q, W_K, W_V, W_O, 1, scale)   # plain causal mask
    mp.setattr(om, "mha_unabsorbed", mha)


def _edit_backward(mp, old, new):
    """Replace one expression in a copy of the oracle's backward."""
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(om.prefill_unabsorbed_backward))
    assert old in src, old
    ns = dict(vars(om))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    mp.setattr(om, "prefill_unabsorbed_backward", ns["prefill_unabsorbed_backward"])


def _mut_bwd_no_softmax_correction(mp):
    _edit_backward(mp, "(dPm - np.sum(dPm * Pm, axis=1, keepdims=True))", "dPm")


def _mut_bwd_scan_not_accumulated(mp):
    _edit_backward(mp, "dU[i] = dCp[i] + dU[i + 1]", "dU[i] = dCp[i]")


def _mut_bwd_no_sigmoid_derivative(mp):
    _edit_backward(mp, "dgate = dw * w * (1.0 - w)", "dgate = dw * w")


def _mut_bwd_transposed_whc(mp):
    _edit_backward(mp, 'W["W_hc"].T @ da', 'W["W_hc"] @ da')


def _mut_bwd_rope_keys_one_head(mp):
    _edit_backward(mp, "dKR += dZ.T @ QR[:, h, :]", "dKR = dZ.T @ QR[:, h, :]")


def _mut_bwd_missing_scale(mp):
    _edit_backward(mp, "keepdims=True)) * scale", "keepdims=True))")


def _edit_rope(mp, old, new):
    import inspect
    import textwrap
    src = textwrap.dedent(inspect.getsource(om.rope_rotate))
    assert old in src, old
    ns = dict(vars(om))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    mp.setattr(om, "rope_rotate", ns["rope_rotate"])


def _mut_rope_sign(mp):
    _edit_rope(mp, "v[..., 0::2] * cs - v[..., 1::2] * sn", "v[..., 0::2] * cs + v[..., 1::2] * sn")


def _mut_rope_exponent(mp):
    _edit_rope(mp, "base ** (-2.0 * np.arange(w // 2) / w)", "base ** (-1.0 * np.arange(w // 2) / w)")


def _mut_rope_half_split(mp):
    def rot(v, pos, base=10000.0):
        w = v.shape[-1]
        theta = base ** (-2.0 * np.arange(w // 2) / w)
        ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
        a, b = v[..., : w // 2], v[..., w // 2:]
        return np.concatenate([a * np.cos(ang) - b * np.sin(ang),
                               a * np.sin(ang) + b * np.cos(ang)], axis=-1)
    mp.setattr(om, "rope_rotate", rot)


MUTANTS = [
    _mut_group_final_zero, _mut_drop_rope, _mut_transpose_whc, _mut_position_by_frame,
    _mut_additive_gate, _mut_no_reset, _mut_rope_key_first_frame, _mut_plain_prefix_sum,
    _mut_bvo_transposed, _mut_a_transposed, _mut_latent_transposed,
    _mut_scale_with_rope_width, _mut_sigmoid_sign, _mut_decode_excludes_newest,
    _mut_chunk_opens_fresh, _mut_chunk_relative_positions, _mut_chunk_state_before_merge,
    _mut_unabsorbed_values_from_keys, _mut_unabsorbed_causal_mask,
    _mut_bwd_no_softmax_correction, _mut_bwd_scan_not_accumulated, _mut_bwd_no_sigmoid_derivative,
    _mut_bwd_transposed_whc, _mut_bwd_rope_keys_one_head, _mut_bwd_missing_scale,
    _mut_rope_sign, _mut_rope_exponent, _mut_rope_half_split,
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_some_pin_catches(mutant, monkeypatch):
    mutant(monkeypatch)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except Exception as e:  # noqa: BLE001 - a crash also counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"{mutant.__name__} passed every pin"
