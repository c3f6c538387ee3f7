"""The seeded input recipe agrees with the oracle's definitions: the rotary
parts of the synthetic inputs are the oracle's decoupled-RoPE inputs of the
same frames, so the library's own RoPE generation and the pre-rotated inputs
the other entry points take describe the same layer."""
import numpy as np

import oracle.mtla as om
import synth
from synth import Dims


def test_synthetic_rotary_inputs_match_oracle_rope():
    dims = Dims(d=64, H=3, d_h=64, r=256, d_hR=32, s=2)
    w = synth.make_weights(dims, 7, "f64", pe_rows=8)
    seq = synth.make_sequence(dims, w, 2, 40, 8, "f64", start=17)
    for b in range(2):
        QR, KR = om.rope_inputs(seq["X"][b], w["W_QR"], w["W_KR"], np.arange(17, 57))
        assert np.max(np.abs(QR - seq["QR"][b])) < 1e-12
        assert np.max(np.abs(KR - seq["KR"][b])) < 1e-12
