"""MI355X-native hot path of Multi-head Temporal Latent Attention (MTLA).

The computation lives in libmtla.so (HIP kernels for gfx950 behind a C ABI,
declared in include/mtla.h); this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    MTLA_BF16, MTLA_F32, OP_BACKWARD, OP_CHUNK, OP_DECODE, OP_MERGE, OP_PREFILL, OP_ROPE,
    OP_UNABSORBED,
    Cache, Dims, GRAD_NAMES, UnabsorbedGrads,
    MtlaError, UnabsorbedWeights, Weights, load_library, make_cache, make_dims,
    make_unabsorbed_weights, make_weights, mtla_append_chunk, mtla_decode_step,
    mtla_gate_content_map, mtla_gate_pos_table, mtla_merge_append, mtla_prefill_strided,
    mtla_prefill_unabsorbed, mtla_prefill_unabsorbed_backward, mtla_rope_inputs,
    mtla_status_string, mtla_workspace_bytes, workspace, dropped_frames)
from .layer import MTLALayer  # noqa: F401
