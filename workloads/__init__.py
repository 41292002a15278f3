"""Seeded synthetic inputs for MLA paged-KV decode.

This package only draws random numbers and lays them out in the shapes the
FlashMLA backend page (``FlashMLABackend.forward_decode`` and
``init_forward_metadata``) hands to its kernels.  It holds none of the
method's arithmetic: no block table, no softmax, no merge.  Both the fp64
oracle (``oracle/``) and the GPU path consume the same bits from here.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    SOFTMAX_SCALE,
    PAGE_SIZE,
    LATENT_DIM,
    V_DIM,
    Workload,
    make_workload,
    workload_seq_lens,
    make_custom,
    poison_unused,
)
