"""MI355X (gfx950) activation-aware dual-codebook 4-bit weight quantizer.

libaaac.so holds every step of the path as hand-written HIP kernels behind the C ABI of
include/aaac.h; `_lib` binds it with ctypes (same names) and `quantize` drives the loop. There is no
CPU fallback: without the built library or a GPU the calls raise.
"""

from ._lib import (  # noqa: F401
    AAACError,
    aaac_assign,
    aaac_assign_batch,
    aaac_assign_refine_batch,
    aaac_awq_prescale,
    aaac_dequant,
    aaac_gemv,
    aaac_gemv_batch,
    aaac_importance,
    aaac_init_quantiles,
    aaac_pack,
    aaac_refine,
    aaac_refine_batch,
    load,
)
from .quantize import (  # noqa: F401
    Layer,
    LayerBuffers,
    Probe,
    QuantizedMatrix,
    Workspaces,
    awq_prescale,
    check_history,
    importance,
    quantize_layer,
    quantize_matrices,
    quantize_matrix,
    quantize_model,
    run_loop,
)
