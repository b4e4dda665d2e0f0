"""MI355X (gfx950) group-shared fixed fan-in output layer.

The compute lives in libhaste.so (hand-written HIP kernels behind the C ABI
of include/haste.h); ``sparse_output_layer_amd.haste`` is the thin ctypes
binding with the same entry-point names.
"""
from . import haste  # noqa: F401  (fails loudly if libhaste.so is missing)
from .haste import (  # noqa: F401
    Bce, HasteError, haste_abi_version, haste_head_bwd, haste_head_fwd,
    haste_head_step, haste_tail_bwd, haste_tail_fwd, haste_tail_group_positives,
    haste_tail_layout, haste_tail_step, haste_tail_validate, haste_topk_merge,
)
