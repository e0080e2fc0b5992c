"""query_adaptive_mixed_amd -- mixed-depth reads of one stored int8 weight
copy on MI355X.

The compute lives in ``libqam.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/qam.h``); this package is the thin Python binding.
Importing it does not load the library; the first call does, and fails
loudly if the library is missing.
"""

from .api import (  # noqa: F401
    LADDER_BITS,
    Decoder,
    Gate,
    GroupedQmatvec,
    LayerDecides,
    LayerDecidesGroup,
    LayerRule,
    LensRules,
    LensSets,
    PackedMatrix,
    Workspace,
    build_level_map,
    build_level_maps,
    build_rung_map,
    escalation_schedule,
    field_width,
    fit_focus_area,
    last_variant,
    layer_levels,
    map_weight_bytes,
    pack_slices,
    packed_bytes,
    qmatvec,
    qmatvec_noalloc,
    status,
    unpack_codes,
    stack_write,
    stack_info,
    stack_read,
    Verifier,
    argmax_rows,
    speculate,
    workspace_bytes,
)
from ._lib import QamError  # noqa: F401
