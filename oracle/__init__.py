"""Plain, slow CPU oracle for mixed-depth reads of one stored int8 weight copy.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP library under
``query_adaptive_mixed_amd/``; the two meet only through the seeded input
generators in ``workloads/``, which hold none of the method's arithmetic.

Every function works in int64 / fp64 and follows the rules in the order the
pages state them; see ``oracle.qam_oracle`` for the citations.
"""

from .qam_oracle import (  # noqa: F401
    LADDER_BITS,
    truncate,
    slice_digits,
    residual_code,
    ceiling,
    profile_stops,
    lens_radius,
    zone_radius,
    field_width,
    level_map,
    mean_bits,
    weight_bytes,
    fit_focus_area,
    layer_scores,
    layer_levels_threshold,
    layer_levels_share,
    qmatvec_ref,
    qmatvec_tolerance,
    escalation_schedule,
    escalation_byte_ratio,
    speculative_decode,
    speculation_byte_ratio,
    uncertainty,
    gate,
    rmsnorm_ref,
    silu_mul_ref,
)
