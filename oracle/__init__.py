"""fp64 CPU oracle for multi-scale retention. Test infrastructure only:
imported by the tests, the smoke check and the benchmark's CPU-baseline leg,
never by the product path."""

from .retention import (  # noqa: F401
    backward,
    chunkwise,
    decay_matrix,
    decode_step,
    half_life,
    head_gammas,
    msr_epilogue,
    parallel,
    recurrent,
    rotate_pairs,
    segmented,
)
