"""Seeded synthetic binary masks shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and paints masks. It contains none of the
distance-transform arithmetic, so both the GPU path and the CPU oracle can be
fed from it without sharing any of the method's code.

Convention: ``uint8`` masks, ``0`` = background, ``1`` = foreground.
"""

from .masks import (  # noqa: F401
    CONFIGS,
    bernoulli_2d,
    bernoulli_3d,
    disks_2d,
    ellipsoids_3d_batch,
    full_row_2d,
    make_config,
    rng_for,
    single_pixel_2d,
    slab_volume,
)
