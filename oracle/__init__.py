"""fp64 CPU oracle of the hybrid gated-linear + window attention layer.

TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU
baseline); the GPU library never imports this package.
"""
from .oracle import (PART_BOTH, PART_GLA, PART_SWA, Oracle, build, compile_source,  # noqa: F401
                     decode_step, default, layer_fwd, num_threads, set_num_threads)
