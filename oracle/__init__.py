"""fp64 CPU oracle of the hybrid gated-linear + window attention layer.

TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU
baseline); the GPU library never imports this package.
"""
from .oracle import (GATE_LOG, GATE_LOG_HEAD, GATE_LOG_TOKEN, GATE_LOGITS,  # noqa: F401
                     PART_BOTH, PART_GLA, PART_SWA, Oracle, build, compile_source,
                     decode_step, default, layer_fwd, num_threads, set_num_threads)
