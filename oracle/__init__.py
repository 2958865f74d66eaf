"""Plain fp64 CPU oracle for gated linear attention (GLA) and gated slot attention (GSA).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU-baseline leg of
the benchmark may import this package.  The product path (the HIP library and its Python
binding) never imports, calls or falls back to it, and this package imports nothing from the
product path.

Everything here evaluates the method in its slowest, most literal form: a step-by-step
recurrence over tokens in float64 NumPy, batched over (batch, head) only.  The chunkwise form
that the GPU kernels use is *not* used here, except in ``gla_chunkwise_fwd``, which exists
solely so the tests can check chunk-size independence of the method against the recurrence.
"""
from .gla_oracle import (  # noqa: F401
    gla_recurrent_fwd, gla_recurrent_bwd, gla_decode_step, gla_chunkwise_fwd,
)
from .gsa_oracle import ACTS as GSA_ACTS, gsa_decode_step, gsa_recurrent_bwd, gsa_recurrent_fwd  # noqa: F401
from .msgla_oracle import msgla_fwd  # noqa: F401
