"""Plain fp64 CPU oracle for the SwiGLU MLP training step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with the HIP path and never calls it; the HIP library never calls it either.

See ``oracle.swiglu`` for the functions and the passages each one follows.
"""
from .swiglu import (  # noqa: F401
    sigmoid, silu, dsilu_form1, dsilu_form2, dsilu_form3, dsilu,
    forward, backward, forward_residual, backward_residual, stack_forward, stack_backward, moe_forward, moe_backward, swiglu_bwd_elementwise, swiglu_fwd_elementwise,
    sampled_forward_backward, gemm_flops, algorithmic_bytes,
)
