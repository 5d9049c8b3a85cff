"""MI355X-native fused affine scans for reinforcement-learning credit assignment.

The seven estimators of the rl-triton summary (GAE, TD(lambda) returns,
discounted returns, V-Trace, Retrace(lambda), eligibility traces, episodic
prefix sums) and the generic affine scan over caller-built coefficients, each
a HIP kernel launch behind the C ABI of include/rlca.h.
PyTorch supplies device memory and the stream; the computation is entirely in
librlca.so, which must be built (``python -m linear_recurrence_scan_row_amd.build``).
"""
from .rlca import (  # noqa: F401
    BACKWARD,
    FORWARD,
    Batch,
    RESET_AFTER_DONE,
    RESET_ON_START,
    RlcaError,
    affine_scan,
    discounted_returns,
    eligibility_traces,
    episodic_prefix_sum,
    gae,
    lib,
    retrace,
    td_lambda,
    vtrace,
)
