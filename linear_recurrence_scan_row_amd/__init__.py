"""MI355X-native fused affine scans for reinforcement-learning credit assignment.

The seven estimators of the rl-triton summary (GAE, TD(lambda) returns,
discounted returns, V-Trace, Retrace(lambda), eligibility traces, episodic
prefix sums), the generic affine scan over caller-built coefficients, batches
of those calls, and the fused PPO consumers of the advantages (gae_stats,
ppo_clip_loss), each HIP kernel launches behind the C ABI of include/rlca.h.
Real-valued arrays may be float32, bfloat16 or float16 (fp32 arithmetic).
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
    gae_stats,
    gae_stats_noalloc,
    lib,
    ppo_clip_loss,
    retrace,
    td_lambda,
    vtrace,
)
