"""CPU oracle for the sparse Mixture-of-Experts feed-forward layer (forward and
backward passes, the per-step load-balancing updates, and the ReLU-routing and
zero-computation-expert variants).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
table or helper with the HIP library; the two meet only at the seeded inputs
that ``moe_inputs`` generates.

Every function computes the plain definition from the pages in NumPy float64
on the exact values of its inputs (bfloat16 and float32 inputs convert to
float64 exactly).  It does not imitate the GPU's roundings; the single place
where the oracle works in float32 on purpose is the selection key with a
selection bias, where the expert set is an integer decision that both sides
must take in the same precision.

Pins: every function here is checked by the ``-m "not gpu"`` tests against
closed forms, special cases that reduce to library routines, hand-worked
golden values and brute force on tiny inputs.  No function is "parity
unpinned".
"""

from .moe_oracle import (  # noqa: F401
    UNLIMITED,
    balance_stats,
    capacity,
    dispatch,
    forward,
    gates,
    moe_output,
    router_logits,
    router_z_loss,
    selection_keys,
    selection_keys_on_probs,
    silu,
    swiglu,
    top_k,
)
from .moe_backward import (  # noqa: F401
    backward,
    balance_logit_grad,
    gate_grad,
    gate_logit_grad,
    objective,
    router_linear_backward,
    silu_grad,
    swiglu_backward,
    z_loss_logit_grad,
)
from .moe_balance import (  # noqa: F401
    adaptive_capacity,
    balance_update,
    load_ema,
    selection_bias_update,
)
from .moe_variants import (  # noqa: F401
    backward_bypass,
    backward_relu,
    bypass_gate_grad,
    bypass_kind,
    bypass_output,
    forward_bypass,
    forward_relu,
    objective_bypass,
    objective_relu,
    relu_gate_logit_grad,
    relu_route,
)
