"""CPU oracle for the batch-invariant fused linear log-probability forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` use it.

The oracle is written from the RL-Kernel pull-request page
"feat(linear-logp): add batch-invariant fused SM90 operator" (PR #337) and
shares no code, constant table or helper with the HIP library.  Every value is
computed in IEEE binary64 from the exact values of the bf16 / fp32 inputs.

Modules
-------
linear_logp
    ``decode_bf16``               exact bf16 -> float64 decode from the bit pattern
    ``linear_logp``               the plain definition (dgemm + explicit max / exp / log)
    ``vocab_splits``              the V-only contiguous split policy
    ``vocab_splits_throughput``   a split policy from N, V and the compute-unit count
                                  (the throughput scheduling the method replaces)
    ``split_merge_linear_logp``   the method's own steps: per-split online
                                  (max, sum-exp) partials, then the ascending combine
    ``brute_force_linear_logp``   pure-Python ``math.fsum`` version for tiny inputs

det_gemm (RL-Kernel PR #395, "feat(musa): add native deterministic gemm kernel")
    ``det_gemm_fwd``              C = A . B^T, float64
    ``det_gemm_da``               dA = dC . B, float64
    ``det_gemm_db``               dB = dC^T . A ([N, K] weight-gradient layout), float64
    ``abs_product``               sums of |terms|: the fp32 rounding-error scale
    ``brute_force_fwd``           pure-Python ``math.fsum`` forward for tiny inputs

linear_logp_grad (the backward: derivatives of PR #337's forward, in PR #395's layouts)
    ``softmax_grad``              dZ = g_lse P + g_logp (onehot - P), float64
    ``linear_logp_backward``      (grad_hidden, grad_weight, grad_bias), float64
    ``grad_hidden_rows``          grad_hidden for a subset of rows
    ``grad_weight_rows``          (grad_weight, grad_bias) for a subset of vocabulary rows
"""

from .linear_logp import (  # noqa: F401
    decode_bf16,
    to_f64,
    linear_logp,
    vocab_splits,
    vocab_splits_throughput,
    split_merge_linear_logp,
    brute_force_linear_logp,
)
from .det_gemm import (  # noqa: F401
    det_gemm_fwd,
    det_gemm_da,
    det_gemm_db,
    abs_product,
    brute_force_fwd,
)
from .linear_logp_grad import (  # noqa: F401
    softmax_grad,
    linear_logp_backward,
    grad_hidden_rows,
    grad_weight_rows,
)
