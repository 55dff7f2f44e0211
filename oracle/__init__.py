"""CPU oracle for the MoE verify-pass layer and the verification round --
TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this
package imports nothing from it.  The arithmetic lives in ``moe_oracle.cpp``
(plain C++, fp64); this module only marshals numpy arrays through ctypes.
"""
from .oracle import (bf16_rne_f64,   # noqa: F401
    F32, BF16, FLAG_BOUNDARY, FLAG_ORDER, Shape, load, bf16_rne, gate_logits,
    route, expert, layer, layer_grouped, dense_mixture, pass_bytes, compact, expert_bytes,
    GREEDY, SAMPLING, sample_index, verify_gate, filter_probs,
)
