"""CPU oracle for the W4A16 verify linear -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it.
"""
from .w4a16_ref import (  # noqa: F401
    CONTRACT_RTOL,
    bf16_bits_to_f64,
    check_contract,
    dequant64,
    linear64,
    linear64_columns,
    linear64_gemm,
    round_to_bf16,
    scales_to_f64,
    unpack_qweight,
    unpack_zeros,
)
from .accept_ref import (  # noqa: F401
    accept_greedy,
    accept_sampled,
    argmax_first,
    decision_margins,
    inverse_cdf,
    softmax64,
)
from .tree_attn_ref import ancestor_masks, attention_weight_mass, tree_attention  # noqa: F401
