"""CPU float64 oracle (test infrastructure only; never on the product path)."""
from .linattn import (  # noqa: F401
    apply_rows,
    apply_state,
    bf16_bits_to_f64,
    kv_state,
    linattn_fp64,
    linattn_from_inputs,
    phi,
    quadratic_fp64,
    state_fp64,
    state_from_inputs,
    to_f64,
)
from .linattn_bwd import (  # noqa: F401,E402
    backward_head,
    linattn_bwd_fp64,
    linattn_bwd_from_inputs,
    state_grad_head,
)
from .linattn_block_causal import (  # noqa: F401,E402
    block_causal_fp64,
    block_causal_from_inputs,
    masked_quadratic_fp64,
)
from .linattn_feature_maps import (  # noqa: F401,E402
    FEATURE_MAPS,
    linattn_fmap_fp64,
    linattn_fmap_from_inputs,
)
from .linattn_qkv import (  # noqa: F401,E402
    project,
    qkv_attention_fp64,
    qkv_attention_from_inputs,
    round_bf16,
)
