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
