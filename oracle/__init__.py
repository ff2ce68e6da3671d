"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .lowbit_oracle import *  # noqa: F401,F403
from .lowbit_oracle import (NonFiniteInput, OracleError, RangeError, dequantize, linear,
                            linear_a8, pack, quantize, quantize_activations_i8,
                            read_code_bitwise, round_to_storage, tolerance, unpack)
