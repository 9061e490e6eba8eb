"""CPU oracle for the BitLinear W1.58A8 forward pass (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does."""
from .bitlinear_oracle import *  # noqa: F401,F403
from .bitlinear_oracle import (absmean_gamma, ternary_codes, pack_ternary,  # noqa: F401
                               unpack_ternary, packed_word_index, quant_act,
                               contract, contract_addsub, dequant, round_output,
                               f32_to_bf16_bits, bf16_bits_to_f32, forward,
                               padded_k, padded_n, packed_bytes, EPS_DEFAULT,
                               rmsnorm, mean_square, NORM_EPS_DEFAULT)
