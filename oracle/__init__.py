"""CPU fp64 oracle of the GPTQ layer solve.

Test infrastructure only: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.
"""
from .gptq_oracle import *  # noqa: F401,F403
from .gptq_oracle import (NotSPD, Prepared, SweepResult, LayerResult, validate_config,  # noqa: F401
                          hessian_sum, finalize_hessian, hessian, damp, act_order, inverse_factor,
                          prepare, quant_params, quantize_values, quantize_layer, naive_obq, rtn,
                          recon_error, recon_error_from_H, packed_words, pack, unpack, dequantize,
                          dequant_matmul, solve_layer)
from . import block_oracle  # noqa: F401,E402
