"""CPU fp64 oracle of the fused-epilogue GEMM -- test infrastructure only.

Imported by tests, the package smoke check and the bench's CPU baseline;
never by the product path.
"""
from .oracle import (EPILOGUES, OracleResult, aux_ld_words, decode, decode_bf16,  # noqa: F401
                     decode_f16, encode, encode_bf16, encode_f16, ffn_block, gelu,
                     gemm_epilogue, pack_mask, round_to_format, unpack_mask)
