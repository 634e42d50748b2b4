"""Seeded synthetic inputs shared by the CPU reference and the GPU path.

This package draws random numbers and lays them out in the cache format; it
performs none of the attention arithmetic.
"""
from .gen import (  # noqa: F401
    BF16_NAN,
    CONFIGS,
    ChunkedPrefillCase,
    DecodeCase,
    PrefillCase,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_case,
    make_chunked_prefill_case,
    make_decode_case,
    make_prefill_case,
)
