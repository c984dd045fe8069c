"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke check.

Holds shapes and input synthesis only; no part of the method's arithmetic."""
from .configs import (DecodeWorkload, PrefillWorkload, FULL, SMALL, TINY_DECODE,
                      LLAMA3_DECODE_32K, TOKEN_HEAD_DECODE_128K, CHUNKED_PREFILL_128K,
                      MLA_TIERED_DECODE_64K, LLAMA3_DECODE_32K_FP8)
from .gen import make_decode_inputs, make_prefill_inputs, make_block_mask
