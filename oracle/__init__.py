"""fp64 CPU oracle for the attention forward pass.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg. The product library never imports it, and
it imports nothing from the product library.
"""
from .attention import (attention, attention_head, attention_rows, attention_varlen,
                        decode, kv_head_of)

__all__ = ["attention", "attention_head", "attention_rows", "attention_varlen", "decode",
           "kv_head_of"]
