"""fp64 CPU oracle for the attention forward pass, its gradients, and the
plain definition of appending tokens to the paged K/V cache.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg. The product library never imports it, and
it imports nothing from the product library.
"""
from .attention import (attention, attention_head, attention_rows, attention_varlen,
                        decode, kv_head_of)
from .backward import attention_grad, attention_head_grad
from .cache import append as cache_append
from .cache import gather as cache_gather

__all__ = ["attention", "attention_head", "attention_rows", "attention_varlen", "decode",
           "kv_head_of", "cache_append", "cache_gather", "attention_grad", "attention_head_grad"]
