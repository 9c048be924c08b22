"""Float64 CPU oracle for paged attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library and never takes
an input from it.

What it computes is the plain definition, written out (FlashAttention and
PagedAttention both reach exactly this result, up to rounding order: the
FlashAttention page's section on FlashAttention being exact rather than
approximate, and the Q&A page's table row saying PagedAttention does not change
the attention mathematics):

* ``pool``      -- its own KV block pool: scatter of written tokens into
                   16-token physical pages, its own fp8 E4M3 quantiser and its
                   own gather through the block table (the paged-loop
                   pseudocode of the "core modules" chapter, section 2.2).
* ``attention`` -- the full score matrix S = scale * Q K^T, causal mask, a
                   two-pass safe softmax, O = P V and LSE = m + ln l, in f64.
* ``fp8_e4m3``  -- the OCP E4M3FN codec from the format's bit definition.
* ``blocks``    -- a plain model of block management: on-demand blocks, shared
                   blocks with reference counts, copy on write before a
                   sequence writes into a shared block (the PagedAttention
                   section of the survey page).
* ``backward``  -- the gradients dQ, dK, dV of the same attention for an
                   upstream dO: the chain rule through the softmax written out
                   with the full probability matrix (the pages describe the
                   backward only as recomputation from kept statistics).

Every function is pinned by the ``-m "not gpu"`` tests in tests/test_oracle.py,
tests/test_blocks.py and tests/test_oracle_backward.py (brute force, closed
forms, finite differences, library special cases and invariants).
"""
from . import fp8_e4m3, pool, attention, blocks, backward  # noqa: F401
from .pool import OraclePool, write_kv, append_kv, copy_blocks, gather_kv  # noqa: F401
from .attention import (attention_two_pass, paged_attention, paged_attention_rows,  # noqa: F401
                        online_softmax_pages, lse_merge)
from .backward import attention_backward_dense, paged_attention_backward  # noqa: F401
