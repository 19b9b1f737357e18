"""CPU float64 oracle for the diffusion-transformer attention hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, constant
table or helper with the HIP library under
``diffusion_transformer_attention_flash_amd/``; the two meet only through
the seeded inputs of ``workloads/``.

What it computes, each written from the plain definition (numpy, float64):

* ``attention``       -- non-causal multi-head scaled-dot-product attention,
                         output O and natural-log LSE per query row
                         (diffusers "Accelerate inference" guide, section
                         "Scaled dot product attention").
* ``merge``           -- combine of partial (O, LSE) pairs computed over
                         disjoint K/V chunks, as each ring-attention rank
                         does after it has seen every K/V block (diffusers
                         "Context parallelism" guide, sections "Ring
                         Attention" and "Ring Anything Attention").
* ``residual_diff``   -- First Block Cache's relative residual difference,
                         sum|a-b| / sum|b| (ParaAttention guide, section
                         "First Block Cache").
* ``fbcache_step``    -- First Block Cache's decision (float32(diff) <
                         threshold) and cached-residual apply, hidden +=
                         cached rounded once to bfloat16 (same section).
* ``layout``          -- seq/head split and concat with uneven and padded
                         parts, the permutations around Ulysses and Ring
                         Anything exchanges (diffusers "Context parallelism"
                         guide).
* ``e4m3_encode`` / ``e4m3_decode`` / ``quant_per_tensor`` /
  ``attention_fp8``   -- per-tensor dynamic fp8 (OCP E4M3FN) quantisation
                         and attention on the dequantised values with the
                         probabilities quantised before the P.V product
                         (ParaAttention guide, section "fp8 quantization").
* ``quant_rows_pow2`` / ``attention_fp8_rows`` -- the row-wise variant the
                         same section names as more accurate: one
                         power-of-two scale per token for Q and K.
* ``attention_fp8_rows_v`` -- the same with V's per-token scale folded into
                         the probabilities and one power-of-two P scale per
                         (query, block of consecutive keys); the block size
                         is an argument.

Every function is pinned by tests in ``tests/test_oracle_pins.py`` against
mathematics it does not share code with (arbitrary-precision brute force,
closed forms, invariants, a library float8 cast). None is "parity unpinned".
"""

from .attention import attention, merge, softmax_rows
from .residual import fbcache_step, residual_diff
from . import layout
from .fp8 import (E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_round, quant_per_tensor,
                  quant_rows_pow2, attention_fp8_rows, attention_fp8_rows_v, p_block_ids,
                  p_block_exponents, pow2_exponent, quant_p_blocks, attention_fp8)

__all__ = [
    "attention", "merge", "softmax_rows", "residual_diff", "fbcache_step", "layout", "E4M3_MAX",
    "e4m3_decode", "e4m3_encode", "e4m3_round", "quant_per_tensor", "attention_fp8",
    "quant_rows_pow2", "attention_fp8_rows", "attention_fp8_rows_v", "p_block_ids",
    "p_block_exponents", "pow2_exponent", "quant_p_blocks",
]
