"""fp64 CPU oracle of the ReplaySSM decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import, call or execute anything in this package.  The product path
(``attention_decode_mamba_amd``) never imports it, and this package imports
nothing from the product path: the two share no code, no headers and no
helpers.  The only module both sides use is ``synth`` (seeded inputs, no
method arithmetic).

What it computes is the plain definition: the stepwise recurrence in float64
with inputs widened exactly from their stored dtype, plus the integer cursor
policy of the checkpoint + ring representation.  Sources (the pages, by title
and section):

* "ReplaySSM caches SSM inputs instead of state ..." (page 4), section "What
  shipped": the Mamba-2 update S_t = a_t S_{t-1} + v_t k_t^T, the window of
  16 buffered records, flush on a full buffer, speculative drafts appended to
  the buffer and committed by a pointer advance, the output-only verify form.
* The Japanese news article on ReplaySSM (page 1), sections on what the method
  does and on what got faster: flush writes the state once per window;
  rollback is a pointer advance; a low-precision read copy never re-enters
  the recurrence.

Pinned by ``tests/test_oracle_*.py`` (brute-force Kronecker unrolling, exact
rational arithmetic, closed-form special cases, published format tables).  The
only parts without an independent pin are listed as "parity unpinned" in the
modules that hold them.
"""
from .recurrence import widen, mamba2_step, gdn_step, kda_step, step, expand_heads
from .quant import (
    e4m3_encode, e4m3_decode, e2m1_encode, e2m1_decode,
    quantize_fp8_blocks, dequantize_fp8_blocks,
    quantize_mxfp4_blocks, dequantize_mxfp4_blocks,
    read_copy_dequant, read_copy_ambiguity,
)
from .model import ReplayOracle, OracleError
from . import replay_forms

__all__ = [
    "widen", "mamba2_step", "gdn_step", "kda_step", "step", "expand_heads",
    "e4m3_encode", "e4m3_decode", "e2m1_encode", "e2m1_decode",
    "quantize_fp8_blocks", "dequantize_fp8_blocks",
    "quantize_mxfp4_blocks", "dequantize_mxfp4_blocks", "read_copy_dequant",
    "read_copy_ambiguity",
    "ReplayOracle", "OracleError", "replay_forms",
]
