"""CPU oracle for the decode step of a Qwen-style decoder stack.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library.

The oracle is the plain definition of what a decode step computes, written
with numpy in float64 by default (float32 on request: the pages' own
references run in fp32).  A KV cache, a split of the key range or a bucket
copy reach this same result exactly up to rounding order, so the oracle is
the definition itself, not any of those algorithms:

* ``decoder``  -- RMSNorm, projections, QK-norm, RoPE, causal GQA attention,
  SwiGLU MLP, final norm and LM head; a per-stream KV cache with bucket
  growth; penalized greedy argmax; the plain LM loop and the two-level
  Talker / Code Predictor frame loop.
* ``brute``    -- a second, loop-only float64 form that recomputes the whole
  sequence from scratch at every step (no cache), for tiny shapes.
* ``codec``    -- the codec decoder's causal dilated and transposed 1-D
  convolutions.
* ``quant``    -- the block-quantized weight formats (int8 and 4-bit codes
  with one fp16 scale per 32 weights): quantize and read back.

Parity status of each function is stated in its docstring.  The whole stack
on random weights has no printed value to compare with: it is pinned by the
closed forms and invariants in the tests (see tests/test_oracle_*.py).
"""

from . import decoder, brute, quant, codec  # noqa: F401
