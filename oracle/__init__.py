"""CPU oracle for the Llama-style decoder forward pass -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it; the only thing both sides use is the seeded input
generator in ``tdf_synth``.

The oracle is the plain definition of what ``decode(batch)`` computes, in
float64, written to be checked by eye against the pages:

* ``ops``      -- RMSNorm, RoPE, SiLU/SwiGLU, causal grouped-query attention.
* ``model``    -- weights (exact widening of the stored bf16/fp32 values).
* ``context``  -- batch validation and defaults, ubatch split, the reference
                  KV-cell allocator, the layer loop, output-row selection,
                  logits and greedy argmax.

Every function is pinned by tests under ``tests/test_oracle_*.py`` against
closed forms, invariants, brute force and an independent library
implementation of the same architecture (Hugging Face ``LlamaForCausalLM``).
"""
from .ops import rms_norm, rope, rope_angles, silu, swiglu_mlp, attend  # noqa: F401
from .model import OracleModel  # noqa: F401
from .context import OracleContext, DecodeResult  # noqa: F401
