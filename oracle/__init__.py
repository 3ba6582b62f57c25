"""CPU oracle for MLA decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything under ``oracle/``.  The HIP product path
never does, and shares no code with it.
"""
from .mla_oracle import (  # noqa: F401
    absorb_out, absorb_q, absorbed_decode, bf16_to_f64, compare, e4m3_to_f64,
    latent_attention, naive_decode, sequence_rows, sparse_decode, visible_rows,
)
