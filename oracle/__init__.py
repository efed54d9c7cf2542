"""fp64 CPU oracle for the KDA chunked forward -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.  The product path never does.
"""
from .kda_oracle import (  # noqa: F401
    backward_states, bwd_dhu, chunk_lengths, chunk_table, chunked, recurrent, sequences, stage_inputs,
)
