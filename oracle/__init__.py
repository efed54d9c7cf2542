"""fp64 CPU oracle for the KDA chunked forward -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.  The product path never does.
"""
from .kda_oracle import recurrent, chunked, chunk_table, chunk_lengths, sequences  # noqa: F401
