"""fp64 CPU oracle of the sparse MLA forward path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` import it. It is written from the pages'
statement of the problem and shares no code with the HIP library.
"""
from . import e4m3, sparse_mla  # noqa: F401
