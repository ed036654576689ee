"""CPU oracle for ResidualQuant (float64 numpy).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import anything under ``oracle/``.  The
product path (the HIP library and its Python binding) never does.
"""
from . import formats, projection, residualquant  # noqa: F401
