"""CPU fp64 oracle for the batch-invariant kernels. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports, calls or links anything here, and this
package imports nothing from the product: the two share no code.

Every function is the plain mathematical definition of the operation,
written out in float64 with numpy. bf16 inputs arrive as raw uint16 bit
patterns and are decoded exactly (a bf16 value is the top half of an fp32).
See ``oracle/bi_oracle.py`` for the citations.
"""
from .bi_oracle import *  # noqa: F401,F403
from .bi_oracle import __all__  # noqa: F401
