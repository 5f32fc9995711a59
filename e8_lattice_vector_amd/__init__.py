"""E8 lattice KV-cache quantization for AMD MI355X (gfx950).

The product is the C-ABI library ``libnq.so`` (include/nq.h) built from
``csrc/``; ``nq`` is its thin ctypes binding, ``synth`` the seeded input
generators and ``workloads`` the named cache shapes.
"""

from . import workloads  # noqa: F401
