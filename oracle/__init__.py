"""CPU oracle for E8 lattice KV-cache quantization.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it.  It shares no code, tables or constants
with the HIP library under ``e8_lattice_vector_amd/``; both sides are written
independently from the same pages:

* NexusQuant blog (nexusquant.hashnode.dev), E8 walkthrough post, sections
  "The E8 Lattice, Briefly", "The Conway-Sloane Nearest-Point Algorithm",
  "Why Per-Group Scaling?", "The Relaxed Parity Discovery",
  "Bit Rate Accounting", "What Makes This Hard in Practice";
* the same blog, post "The E8 lattice quantizes 8 numbers at once",
  section "Handling outliers" (Hadamard rotation);
* nexusquant-kv 0.5.1 README, sections "How it works" and "API reference";
* Nedelkoski et al., "E8 Lattice Key Quantization for Low-Bit KV-Cache
  Compression", Abstract and Tables 2-3 (table-based asymmetric scoring).

Everything that yields a floating-point result is computed in fp64.  Integer
decisions (the lattice code) are taken on the fp32 value ``y`` that the codec
defines, exactly (fp64 comparisons with an exact rational fallback at
near-ties), so that oracle and kernel decide on the same number.

Parity status per function is recorded in each module's header.
"""

from . import lattice, transform, codec  # noqa: F401
