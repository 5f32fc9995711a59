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

Everything is computed in fp64 from the exact input values, including the
value ``y`` that decides each lattice code; the decision itself is exact for
that fp64 value (fp64 comparisons, with exact rational arithmetic wherever
two compared costs are too close for fp64 to separate).  Functions that
compute in fp32 (``transform.*_f32``, ``codec.compute_y_f32_stage_order``)
are diagnostics: tests use them to bound the error of an fp32 computation of
y; no acceptance decision rests on them.

Parity status per function is recorded in each module's header.
"""

from . import lattice, transform, codec  # noqa: F401
