"""CPU oracle for the LLaMA decoder-block forward pass (TEST INFRASTRUCTURE ONLY).

Plain, slow, float64 numpy code that states what the block computes, one step
per function, each citing the page passage it follows.  It shares no code with
the HIP path and imports nothing from it.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
use it; the product path never does.

``oracle.block``  - numpy float64 definition of every step.
``oracle.brute``  - pure-Python loop version of the same definition for tiny
                    shapes (explicit complex rotation, explicit -inf mask,
                    explicit repeat_kv copy), used to cross-check ``block``.

Every function is pinned by a CPU test in ``tests/test_oracle_pins.py``
against what the pages and the mathematics fix (printed values, closed forms,
invariants, special cases).  End-to-end block values have no printed example
on the pages; they are pinned through those properties only.
"""
from . import block, brute  # noqa: F401
