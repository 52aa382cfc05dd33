"""CPU oracle (fp64 numpy) for the GPT training step.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``.  The GPU path does not import it.
"""
