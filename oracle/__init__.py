"""CPU oracle (float64 numpy).  TEST INFRASTRUCTURE ONLY: imported by
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg,
never by the product package."""
