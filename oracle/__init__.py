"""CPU oracle (fp64 C + a Python page-pool model).  Test infrastructure only:
imported by tests/, the smoke check and bench.py's CPU-baseline leg, never by
the product package."""
