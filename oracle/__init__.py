"""CPU oracle for the Graft per-step path.

TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and the benchmark's
CPU-baseline leg import this package.  It shares no code with the HIP path.
"""
