"""CPU oracle for the DSpark cross-layer context-KV write.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path. It shares no code
with the HIP library.
"""
