"""Plain fp64 CPU oracle for the per-rank Ulysses attention path.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path never does.
"""
