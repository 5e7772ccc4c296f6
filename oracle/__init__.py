"""fp64 CPU oracle for the KDA forward pass.

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the benchmark's
cpu_baseline leg; never imported by the product package.
"""
