"""CPU reference oracle for the MoE layer: test infrastructure only.

Imported by the tests, the package smoke check and the benchmark's
CPU-baseline leg; never by the product path.
"""
