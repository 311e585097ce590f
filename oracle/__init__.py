"""CPU oracle for the routed-MoE layer -- test infrastructure only.

Importable by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the product path.
"""
