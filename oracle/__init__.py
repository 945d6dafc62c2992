"""CPU oracle of the MoE FFN layer forward -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package; the product path never does.
"""
