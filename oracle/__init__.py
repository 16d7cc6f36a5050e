"""CPU oracle of the sparse-MoE FFN layer forward pass (test infrastructure).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package; the product path never does.
"""
