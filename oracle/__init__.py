"""CPU oracle of the latent-MoE layer tail -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the product library never does.
"""
