"""float64 CPU oracle of the sparse MoE FFN layer (test infrastructure only).

Only tests/, the graft entry point's smoke check and the benchmark's CPU
baseline may import this package; the HIP library never does.
"""
