"""fp64 CPU oracle for packed-tree SSD verification (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product path never does.
"""
