"""CPU oracle for the contextual-sparsity FFN step (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg may import
anything in this directory; the product path never does.
"""
