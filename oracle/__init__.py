"""CPU oracle for LLSA (test infrastructure only).

Only the test suite, the package entry point's smoke check and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its Python binding)
never imports or calls it.
"""
