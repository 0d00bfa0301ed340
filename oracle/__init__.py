"""fp64 CPU oracle for IKBO target attention (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may use this package; the HIP library neither imports nor calls it.
"""
