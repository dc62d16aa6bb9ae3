"""fp64 CPU oracle of the paged decode step.

TEST INFRASTRUCTURE ONLY: only the test suite, the package entry file's smoke
check and the benchmark's CPU-baseline leg may import this package.
"""
