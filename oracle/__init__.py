"""fp64 CPU oracle for the DoRA module -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP product library.
"""
