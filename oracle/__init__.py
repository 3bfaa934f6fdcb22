"""CPU oracle for the collective primitives (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP path.
"""
