"""fp64 CPU oracle of the sparse MoE feed-forward layer: test infrastructure.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import anything here.  It shares no code with the HIP library.
"""
