"""fp64 CPU oracle for the Sol-Attn forward pass -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The GPU library neither imports nor links it, and it imports nothing from the GPU
library.  ``oracle.oracle`` wraps the C implementation (``sol_oracle.c``); ``oracle.brute`` holds
whole-matrix numpy references used to pin it.
"""
