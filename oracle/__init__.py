"""Parity oracle (test infrastructure only): exact fp64 attention on the CPU.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It shares no code with the GPU library.
"""
