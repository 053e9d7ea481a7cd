"""CPU oracle of the HSTU layer forward (float64) -- test infrastructure only.

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg; never by the
HIP library or its binding.
"""
