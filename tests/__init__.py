"""Tests of the float64 oracle, the C ABI and the HIP kernels against the oracle."""
