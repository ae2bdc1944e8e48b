"""Measurement helpers of the benchmark: ceiling probes built from ``measure/csrc/ceilings.hip``."""
