"""Seeded synthetic inputs for the DSA hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  FP8 quantisation of the indexer's q / k is left to each
consumer: the HIP library quantises on the GPU, the oracle with its own codec.
It is the one module that both sides import.
"""

from .gen import CONFIG_NAMES, Workload, make_config, make_custom  # noqa: F401
