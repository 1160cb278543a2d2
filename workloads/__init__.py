"""Seeded synthetic workloads shared by the tests, the benchmark and the oracle harness.

This package holds shapes, seeds, random draws and FLOP/byte bookkeeping only.  It contains
none of the attention arithmetic, so both the fp64 oracle and the HIP path can take their
inputs from here without sharing any of the method's code.
"""
from .configs import CONFIGS, Config, get_config, fwd_flops, bwd_flops, visible_pairs
from .gen import make_inputs, make_inputs_like, make_qk_packed, rotary_tables

__all__ = ["CONFIGS", "Config", "get_config", "fwd_flops", "bwd_flops", "visible_pairs",
           "make_inputs", "make_inputs_like", "make_qk_packed", "rotary_tables"]
