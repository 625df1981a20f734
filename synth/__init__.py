"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package only draws random numbers and lays them out in storage formats
(bf16 bit patterns, OCP e4m3 bytes).  It holds none of the scoring arithmetic:
no normalisation, attention, log-sum-exp or path sums live here.
"""
from .gen import (CONFIGS, Config, make_inputs, make_labels, running_example_labels,
                  zipf_copy_prefix_labels, labels_to_csr, csr_to_labels, config)

__all__ = ["CONFIGS", "Config", "make_inputs", "make_labels", "running_example_labels",
           "zipf_copy_prefix_labels", "labels_to_csr", "csr_to_labels", "config"]
