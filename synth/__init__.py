"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

Holds no arithmetic of the method itself (see workloads.py)."""
from .workloads import (WORKLOADS, Workload, GQACase, GQALayer, MLACase, make_block_table,  # noqa: F401
                        make_gqa_case, make_gqa_layer, make_gqa_calibration, make_mla_case,
                        make_mla_calibration, population_basis, bf16_bits, seed_for)
