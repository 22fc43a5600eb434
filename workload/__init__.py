"""Seeded synthetic workloads for the flow-matching action expert.

This package only draws random numbers and lays them out in the storage
formats the library accepts (fp32, bf16 bits, OCP FP8 E4M3 bytes with
per-output-channel scales). It holds none of the method's arithmetic: both the
GPU library and the CPU oracle consume exactly these arrays.
"""
from .configs import AEConfig, CONFIGS, config_by_name  # noqa: F401
from .gen import (  # noqa: F401
    make_weights, make_prefix_kv, make_noise, make_draft, make_verify_case, weight_names,
)
