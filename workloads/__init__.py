"""Seeded synthetic inputs and workload definitions shared by the tests, the
bench and the oracle checks.  Nothing in this package computes any part of the
attention method: it only draws random numbers and rounds them to the storage
dtype."""
from .configs import CONFIGS, Workload, get  # noqa: F401
from .generate import (  # noqa: F401
    TENSORS,
    layer_inputs_host,
    layer_inputs_device,
    group_inputs_device,
    block_inputs_host,
    block_inputs_device,
    heavy_token_positions,
    to_f64,
)
