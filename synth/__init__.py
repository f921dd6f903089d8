"""Seeded synthetic inputs and the workload definitions.

This module holds no arithmetic of the method: it only draws random numbers
and names shapes.  Both the oracle-side tests and the device path take
their inputs from here, so the two see identical values.
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import normal, normal_chunked_rows, page_toy_hidden, tensor_seed  # noqa: F401
