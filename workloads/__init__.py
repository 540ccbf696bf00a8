"""Seeded synthetic inputs for paged-KV attention.

This package is the only code the oracle and the HIP path both consume.  It
draws sequence lengths, block assignments, slot mappings and Q/K/V values; it
contains none of the attention arithmetic and imports neither side.
"""

from .configs import (Workload, build_workload, make_config, make_spec_verify,  # noqa: F401
                      CONFIG_NAMES, SPEC_VERIFY_NAME)
