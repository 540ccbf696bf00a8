"""The HIP path driven by the host block manager's serving loop: prefix
reuse, copy-on-write of forked sequences, eviction and preemption under KV
pressure, with every step's appends and split-K decode checked against the
fp64 oracle applying the same operations to its own pool."""

import numpy as np
import pytest

from tests import serving_sim as sim
from tests.gpu_helpers import TOL

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("num_blocks,ps", [(24, 32), (60, 64)])
def test_serving_loop_on_gpu_matches_oracle(num_blocks, ps):
    worst = [0.0]

    def compare(got, ref):
        assert np.all(np.isfinite(got)), "non-finite output"
        err = float(np.max(np.abs(got - ref)))
        worst[0] = max(worst[0], err)
        assert err <= TOL["bf16"], err

    backend = sim.PairedBackend(sim.GpuBackend(num_blocks, ps), sim.OracleBackend(num_blocks),
                                compare)
    mgr, steps, rows, _ = sim.run(backend, num_blocks, seed=11)
    assert rows > 100 and mgr.stats["cow_copies"] > 0 and mgr.stats["prefix_hit_blocks"] > 0
    if num_blocks == 24:
        assert mgr.stats["preemptions"] > 0
    assert all(r == 0 for r in mgr.pool.ref)
