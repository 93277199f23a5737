"""GPU parity at the full sizes of the decode workloads (2K/32K/256K/1M context),
in the launch configuration the benchmark times: every row is checked against
the CPU oracle (the oracle finishes a 1M-key row in about two seconds)."""
import pytest
import torch

from kv_reuse_amd import workloads as wl
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["decode_32k_b16", "decode_256k_b4_drift", "decode_1m_b1_heavy"])
def test_full_size_decode_workload(name):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w = wl.WORKLOADS[name]
    gh.log(f"[workload] {name}: generating")
    x = wl.generate(w)
    gh.log(f"[workload] {name}: GPU step")
    res = gh.run_step(w, x)
    gh.log(f"[workload] {name}: oracle compare")
    stats = gh.compare_step(w, x, res)
    gh.log(f"[workload] {name}: {stats}")
