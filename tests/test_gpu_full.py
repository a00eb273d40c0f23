"""GPU parity at the workloads' full sizes (d = 4096 / 8192, |V| = 128256) in
the launch configuration the benchmark times.  Per draft step the oracle
recomputes sampled rows from the GPU's inputs of that step (teacher forcing);
tree structure, accepted lengths and tokens are compared bit for bit on every
request (protocol in tests/parity.py)."""
import pytest

from eagle_feature_space_amd import configs as C

pytestmark = pytest.mark.gpu

# (workload, rows checked per draft step; None = all).  Sampled rows are
# spread evenly over the step, so at 512 rows the 16 rows fall in every
# 64-row band of both 256-row tiles of the tiled kernels.
FULL = [("c1_8b_static", None), ("c2_8b_dynamic", 12), ("c3_8b_eagle3", 8),
        ("c4_70b_dynamic", 16), ("c5_8b_eagle3_steady", 8), ("c6_8b_target", None),
        ("c7_8b_dynamic_steady", 8), ("c8_8b_dynamic_sampled", 8)]


@pytest.mark.parametrize("name,rows", FULL, ids=[f[0] for f in FULL])
def test_full_workload_parity(name, rows):
    from tests.parity import full_check
    print(f"\n[parity-full] {name}", flush=True)
    rep = full_check(C.CONFIGS[name], rows_per_step=rows)
    print(f"[parity-full] {name}: {rep}", flush=True)
