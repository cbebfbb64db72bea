"""GPU tests of the boundary's auxiliary calls: the plan search, per-kernel
profiling and the device probes.  The searched plan is also checked against
the oracle (any plan must reproduce the unsplit layer)."""
import numpy as np
import pytest
import torch

from intra_operation_overlap_amd import binding as B
from tests import gpu_harness as GH
from tests.test_gpu_parity import SMALL_BF16, _full_check

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

KINDS = ("rmsnorm_attn", "gemm_qkv", "rope_kv_append", "attention", "gemm_o_residual", "rmsnorm_ffn",
         "gemm_gate_up_swiglu", "gemm_down_residual")


@pytest.fixture(scope="module")
def small():
    return GH.setup(SMALL_BF16)


def test_plan_search_returns_a_valid_plan_that_matches_the_oracle(small):
    T = small.batch.n_tokens
    k0, v0 = small.k.clone(), small.v.clone()
    plan, (ms, n_cands) = small.layer.search(small.pool, small.hb, max_count=3, warmup=1, reps=2, top_k=4,
                                              stream=GH.stream())
    torch.cuda.synchronize()
    small.k.copy_(k0)
    small.v.copy_(v0)
    GH.log(f"searched {B.plan_dict(plan)} {ms:.3f} ms over {int(n_cands)} candidates")
    assert 1 <= plan.count <= 3 and sum(list(plan.sizes)[:plan.count]) == T
    assert ms > 0 and n_cands >= 1
    assert B.plan_dict(small.layer.get_plan()) == B.plan_dict(plan)
    _full_check(small, "searched", plan)


def test_profile_reports_every_kernel_kind_and_filters(small):
    small.layer.set_plan(B.make_plan(1, [small.batch.n_tokens]))
    small.layer.profile_enable(True)
    for _ in range(2):
        small.layer.step(small.pool, small.hb, GH.stream())
    prof = small.layer.profile_read()
    small.layer.profile_enable(False)
    for k in KINDS:
        assert k in prof, (k, sorted(prof))
        launches, ms = prof[k]
        assert launches >= 2 and ms > 0
    small.layer.profile_enable(True, "attention")
    small.layer.step(small.pool, small.hb, GH.stream())
    only = small.layer.profile_read()
    small.layer.profile_enable(False)
    assert set(only) == {"attention"}
    with pytest.raises(B.NfError):
        small.layer.profile_enable(True, "no_such_kind")


def test_device_probes_are_plausible():
    tf = B.probe_mfma_bf16_tflops()
    gbps = B.probe_hbm_read_gbps(1 << 30)
    GH.log(f"bf16 MFMA {tf:.0f} TFLOP/s, HBM read {gbps:.0f} GB/s")
    assert 500 < tf < 3000
    assert 1000 < gbps < 9000
    xcc = B.probe_cu_map(256)
    assert len(set(xcc)) == 8 and all(0 <= x < 8 for x in xcc)
    ms, cfg, splits = B.probe_gemm_bf16_ms(256, 1024, 1024, 0, -1, 0, 256, 3)
    assert ms > 0 and cfg >= 0 and splits >= 1
