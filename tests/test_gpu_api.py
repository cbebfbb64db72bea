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
    """The search times its candidates on scratch copies of the pages the
    batch writes: the pool is left bit-identical."""
    T = small.batch.n_tokens
    k0, v0 = small.k.clone(), small.v.clone()
    plan, (ms, n_cands) = small.layer.search(small.pool, small.hb, max_count=3, warmup=1, reps=2, top_k=4,
                                              stream=GH.stream())
    torch.cuda.synchronize()
    assert torch.equal(small.k, k0) and torch.equal(small.v, v0)
    GH.log(f"searched {B.plan_dict(plan)} {ms:.3f} ms over {int(n_cands)} candidates")
    assert 1 <= plan.count <= 3 and sum(list(plan.sizes)[:plan.count]) == T
    assert ms > 0 and n_cands >= 1
    assert B.plan_dict(small.layer.get_plan()) == B.plan_dict(plan)
    rep = small.layer.search_report()
    GH.log("search report: " + "; ".join(f"{d} predicted {p:.3f} measured {m:.3f}{' (calibration)' if c else ''}"
                                         for d, p, m, c in rep))
    assert any(d == B.plan_dict(plan) and not c for d, _, _, c in rep)
    assert all(p > 0 and m > 0 for _, p, m, _ in rep)
    assert min(m for d, _, m, c in rep if d == B.plan_dict(plan) and not c) == pytest.approx(ms)
    # the calibration runs come first; the model meets each of them (its wait is fitted)
    cal = [c for *_, c in rep]
    assert cal == sorted(cal, reverse=True)
    # (a wait only lengthens the prediction, so none falls short of its run)
    assert all(p >= m * 0.998 for _, p, m, c in rep if c)
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
    ms, cfg, splits = B.probe_gemm_bf16_ms(256, 1024, 1024, 0, -1, 0, 256, 3)
    assert ms > 0 and cfg >= 0 and splits >= 1


def test_cu_mask_map_is_measured_and_budgets_land_on_their_cus():
    """Every CU-mask bit maps to a distinct (XCD, CU); a plan-style budget of
    CUs [first, first + count) per XCD runs exactly on the CUs the map names."""
    n = torch.cuda.get_device_properties(0).multi_processor_count
    xcc, cu = B.probe_cu_map(n)
    GH.log(f"CU map: xcc {xcc[:16]}..., cu {cu[:16]}...")
    assert all(0 <= x < 8 for x in xcc) and all(c >= 0 for c in cu)
    pairs = list(zip(xcc, cu))
    assert len(set(pairs)) == n
    assert all(xcc.count(x) == n // 8 for x in range(8))
    per = n // 8
    for first, count in ((0, 16), (16, 16), (0, 24), (24, 8), (per - 4, 4)):
        want = sorted({(xcc[b], cu[b]) for b in range(n) if first <= b // 8 < first + count})
        got = B.probe_budget_cus(first, count)
        assert got == want, (first, count)
        assert len({x for x, _ in got}) == 8
    with pytest.raises(B.NfError) as e:
        B.probe_budget_cus(per - 2, 4)
    assert e.value.status == B.NF_ERR_OUT_OF_RANGE


def test_debug_capture_switches_the_intermediates_off_and_on(small):
    """With capture off nf_layer_intermediate refuses every index; switched on
    again, the next step's q_rot / attn / x1 / act are readable and match the
    oracle."""
    small.layer.debug_capture(False)
    for which in (0, 1, 2, 3):
        with pytest.raises(B.NfError) as e:
            small.layer.intermediate(which)
        assert e.value.status == B.NF_ERR_UNSUPPORTED
    small.layer.debug_capture(True)
    _full_check(small, "capture_on", B.make_plan(1, [small.batch.n_tokens]))
