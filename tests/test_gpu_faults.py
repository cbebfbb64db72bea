"""Host-side fault injection (NF_FAULT=after:<n>): inside the next step, the
n-th checked HIP call is not made and reports failure instead.  No device
work is touched -- the call is skipped -- so the GPU never sees a fault.

For every n up to the number of HIP calls a step makes, under an unsplit plan
and under two nano-batches on two CU-masked streams:
- the step returns NF_ERR_HIP and the error text names the injection;
- the next step without injection gives the same output and pool bits as a
  step that never failed (the failed step's enqueued work drained, nothing
  left half-configured: streams, events, staging buffers, workspace).
"""
import os

import pytest
import torch

from intra_operation_overlap_amd import binding as B
from intra_operation_overlap_amd import workload as W
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

SMALL = W.Workload("faults", W.Shape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=688, dtype="bf16",
                                     rope_theta=5e5),
                   n_decode=24, ctx_range=(1, 200), prefill=(20, 30), seed=91)


@pytest.fixture(scope="module")
def S():
    return GH.setup(SMALL)


def _plans(T):
    half = [T // 2, T - T // 2]
    return {"k1": B.make_plan(1, [T]),
            "k2_masked": B.make_plan(2, half, n_streams=2, gemm_cus_per_xcd=20, attn_cus_per_xcd=12),
            "k2_deep": B.make_plan(2, half, order=B.NF_ORDER_DEEP, n_streams=2),
            "k3_lanes": B.make_plan(3, [T // 3, T // 3, T - 2 * (T // 3)], order=B.NF_ORDER_LANES, n_streams=2)}


def _step_bits(S):
    k0, v0 = S.k.clone(), S.v.clone()
    GH.run_step(S)
    torch.cuda.synchronize()
    got = (S.out.clone(), S.k.clone(), S.v.clone())
    S.k.copy_(k0)
    S.v.copy_(v0)
    return got, (k0, v0)


@pytest.mark.parametrize("plan_name", ["k1", "k2_masked", "k2_deep", "k3_lanes"])
def test_every_injected_hip_failure_is_reported_and_recovered(S, plan_name):
    S.layer.set_plan(_plans(S.batch.n_tokens)[plan_name])
    want, _ = _step_bits(S)
    n = 0
    try:
        while True:
            assert n < 400, "the step never ran to the end"
            os.environ["NF_FAULT"] = f"after:{n}"
            k0, v0 = S.k.clone(), S.v.clone()
            torch.cuda.synchronize()
            try:
                GH.run_step(S)
                failed = False
            except B.NfError as e:
                failed = True
                assert e.status == B.NF_ERR_HIP, str(e)
                assert "injected failure" in str(e), str(e)
            del os.environ["NF_FAULT"]
            torch.cuda.synchronize()
            S.k.copy_(k0)
            S.v.copy_(v0)
            if not failed:
                break
            # the next plain step equals one that never followed a failure
            got, _ = _step_bits(S)
            for a, b in zip(want, got):
                assert torch.equal(a, b), (plan_name, n)
            n += 1
    finally:
        os.environ.pop("NF_FAULT", None)
    GH.log(f"{plan_name}: {n} checked HIP calls per step, each failure reported and recovered")
    assert n >= 10
