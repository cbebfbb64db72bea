"""The emulated tensor-parallel all-reduce (nf_layer_set_allreduce_emulation)
through the C ABI.  On one GPU the all-reduce of a row-parallel output is the
identity, so a step with the emulation must give the same bits as without it,
in every plan shape and order, on the copy engines and with a copy kernel.
The FFN half reads the all-reduced copy of x1 and the step's output is the
all-reduced copy of the down projection's: a missing wait would leave stale
rows, which a second step on other inputs exposes."""
import numpy as np
import pytest
import torch

from intra_operation_overlap_amd import binding as B
from intra_operation_overlap_amd import workload as W
from tests import gpu_harness as GH
from tests.test_gpu_parity import SMALL_BF16, SMALL_MOE

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _plans(T):
    h = T // 2
    t3 = [T // 3, T // 3, T - 2 * (T // 3)]
    return {
        "k1": B.make_plan(1, [T]),
        "k2_pipelined": B.make_plan(2, [h, T - h], n_streams=2),
        "k2_sequential_one_stream": B.make_plan(2, [h, T - h], order=B.NF_ORDER_SEQUENTIAL),
        "k3_deep": B.make_plan(3, t3, order=B.NF_ORDER_DEEP, n_streams=2),
        "k3_deep_one_stream": B.make_plan(3, t3, order=B.NF_ORDER_DEEP),
        "k2_masked16_waves4": B.make_plan(2, [h, T - h], n_streams=2, gemm_cus_per_xcd=16, attn_waves_per_cu=4),
        "k3_lanes": B.make_plan(3, t3, order=B.NF_ORDER_LANES, n_streams=2),
    }


def _step(S, x):
    S.acts["x"].copy_(x)
    k0, v0 = S.k.clone(), S.v.clone()
    GH.run_step(S)
    out = S.out.clone()
    S.k.copy_(k0)
    S.v.copy_(v0)
    return out


@pytest.mark.parametrize("wl", [SMALL_BF16, SMALL_MOE], ids=["dense", "moe"])
def test_allreduce_emulation_is_bit_identical(wl):
    S = GH.setup(wl)
    T = S.batch.n_tokens
    x_a = S.acts["x"].clone()
    x_b = (torch.randn_like(x_a.float()) * 1.5).to(x_a.dtype)
    for name, plan in _plans(T).items():
        S.layer.set_plan(plan)
        S.layer.set_allreduce_emulation(0)
        ref_a, ref_b = _step(S, x_a), _step(S, x_b)
        for mode in (1, 2):
            GH.log(f"{wl.name} plan={name} emulation mode {mode}")
            S.layer.set_allreduce_emulation(mode, 8)
            got_a, got_b = _step(S, x_a), _step(S, x_b)
            assert torch.equal(got_a, ref_a), (name, mode, "a")
            assert torch.equal(got_b, ref_b), (name, mode, "b")
        S.layer.set_allreduce_emulation(0)
    S.acts["x"].copy_(x_a)


def test_allreduce_emulation_step_matches_oracle():
    """One full oracle check with the emulation on (deep order, two streams)."""
    from tests.test_gpu_parity import _full_check
    S = GH.setup(SMALL_BF16)
    T = S.batch.n_tokens
    S.layer.set_allreduce_emulation(1)
    _full_check(S, "k3_deep_emulated_allreduce",
                B.make_plan(3, [T // 3, T // 3, T - 2 * (T // 3)], order=B.NF_ORDER_DEEP, n_streams=2))


def test_allreduce_emulation_rejects_bad_arguments():
    S = GH.setup(SMALL_BF16)
    for mode, wgs in ((3, 8), (-1, 8), (2, 0)):
        with pytest.raises(B.NfError) as e:
            S.layer.set_allreduce_emulation(mode, wgs)
        assert e.value.status == B.NF_ERR_INVALID_ARG
