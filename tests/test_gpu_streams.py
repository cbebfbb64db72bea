"""CU-masked stream pairs belong to the device: every layer shares them, at
most two stay alive, and the least recently used one is drained and destroyed
when a third budget is needed.  A step holds its pair while it enqueues.

Two layers, stepped from two host threads, cycle through three masked budgets
(so pairs are evicted while the other thread may be enqueuing on one).  Each
step must give the same bits as that layer's step under the same plan run
alone beforehand: the step is deterministic for a given plan, and a step
rewrites the pool slots of its own batch with the same values.
"""
import threading

import pytest
import torch

from intra_operation_overlap_amd import binding as B
from intra_operation_overlap_amd import workload as W
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _workload(seed):
    return W.Workload(f"streams{seed}", W.Shape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=688,
                                                 dtype="bf16", rope_theta=5e5),
                      n_decode=24, ctx_range=(1, 200), prefill=(20, 30), seed=seed)


BUDGETS = {"g20a12": (20, 12), "g16a16": (16, 16), "g24a8": (24, 8)}


def _plans(T):
    half = [T // 2, T - T // 2]
    return {n: B.make_plan(2, half, n_streams=2, gemm_cus_per_xcd=g, attn_cus_per_xcd=a)
            for n, (g, a) in BUDGETS.items()}


def test_shared_masked_pairs_survive_eviction_across_threads():
    setups = [GH.setup(_workload(seed)) for seed in (131, 132)]
    refs = []
    for S in setups:
        ref = {}
        for name, plan in _plans(S.batch.n_tokens).items():
            S.layer.set_plan(plan)
            GH.run_step(S)
            ref[name] = S.out.clone()
        refs.append(ref)
    names = list(BUDGETS)
    errors = []

    def worker(S, ref, offset, n):
        try:
            s = torch.cuda.Stream()
            plans = _plans(S.batch.n_tokens)
            with torch.cuda.stream(s):
                for i in range(n):
                    name = names[(i + offset) % len(names)]
                    S.layer.set_plan(plans[name])
                    S.layer.step(S.pool, S.hb, s.cuda_stream)
                    s.synchronize()
                    if not torch.equal(S.out, ref[name]):
                        errors.append(f"offset {offset} step {i} plan {name}: output differs")
        except Exception as e:          # reported below, in the test's own thread
            errors.append(f"offset {offset}: {e!r}")

    threads = [threading.Thread(target=worker, args=(S, ref, k, 24)) for k, (S, ref) in
               enumerate(zip(setups, refs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    assert not any(t.is_alive() for t in threads), "a stepping thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors[:5]
    GH.log("two threads x 24 steps over three masked budgets: every step bit-identical")
