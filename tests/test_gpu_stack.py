"""Multi-layer step (nf_stack_step) and its HIP graph (nf_stack_graph_create)
through the C ABI.

- Parity: a stack of layers with their own weights and KV pools against the
  fp64 oracle applied layer by layer (each layer's output is the next one's
  input).  Tolerance: normwise 2e-2 for bf16, 1e-4 for fp32, on the last
  layer's output and on every layer's written pool slots.
- The stack equals nf_layer_step applied layer by layer, bit for bit, for
  every plan shape: the nano-batch pipeline across layers reorders launches
  only.
- Graph replays equal the eager step bit for bit, replay after replay, with
  the program's own eager work and synchronisations between replays.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from intra_operation_overlap_amd import binding as B
from intra_operation_overlap_amd import workload as W
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

N_LAYERS = 3

SMALL_BF16 = W.Workload("stack_bf16",
                        W.Shape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=688, dtype="bf16",
                                rope_theta=5e5),
                        n_decode=40, ctx_range=(1, 300), prefill=(37, 45), seed=91)

SMALL_MOE = W.Workload("stack_moe",
                       W.Shape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=384, n_experts=8, top_k=2,
                               dtype="bf16", rope_theta=1e6),
                       n_decode=70, ctx_range=(1, 200), prefill=(10, 30), seed=92)


class Stack:
    """n layers over one batch: layer l has weights and pool drawn with seed
    wl.seed + 1000 l; the batch, its input x and router logits are layer 0's."""

    def __init__(self, wl, n):
        self.wl = wl
        self.batch = W.make_batch(wl)
        self.S = []
        for l in range(n):
            seed = wl.seed + 1000 * l
            S = GH.setup(wl, batch=self.batch, weights=W.make_weights(wl, "cuda", seed=seed))
            k, v = W.make_pool(wl, self.batch.n_pages, "cuda", seed=seed)
            B.kv_pool_import(S.pool, k, v, None, GH.stream())
            torch.cuda.synchronize()
            S.k_plain, S.v_plain = k, v
            self.S.append(S)
        s0 = self.S[0]
        self.x = s0.acts["x"]
        self.out = torch.empty_like(self.x)
        logits = s0.acts.get("router_logits")
        self.logits = logits
        self.hb = B.HostBatch(self.batch, self.x.data_ptr(), self.out.data_ptr(),
                              logits.data_ptr() if logits is not None else None)
        self.layers = [S.layer for S in self.S]
        self.pools = [S.pool for S in self.S]

    def save_pools(self):
        return [(S.k.clone(), S.v.clone()) for S in self.S]

    def restore_pools(self, saved):
        for S, (k, v) in zip(self.S, saved):
            S.k.copy_(k)
            S.v.copy_(v)

    def pools_now(self):
        return [(S.k.clone(), S.v.clone()) for S in self.S]

    def set_plan(self, plan):
        for L in self.layers:
            L.set_plan(plan)


def _plans(T):
    half = T // 2
    return {
        "k1": B.make_plan(1, [T]),
        "k2_two_streams_pipelined": B.make_plan(2, [half, T - half], n_streams=2),
        "k3_two_streams_pipelined": B.make_plan(3, [T // 3, T // 3, T - 2 * (T // 3)], n_streams=2),
        "k2_masked16": B.make_plan(2, [half, T - half], n_streams=2, gemm_cus_per_xcd=16),
        "k2_sequential_one_stream": B.make_plan(2, [half, T - half], order=B.NF_ORDER_SEQUENTIAL),
        "k2_lanes": B.make_plan(2, [half, T - half], order=B.NF_ORDER_LANES, n_streams=2),
    }


def _oracle_chain(st):
    """The oracle layer by layer on the generator's caches (the pools before
    the step); returns the last output and each layer's pools after its step
    (fp64, plain layout)."""
    b = st.batch
    x = GH.f64(st.x)
    after = []
    for S in st.S:
        bd = dict(x=x, req_q_start=b.req_q_start, req_q_len=b.req_q_len, req_pos0=b.req_pos0, pos=b.pos,
                  page_indptr=b.page_indptr, page_indices=np.asarray(b.page_indices, np.int64))
        if st.logits is not None:
            bd["router_logits"] = GH.f64(st.logits)
        res = oracle.layer_step(st.wl.shape.as_dict(), GH.weights_np(S), bd, GH.f64(S.k_plain),
                                GH.f64(S.v_plain))
        after.append((res["k_pool"], res["v_pool"]))
        x = res["out"]
    return x, after


def _written(k_before, k_after_ref, k_gpu):
    """Normwise error over the pool elements the oracle step changed (plain
    layouts)."""
    ref = np.asarray(k_after_ref)
    before = GH.f64(k_before)
    changed = ref != before
    assert changed.any()
    return GH.normwise(GH.f64(k_gpu)[changed], ref[changed])


def _parity(st, plan_name, plan):
    GH.log(f"stack {st.wl.name} x{len(st.layers)} plan={plan_name} T={st.batch.n_tokens}")
    st.set_plan(plan)
    before = st.save_pools()
    B.stack_step(st.layers, st.pools, st.hb, GH.stream())
    torch.cuda.synchronize()
    ref_out, ref_pools = _oracle_chain(st)
    tol = GH.tolerance(st.wl)
    e = GH.normwise(GH.f64(st.out), ref_out)
    GH.log(f"  out error {e:.3e}")
    assert e <= tol, (plan_name, e)
    for l, (S, (kr, vr)) in enumerate(zip(st.S, ref_pools)):
        kg, vg = GH.pool_plain(S)
        ek, ev = _written(S.k_plain, kr, kg), _written(S.v_plain, vr, vg)
        assert ek <= tol and ev <= tol, (plan_name, l, ek, ev)
    st.restore_pools(before)


@pytest.fixture(scope="module")
def bf16_stack():
    return Stack(SMALL_BF16, N_LAYERS)


@pytest.mark.parametrize("plan_name", list(_plans(85)))
def test_stack_bf16_matches_oracle_chain(bf16_stack, plan_name):
    _parity(bf16_stack, plan_name, _plans(bf16_stack.batch.n_tokens)[plan_name])


def test_stack_fp32_matches_oracle_chain():
    st = Stack(W.WORKLOADS["c1"], N_LAYERS)
    for name in ("k1", "k2_two_streams_pipelined"):
        _parity(st, name, _plans(st.batch.n_tokens)[name])


def _chained_steps(st):
    """nf_layer_step layer by layer through temporaries: (last output, pools)."""
    x = st.x
    for l, S in enumerate(st.S):
        out = torch.empty_like(x)
        hb = B.HostBatch(st.batch, x.data_ptr(), out.data_ptr(),
                         st.logits.data_ptr() if st.logits is not None else None)
        S.layer.step(S.pool, hb, GH.stream())
        torch.cuda.synchronize()
        x = out
    return x.clone(), st.pools_now()


@pytest.mark.parametrize("wl", [SMALL_BF16, SMALL_MOE], ids=["dense", "moe"])
def test_stack_equals_layer_by_layer_bit_exact(wl):
    st = Stack(wl, N_LAYERS)
    T = st.batch.n_tokens
    for name, plan in _plans(T).items():
        GH.log(f"stack vs chained steps {wl.name} plan={name}")
        st.set_plan(plan)
        before = st.save_pools()
        B.stack_step(st.layers, st.pools, st.hb, GH.stream())
        torch.cuda.synchronize()
        out_s, pools_s = st.out.clone(), st.pools_now()
        st.restore_pools(before)
        out_c, pools_c = _chained_steps(st)
        st.restore_pools(before)
        assert torch.equal(out_s, out_c), name
        for (ks, vs), (kc, vc) in zip(pools_s, pools_c):
            assert torch.equal(ks, kc) and torch.equal(vs, vc), name


def test_stack_rejects_repeated_layer_and_foreign_pool(bf16_stack):
    st = bf16_stack
    with pytest.raises(B.NfError) as e:
        B.stack_step([st.layers[0], st.layers[0]], [st.pools[0], st.pools[0]], st.hb, GH.stream())
    assert e.value.status == B.NF_ERR_INVALID_ARG
    with pytest.raises(B.NfError) as e:
        B.stack_step(st.layers[:2], [st.pools[1], st.pools[0]], st.hb, GH.stream())
    assert e.value.status == B.NF_ERR_INVALID_ARG


@pytest.mark.parametrize("plan_name", ["k1", "k2_two_streams_pipelined", "k2_lanes"])
def test_graph_replays_equal_eager_step(bf16_stack, plan_name):
    st = bf16_stack
    T = st.batch.n_tokens
    st.set_plan(_plans(T)[plan_name])
    before = st.save_pools()
    B.stack_step(st.layers, st.pools, st.hb, GH.stream())
    torch.cuda.synchronize()
    ref_out, ref_pools = st.out.clone(), st.pools_now()
    st.restore_pools(before)
    GH.log(f"graph {plan_name}: capture")
    g = B.StackGraph(st.layers, st.pools, st.hb, GH.stream())
    torch.cuda.synchronize()
    assert torch.equal(st.out, ref_out)
    a = torch.randn(512, 512, device="cuda")
    for rep in range(3):
        st.out.fill_(float("nan"))
        st.restore_pools(before)
        torch.cuda.synchronize()
        g.launch(GH.stream())
        torch.cuda.synchronize()
        GH.log(f"  replay {rep}")
        assert torch.equal(st.out, ref_out), rep
        for (k, v), (kr, vr) in zip(st.pools_now(), ref_pools):
            assert torch.equal(k, kr) and torch.equal(v, vr), rep
        # the program's own work between replays: an eager step of the same
        # layers, and unrelated device work
        B.stack_step(st.layers, st.pools, st.hb, GH.stream())
        (a @ a).sum().item()
        torch.cuda.synchronize()
        assert torch.equal(st.out, ref_out), rep
    g.close()
    st.restore_pools(before)


def test_graph_refuses_cu_split_plan(bf16_stack):
    st = bf16_stack
    st.set_plan(_plans(st.batch.n_tokens)["k2_masked16"])
    with pytest.raises(B.NfError) as e:
        B.StackGraph(st.layers, st.pools, st.hb, GH.stream())
    assert e.value.status == B.NF_ERR_UNSUPPORTED
    st.set_plan(B.make_plan(1, [st.batch.n_tokens]))
