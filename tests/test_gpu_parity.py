"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances (normwise max relative error, per tensor): 1e-4 for fp32 layers,
2e-2 for bf16 layers; index handling (which pool slots change, which key a
one-hot query selects, MoE routing and permutation) must be bit-exact."""
import dataclasses

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


def _plans_for(T):
    half = T // 2
    return {
        "k1_one_stream": B.make_plan(1, [T]),
        "k2_two_streams_unmasked": B.make_plan(2, [half, T - half], n_streams=2),
        "k2_masked16": B.make_plan(2, [half, T - half], n_streams=2, gemm_cus_per_xcd=16),
        "k3_sequential_masked8": B.make_plan(3, [T // 3, T // 3, T - 2 * (T // 3)], order=B.NF_ORDER_SEQUENTIAL,
                                             n_streams=2, gemm_cus_per_xcd=8),
        "k4_masked24": B.make_plan(4, [T // 4] * 3 + [T - 3 * (T // 4)], n_streams=2, gemm_cus_per_xcd=24),
        "k3_deep_two_streams": B.make_plan(3, [T // 3, T // 3, T - 2 * (T // 3)], order=B.NF_ORDER_DEEP,
                                           n_streams=2),
        # persistent one-wave attention grids (split page ranges + merge)
        "k1_attn_waves1": B.make_plan(1, [T], n_streams=2, attn_waves_per_cu=1),
        "k2_attn_waves4": B.make_plan(2, [half, T - half], n_streams=2, attn_waves_per_cu=4),
        "k2_attn_waves1_masked16": B.make_plan(2, [half, T - half], n_streams=2, gemm_cus_per_xcd=16,
                                               attn_waves_per_cu=1),
        # grids far smaller than the work list: every workgroup loops
        "k2_attn_waves4_on2cus": B.make_plan(2, [half, T - half], n_streams=2, attn_cus_per_xcd=2,
                                             attn_waves_per_cu=4),
        "k1_attn_waves2_on2cus": B.make_plan(1, [T], n_streams=2, attn_cus_per_xcd=2, attn_waves_per_cu=2),
        # lanes: nano-batch j on stream j % 2, each lane's GEMMs tiled for half
        # the chip (own split-K partials), under CU budgets, with a bounded
        # attention grid, and with three nano-batches (two share lane 0)
        "k2_lanes": B.make_plan(2, [half, T - half], order=B.NF_ORDER_LANES, n_streams=2),
        "k2_lanes_masked16": B.make_plan(2, [half, T - half], order=B.NF_ORDER_LANES, n_streams=2,
                                         gemm_cus_per_xcd=16, attn_cus_per_xcd=16),
        "k2_lanes_attn_waves8": B.make_plan(2, [half, T - half], order=B.NF_ORDER_LANES, n_streams=2,
                                            attn_waves_per_cu=8),
        "k3_lanes": B.make_plan(3, [T // 3, T // 3, T - 2 * (T // 3)], order=B.NF_ORDER_LANES, n_streams=2),
        "k4_lanes": B.make_plan(4, [T // 4] * 3 + [T - 3 * (T // 4)], order=B.NF_ORDER_LANES, n_streams=2),
    }


def _check(S, where, requests=None, w_np=None):
    """One step under the layer's plan, then every compared tensor against the
    oracle on `requests` (all by default) and the pool sentinel; the pool's
    own buffers are restored afterwards."""
    k0, v0 = S.k.clone(), S.v.clone()
    GH.run_step(S)
    k_after, v_after = GH.pool_plain(S)
    GH.check_sentinel(S, k_after, v_after)
    reqs = list(range(S.batch.n_requests)) if requests is None else requests
    GH.log(f"  oracle on {len(reqs)} requests")
    res, rows, pages = GH.oracle_subset(S, reqs, w_np)
    errs = GH.compare_rows(S, res, rows, pages, reqs, k_after, v_after)
    GH.log(f"  errors {errs}")
    GH.assert_errors(errs, GH.tolerance(S.wl), where)
    S.k.copy_(k0)
    S.v.copy_(v0)
    return res, rows, errs


def _full_check(S, plan_name, plan):
    GH.log(f"step {S.wl.name} plan={plan_name} T={S.batch.n_tokens}")
    S.layer.set_plan(plan)
    return _check(S, plan_name)[2]


# ---------------------------------------------------------------- tiny fp32 layer

@pytest.fixture(scope="module")
def c1():
    return GH.setup(W.WORKLOADS["c1"])


@pytest.mark.parametrize("plan_name", [p for p in _plans_for(16) if "attn_waves" not in p])
def test_c1_fp32_full_parity(c1, plan_name):
    _full_check(c1, plan_name, _plans_for(c1.batch.n_tokens)[plan_name])


# ---------------------------------------------------------------- small bf16 layer

SMALL_BF16 = W.Workload("small_bf16",
                        W.Shape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=688, dtype="bf16",
                                rope_theta=5e5),
                        n_decode=40, ctx_range=(1, 300), prefill=(37, 45), seed=77)


@pytest.fixture(scope="module")
def small():
    return GH.setup(SMALL_BF16)


@pytest.mark.parametrize("plan_name", list(_plans_for(85)))
def test_small_bf16_full_parity(small, plan_name):
    _full_check(small, plan_name, _plans_for(small.batch.n_tokens)[plan_name])


def test_small_bf16_prefill_from_zero_and_g8():
    wl = W.Workload("g8", W.Shape(hidden=1024, n_q_heads=8, n_kv_heads=1, head_dim=128, ffn=512, dtype="bf16",
                                  rope_theta=1e4),
                    n_decode=9, ctx_range=(100, 200), prefill=(0, 70), seed=78)
    S = GH.setup(wl)
    T = S.batch.n_tokens
    _full_check(S, "k1", B.make_plan(1, [T]))
    _full_check(S, "k2_split_prefill", B.make_plan(2, [40, T - 40], n_streams=2, gemm_cus_per_xcd=16))
    _full_check(S, "k2_split_prefill_attn_waves4", B.make_plan(2, [40, T - 40], n_streams=2, attn_waves_per_cu=4))
    _full_check(S, "k1_attn_waves1", B.make_plan(1, [T], n_streams=2, attn_waves_per_cu=1))


# Seeded shape sweep: GQA groups 1, 2 and 8, hidden not a multiple of 64 (the
# GEMMs' non-pipelined configurations), ragged FFN widths, prefill chunks from
# position 0 and mid-context, a decode-only batch with long contexts, contexts
# of 6K-16K tokens, and an fp32 layer with head_dim 64 (the generic attention
# kernel).
SWEEP = {
    "g1_prefill_from_0": W.Workload("sw_g1", W.Shape(hidden=256, n_q_heads=8, n_kv_heads=8, head_dim=128, ffn=344,
                                                     dtype="bf16", rope_theta=1e4),
                                    n_decode=17, ctx_range=(1, 64), prefill=(0, 33), seed=101),
    "g2_hidden520": W.Workload("sw_g2", W.Shape(hidden=520, n_q_heads=8, n_kv_heads=4, head_dim=128, ffn=720,
                                                dtype="bf16", rope_theta=5e5),
                               n_decode=33, ctx_range=(20, 400), prefill=(50, 20), seed=102),
    "g8_long_decode": W.Workload("sw_g8", W.Shape(hidden=1024, n_q_heads=16, n_kv_heads=2, head_dim=128, ffn=1000,
                                                  dtype="bf16", rope_theta=1e6),
                                 n_decode=50, ctx_range=(1, 700), prefill=None, seed=103),
    # contexts of 6K-16K tokens: long items split into page ranges whose
    # partials several merge items combine, and a prefill chunk deep in context
    "g4_long_context": W.Workload("sw_long", W.Shape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=688,
                                                     dtype="bf16", rope_theta=1e6),
                                  n_decode=5, ctx_range=(6000, 16000), prefill=(9000, 40), seed=105),
    "fp32_d64": W.Workload("sw_f32", W.Shape(hidden=384, n_q_heads=6, n_kv_heads=2, head_dim=64, ffn=520,
                                             dtype="f32", rope_theta=1e4),
                           n_decode=12, ctx_range=(1, 150), prefill=(10, 27), seed=104),
}


@pytest.mark.parametrize("case", list(SWEEP))
def test_shape_sweep_parity(case):
    S = GH.setup(SWEEP[case])
    T = S.batch.n_tokens
    _full_check(S, f"{case} k1", B.make_plan(1, [T]))
    _full_check(S, f"{case} k2", B.make_plan(2, [T // 2, T - T // 2], n_streams=2))
    if S.wl.shape.dtype == "bf16":      # the one-wave kernel: bf16, head_dim 128
        _full_check(S, f"{case} k2 attn_waves4", B.make_plan(2, [T // 2, T - T // 2], n_streams=2,
                                                              attn_waves_per_cu=4))
        _full_check(S, f"{case} k1 attn_waves1", B.make_plan(1, [T], n_streams=2, attn_waves_per_cu=1))


def test_degenerate_batches_parity():
    """A single token at position 0 (one key, one page slot); decode tokens on
    the last slot of a page and the first slot of the next; a prefill chunk of
    exactly one page from position 0."""
    shape = W.Shape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=688, dtype="bf16", rope_theta=1e4)
    one = GH.setup(W.Workload("one_tok", shape, n_decode=1, ctx_range=(0, 0), prefill=None, seed=111))
    _full_check(one, "one token k1", B.make_plan(1, [1]))
    _full_check(one, "one token two streams attn_waves1", B.make_plan(1, [1], n_streams=2, attn_waves_per_cu=1))
    edges = GH.setup(W.Workload("page_edges", shape, n_decode=6, ctx_range=(15, 16), prefill=(0, 16), seed=112))
    T = edges.batch.n_tokens
    assert set(edges.batch.pos[:6].tolist()) <= {15, 16} and edges.batch.req_q_len[-1] == 16
    _full_check(edges, "page edges k1", B.make_plan(1, [T]))
    _full_check(edges, "page edges k2", B.make_plan(2, [6, T - 6], n_streams=2))
    _full_check(edges, "page edges k2 attn_waves4", B.make_plan(2, [6, T - 6], n_streams=2, attn_waves_per_cu=4))


def test_split_k_small_batch_parity():
    """Decode-sized nano-batches take the split-K GEMM path (fused reduction)."""
    wl = W.Workload("splitk", W.Shape(hidden=2048, n_q_heads=8, n_kv_heads=4, head_dim=128, ffn=1536,
                                      dtype="bf16", rope_theta=5e5),
                    n_decode=20, ctx_range=(5, 90), prefill=None, seed=80)
    S = GH.setup(wl)
    _full_check(S, "k1", B.make_plan(1, [20]))
    _full_check(S, "k2_masked", B.make_plan(2, [7, 13], n_streams=2, gemm_cus_per_xcd=20))


@pytest.mark.parametrize("wl_name", ["small_bf16", "splitk"])
def test_attention_norm_kernel_and_fold_both_match_the_oracle(wl_name, monkeypatch):
    """bf16 layers fold the attention RMSNorm into the QKV projection (gain in
    the weights, 1 / RMS applied in RoPE/append, also on the split-K
    partials); NF_NORM_FOLD=0 keeps the norm as a kernel of its own.  Both
    layers match the oracle, and each other within the bf16 tolerance."""
    wl = SMALL_BF16 if wl_name == "small_bf16" else W.Workload(
        "splitk_nofold", W.Shape(hidden=2048, n_q_heads=8, n_kv_heads=4, head_dim=128, ffn=1536, dtype="bf16",
                                 rope_theta=5e5), n_decode=20, ctx_range=(5, 90), prefill=None, seed=81)
    outs = []
    for fold in ("0", "1"):
        monkeypatch.setenv("NF_NORM_FOLD", fold)
        S = GH.setup(wl)
        T = S.batch.n_tokens
        _full_check(S, f"fold={fold} k1", B.make_plan(1, [T]))
        outs.append(S.out.clone())
        _full_check(S, f"fold={fold} k2", B.make_plan(2, [T // 2, T - T // 2], n_streams=2))
    e = GH.normwise(GH.f64(outs[1]), GH.f64(outs[0]))
    GH.log(f"  folded vs unfolded {e:.2e}")
    assert e <= GH.tolerance(wl)


def test_plan_invariance_bit_exact(small):
    """Same nano-batch sizes and the same CU budget give bit-identical outputs
    whatever the stream count and operation order."""
    T = small.batch.n_tokens
    outs = []
    for plan in (B.make_plan(2, [30, T - 30]),
                 B.make_plan(2, [30, T - 30], order=B.NF_ORDER_SEQUENTIAL),
                 B.make_plan(2, [30, T - 30], n_streams=2),
                 B.make_plan(2, [30, T - 30], order=B.NF_ORDER_DEEP, n_streams=2),
                 B.make_plan(2, [30, T - 30], order=B.NF_ORDER_DEEP)):
        small.layer.set_plan(plan)
        k0, v0 = small.k.clone(), small.v.clone()
        GH.run_step(small)
        outs.append((small.out.clone(), small.k.clone(), small.v.clone()))
        small.k.copy_(k0)
        small.v.copy_(v0)
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)


def test_caller_stream_kind_does_not_change_results(small):
    """Two-stream plans give the same bits on the null stream (whose implicit
    synchronisation with the blocking CU-masked streams the executor steps
    around) and on a non-blocking caller stream."""
    T = small.batch.n_tokens
    half = [T // 2, T - T // 2]
    side = torch.cuda.Stream()
    for plan in (B.make_plan(2, half, n_streams=2),
                 B.make_plan(2, half, n_streams=2, attn_cus_per_xcd=24),
                 B.make_plan(2, half, n_streams=2, gemm_cus_per_xcd=16, attn_cus_per_xcd=16),
                 B.make_plan(2, half, order=B.NF_ORDER_DEEP, n_streams=2, gemm_cus_per_xcd=20),
                 B.make_plan(2, half, order=B.NF_ORDER_LANES, n_streams=2),
                 B.make_plan(3, [28, 28, T - 56], order=B.NF_ORDER_LANES, n_streams=2, gemm_cus_per_xcd=16,
                             attn_cus_per_xcd=16)):
        small.layer.set_plan(plan)
        outs = []
        for s in (None, side):
            k0, v0 = small.k.clone(), small.v.clone()
            torch.cuda.synchronize()
            if s is None:
                GH.run_step(small)
            else:
                with torch.cuda.stream(s):
                    GH.run_step(small)
            torch.cuda.synchronize()
            outs.append((small.out.clone(), small.k.clone(), small.v.clone()))
            small.k.copy_(k0)
            small.v.copy_(v0)
        for a, b in zip(*outs):
            assert torch.equal(a, b), B.plan_dict(plan)


def test_repeated_steps_are_idempotent(small):
    small.layer.set_plan(B.make_plan(2, [42, small.batch.n_tokens - 42], n_streams=2, gemm_cus_per_xcd=12))
    GH.run_step(small)
    a = (small.out.clone(), small.k.clone())
    for _ in range(3):
        GH.run_step(small)
    assert torch.equal(a[0], small.out) and torch.equal(a[1], small.k)


def test_empty_batch_is_a_no_op(small):
    empty = W.Batch(0, np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32),
                    np.zeros(1, np.int32), np.zeros(0, np.int32), small.batch.n_pages)
    hb = B.HostBatch(empty, small.acts["x"].data_ptr(), small.out.data_ptr())
    small.layer.set_plan(B.make_plan(1, [0]))
    k0 = small.k.clone()
    small.layer.step(small.pool, hb, GH.stream())
    torch.cuda.synchronize()
    assert torch.equal(k0, small.k)


def test_invalid_batch_launches_nothing(small):
    bad = dataclasses.replace(small.batch, page_indices=small.batch.page_indices.copy())
    bad.page_indices[0] = small.batch.n_pages + 5
    hb = B.HostBatch(bad, small.acts["x"].data_ptr(), small.out.data_ptr())
    small.out.fill_(7.0)
    with pytest.raises(B.NfError) as e:
        small.layer.step(small.pool, hb, GH.stream())
    torch.cuda.synchronize()
    assert e.value.status == B.NF_ERR_OUT_OF_RANGE
    assert bool((small.out == 7.0).all())


# ---------------------------------------------------------------- one-hot probe

@pytest.mark.parametrize("wl_name", ["c1", "small_bf16"])
def test_one_hot_attention_selects_exact_key(wl_name):
    """Prior keys crafted so one chosen position's score beats every other by
    >= 100: attention must return that position's value bit-exactly, which
    pins the page-table lookup and the slot arithmetic.  The keys are written
    into the plain paged cache and imported into the pool."""
    wl = W.WORKLOADS["c1"] if wl_name == "c1" else SMALL_BF16
    S = GH.setup(wl)
    b = S.batch
    S.layer.set_plan(B.make_plan(1, [b.n_tokens]))
    GH.run_step(S)
    s = wl.shape
    dt = torch.float32 if s.dtype == "f32" else torch.bfloat16
    q = GH.intermediate(S, 0, b.n_tokens, s.n_q_heads * s.head_dim, dt).float().view(b.n_tokens, s.n_q_heads, s.head_dim)
    rng = np.random.Generator(np.random.PCG64(5))
    G = s.n_q_heads // s.n_kv_heads
    kp = S.k_plain.clone()
    chosen = {}
    for r in range(b.n_requests):
        if b.req_q_len[r] != 1 or b.req_pos0[r] < 1:
            continue
        t = b.req_q_start[r]
        p0 = int(b.req_pos0[r])
        j = int(rng.integers(0, p0))          # a cached position
        pages = torch.as_tensor(b.page_indices[b.page_indptr[r]:b.page_indptr[r + 1]].astype(np.int64), device="cuda")
        slots = torch.arange(p0, device="cuda")
        for kh in range(s.n_kv_heads):
            # zero every cached key of this request ...
            kp[pages[slots // 16], kh, slots % 16] = 0
            # ... then point key j along the group's first query head: score 400
            qh = q[t, kh * G]
            kp[int(pages[j // 16]), kh, j % 16] = (qh * (400.0 * s.head_dim ** 0.5 / float(qh.norm()) ** 2)).to(dt)
        chosen[r] = j
    B.kv_pool_import(S.pool, kp, S.v_plain, None, GH.stream())
    # only the group's first head is aligned with the key; the check uses it alone
    GH.run_step(S)
    attn = GH.intermediate(S, 1, b.n_tokens, s.n_q_heads * s.head_dim, dt).view(b.n_tokens, s.n_q_heads, s.head_dim)
    checked = 0
    for r, j in chosen.items():
        t = b.req_q_start[r]
        page = int(b.page_indices[b.page_indptr[r] + j // 16])
        for kh in range(s.n_kv_heads):
            assert torch.equal(attn[t, kh * G], S.v_plain[page, kh, j % 16]), (r, kh, j)
            checked += 1
    assert checked > 0


def test_pool_import_matches_documented_layout_and_round_trips():
    """nf_kv_pool_import places plain [page][head][slot][dim] values where the
    boundary's block layout says (an enumeration of the attention operand
    loads, tests/kv_layout.py); export returns them bit for bit, also for a
    page list; a step on the imported pool is checked by every parity test."""
    from tests import kv_layout as KV
    for wl in (SMALL_BF16, W.WORKLOADS["c1"]):
        S = GH.setup(wl)
        s = wl.shape
        kmap, vmap = KV.maps(s.head_dim)
        km = torch.as_tensor(kmap.reshape(-1), device="cuda")
        vm = torch.as_tensor(vmap.reshape(-1), device="cuda")
        P, nkv = S.batch.n_pages, s.n_kv_heads
        want_k = torch.empty_like(S.k)
        want_v = torch.empty_like(S.v)
        want_k[:, :, km] = S.k_plain.reshape(P, nkv, -1)
        want_v[:, :, vm] = S.v_plain.reshape(P, nkv, -1)
        assert torch.equal(S.k, want_k) and torch.equal(S.v, want_v)
        k_back, v_back = GH.pool_plain(S)
        assert torch.equal(k_back, S.k_plain) and torch.equal(v_back, S.v_plain)
        # a page list, with a repeated page, both ways
        pages = np.array([3, 0, P - 1, 3, 7], np.int32)
        ke = torch.empty(len(pages), nkv, 16, s.head_dim, dtype=S.k.dtype, device="cuda")
        ve = torch.empty_like(ke)
        B.kv_pool_export(S.pool, ke, ve, pages, GH.stream())
        torch.cuda.synchronize()
        idx = torch.as_tensor(pages.astype(np.int64), device="cuda")
        assert torch.equal(ke, S.k_plain[idx]) and torch.equal(ve, S.v_plain[idx])
        ki, vi = torch.randn_like(ke.float()).to(ke.dtype), torch.randn_like(ve.float()).to(ve.dtype)
        B.kv_pool_import(S.pool, ki[:3], vi[:3], pages[:3], GH.stream())
        k2, v2 = GH.pool_plain(S)
        assert torch.equal(k2[idx[:3]], ki[:3]) and torch.equal(v2[idx[:3]], vi[:3])
        rest = torch.ones(P, dtype=torch.bool, device="cuda")
        rest[idx[:3]] = False
        assert torch.equal(k2[rest], S.k_plain[rest]) and torch.equal(v2[rest], S.v_plain[rest])
        with pytest.raises(B.NfError) as e:
            B.kv_pool_export(S.pool, ke, ve, np.array([P], np.int32), GH.stream())
        assert e.value.status == B.NF_ERR_OUT_OF_RANGE
        S.pool.close()
        S.layer.close()


# ---------------------------------------------------------------- full-size workloads

def _sampled_check(S, requests, w_np=None):
    GH.log(f"step {S.wl.name} T={S.batch.n_tokens} plan={B.plan_dict(S.layer.get_plan())}")
    res, rows, _ = _check(S, S.wl.name, requests, w_np)
    return res, rows


def _sample_requests(b, n, seed=3):
    rng = np.random.Generator(np.random.PCG64(seed))
    dec = [r for r in range(b.n_requests) if b.req_q_len[r] == 1]
    pick = sorted(rng.choice(dec, size=min(n, len(dec)), replace=False).tolist())
    pre = [r for r in range(b.n_requests) if b.req_q_len[r] > 1]
    return pick + pre


@pytest.mark.slow
def test_c2_full_size_every_request():
    S = GH.setup(W.WORKLOADS["c2"])
    S.layer.set_plan(B.make_plan(1, [S.batch.n_tokens]))
    _sampled_check(S, list(range(S.batch.n_requests)), GH.weights_np(S))


@pytest.mark.slow
@pytest.mark.parametrize("wl_name", ["c3", "c4"])
def test_mixed_full_size_sampled(wl_name):
    S = GH.setup(W.WORKLOADS[wl_name])
    T = S.batch.n_tokens
    w_np = GH.weights_np(S)
    S.layer.set_plan(B.make_plan(2, [T // 2, T - T // 2], n_streams=2, gemm_cus_per_xcd=16))
    _sampled_check(S, _sample_requests(S.batch, 16), w_np)
    S.layer.set_plan(B.make_plan(1, [T]))
    _sampled_check(S, _sample_requests(S.batch, 16, seed=4), w_np)
    S.layer.set_plan(B.make_plan(2, [T // 2, T - T // 2], n_streams=2, attn_waves_per_cu=4))
    _sampled_check(S, _sample_requests(S.batch, 8, seed=5), w_np)
    # two lanes, each tiling its GEMMs for half the chip
    S.layer.set_plan(B.make_plan(2, [T // 2, T - T // 2], order=B.NF_ORDER_LANES, n_streams=2))
    _sampled_check(S, _sample_requests(S.batch, 8, seed=6), w_np)


# ---------------------------------------------------------------- mixture of experts

SMALL_MOE = W.Workload("small_moe",
                       W.Shape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=384, n_experts=8, top_k=2,
                               dtype="bf16", rope_theta=1e6),
                       n_decode=70, ctx_range=(1, 200), prefill=(10, 30), seed=79)


def _route_check(S, t0, t1, j):
    """GPU routing of tokens t0..t1 (nano-batch j) == oracle routing, exactly."""
    s = S.wl.shape
    k = s.top_k
    T = S.batch.n_tokens
    logits = GH.f64(S.acts["router_logits"][t0:t1])
    idx, w, perm, offsets = oracle.moe_route(logits, k)
    gi = torch.empty(T * k, dtype=torch.int32, device="cuda")
    gw = torch.empty(T * k, dtype=torch.float32, device="cuda")
    gp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    go = torch.empty(4 * (s.n_experts + 1), dtype=torch.int32, device="cuda")
    for which, t in ((5, gi), (6, gw), (7, gp), (8, go)):
        ptr, _ = S.layer.intermediate(which)
        B.copy_device(t, ptr, t.numel() * t.element_size())
    gi = gi.cpu().numpy()[t0 * k:t1 * k].reshape(-1, k)
    gw = gw.cpu().numpy()[t0 * k:t1 * k].reshape(-1, k)
    gp = gp.cpu().numpy()[t0 * k:t1 * k]
    go = go.cpu().numpy()[j * (s.n_experts + 1):(j + 1) * (s.n_experts + 1)]
    assert np.array_equal(gi, idx)
    assert np.array_equal(gp, perm)
    assert np.array_equal(go, offsets)
    assert np.max(np.abs(gw - w)) < 1e-6


def test_small_moe_full_parity():
    S = GH.setup(SMALL_MOE)
    T = S.batch.n_tokens
    for name, plan in (("k1", B.make_plan(1, [T])),
                       ("k3", B.make_plan(3, [33, 33, T - 66], n_streams=2, gemm_cus_per_xcd=16)),
                       ("k3_lanes", B.make_plan(3, [33, 33, T - 66], order=B.NF_ORDER_LANES, n_streams=2))):
        _full_check(S, name, plan)
        sizes = list(plan.sizes)[:plan.count]
        t0 = 0
        for j, n in enumerate(sizes):
            _route_check(S, t0, t0 + n, j)
            t0 += n


SKEWED_MOE = W.Workload("skewed_moe",
                        W.Shape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=384, n_experts=8,
                                top_k=2, dtype="bf16", rope_theta=1e6),
                        n_decode=200, ctx_range=(1, 64), prefill=(10, 30), seed=83)


def test_skewed_moe_routing_multi_pass_and_empty_expert():
    """Router logits biased so that one expert receives every token (230
    rows: more than one 160-row pass of the expert GEMMs) and another expert
    none (an empty group), under one and two nano-batches."""
    S = GH.setup(SKEWED_MOE)
    logits = S.acts["router_logits"]
    logits[:, 3] += 8.0
    logits[:, 5] -= 8.0
    torch.cuda.synchronize()
    T = S.batch.n_tokens
    assert T > 160
    for name, plan in (("k1", B.make_plan(1, [T])), ("k2", B.make_plan(2, [T // 2, T - T // 2]))):
        _full_check(S, name, plan)
        t0 = 0
        for j, n in enumerate(list(plan.sizes)[:plan.count]):
            _route_check(S, t0, t0 + n, j)
            t0 += n


@pytest.mark.slow
def test_c5_full_size_sampled():
    S = GH.setup(W.WORKLOADS["c5"])
    T = S.batch.n_tokens
    w_np = GH.weights_np(S)
    S.layer.set_plan(B.make_plan(2, [T // 2, T - T // 2], n_streams=2, gemm_cus_per_xcd=16))
    _sampled_check(S, _sample_requests(S.batch, 8), w_np)
    _route_check(S, 0, T // 2, 0)
    _route_check(S, T // 2, T, 1)
    S.layer.set_plan(B.make_plan(1, [T]))
    _sampled_check(S, _sample_requests(S.batch, 8, seed=4), w_np)
    _route_check(S, 0, T, 0)
    # two lanes: each lane's expert GEMMs with split-K partials of its own
    S.layer.set_plan(B.make_plan(2, [T // 2, T - T // 2], order=B.NF_ORDER_LANES, n_streams=2))
    _sampled_check(S, _sample_requests(S.batch, 6, seed=7), w_np)
    _route_check(S, 0, T // 2, 0)
    _route_check(S, T // 2, T, 1)
