"""KV offload to host (nf_kv_offload) through the C ABI: the host copy of
each listed page equals the pool's page bit for bit (K and V, every KV
head), alone and while a layer step runs on another stream; out-of-range
pages are refused before anything is launched."""
import numpy as np
import pytest
import torch

from intra_operation_overlap_amd import binding as B
from intra_operation_overlap_amd import workload as W
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

SMALL = W.Workload("offload_bf16",
                   W.Shape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=688, dtype="bf16",
                           rope_theta=5e5),
                   n_decode=40, ctx_range=(1, 300), prefill=(37, 45), seed=93)


def _host_like(pool, n):
    return torch.empty((n,) + tuple(pool.shape[1:]), dtype=pool.dtype, pin_memory=True)


def _written_pages(batch):
    """Pool pages holding a position the step writes."""
    out = set()
    for r in range(batch.n_requests):
        p0, ql = int(batch.req_pos0[r]), int(batch.req_q_len[r])
        start = int(batch.page_indptr[r])
        for p in range(p0, p0 + ql):
            out.add(int(batch.page_indices[start + p // 16]))
    return out


@pytest.fixture(scope="module")
def S():
    return GH.setup(SMALL)


def test_offload_copies_pages_bit_exact(S):
    rng = np.random.Generator(np.random.PCG64(5))
    n_pages = S.k.shape[0]
    pages = np.concatenate([[0, n_pages - 1], rng.integers(0, n_pages, 35)]).astype(np.int32)   # repeats allowed
    hk, hv = _host_like(S.k, len(pages)), _host_like(S.v, len(pages))
    B.kv_offload(S.pool, pages, hk, hv, GH.stream())
    torch.cuda.synchronize()
    idx = torch.as_tensor(pages, dtype=torch.int64, device="cuda")
    assert torch.equal(hk, S.k[idx].cpu())
    assert torch.equal(hv, S.v[idx].cpu())
    B.kv_offload(S.pool, np.zeros(0, np.int32), hk, hv, GH.stream())       # n = 0: nothing to do


def test_offload_refuses_out_of_range_page(S):
    hk, hv = _host_like(S.k, 2), _host_like(S.v, 2)
    hk.fill_(7)
    for bad in ([0, S.k.shape[0]], [-1, 0]):
        with pytest.raises(B.NfError) as e:
            B.kv_offload(S.pool, np.array(bad, np.int32), hk, hv, GH.stream())
        assert e.value.status == B.NF_ERR_OUT_OF_RANGE
    torch.cuda.synchronize()
    assert (hk == 7).all()


def test_offload_beside_a_step(S):
    """An offload on its own stream while a step runs: both results equal
    the ones each gives alone (the offloaded pages are ones the step only
    reads)."""
    k0, v0 = S.k.clone(), S.v.clone()
    GH.run_step(S)
    ref_out, ref_k, ref_v = S.out.clone(), S.k.clone(), S.v.clone()
    S.k.copy_(k0)
    S.v.copy_(v0)
    written = _written_pages(S.batch)
    pages = np.array([p for p in range(S.k.shape[0]) if p not in written], np.int32)
    assert len(pages) > 100
    hk, hv = _host_like(S.k, len(pages)), _host_like(S.v, len(pages))
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    B.kv_offload(S.pool, pages, hk, hv, side.cuda_stream)
    S.layer.step(S.pool, S.hb, GH.stream())
    torch.cuda.synchronize()
    idx = torch.as_tensor(pages, dtype=torch.int64, device="cuda")
    assert torch.equal(hk, k0[idx].cpu()) and torch.equal(hv, v0[idx].cpu())
    assert torch.equal(S.out, ref_out) and torch.equal(S.k, ref_k) and torch.equal(S.v, ref_v)
    S.k.copy_(k0)
    S.v.copy_(v0)
