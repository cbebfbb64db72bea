"""nf_gemm_bf16_noalloc through the C ABI: the same bits as nf_gemm_bf16 (its
split-K partials live in the library's fixed device array instead of an
allocated workspace), on two calls in a row, the second smaller, for every
mode; larger partials than the array holds and the weight-streaming
configurations are refused before anything is launched."""
import pytest
import torch

from intra_operation_overlap_amd import binding as B

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _operands(M, N, K, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    A = (torch.rand(M, K, generator=g, device="cuda") * 2 - 1).to(torch.bfloat16)
    Bm = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    B2 = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    R = torch.randn(M, N, generator=g, device="cuda").to(torch.bfloat16)
    return A, Bm, B2, R


def _reference(mode, A, Bm, B2, R):
    acc = A.float() @ Bm.float().t()
    if mode == 1:
        return acc + R.float()
    if mode == 2:
        up = A.float() @ B2.float().t()
        return acc * torch.sigmoid(acc) * up
    return acc


def _run(fn, mode, M, N, K, A, Bm, B2, R, splits):
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    cfg, z = fn(M, N, K, mode, A.data_ptr(), K, Bm.data_ptr(), B2.data_ptr(), K, R.data_ptr(), N, C.data_ptr(), N,
                -1, splits, 0, s)
    torch.cuda.synchronize()
    return C, cfg, z


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_noalloc_gemm_equals_allocating_gemm_twice(mode):
    # first call large (partials 256 x 1024 x 4 slices), second smaller and ragged
    for (M, N, K, splits, seed) in ((256, 1024, 4096, 4, 11), (100, 520, 2048, 3, 12)):
        A, Bm, B2, R = _operands(M, N, K, seed + mode)
        got, cfg, z = _run(B.gemm_bf16_noalloc, mode, M, N, K, A, Bm, B2, R, splits)
        want, cfg2, z2 = _run(B.gemm_bf16, mode, M, N, K, A, Bm, B2, R, splits)
        assert (cfg, z) == (cfg2, z2) and z == splits
        assert torch.equal(got, want), (mode, M, N, K)
        ref = _reference(mode, A, Bm, B2, R)
        err = float((got.float() - ref).abs().max() / ref.abs().max())
        assert err <= 2e-2, (mode, M, err)


def test_noalloc_gemm_refuses_oversized_partials_and_streaming_configs():
    M, N, K = 2048, 4096, 4096            # 4 slices of 2048 x 4096 fp32: 128 MiB > 64 MiB
    A, Bm, B2, R = _operands(M, N, K, 13)
    C = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    with pytest.raises(B.NfError) as e:
        B.gemm_bf16_noalloc(M, N, K, 0, A.data_ptr(), K, Bm.data_ptr(), None, K, None, 0, C.data_ptr(), N, 13, 4, 0, s)
    assert e.value.status == B.NF_ERR_OUT_OF_RANGE
    with pytest.raises(B.NfError) as e:
        B.gemm_bf16_noalloc(M, N, K, 0, A.data_ptr(), K, Bm.data_ptr(), None, K, None, 0, C.data_ptr(), N, 46, 1, 0, s)
    assert e.value.status == B.NF_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((C == 0).all())
