"""The layer's bf16 GEMM kernels one call at a time (nf_gemm_bf16), against a
plain PyTorch fp32 reference of the same op: the same bf16 inputs, fp32
products and sums, one rounding of the output.

Shapes are ragged in M and N (partial tiles in both), every LDS-tiled
configuration runs with and without split-K, and a row stride that is not a
multiple of 8 sends the output through the scalar epilogue instead of the
LDS-staged 16-byte one; the two epilogues must agree bit for bit.
"""
import pytest
import torch

from intra_operation_overlap_amd import binding as B

pytestmark = pytest.mark.gpu

CFGS = [0, 10, 13, 14, 15, 16, 21, 22, 26, 27, 30]


def _case(M, N, K, mode, seed):
    g = torch.Generator().manual_seed(seed)
    A = torch.randn(M, K, generator=g).to(torch.bfloat16)
    Bm = (torch.randn(N, K, generator=g) * 0.05).to(torch.bfloat16)
    B2 = (torch.randn(N, K, generator=g) * 0.05).to(torch.bfloat16) if mode == 2 else None
    R = torch.randn(M, N, generator=g).to(torch.bfloat16) if mode == 1 else None
    return A, Bm, B2, R


def _reference(mode, A, Bm, B2, R):
    a = A.float()
    y = a @ Bm.float().T
    if mode == 1:
        y = y + R.float()
    elif mode == 2:
        y = torch.nn.functional.silu(y) * (a @ B2.float().T)
    return y


def _run(M, N, K, mode, cfg, ks, ld_pad, case):
    A, Bm, B2, R = case
    ld = N + ld_pad
    dA, dB = A.cuda(), Bm.cuda()
    dB2 = B2.cuda() if B2 is not None else None
    dR = None
    if R is not None:
        dR = torch.zeros(M, ld, dtype=torch.bfloat16, device="cuda")
        dR[:, :N] = R.cuda()
    C = torch.full((M, ld), float("nan"), dtype=torch.bfloat16, device="cuda")
    ran = B.gemm_bf16(M, N, K, mode, dA.data_ptr(), K, dB.data_ptr(), dB2.data_ptr() if dB2 is not None else None,
                      K, dR.data_ptr() if dR is not None else None, ld, C.data_ptr(), ld, cfg, ks)
    torch.cuda.synchronize()
    out = C.cpu()
    if ld_pad:
        assert torch.isnan(out[:, N:].float()).all(), "wrote past N"
    return out[:, :N], ran


@pytest.mark.parametrize("cfg", CFGS)
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_gemm_config_matches_fp32_reference(cfg, mode):
    M, N, K = 300, 264, 512
    case = _case(M, N, K, mode, seed=10 * cfg + mode)
    want = _reference(mode, *case)
    for ks in (1, 2):
        got, ran = _run(M, N, K, mode, cfg, ks, 0, case)
        assert ran == (cfg, ks)
        assert not torch.isnan(got.float()).any(), f"cfg {cfg} split {ks}: rows or columns left unwritten"
        err = ((got.float() - want).norm() / want.norm()).item()
        assert err < 5e-3, f"cfg {cfg} mode {mode} split {ks}: normwise relative error {err:.2e}"
        # the scalar epilogue (row stride not a multiple of 8) gives the same bits
        got_s, _ = _run(M, N, K, mode, cfg, ks, 4, case)
        assert torch.equal(got.view(torch.int16), got_s.view(torch.int16)), f"cfg {cfg} split {ks}: epilogues differ"


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_gemm_library_choice_on_a_large_ragged_problem(mode):
    """The library's own tile and split choice on a large ragged problem."""
    M, N, K = 2000, (6152 if mode == 2 else 12296), 1024
    case = _case(M, N, K, mode, seed=99 + mode)
    want = _reference(mode, *case)
    got, ran = _run(M, N, K, mode, -1, 0, 0, case)
    err = ((got.float() - want).norm() / want.norm()).item()
    assert err < 5e-3, f"choice {ran}: normwise relative error {err:.2e}"



# weight-streaming configurations: (cfg, rows per pass) for one n-block per
# wave (modes 0, 1) and two (SwiGLU)
STREAM_1 = [40, 41, 44, 46, 48, 50]
STREAM_2 = [42, 43, 45, 47, 49, 51]


@pytest.mark.parametrize("cfg", STREAM_1 + STREAM_2)
def test_streaming_config_matches_fp32_reference(cfg):
    """The weight-streaming kernels (B copied into MFMA operand order first),
    with M ragged against their 32-row blocks, one pass or several, and
    split-K with ragged chunk counts per piece."""
    modes = [2] if cfg in STREAM_2 else [0, 1]
    N, K = 192, 1024
    for mode in modes:
        for M in (20, 64, 170):
            case = _case(M, N, K, mode, seed=1000 + 7 * cfg + M + mode)
            want = _reference(mode, *case)
            for ks in (1, 3):
                got, ran = _run(M, N, K, mode, cfg, ks, 0, case)
                assert ran[0] == cfg
                assert not torch.isnan(got.float()).any(), f"cfg {cfg} M {M} split {ks}: unwritten outputs"
                err = ((got.float() - want).norm() / want.norm()).item()
                assert err < 5e-3, f"cfg {cfg} mode {mode} M {M} split {ks}: normwise relative error {err:.2e}"
