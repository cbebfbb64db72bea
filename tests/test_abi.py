"""C-ABI checks that need no GPU: the library loads, exports every function
include/nf.h declares, and its host-side validation returns the documented
status codes before anything would launch."""
import ctypes
import os
import re

import numpy as np
import pytest

from intra_operation_overlap_amd import binding as B
from intra_operation_overlap_amd import workload as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "nf.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nf_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 18
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in B._SIGS, f"binding lacks {n}"


def test_status_strings():
    L = B.lib()
    assert L.nf_status_string(B.NF_OK) == b"ok"
    assert L.nf_status_string(B.NF_ERR_NO_PLAN) == b"no plan"


def _small():
    wl = W.WORKLOADS["c1"]
    batch = W.make_batch(wl)
    shape = B.make_shape(wl.shape, max_tokens=64, max_pos=512)
    return wl, batch, shape


def _validate(shape, batch, n_pages=None, page_size=16, plan=None, x=0x1000, out=0x2000, logits=None):
    hb = B.HostBatch(batch, x, out, logits)
    return B.batch_validate(shape, batch.n_pages if n_pages is None else n_pages, page_size, hb, plan)


def _copy(batch, **kw):
    import dataclasses
    arrays = {k: np.array(getattr(batch, k), copy=True) for k in
              ("req_q_start", "req_q_len", "req_pos0", "pos", "page_indptr", "page_indices")}
    arrays.update(kw)
    return dataclasses.replace(batch, **arrays)


def test_validate_accepts_valid_batch_and_plans():
    wl, batch, shape = _small()
    assert _validate(shape, batch) == B.NF_OK
    assert _validate(shape, batch, plan=B.make_plan(2, [8, 8], n_streams=2, gemm_cus_per_xcd=16)) == B.NF_OK
    assert _validate(shape, batch, plan=B.make_plan(1, [0])) == B.NF_OK


def test_validate_rejects_bad_batches():
    wl, batch, shape = _small()
    # page index outside the pool
    bad = _copy(batch)
    bad.page_indices[3] = batch.n_pages
    assert _validate(shape, bad) == B.NF_ERR_OUT_OF_RANGE
    # one page owned by two requests
    bad = _copy(batch)
    r0 = bad.page_indices[bad.page_indptr[0]]
    bad.page_indices[bad.page_indptr[1]] = r0
    assert _validate(shape, bad) == B.NF_ERR_INVALID_ARG
    # positions inconsistent with pos0
    bad = _copy(batch)
    bad.pos[2] += 1
    assert _validate(shape, bad) == B.NF_ERR_INVALID_ARG
    # too few pages for the new position
    bad = _copy(batch)
    bad.req_pos0[0] = (bad.page_indptr[1] - bad.page_indptr[0]) * 16
    bad.pos[0] = bad.req_pos0[0]
    assert _validate(shape, bad) == B.NF_ERR_OUT_OF_RANGE
    # requests not contiguous
    bad = _copy(batch)
    bad.req_q_start[1] = 2
    assert _validate(shape, bad) == B.NF_ERR_INVALID_ARG
    # a q_len so large that a 32-bit running token count would wrap
    bad = _copy(batch)
    bad.req_q_len[1] = 2 ** 31 - 1
    assert _validate(shape, bad) == B.NF_ERR_INVALID_ARG
    # out aliasing x
    assert _validate(shape, batch, x=0x1000, out=0x1000) == B.NF_ERR_INVALID_ARG
    # unsupported page size
    assert _validate(shape, batch, page_size=8) == B.NF_ERR_UNSUPPORTED


def test_validate_rejects_capacity_and_plan_errors():
    wl, batch, shape = _small()
    small = B.make_shape(wl.shape, max_tokens=8, max_pos=512)
    assert _validate(small, batch) == B.NF_ERR_OUT_OF_RANGE
    short = B.make_shape(wl.shape, max_tokens=64, max_pos=int(batch.pos.max()))
    assert _validate(short, batch) == B.NF_ERR_OUT_OF_RANGE
    assert _validate(shape, batch, plan=B.make_plan(2, [8, 7])) == B.NF_ERR_NO_PLAN
    assert _validate(shape, batch, plan=B.make_plan(2, [16, 0])) == B.NF_ERR_NO_PLAN
    assert _validate(shape, batch, plan=B.make_plan(5, [4, 4, 4, 4])) == B.NF_ERR_INVALID_ARG
    assert _validate(shape, batch, plan=B.make_plan(1, [16], n_streams=1, gemm_cus_per_xcd=8)) == B.NF_ERR_INVALID_ARG
    assert _validate(shape, batch, plan=B.make_plan(1, [16], n_streams=2, gemm_cus_per_xcd=32)) == B.NF_ERR_OUT_OF_RANGE
    # lanes need two streams; an unknown order is refused
    assert _validate(shape, batch, plan=B.make_plan(2, [8, 8], order=B.NF_ORDER_LANES)) == B.NF_ERR_INVALID_ARG
    assert _validate(shape, batch, plan=B.make_plan(2, [8, 8], order=B.NF_ORDER_LANES, n_streams=2)) == B.NF_OK
    assert _validate(shape, batch, plan=B.make_plan(2, [8, 8], order=4, n_streams=2)) == B.NF_ERR_INVALID_ARG


def test_validate_rejects_gemm_operands_over_4gib():
    """bf16 GEMMs address operands with 32-bit byte offsets: a capacity whose
    widest activation (T x ffn bf16) reaches 4 GiB is refused up front."""
    wl = W.WORKLOADS["c2"]
    batch = W.make_batch(wl)
    ok = B.make_shape(wl.shape, max_tokens=(1 << 32) // (2 * wl.shape.ffn) - 1, max_pos=4096)
    assert _validate(ok, batch) == B.NF_OK
    big = B.make_shape(wl.shape, max_tokens=(1 << 32) // (2 * wl.shape.ffn) + 1, max_pos=4096)
    assert _validate(big, batch) == B.NF_ERR_OUT_OF_RANGE


def test_gemm_rejects_bad_arguments_before_launching():
    with pytest.raises(B.NfError) as e:
        B.gemm_bf16(64, 64, 96, 0, 1, 96, 1, None, 96, None, 64, 1, 64, 14, 1)    # cfg 14 needs K % 64
    assert e.value.status == B.NF_ERR_INVALID_ARG
    with pytest.raises(B.NfError) as e:
        B.gemm_bf16(64, 60, 64, 0, 1, 64, 1, None, 64, None, 60, 1, 60)           # N % 8
    assert e.value.status == B.NF_ERR_INVALID_ARG
    with pytest.raises(B.NfError) as e:
        B.gemm_bf16(64, 64, 64, 2, 1, 64, 1, None, 64, None, 64, 1, 64)           # SwiGLU without B2
    assert e.value.status == B.NF_ERR_INVALID_ARG
    with pytest.raises(B.NfError) as e:
        B.gemm_bf16(64, 64, 64, 0, 1, 64, 1, None, 64, None, 64, 1, 64, 40, 1)    # streaming tiles need packing
    assert e.value.status == B.NF_ERR_INVALID_ARG


def test_gemm_probe_rejects_bad_arguments_before_allocating():
    """The probe checks its configuration like nf_gemm_bf16 before any HIP call."""
    bad = [(64, 64, 64, 0, 45, 1, 5),      # a two-n-block streaming configuration for a plain GEMM
           (64, 64, 64, 2, 46, 1, 5),      # a one-n-block streaming configuration for SwiGLU
           (64, 64, 96, 0, 14, 1, 5),      # a pipelined configuration with K % 64 != 0
           (64, 60, 64, 0, -1, 0, 5),      # N % 8
           (64, 64, 64, 0, 7, 1, 5),       # no configuration 7
           (64, 64, 64, 0, -1, 0, 0)]      # reps <= 0
    for M, N, K, mode, cfg, ks, reps in bad:
        with pytest.raises(B.NfError) as e:
            B.probe_gemm_bf16_ms(M, N, K, mode, cfg, ks, 256, reps)
        assert e.value.status == B.NF_ERR_INVALID_ARG, (M, N, K, mode, cfg, reps)


def test_validate_moe_needs_logits_and_shape_rules():
    wl = W.WORKLOADS["c5"]
    batch = W.make_batch(wl, n_decode=4)
    shape = B.make_shape(wl.shape, max_tokens=64, max_pos=4096)
    assert _validate(shape, batch) == B.NF_ERR_INVALID_ARG
    assert _validate(shape, batch, logits=0x3000) == B.NF_OK
    bad = B.make_shape(W.Shape(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=688), 64, 512)
    assert _validate(bad, batch) == B.NF_ERR_UNSUPPORTED           # bf16 needs head_dim 128
    bad = B.make_shape(W.Shape(hidden=256, n_q_heads=6, n_kv_heads=4, head_dim=128, ffn=688), 64, 512)
    assert _validate(bad, batch) == B.NF_ERR_INVALID_ARG


def test_empty_batch_is_valid():
    wl, batch, shape = _small()
    empty = W.Batch(0, np.zeros(0, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32),
                    np.zeros(0, np.int32), np.zeros(1, np.int32), np.zeros(0, np.int32), 4)
    assert _validate(shape, empty) == B.NF_OK


def test_kv_pool_bytes():
    wl, batch, shape = _small()
    kb, vb = B.kv_pool_bytes(shape, 10, 16)
    assert kb == vb == 10 * 2 * 16 * 64 * 4
    with pytest.raises(B.NfError) as e:
        B.kv_pool_bytes(shape, 10, 32)
    assert e.value.status == B.NF_ERR_UNSUPPORTED


def test_stack_and_graph_reject_bad_arguments_before_launching():
    L = B.lib()
    _, batch, _ = _small()
    hb = B.HostBatch(batch, 0x1000, 0x2000)
    one = (ctypes.c_void_p * 1)(None)
    # null arrays, no layers, null handles: rejected before any HIP call
    assert L.nf_stack_step(None, None, 1, ctypes.byref(hb.c), None) == B.NF_ERR_INVALID_ARG
    assert L.nf_stack_step(one, one, 0, ctypes.byref(hb.c), None) == B.NF_ERR_INVALID_ARG
    assert L.nf_stack_step(one, one, 1, ctypes.byref(hb.c), None) == B.NF_ERR_INVALID_ARG
    assert L.nf_stack_step(one, one, 1, None, None) == B.NF_ERR_INVALID_ARG
    out = ctypes.c_void_p()
    assert L.nf_stack_graph_create(one, one, 1, ctypes.byref(hb.c), None, None) == B.NF_ERR_INVALID_ARG
    assert L.nf_stack_graph_create(one, one, 0, ctypes.byref(hb.c), None, ctypes.byref(out)) == B.NF_ERR_INVALID_ARG
    assert out.value is None
    assert L.nf_graph_launch(None, None) == B.NF_ERR_INVALID_ARG
    L.nf_graph_destroy(None)                      # a no-op


def test_kv_offload_rejects_bad_arguments_before_launching():
    L = B.lib()
    pages = (ctypes.c_int32 * 2)(0, 1)
    assert L.nf_kv_offload(None, pages, 2, 1, 1, None) == B.NF_ERR_INVALID_ARG
    assert L.nf_kv_offload(ctypes.c_void_p(8), pages, -1, 1, 1, None) == B.NF_ERR_INVALID_ARG
    assert L.nf_kv_offload(ctypes.c_void_p(8), None, 2, 1, 1, None) == B.NF_ERR_INVALID_ARG
    assert L.nf_kv_offload(ctypes.c_void_p(8), pages, 2, None, 1, None) == B.NF_ERR_INVALID_ARG


def test_kv_pool_import_export_reject_bad_arguments_before_launching():
    L = B.lib()
    pages = (ctypes.c_int32 * 2)(0, 1)
    for fn in (L.nf_kv_pool_import, L.nf_kv_pool_export):
        assert fn(None, pages, 2, 1, 1, None) == B.NF_ERR_INVALID_ARG
        assert fn(ctypes.c_void_p(8), pages, -1, 1, 1, None) == B.NF_ERR_INVALID_ARG
        assert fn(ctypes.c_void_p(8), pages, 2, None, 1, None) == B.NF_ERR_INVALID_ARG
        assert fn(ctypes.c_void_p(8), None, 2, 1, None, None) == B.NF_ERR_INVALID_ARG


def test_cu_map_probes_reject_bad_arguments_before_launching():
    L = B.lib()
    buf = (ctypes.c_int32 * 8)()
    n = ctypes.c_int32()
    assert L.nf_probe_cu_map(None, None, 8) == B.NF_ERR_INVALID_ARG
    assert L.nf_probe_cu_map(buf, None, 0) == B.NF_ERR_INVALID_ARG
    assert L.nf_probe_budget_cus(0, 4, None, 8, ctypes.byref(n)) == B.NF_ERR_INVALID_ARG
    assert L.nf_probe_budget_cus(-1, 4, buf, 8, ctypes.byref(n)) == B.NF_ERR_INVALID_ARG
    assert L.nf_probe_budget_cus(0, 0, buf, 8, ctypes.byref(n)) == B.NF_ERR_INVALID_ARG


def test_binding_has_every_name_the_gpu_tests_and_bench_use():
    """The GPU tests skip on a machine without a GPU; their use of the binding
    is checked here so a missing name fails on the CPU first."""
    names = set()
    for f in ("tests/test_gpu_parity.py", "tests/test_gpu_collective.py", "tests/test_gpu_api.py",
              "tests/test_gpu_stack.py", "tests/test_gpu_offload.py", "tests/test_gpu_gemm.py",
              "tests/test_zz_no_alloc.py", "tests/gpu_harness.py", "bench.py", "__graft_entry__.py"):
        names |= set(re.findall(r"\bB\.([A-Za-z_][A-Za-z0-9_]*)", open(os.path.join(ROOT, f)).read()))
    missing = sorted(n for n in names if not hasattr(B, n))
    assert not missing, missing


def test_loop_rejects_bad_arguments_before_launching():
    L = B.lib()
    o = B.nf_loop_opts(16, 16, 1, 10.0)
    h = ctypes.c_void_p()
    assert L.nf_loop_create(None, None, ctypes.byref(o), ctypes.byref(h)) == B.NF_ERR_INVALID_ARG
    rid = ctypes.c_int32()
    assert L.nf_loop_add_request(None, 4, 8, 16, 16, ctypes.byref(rid)) == B.NF_ERR_INVALID_ARG
    assert L.nf_loop_run(None, None, None) == B.NF_ERR_INVALID_ARG
    n = ctypes.c_int32()
    assert L.nf_loop_request_length(None, 0, ctypes.byref(n)) == B.NF_ERR_INVALID_ARG
    L.nf_loop_destroy(None)


def test_debug_capture_and_intermediate_reject_null_layers():
    L = B.lib()
    assert L.nf_layer_debug_capture(None, 1) == B.NF_ERR_INVALID_ARG
    ptr, stride = ctypes.c_void_p(), ctypes.c_int64()
    assert L.nf_layer_intermediate(None, 0, ctypes.byref(ptr), ctypes.byref(stride)) == B.NF_ERR_INVALID_ARG
