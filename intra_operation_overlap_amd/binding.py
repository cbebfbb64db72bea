"""ctypes binding of libnf.so (declarations in include/nf.h).

Argument marshalling only: every step of the layer runs in the HIP library.
The functions keep the C names; the small classes below only hold handles
and keep the caller's tensors alive.  Loading fails loudly when the library
has not been built -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnf.so")

NF_OK, NF_ERR_INVALID_ARG, NF_ERR_OUT_OF_RANGE, NF_ERR_UNSUPPORTED, NF_ERR_NO_PLAN, NF_ERR_HIP = range(6)
NF_F32, NF_BF16 = 0, 1
NF_ORDER_PIPELINED, NF_ORDER_SEQUENTIAL, NF_ORDER_DEEP, NF_ORDER_LANES = 0, 1, 2, 3
NF_MAX_NANO = 4

i32 = ctypes.c_int32
i64 = ctypes.c_int64
vp = ctypes.c_void_p
P_i32 = ctypes.POINTER(ctypes.c_int32)


class nf_shape(ctypes.Structure):
    _fields_ = [("hidden", i32), ("n_q_heads", i32), ("n_kv_heads", i32), ("head_dim", i32),
                ("ffn", i32), ("n_experts", i32), ("top_k", i32), ("dtype", i32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_double),
                ("max_tokens", i32), ("max_pos", i32)]


class nf_weights(ctypes.Structure):
    _fields_ = [(n, vp) for n in ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate", "w_up", "w_down")]


class nf_batch(ctypes.Structure):
    _fields_ = [("n_tokens", i32), ("n_requests", i32), ("x", vp), ("out", vp),
                ("req_q_start", P_i32), ("req_q_len", P_i32), ("req_pos0", P_i32), ("pos", P_i32),
                ("page_indptr", P_i32), ("page_indices", P_i32),
                ("router_logits", ctypes.POINTER(ctypes.c_float))]


class nf_plan(ctypes.Structure):
    _fields_ = [("count", i32), ("sizes", i32 * NF_MAX_NANO), ("order", i32), ("n_streams", i32),
                ("gemm_cus_per_xcd", i32), ("attn_cus_per_xcd", i32), ("attn_waves_per_cu", i32)]


NF_PROFILE_POINTS = 8


class nf_plan_profile(ctypes.Structure):
    _fields_ = [("n_points", i32), ("tokens", ctypes.c_double * NF_PROFILE_POINTS),
                ("front_us", ctypes.c_double * NF_PROFILE_POINTS), ("oproj_us", ctypes.c_double * NF_PROFILE_POINTS),
                ("ffn_us", ctypes.c_double * NF_PROFILE_POINTS), ("attn_base_us", ctypes.c_double),
                ("attn_us_per_page", ctypes.c_double), ("gap_us", ctypes.c_double), ("slow_gemm", ctypes.c_double),
                ("slow_attn", ctypes.c_double), ("wait_us", ctypes.c_double), ("scale_gemm", ctypes.c_double),
                ("scale_attn", ctypes.c_double), ("lane_rate", ctypes.c_double)]


class nf_loop_opts(ctypes.Structure):
    _fields_ = [("max_tokens", i32), ("max_prefill_tokens", i32), ("async_", i32), ("eos_threshold", ctypes.c_float)]


class nf_loop_stats(ctypes.Structure):
    _fields_ = [("iterations", i32), ("finished", i32), ("tokens", i64), ("wasted_tokens", i64),
                ("host_us", ctypes.c_double), ("wall_us", ctypes.c_double)]


class nf_search_opts(ctypes.Structure):
    _fields_ = [("max_count", i32), ("warmup", i32), ("reps", i32), ("top_k", i32)]


# name -> (restype, argtypes), mirroring include/nf.h
_SIGS = {
    "nf_layer_create": (i32, [ctypes.POINTER(nf_shape), ctypes.POINTER(nf_weights), ctypes.POINTER(vp)]),
    "nf_layer_destroy": (None, [vp]),
    "nf_kv_pool_bytes": (i32, [ctypes.POINTER(nf_shape), i32, i32, ctypes.POINTER(ctypes.c_size_t),
                               ctypes.POINTER(ctypes.c_size_t)]),
    "nf_kv_pool_create": (i32, [vp, i32, i32, vp, vp, ctypes.POINTER(vp)]),
    "nf_kv_pool_destroy": (None, [vp]),
    "nf_plan_set": (i32, [vp, ctypes.POINTER(nf_plan)]),
    "nf_plan_get": (i32, [vp, ctypes.POINTER(nf_plan)]),
    "nf_batch_validate": (i32, [ctypes.POINTER(nf_shape), i32, i32, ctypes.POINTER(nf_batch),
                                ctypes.POINTER(nf_plan)]),
    "nf_layer_step": (i32, [vp, vp, ctypes.POINTER(nf_batch), vp]),
    "nf_layer_set_allreduce_emulation": (i32, [vp, i32, i32]),
    "nf_stack_step": (i32, [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, ctypes.POINTER(nf_batch), vp]),
    "nf_stack_graph_create": (i32, [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, ctypes.POINTER(nf_batch), vp,
                                    ctypes.POINTER(vp)]),
    "nf_graph_launch": (i32, [vp, vp]),
    "nf_kv_offload": (i32, [vp, P_i32, i32, vp, vp, vp]),
    "nf_loop_create": (i32, [vp, vp, ctypes.POINTER(nf_loop_opts), ctypes.POINTER(vp)]),
    "nf_loop_add_request": (i32, [vp, i32, i32, vp, vp, P_i32]),
    "nf_loop_run": (i32, [vp, vp, ctypes.POINTER(nf_loop_stats)]),
    "nf_loop_request_length": (i32, [vp, i32, P_i32]),
    "nf_loop_destroy": (None, [vp]),
    "nf_kv_pool_import": (i32, [vp, P_i32, i32, vp, vp, vp]),
    "nf_kv_pool_export": (i32, [vp, P_i32, i32, vp, vp, vp]),
    "nf_graph_destroy": (None, [vp]),
    "nf_plan_search": (i32, [vp, vp, ctypes.POINTER(nf_batch), ctypes.POINTER(nf_search_opts),
                             ctypes.POINTER(nf_plan), ctypes.POINTER(ctypes.c_double), vp]),
    "nf_plan_search_report": (i32, [vp, i32, ctypes.POINTER(nf_plan), ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32), ctypes.POINTER(i32)]),
    "nf_plan_predict": (i32, [ctypes.POINTER(nf_plan_profile), ctypes.POINTER(nf_shape), ctypes.POINTER(nf_plan),
                              ctypes.POINTER(nf_batch), ctypes.POINTER(ctypes.c_double)]),
    "nf_layer_intermediate": (i32, [vp, i32, ctypes.POINTER(vp), ctypes.POINTER(i64)]),
    "nf_layer_debug_capture": (i32, [vp, i32]),
    "nf_profile_enable": (i32, [vp, i32, ctypes.c_char_p]),
    "nf_profile_read": (i32, [vp, i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(i64),
                              ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]),
    "nf_probe_mfma_bf16_tflops": (i32, [ctypes.POINTER(ctypes.c_double)]),
    "nf_probe_hbm_read_gbps": (i32, [ctypes.c_size_t, ctypes.POINTER(ctypes.c_double)]),
    "nf_probe_cu_map": (i32, [P_i32, P_i32, i32]),
    "nf_probe_budget_cus": (i32, [i32, i32, P_i32, i32, P_i32]),
    "nf_probe_gemm_bf16_ms": (i32, [i32, i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_double),
                                    P_i32, P_i32]),
    "nf_gemm_bf16": (i32, [i32, i32, i32, i32, vp, i64, vp, vp, i64, vp, i64, vp, i64, i32, i32, i32, vp,
                           P_i32, P_i32]),
    "nf_gemm_bf16_noalloc": (i32, [i32, i32, i32, i32, vp, i64, vp, vp, i64, vp, i64, vp, i64, i32, i32, i32, vp,
                                   P_i32, P_i32]),
    "nf_last_error": (ctypes.c_char_p, []),
    "nf_status_string": (ctypes.c_char_p, [i32]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m intra_operation_overlap_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class NfError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().nf_last_error().decode()
        super().__init__(f"{where}: {lib().nf_status_string(status).decode()} ({status}): {msg}")


def check(status: int, where: str) -> None:
    if status != NF_OK:
        raise NfError(status, where)


# ---------------------------------------------------------------- helpers

def make_shape(s, max_tokens: int, max_pos: int) -> nf_shape:
    """nf_shape from a workload Shape (any object with the same field names)."""
    return nf_shape(s.hidden, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn, s.n_experts, s.top_k,
                    NF_BF16 if s.dtype == "bf16" else NF_F32, s.rms_eps, s.rope_theta, max_tokens, max_pos)


def _i32p(a: np.ndarray):
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(P_i32)


class HostBatch:
    """Keeps the host arrays of one batch alive and exposes an nf_batch."""

    def __init__(self, batch, x_ptr: int, out_ptr: int, logits_ptr: Optional[int] = None):
        self.arrays = [np.ascontiguousarray(a, dtype=np.int32) for a in
                       (batch.req_q_start, batch.req_q_len, batch.req_pos0, batch.pos,
                        batch.page_indptr, batch.page_indices)]
        if self.arrays[5].size == 0:
            self.arrays[5] = np.zeros(1, np.int32)
        a = self.arrays
        self.c = nf_batch(batch.n_tokens, batch.n_requests, x_ptr, out_ptr, _i32p(a[0]), _i32p(a[1]),
                          _i32p(a[2]), _i32p(a[3]), _i32p(a[4]), _i32p(a[5]),
                          ctypes.cast(logits_ptr or 0, ctypes.POINTER(ctypes.c_float)))


def make_plan(count=1, sizes: Sequence[int] = (0,), order=NF_ORDER_PIPELINED, n_streams=1,
              gemm_cus_per_xcd=0, attn_cus_per_xcd=0, attn_waves_per_cu=0) -> nf_plan:
    s = list(sizes) + [0] * (NF_MAX_NANO - len(sizes))
    return nf_plan(count, (i32 * NF_MAX_NANO)(*s), order, n_streams, gemm_cus_per_xcd, attn_cus_per_xcd,
                   attn_waves_per_cu)


def plan_dict(p: nf_plan) -> dict:
    return {"count": p.count, "sizes": list(p.sizes)[:p.count], "order": p.order,
            "n_streams": p.n_streams, "gemm_cus_per_xcd": p.gemm_cus_per_xcd,
            "attn_cus_per_xcd": p.attn_cus_per_xcd, "attn_waves_per_cu": p.attn_waves_per_cu}


def batch_validate(shape: nf_shape, n_pages: int, page_size: int, hb: HostBatch,
                   plan: Optional[nf_plan] = None) -> int:
    return lib().nf_batch_validate(ctypes.byref(shape), n_pages, page_size, ctypes.byref(hb.c),
                                   ctypes.byref(plan) if plan is not None else None)


class Layer:
    """nf_layer over caller-owned torch weights (kept referenced here)."""

    def __init__(self, shape, weights: Dict[str, "torch.Tensor"], max_tokens: int, max_pos: int):
        self.shape = make_shape(shape, max_tokens, max_pos)
        self._weights = weights
        w = nf_weights(*(weights[n].data_ptr() for n in
                         ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate", "w_up", "w_down")))
        h = vp()
        check(lib().nf_layer_create(ctypes.byref(self.shape), ctypes.byref(w), ctypes.byref(h)), "nf_layer_create")
        self.h = h

    def close(self):
        if self.h:
            lib().nf_layer_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_plan(self, plan: nf_plan) -> None:
        check(lib().nf_plan_set(self.h, ctypes.byref(plan)), "nf_plan_set")

    def get_plan(self) -> nf_plan:
        p = nf_plan()
        check(lib().nf_plan_get(self.h, ctypes.byref(p)), "nf_plan_get")
        return p

    def set_allreduce_emulation(self, mode: int, copy_workgroups: int = 16) -> None:
        check(lib().nf_layer_set_allreduce_emulation(self.h, mode, copy_workgroups),
              "nf_layer_set_allreduce_emulation")

    def step(self, pool: "KVPool", hb: HostBatch, stream: int = 0) -> None:
        check(lib().nf_layer_step(self.h, pool.h, ctypes.byref(hb.c), stream), "nf_layer_step")

    def search(self, pool: "KVPool", hb: HostBatch, max_count=4, warmup=2, reps=5, top_k=8, stream: int = 0):
        opts = nf_search_opts(max_count, warmup, reps, top_k)
        p = nf_plan()
        t = (ctypes.c_double * 2)()
        check(lib().nf_plan_search(self.h, pool.h, ctypes.byref(hb.c), ctypes.byref(opts), ctypes.byref(p), t,
                                   stream), "nf_plan_search")
        return p, (t[0], t[1])

    def search_report(self, max_entries: int = 64):
        """[(plan dict, predicted ms, measured ms, calibration run?)] of the last plan search."""
        plans = (nf_plan * max_entries)()
        pr = (ctypes.c_double * max_entries)()
        me = (ctypes.c_double * max_entries)()
        cal = (i32 * max_entries)()
        n = i32()
        check(lib().nf_plan_search_report(self.h, max_entries, plans, pr, me, cal, ctypes.byref(n)),
              "nf_plan_search_report")
        return [(plan_dict(plans[i]), pr[i], me[i], bool(cal[i])) for i in range(min(n.value, max_entries))]

    def intermediate(self, which: int):
        ptr, stride = vp(), i64()
        check(lib().nf_layer_intermediate(self.h, which, ctypes.byref(ptr), ctypes.byref(stride)),
              "nf_layer_intermediate")
        return ptr.value, stride.value

    def debug_capture(self, on: bool) -> None:
        check(lib().nf_layer_debug_capture(self.h, 1 if on else 0), "nf_layer_debug_capture")

    def profile_enable(self, on: bool, only_kind: Optional[str] = None) -> None:
        check(lib().nf_profile_enable(self.h, 1 if on else 0, only_kind.encode() if only_kind else None),
              "nf_profile_enable")

    def profile_read(self) -> Dict[str, tuple]:
        n = 32
        names = (ctypes.c_char_p * n)()
        launches = (i64 * n)()
        ms = (ctypes.c_double * n)()
        k = i32()
        check(lib().nf_profile_read(self.h, n, names, launches, ms, ctypes.byref(k)), "nf_profile_read")
        return {names[i].decode(): (launches[i], ms[i]) for i in range(min(k.value, n))}


class KVPool:
    """nf_kv_pool over caller-owned K / V buffers in the pool's layout."""

    def __init__(self, layer: Layer, n_pages: int, page_size: int, k, v):
        self._keep = (k, v)
        self.k, self.v = k, v
        h = vp()
        check(lib().nf_kv_pool_create(layer.h, n_pages, page_size, k.data_ptr(), v.data_ptr(), ctypes.byref(h)),
              "nf_kv_pool_create")
        self.h = h
        self.layer = layer

    @classmethod
    def from_plain(cls, layer: Layer, k_plain, v_plain, stream: int = 0) -> "KVPool":
        """A pool holding the plain paged cache k_plain / v_plain
        ([P][nkv][16][d] device tensors): buffers of the pool's size are
        allocated with torch and filled by nf_kv_pool_import."""
        import torch
        P, nkv, S, d = (int(x) for x in k_plain.shape)
        kb, _ = kv_pool_bytes(layer.shape, P, S)
        k = torch.empty(kb // k_plain.element_size(), dtype=k_plain.dtype, device=k_plain.device).view(P, nkv, S * d)
        v = torch.empty_like(k)
        pool = cls(layer, P, S, k, v)
        kv_pool_import(pool, k_plain, v_plain, None, stream)
        return pool

    def to_plain(self, stream: int = 0):
        """(K, V) of every page as plain [P][nkv][16][d] tensors (nf_kv_pool_export)."""
        import torch
        P, nkv, Sd = (int(x) for x in self.k.shape)
        d = int(self.layer.shape.head_dim)
        k = torch.empty(P, nkv, Sd // d, d, dtype=self.k.dtype, device=self.k.device)
        v = torch.empty_like(k)
        kv_pool_export(self, k, v, None, stream)
        return k, v

    def close(self):
        if self.h:
            lib().nf_kv_pool_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Loop:
    """nf_loop over a layer and a pool (the requests' row tensors are kept referenced)."""

    def __init__(self, layer: Layer, pool: KVPool, max_tokens: int, max_prefill_tokens: int, async_: bool,
                 eos_threshold: float):
        self._keep = [layer, pool]
        h = vp()
        o = nf_loop_opts(max_tokens, max_prefill_tokens, 1 if async_ else 0, eos_threshold)
        check(lib().nf_loop_create(layer.h, pool.h, ctypes.byref(o), ctypes.byref(h)), "nf_loop_create")
        self.h = h

    def add(self, prompt_len: int, rows_in, rows_out) -> int:
        self._keep += [rows_in, rows_out]
        rid = i32()
        check(lib().nf_loop_add_request(self.h, prompt_len, int(rows_in.shape[0]), rows_in.data_ptr(),
                                        rows_out.data_ptr(), ctypes.byref(rid)), "nf_loop_add_request")
        return rid.value

    def run(self, stream: int = 0) -> dict:
        st = nf_loop_stats()
        check(lib().nf_loop_run(self.h, stream, ctypes.byref(st)), "nf_loop_run")
        return {k: getattr(st, k) for k, _ in nf_loop_stats._fields_}

    def length(self, rid: int) -> int:
        n = i32()
        check(lib().nf_loop_request_length(self.h, rid, ctypes.byref(n)), "nf_loop_request_length")
        return n.value

    def close(self):
        if self.h:
            lib().nf_loop_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _handles(objs) -> "ctypes.Array":
    return (vp * len(objs))(*(o.h for o in objs))


def stack_step(layers: List[Layer], pools: List[KVPool], hb: HostBatch, stream: int = 0) -> None:
    """nf_stack_step: the layers in order on one batch (hb.x in, hb.out out)."""
    check(lib().nf_stack_step(_handles(layers), _handles(pools), len(layers), ctypes.byref(hb.c), stream),
          "nf_stack_step")


class StackGraph:
    """nf_stack_graph_create / nf_graph_launch / nf_graph_destroy."""

    def __init__(self, layers: List[Layer], pools: List[KVPool], hb: HostBatch, stream: int = 0):
        self._keep = (layers, pools, hb)
        h = vp()
        check(lib().nf_stack_graph_create(_handles(layers), _handles(pools), len(layers), ctypes.byref(hb.c), stream,
                                          ctypes.byref(h)), "nf_stack_graph_create")
        self.h = h

    def launch(self, stream: int = 0) -> None:
        check(lib().nf_graph_launch(self.h, stream), "nf_graph_launch")

    def close(self):
        if self.h:
            lib().nf_graph_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def kv_offload(pool: KVPool, pages, host_k, host_v, stream: int = 0) -> None:
    """nf_kv_offload: pool pages `pages` (int32) to host tensors host_k / host_v."""
    a = np.ascontiguousarray(np.asarray(pages, np.int32))
    check(lib().nf_kv_offload(pool.h, _i32p(a), len(a), host_k.data_ptr(), host_v.data_ptr(), stream),
          "nf_kv_offload")


def kv_pool_import(pool: KVPool, k_src, v_src, pages=None, stream: int = 0) -> None:
    """nf_kv_pool_import: plain [n][nkv][16][d] device tensors into the pool
    (pages None: pool pages 0..n-1)."""
    n = int(k_src.shape[0])
    a = None if pages is None else np.ascontiguousarray(np.asarray(pages, np.int32))
    check(lib().nf_kv_pool_import(pool.h, _i32p(a) if a is not None else None, n, k_src.data_ptr(),
                                  v_src.data_ptr(), stream), "nf_kv_pool_import")


def kv_pool_export(pool: KVPool, k_dst, v_dst, pages=None, stream: int = 0) -> None:
    """nf_kv_pool_export: pool pages into plain [n][nkv][16][d] device tensors."""
    n = int(k_dst.shape[0])
    a = None if pages is None else np.ascontiguousarray(np.asarray(pages, np.int32))
    check(lib().nf_kv_pool_export(pool.h, _i32p(a) if a is not None else None, n, k_dst.data_ptr(),
                                  v_dst.data_ptr(), stream), "nf_kv_pool_export")


def plan_predict(profile: nf_plan_profile, shape: nf_shape, plan: nf_plan, hb: HostBatch) -> float:
    """nf_plan_predict: the model's step time (microseconds), host only."""
    us = ctypes.c_double()
    check(lib().nf_plan_predict(ctypes.byref(profile), ctypes.byref(shape), ctypes.byref(plan), ctypes.byref(hb.c),
                                ctypes.byref(us)), "nf_plan_predict")
    return us.value


def kv_pool_bytes(shape: nf_shape, n_pages: int, page_size: int):
    kb, vb = ctypes.c_size_t(), ctypes.c_size_t()
    check(lib().nf_kv_pool_bytes(ctypes.byref(shape), n_pages, page_size, ctypes.byref(kb), ctypes.byref(vb)),
          "nf_kv_pool_bytes")
    return kb.value, vb.value


def probe_mfma_bf16_tflops() -> float:
    v = ctypes.c_double()
    check(lib().nf_probe_mfma_bf16_tflops(ctypes.byref(v)), "nf_probe_mfma_bf16_tflops")
    return v.value


def probe_hbm_read_gbps(nbytes: int = 4 << 30) -> float:
    v = ctypes.c_double()
    check(lib().nf_probe_hbm_read_gbps(nbytes, ctypes.byref(v)), "nf_probe_hbm_read_gbps")
    return v.value


def probe_cu_map(n: int):
    """(xcc, cu): per CU-mask bit, its XCD and its CU field of HW_ID (-1: unknown)."""
    a = np.zeros(n, np.int32)
    c = np.zeros(n, np.int32)
    check(lib().nf_probe_cu_map(_i32p(a), _i32p(c), n), "nf_probe_cu_map")
    return a.tolist(), c.tolist()


def probe_budget_cus(first: int, count: int, max_pairs: int = 1024) -> List[tuple]:
    """Distinct (XCD, CU field) pairs a stream masked to CUs first..first+count-1
    of every XCD ran on."""
    a = np.zeros(max_pairs, np.int32)
    n = i32()
    check(lib().nf_probe_budget_cus(first, count, _i32p(a), max_pairs, ctypes.byref(n)), "nf_probe_budget_cus")
    return [(int(v) >> 16, int(v) & 0xFFFF) for v in a[:min(n.value, max_pairs)]]


def probe_gemm_bf16_ms(M, N, K, mode=0, tile_cfg=-1, k_splits=0, cus=256, reps=20):
    """(ms, cfg, splits) of one GEMM launch on library-owned buffers."""
    v = ctypes.c_double()
    c, s = i32(), i32()
    check(lib().nf_probe_gemm_bf16_ms(M, N, K, mode, tile_cfg, k_splits, cus, reps, ctypes.byref(v),
                                      ctypes.byref(c), ctypes.byref(s)), "nf_probe_gemm_bf16_ms")
    return v.value, c.value, s.value


def gemm_bf16(M, N, K, mode, A, lda, B, B2, ldb, R, ldr, C, ldc, tile_cfg=-1, k_splits=0, cus=0, stream=None):
    """One layer GEMM on caller device pointers; returns (cfg, splits) that ran."""
    c, s = i32(), i32()
    check(lib().nf_gemm_bf16(M, N, K, mode, A, lda, B, B2, ldb, R, ldr, C, ldc, tile_cfg, k_splits, cus, stream,
                             ctypes.byref(c), ctypes.byref(s)), "nf_gemm_bf16")
    return c.value, s.value


def gemm_bf16_noalloc(M, N, K, mode, A, lda, B, B2, ldb, R, ldr, C, ldc, tile_cfg=-1, k_splits=0, cus=0,
                      stream=None):
    """nf_gemm_bf16_noalloc (enqueue only, no allocation); returns (cfg, splits)."""
    c, s = i32(), i32()
    check(lib().nf_gemm_bf16_noalloc(M, N, K, mode, A, lda, B, B2, ldb, R, ldr, C, ldc, tile_cfg, k_splits, cus,
                                     stream, ctypes.byref(c), ctypes.byref(s)), "nf_gemm_bf16_noalloc")
    return c.value, s.value


# device-to-device copy of raw library memory into a torch tensor (plumbing)
_hip = None


def copy_device(dst_tensor, src_ptr: int, nbytes: int) -> None:
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.restype = ctypes.c_int
        _hip.hipMemcpy.argtypes = [vp, vp, ctypes.c_size_t, ctypes.c_int]
    rc = _hip.hipMemcpy(dst_tensor.data_ptr(), src_ptr, nbytes, 3)   # hipMemcpyDeviceToDevice
    if rc != 0:
        raise RuntimeError(f"hipMemcpy failed: {rc}")
