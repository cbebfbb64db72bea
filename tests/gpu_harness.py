"""Shared set-up for the GPU parity tests: seeded inputs on the device, the
library objects over them, and oracle inputs built from the same tensors.
(Expected values always come from the oracle, never from the GPU path.)"""
from __future__ import annotations

import dataclasses
import sys
import time
from typing import List, Optional

import numpy as np
import torch

import oracle
from intra_operation_overlap_amd import binding as B
from intra_operation_overlap_amd import workload as W


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


@dataclasses.dataclass
class Setup:
    wl: W.Workload
    batch: W.Batch
    weights: dict
    acts: dict
    k: torch.Tensor          # the pool's own buffers (the library's block layout)
    v: torch.Tensor
    out: torch.Tensor
    layer: B.Layer
    pool: B.KVPool
    hb: B.HostBatch
    max_tokens: int
    max_pos: int
    k_plain: torch.Tensor    # the generator's paged cache [P][nkv][16][d]: the oracle's input
    v_plain: torch.Tensor


def setup(wl: W.Workload, batch: Optional[W.Batch] = None, max_tokens: Optional[int] = None,
          max_pos: Optional[int] = None, weights=None) -> Setup:
    dev = "cuda"
    batch = batch if batch is not None else W.make_batch(wl)
    weights = weights if weights is not None else W.make_weights(wl, dev)
    acts = W.make_activations(wl, batch, dev)
    kp, vp = W.make_pool(wl, batch.n_pages, dev)
    mt = max_tokens or max(batch.n_tokens, 1)
    if max_pos is not None:
        mp = max_pos
    else:
        mp = int(batch.pos.max()) + 1 if batch.n_tokens else 16
    layer = B.Layer(wl.shape, weights, mt, mp)
    pool = B.KVPool.from_plain(layer, kp, vp, stream())
    torch.cuda.synchronize()
    out = torch.empty_like(acts["x"])
    hb = B.HostBatch(batch, acts["x"].data_ptr(), out.data_ptr(),
                     acts["router_logits"].data_ptr() if "router_logits" in acts else None)
    return Setup(wl, batch, weights, acts, pool.k, pool.v, out, layer, pool, hb, mt, mp, kp, vp)


def pool_plain(S: Setup):
    """The pool's current contents as plain [P][nkv][16][d] tensors (read back
    through nf_kv_pool_export)."""
    k, v = S.pool.to_plain(stream())
    torch.cuda.synchronize()
    return k, v


def stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def run_step(S: Setup) -> None:
    S.layer.step(S.pool, S.hb, stream())
    torch.cuda.synchronize()


def intermediate(S: Setup, which: int, rows: int, cols: int, dtype) -> torch.Tensor:
    ptr, stride = S.layer.intermediate(which)
    assert stride == cols
    t = torch.empty(rows, cols, dtype=dtype, device="cuda")
    B.copy_device(t, ptr, t.numel() * t.element_size())
    return t


def f64(t: torch.Tensor) -> np.ndarray:
    return W.to_f64(t)


def weights_np(S: Setup) -> dict:
    """Exact values of the weights; float32 arrays hold bf16 values exactly and
    numpy promotes them to fp64 inside the oracle's products."""
    return {k: v.detach().to("cpu", torch.float32).numpy() for k, v in S.weights.items()}


def oracle_subset(S: Setup, requests: List[int], w_np: Optional[dict] = None):
    """Runs the oracle on the given requests only (rows are independent), on
    the generator's paged cache (the pool before the step).  Pool pages of
    those requests are gathered into a compact pool.
    Returns (oracle result, token rows of the full batch, page map)."""
    sub, rows = W.sub_batch(S.batch, requests)
    pages = np.asarray(sub.page_indices, np.int64)
    remap = np.arange(len(pages))
    kp = f64(S.k_plain[torch.as_tensor(pages, device=S.k_plain.device)])
    vp = f64(S.v_plain[torch.as_tensor(pages, device=S.v_plain.device)])
    x = f64(S.acts["x"][torch.as_tensor(rows, device="cuda")])
    bd = dict(x=x, req_q_start=sub.req_q_start, req_q_len=sub.req_q_len, req_pos0=sub.req_pos0,
              pos=sub.pos, page_indptr=sub.page_indptr, page_indices=remap)
    if "router_logits" in S.acts:
        bd["router_logits"] = f64(S.acts["router_logits"][torch.as_tensor(rows, device="cuda")])
    res = oracle.layer_step(S.wl.shape.as_dict(), w_np if w_np is not None else weights_np(S), bd, kp, vp)
    return res, rows, pages


def normwise(g: np.ndarray, r: np.ndarray) -> float:
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    den = np.max(np.abs(r)) if r.size else 1.0
    return float(np.max(np.abs(g - r)) / den) if r.size else 0.0


def storage_ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """One unit in the last place of each |v| in the storage type (bf16: 8
    significant bits, fp32: 24)."""
    a = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - (7 if dtype == "bf16" else 23))


def rounding_allowance(stored_sum_gpu, stored_sum_ref, dtype) -> np.ndarray:
    """Round-to-nearest moves a sum by at most half an ulp of its binade.  The
    GPU's unrounded sum is not observable: it lies within that half ulp of
    the stored value, which may sit one binade above or below the fp64
    reference near a power of two, so the larger ulp of the two is taken."""
    return 0.5 * np.maximum(storage_ulp(stored_sum_gpu, dtype), storage_ulp(stored_sum_ref, dtype))


def delta_error(g_delta, r_delta, stored_sum_gpu, stored_sum_ref, dtype) -> float:
    """Normwise error of a residual branch recovered as (stored sum - input):
    the sum is held in the storage type, so each element may carry up to half
    a storage ulp of the sum on top of the branch's own error; that allowance
    is subtracted before normalising by the branch's largest magnitude."""
    r_delta = np.asarray(r_delta, np.float64)
    if not r_delta.size:
        return 0.0
    den = np.max(np.abs(r_delta))
    excess = np.abs(np.asarray(g_delta) - r_delta) - rounding_allowance(stored_sum_gpu, stored_sum_ref, dtype)
    return float(max(0.0, np.max(excess)) / den)


def raw_delta_bound(r_delta, stored_sum_ref, dtype, tol) -> float:
    """Bound on the plain normwise error of a branch recovered as (stored sum
    - input): the tolerance plus one storage ulp of the largest stored sum
    (half an ulp of rounding, doubled for a binade of slack), relative to
    the branch's largest magnitude."""
    r_delta = np.asarray(r_delta, np.float64)
    if not r_delta.size:
        return tol
    return tol + float(np.max(storage_ulp(stored_sum_ref, dtype))) / float(np.max(np.abs(r_delta)))


def elementwise(g: np.ndarray, r: np.ndarray) -> float:
    """Diagnostic: max |g - r| / (|r| + rms(r))."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    if not r.size:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    return float(np.max(np.abs(g - r) / (np.abs(r) + rms)))


def tolerance(wl: W.Workload) -> float:
    return 1e-4 if wl.shape.dtype == "f32" else 2e-2


def written_slots(batch: W.Batch, requests: Optional[List[int]] = None):
    """(page, slot) of every position the step writes, per token in batch order."""
    reqs = range(batch.n_requests) if requests is None else requests
    out = []
    for r in reqs:
        for i in range(batch.req_q_len[r]):
            p = batch.req_pos0[r] + i
            out.append((int(batch.page_indices[batch.page_indptr[r] + p // 16]), int(p % 16)))
    return out


def check_sentinel(S: Setup, k_after: torch.Tensor, v_after: torch.Tensor) -> None:
    """Every pool slot the step does not name must be bit-identical to the
    generator's cache (plain layouts on both sides)."""
    P = S.batch.n_pages
    mask = torch.ones(P, 16, dtype=torch.bool, device="cuda")
    ws = written_slots(S.batch)
    if ws:
        idx = torch.as_tensor(ws, device="cuda")
        mask[idx[:, 0], idx[:, 1]] = False
    kd = (k_after != S.k_plain).any(dim=-1).any(dim=1)     # [P, 16]
    vd = (v_after != S.v_plain).any(dim=-1).any(dim=1)
    assert not bool((kd & mask).any()), "K pool changed outside the written slots"
    assert not bool((vd & mask).any()), "V pool changed outside the written slots"


def compare_rows(S: Setup, res: dict, rows: np.ndarray, pages: np.ndarray, requests: List[int],
                 k_after: torch.Tensor, v_after: torch.Tensor) -> dict:
    """Errors of out, x1, the two branch deltas, q_rot, attn, act and the K/V
    values written for the given rows (normwise; the keys ending in _raw and
    _elem and the bound_ keys are diagnostics and bounds)."""
    s = S.wl.shape
    T = S.batch.n_tokens
    dt = torch.float32 if s.dtype == "f32" else torch.bfloat16
    tol = tolerance(S.wl)
    ridx = torch.as_tensor(rows, device="cuda")
    out = f64(S.out[ridx])
    x = f64(S.acts["x"][ridx])
    x1 = f64(intermediate(S, 2, T, s.hidden, dt)[ridx])
    q_rot = f64(intermediate(S, 0, T, s.n_q_heads * s.head_dim, dt)[ridx])
    attn = f64(intermediate(S, 1, T, s.n_q_heads * s.head_dim, dt)[ridx])
    errs = {
        "out": normwise(out, res["out"]),
        "x1": normwise(x1, res["x1"]),
        "d_attn": delta_error(x1 - x, res["x1"] - x, x1, res["x1"], s.dtype),
        "d_ffn": delta_error(out - x1, res["out"] - res["x1"], out, res["out"], s.dtype),
        "d_attn_raw": normwise(x1 - x, res["x1"] - x),
        "d_ffn_raw": normwise(out - x1, res["out"] - res["x1"]),
        "bound_d_attn_raw": raw_delta_bound(res["x1"] - x, res["x1"], s.dtype, tol),
        "bound_d_ffn_raw": raw_delta_bound(res["out"] - res["x1"], res["out"], s.dtype, tol),
        "q_rot": normwise(q_rot, res["q_rot"].reshape(len(rows), -1)),
        "attn": normwise(attn, res["attn"]),
        "out_elem": elementwise(out, res["out"]),
        "attn_elem": elementwise(attn, res["attn"]),
    }
    if s.n_experts == 1:
        act = f64(intermediate(S, 3, T, s.ffn, dt)[ridx])
        errs["act"] = normwise(act, res["act"])
        errs["act_elem"] = elementwise(act, res["act"])
    # K/V written: slot values of the sampled requests' new positions
    ws_full = written_slots(S.batch, requests)
    page_pos = {int(p): i for i, p in enumerate(pages)}     # pool page -> compact oracle page
    pg = torch.as_tensor([p for p, _ in ws_full], device="cuda")
    sl = torch.as_tensor([s_ for _, s_ in ws_full], device="cuda")
    kg = f64(k_after[pg, :, sl])                          # [n, nkv, d]
    vg = f64(v_after[pg, :, sl])
    kr = np.stack([res["k_pool"][page_pos[p], :, s_] for p, s_ in ws_full])
    vr = np.stack([res["v_pool"][page_pos[p], :, s_] for p, s_ in ws_full])
    errs["k_new"] = normwise(kg, kr)
    errs["v_new"] = normwise(vg, vr)
    return errs


def assert_errors(errs: dict, tol: float, where) -> None:
    """Every checked error within the tolerance, the raw branch deltas within
    their bound; diagnostics (_elem) are only reported."""
    for k, e in errs.items():
        if k.startswith("bound_") or k.endswith("_elem"):
            continue
        if k.endswith("_raw"):
            assert e <= errs["bound_" + k], (where, k, e, errs["bound_" + k])
        else:
            assert e <= tol, (where, k, e)
