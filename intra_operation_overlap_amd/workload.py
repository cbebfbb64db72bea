"""Seeded synthetic inputs for one decoder-layer step.

This module only draws random numbers and lays out batches; it holds none of
the layer's arithmetic. Both the GPU path and the CPU oracle are fed from it.

Workload shapes follow the model families the Nanoflow README names among its
supported and evaluated models (Llama-2/3 and Mixtral 8x7B, "News" and
"Abstract" of the README on the ossradar page) and the constant 1024-in /
512-out load of its "Feasibility" benchmark: decode requests mid-generation
hold 1024..1536 cached tokens.  The traces the pages evaluate on are not
available, so uniform context ranges stand in for them.

Recipe (same for every config):
  * host metadata: numpy PCG64 seeded with ``seed``; per-request context
    lengths uniform over an inclusive integer range; decode requests first,
    the prefill chunk (if any) last; pages per request
    ceil((pos0 + q_len) / page_size); pool pages = sum + ceil(5% of sum) + 1;
    pages handed out from one seeded permutation of the pool, request by
    request;
  * tensors: torch generators on the target device, one stream per tensor
    (seed * 1000 + tensor id); weights N(0, 0.02), norm gains U[0.5, 1.5],
    activations and every pool slot N(0, 1), router logits N(0, 1) in fp32;
    bf16 tensors are drawn in fp32 and rounded to nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

PAGE_SIZE = 16


@dataclasses.dataclass(frozen=True)
class Shape:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    n_experts: int = 1
    top_k: int = 1
    dtype: str = "bf16"          # "bf16" or "f32"
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0
    page_size: int = PAGE_SIZE

    @property
    def qkv_cols(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def as_dict(self) -> dict:
        return dataclasses.asdict(self)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    n_decode: int
    ctx_range: Tuple[int, int]            # inclusive range of cached tokens
    prefill: Optional[Tuple[int, int]]    # (chunk start position, chunk length)
    seed: int
    plan_sizes: Optional[Tuple[int, ...]] = None   # fixed nano-batch sizes, or None
    description: str = ""


LLAMA3_8B = dict(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=14336)

WORKLOADS: Dict[str, Workload] = {
    "c1": Workload(
        "c1", Shape(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=688,
                    dtype="f32", rope_theta=1e4),
        n_decode=16, ctx_range=(32, 128), prefill=None, seed=1001, plan_sizes=(8, 8),
        description="tiny fp32 layer, 16 decode requests, 2 nano-batches of 8"),
    "c2": Workload(
        "c2", Shape(**LLAMA3_8B, dtype="bf16", rope_theta=5e5),
        n_decode=64, ctx_range=(512, 512), prefill=None, seed=1002, plan_sizes=(64,),
        description="Llama-3-8B-shaped layer, 64 decode requests at context 512, one batch"),
    "c3": Workload(
        "c3", Shape(**LLAMA3_8B, dtype="bf16", rope_theta=5e5),
        n_decode=768, ctx_range=(1024, 1536), prefill=(768, 256), seed=1003,
        description="Llama-3-8B-shaped layer, 768 decode requests (context 1024-1536) "
                    "+ the last 256-token prefill chunk of a 1024-token prompt"),
    "c4": Workload(
        "c4", Shape(hidden=8192, n_q_heads=8, n_kv_heads=1, head_dim=128, ffn=3584,
                    dtype="bf16", rope_theta=1e4),
        n_decode=1536, ctx_range=(1024, 1536), prefill=(512, 512), seed=1004,
        description="Llama-2-70B 1/8 tensor-parallel shard, 1536 decode requests "
                    "(context 1024-1536) + a 512-token prefill chunk"),
    "c5": Workload(
        "c5", Shape(**LLAMA3_8B, n_experts=8, top_k=2, dtype="bf16", rope_theta=1e6),
        n_decode=512, ctx_range=(512, 2048), prefill=None, seed=1005,
        description="Mixtral-8x7B-shaped MoE layer (8 experts, top-2), "
                    "512 decode requests (context 512-2048)"),
}


@dataclasses.dataclass
class Batch:
    """Host-side description of one step's batch (all int32 numpy arrays)."""
    n_tokens: int
    req_q_start: np.ndarray
    req_q_len: np.ndarray
    req_pos0: np.ndarray
    pos: np.ndarray
    page_indptr: np.ndarray
    page_indices: np.ndarray
    n_pages: int

    @property
    def n_requests(self) -> int:
        return int(self.req_q_len.shape[0])


def build_batch(req_pos0: List[int], req_q_len: List[int], page_size: int,
                rng: np.random.Generator, spare_frac: float = 0.05) -> Batch:
    """Lay out requests (tokens contiguous per request) and hand out pages from a
    seeded permutation of the pool."""
    pos0 = np.asarray(req_pos0, dtype=np.int64)
    qlen = np.asarray(req_q_len, dtype=np.int64)
    q_start = np.concatenate([[0], np.cumsum(qlen)[:-1]]) if len(qlen) else np.zeros(0, np.int64)
    n_tokens = int(qlen.sum())
    pages_per_req = (pos0 + qlen + page_size - 1) // page_size
    used = int(pages_per_req.sum())
    n_pages = used + int(math.ceil(spare_frac * used)) + 1
    perm = rng.permutation(n_pages)
    indptr = np.concatenate([[0], np.cumsum(pages_per_req)])
    indices = perm[:used]
    pos = np.concatenate([np.arange(p, p + q) for p, q in zip(pos0, qlen)]) if n_tokens else np.zeros(0, np.int64)
    i32 = lambda a: np.ascontiguousarray(a, dtype=np.int32)
    return Batch(n_tokens, i32(q_start), i32(qlen), i32(pos0), i32(pos), i32(indptr),
                 i32(indices), n_pages)


def make_batch(wl: Workload, n_decode: Optional[int] = None) -> Batch:
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    nd = wl.n_decode if n_decode is None else n_decode
    lo, hi = wl.ctx_range
    ctx = rng.integers(lo, hi + 1, size=nd)
    pos0 = list(ctx)
    qlen = [1] * nd
    if wl.prefill is not None:
        pos0.append(wl.prefill[0])
        qlen.append(wl.prefill[1])
    return build_batch(pos0, qlen, wl.shape.page_size, rng)


def sub_batch(batch: Batch, requests: List[int]) -> Tuple[Batch, np.ndarray]:
    """Batch holding only ``requests`` (same pool pages, same positions).

    Returns the sub-batch and the token rows of the full batch it covers."""
    pos0 = batch.req_pos0[requests]
    qlen = batch.req_q_len[requests]
    rows = np.concatenate([np.arange(batch.req_q_start[r], batch.req_q_start[r] + batch.req_q_len[r])
                           for r in requests]).astype(np.int64)
    pages = [batch.page_indices[batch.page_indptr[r]:batch.page_indptr[r + 1]] for r in requests]
    indptr = np.concatenate([[0], np.cumsum([len(p) for p in pages])]).astype(np.int32)
    q_start = np.concatenate([[0], np.cumsum(qlen)[:-1]]).astype(np.int32)
    b = Batch(int(qlen.sum()), q_start, qlen.astype(np.int32), pos0.astype(np.int32),
              batch.pos[rows].astype(np.int32), indptr,
              np.concatenate(pages).astype(np.int32), batch.n_pages)
    return b, rows


# ----------------------------------------------------------------------------
# tensors (torch is used here only as a seeded random source and as storage)
# ----------------------------------------------------------------------------

_TENSOR_IDS = {"attn_norm": 1, "w_qkv": 2, "w_o": 3, "ffn_norm": 4, "w_gate": 5,
               "w_up": 6, "w_down": 7, "x": 8, "k_pool": 9, "v_pool": 10,
               "router_logits": 11}


def _torch_dtype(shape: Shape):
    import torch
    return torch.bfloat16 if shape.dtype == "bf16" else torch.float32


def _gen(seed: int, name: str, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + _TENSOR_IDS[name])
    return g


def _draw(seed, name, dims, dist, dtype, device, chunk_elems=1 << 28):
    """Draw a tensor in fp32 chunks along dim 0 and store it in ``dtype``."""
    import torch
    g = _gen(seed, name, device)
    out = torch.empty(dims, dtype=dtype, device=device)
    flat = out.view(dims[0], -1) if len(dims) > 1 else out.view(-1, 1)
    row_elems = max(1, flat.shape[1])
    rows_per = max(1, chunk_elems // row_elems)
    for r0 in range(0, flat.shape[0], rows_per):
        r1 = min(flat.shape[0], r0 + rows_per)
        n = (r1 - r0) * flat.shape[1]
        if dist[0] == "normal":
            v = torch.randn(n, generator=g, device=device, dtype=torch.float32) * dist[1]
        else:
            lo, hi = dist[1], dist[2]
            v = torch.rand(n, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo
        flat[r0:r1].copy_(v.view(r1 - r0, -1).to(dtype))
    return out


def make_weights(wl: Workload, device="cpu", seed: Optional[int] = None) -> Dict[str, "torch.Tensor"]:
    """Layer weights in the boundary's documented layouts:
    attn_norm/ffn_norm [H]; w_qkv [(nq+2nkv)*d, H]; w_o [H, nq*d];
    w_gate, w_up [E, F, H]; w_down [E, H, F] (each matrix row-major,
    output features first)."""
    s = wl.shape
    seed = wl.seed if seed is None else seed
    dt = _torch_dtype(s)
    H, F, E = s.hidden, s.ffn, s.n_experts
    return {
        "attn_norm": _draw(seed, "attn_norm", (H,), ("uniform", 0.5, 1.5), dt, device),
        "w_qkv": _draw(seed, "w_qkv", (s.qkv_cols, H), ("normal", 0.02), dt, device),
        "w_o": _draw(seed, "w_o", (H, s.n_q_heads * s.head_dim), ("normal", 0.02), dt, device),
        "ffn_norm": _draw(seed, "ffn_norm", (H,), ("uniform", 0.5, 1.5), dt, device),
        "w_gate": _draw(seed, "w_gate", (E, F, H), ("normal", 0.02), dt, device),
        "w_up": _draw(seed, "w_up", (E, F, H), ("normal", 0.02), dt, device),
        "w_down": _draw(seed, "w_down", (E, H, F), ("normal", 0.02), dt, device),
    }


def make_activations(wl: Workload, batch: Batch, device="cpu", seed: Optional[int] = None):
    """x [T, H] and, for MoE layers, router logits [T, E] (fp32)."""
    import torch
    s = wl.shape
    seed = wl.seed if seed is None else seed
    out = {"x": _draw(seed, "x", (batch.n_tokens, s.hidden), ("normal", 1.0), _torch_dtype(s), device)}
    if s.n_experts > 1:
        out["router_logits"] = _draw(seed, "router_logits", (batch.n_tokens, s.n_experts),
                                     ("normal", 1.0), torch.float32, device)
    return out


def make_pool(wl: Workload, n_pages: int, device="cpu", seed: Optional[int] = None):
    """The plain paged K and V caches [P, nkv, page_size, d] (page, KV head,
    key slot, dimension); every element N(0, 1), cached prefix values and
    never-written slots alike."""
    s = wl.shape
    seed = wl.seed if seed is None else seed
    dt = _torch_dtype(s)
    dims = (n_pages, s.n_kv_heads, s.page_size, s.head_dim)
    k = _draw(seed, "k_pool", dims, ("normal", 1.0), dt, device)
    v = _draw(seed, "v_pool", dims, ("normal", 1.0), dt, device)
    return k, v


def layer_flops_per_token(shape: Shape) -> float:
    """2 x active weight parameters per token (dense GEMMs only)."""
    H, F = shape.hidden, shape.ffn
    attn = shape.qkv_cols * H + H * shape.n_q_heads * shape.head_dim
    ffn = 3 * H * F * (shape.top_k if shape.n_experts > 1 else 1)
    return 2.0 * (attn + ffn)


def to_f64(t) -> np.ndarray:
    """Exact fp64 copy of a (bf16 or fp32) torch tensor."""
    import torch
    return t.detach().to("cpu", torch.float64).numpy()
