"""CPU fp64 oracle for one decoder-layer step over a mixed prefill+decode batch.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library and imports
nothing from the product package: every input arrives as numpy arrays.

What it computes.  Nanoflow reaches the result of the unsplit layer: splitting
a batch into nano-batches only duplicates each operation over a portion of the
rows so that the portions can overlap (abstract on the codewithpapers page
"NanoFlow: Towards Optimal Large Language Model Serving Throughput"; README
"Introduction" on the ossradar page).  So the oracle is the plain definition of
the layer, computed once over the whole batch, in fp64, with no blocking,
fusion or reordering beyond a library matmul per projection.

The layer is the Llama-family pre-norm block of the model families the README
lists (README "News"; Mixtral 8x7B in the abstract): RMSNorm -> QKV projection
-> rotary embedding (rotate-half pairing) -> paged KV append -> causal GQA
attention over the paged cache -> O projection + residual -> RMSNorm ->
SwiGLU FFN (or a top-k mixture of SwiGLU experts) + residual.  The paged KV
cache is the PagedAttention block-pool substrate the pages name (p1 "How it
differs from vLLM and TensorRT-LLM"; p4 References).

Layouts (the weights as the boundary documents them, restated here
independently): w_qkv [(nq + 2 nkv) d, H]: output columns are Q heads, then
K heads, then V heads, each head's d columns contiguous; w_o [H, nq d];
w_gate, w_up [E, F, H]; w_down [E, H, F].  The K and V pools are the plain
paged cache [P, nkv, 16, d]: pool page, KV head, key slot, dimension.
Request r's logical page i is pool page page_indices[page_indptr[r] + i];
position p lives in logical page p // 16 at slot p % 16.  How a device lays
out a block inside its memory is not the oracle's concern: the tests convert
a device pool to this layout before comparing.

The one rounding the oracle applies is the write into the KV pool, which is a
typed data structure (bf16 round-to-nearest-even or fp32); keys and values of
the current step are read back from the pool, as the GPU does.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np


# ----------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------

def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of each fp64 element, as fp64.

    bf16 keeps 8 significant bits (7 stored + the implicit one) and fp32's
    exponent range.  Rounding is done on the fp64 value directly (no detour
    through fp32), by scaling each element so that its bf16 ulp is 1 and using
    numpy's round-half-even."""
    a = np.asarray(a, dtype=np.float64)
    out = np.array(a, copy=True)
    finite = np.isfinite(a) & (a != 0)
    m, e = np.frexp(a[finite])             # a = m * 2**e, 0.5 <= |m| < 1
    # bf16 normals: 8 significant bits -> ulp = 2**(e - 8); subnormals share
    # the fixed ulp 2**-133 (fp32's minimum exponent -126 less 7 bits).
    ulp_exp = np.maximum(e - 8, -133)
    out[finite] = np.round(np.ldexp(a[finite], -ulp_exp)) * np.ldexp(1.0, ulp_exp)
    big = np.abs(out) >= 2.0 ** 128      # rounded past the largest finite bf16
    out[big] = np.sign(out[big]) * np.inf
    return out


def round_to_f32(a: np.ndarray) -> np.ndarray:
    """Nearest fp32 value (ties to even; past the largest finite fp32 value
    by half an ulp or more: infinity) of each fp64 element, as fp64, through
    numpy's IEEE-754 conversion."""
    with np.errstate(over="ignore"):
        return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def store_round(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(a)
    if dtype == "f32":
        return round_to_f32(a)
    if dtype == "f64":          # exact pool, used only by invariance checks
        return np.asarray(a, dtype=np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# layer pieces
# ----------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Row-wise RMS normalisation with a per-feature gain:
    x / sqrt(mean(x^2) + eps) * g."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_cos_sin(pos: np.ndarray, head_dim: int, theta: float):
    """Angles p * theta^(-2j/d) for j < d/2, per position."""
    half = head_dim // 2
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / head_dim)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def rope(v: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding, rotate-half pairing: element j pairs with j + d/2 and
    the pair (a, b) turns by the angle of position p at frequency j.
    v: [T, heads, d]."""
    d = v.shape[-1]
    half = d // 2
    cos, sin = rope_cos_sin(pos, d, theta)
    cos = cos[:, None, :]
    sin = sin[:, None, :]
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(h: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray):
    """SwiGLU FFN for one expert: act = silu(h Wg^T) * (h Wu^T); y = act Wd^T."""
    act = silu(h @ w_gate.T) * (h @ w_up.T)
    return act, act @ w_down.T


PAGE = 16


def page_slots(page_indptr, page_indices, r: int, n_keys: int, page_size: int):
    """(pool page, slot) of each of request r's first n_keys positions."""
    j = np.arange(n_keys)
    pages = np.asarray(page_indices)[page_indptr[r] + j // page_size]
    return pages, j % page_size


def kv_append(k_pool, v_pool, k_new, v_new, tok_req, pos, page_indptr, page_indices,
              page_size: int, dtype: str) -> None:
    """Write each token's rotated key and its value into the pool slot of its
    position, rounded to the pool's storage type.  k_new, v_new: [T, nkv, d];
    pools [P, nkv, page_size, d]."""
    assert page_size == PAGE
    for t in range(k_new.shape[0]):
        r = tok_req[t]
        p = int(pos[t])
        page = page_indices[page_indptr[r] + p // page_size]
        slot = p % page_size
        k_pool[page, :, slot, :] = store_round(k_new[t], dtype)
        v_pool[page, :, slot, :] = store_round(v_new[t], dtype)


def attention_weights(q: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """softmax over keys of q.k / sqrt(d), max-subtracted.  q: [G, d]; keys: [L, d]."""
    s = q @ keys.T / math.sqrt(q.shape[-1])
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def paged_attention(q_rot, k_pool, v_pool, req_q_start, req_q_len, pos,
                    page_indptr, page_indices, page_size: int, n_kv_heads: int):
    """Causal GQA attention read through the page tables.

    Query head h of a token at position p attends to keys 0..p of its own
    request, held by KV head h // (nq / nkv).  Pools [P, nkv, page_size, d].
    Returns [T, nq, d]."""
    T, nq, d = q_rot.shape
    G = nq // n_kv_heads
    assert page_size == PAGE
    out = np.zeros_like(q_rot)
    for r in range(len(req_q_len)):
        t0, n = int(req_q_start[r]), int(req_q_len[r])
        if n == 0:
            continue
        last = int(pos[t0 + n - 1])
        pages, slots = page_slots(page_indptr, page_indices, r, last + 1, page_size)
        for kh in range(n_kv_heads):
            K = k_pool[pages, kh, slots]      # [L, d]
            V = v_pool[pages, kh, slots]      # [L, d]
            for t in range(t0, t0 + n):
                p = int(pos[t])
                w = attention_weights(q_rot[t, kh * G:(kh + 1) * G], K[:p + 1])
                out[t, kh * G:(kh + 1) * G] = w @ V[:p + 1]
    return out


def moe_route(logits: np.ndarray, top_k: int):
    """Top-k experts per token (larger logit first; equal logits: lower expert
    index first), gate weights = softmax over the selected logits, and the
    assignments (token t, slot s) -> id t*top_k + s counting-sorted by expert
    (stable in id).  Returns idx [T,k], w [T,k], perm [T*k], offsets [E+1]."""
    T, E = logits.shape
    idx = np.zeros((T, top_k), dtype=np.int64)
    w = np.zeros((T, top_k), dtype=np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:top_k]
        idx[t] = order
        sel = np.array([float(logits[t, e]) for e in order])
        ex = np.exp(sel - sel.max())
        w[t] = ex / ex.sum()
    counts = np.bincount(idx.reshape(-1), minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.zeros(T * top_k, dtype=np.int64)
    fill = offsets[:-1].copy()
    for a in range(T * top_k):
        e = idx.reshape(-1)[a]
        perm[fill[e]] = a
        fill[e] += 1
    return idx, w, perm, offsets


# ----------------------------------------------------------------------------
# the whole step
# ----------------------------------------------------------------------------

def layer_step(shape: Dict, w: Dict[str, np.ndarray], batch: Dict[str, np.ndarray],
               k_pool: np.ndarray, v_pool: np.ndarray,
               pool_dtype: Optional[str] = None) -> Dict[str, np.ndarray]:
    """One decoder-layer step, unsplit, in fp64.

    shape: hidden, n_q_heads, n_kv_heads, head_dim, ffn, n_experts, top_k,
           dtype, rms_eps, rope_theta, page_size
    w:     attn_norm, w_qkv, w_o, ffn_norm, w_gate, w_up, w_down (fp64 values)
    batch: x [T,H], req_q_start, req_q_len, req_pos0, pos, page_indptr,
           page_indices, optional router_logits [T,E]
    k_pool, v_pool: fp64 values of the pool before the step (not modified).

    Returns out, x1, q_rot, attn, act (dense layers), route (MoE layers) and
    the pool after the step."""
    H = shape["hidden"]
    nq, nkv, d = shape["n_q_heads"], shape["n_kv_heads"], shape["head_dim"]
    S = shape["page_size"]
    eps, theta = shape["rms_eps"], shape["rope_theta"]
    E, top_k = shape.get("n_experts", 1), shape.get("top_k", 1)
    pool_dtype = pool_dtype or shape["dtype"]

    x = np.asarray(batch["x"], dtype=np.float64)
    T = x.shape[0]
    q_start = np.asarray(batch["req_q_start"])
    q_len = np.asarray(batch["req_q_len"])
    pos0 = np.asarray(batch["req_pos0"])
    pos = np.asarray(batch["pos"])
    indptr = np.asarray(batch["page_indptr"])
    indices = np.asarray(batch["page_indices"])
    tok_req = np.repeat(np.arange(len(q_len)), q_len)
    for r in range(len(q_len)):        # positions follow from pos0 (boundary contract)
        assert np.array_equal(pos[q_start[r]:q_start[r] + q_len[r]],
                              pos0[r] + np.arange(q_len[r]))

    # attention branch
    h = rmsnorm(x, w["attn_norm"], eps)
    qkv = h @ w["w_qkv"].T
    q = qkv[:, :nq * d].reshape(T, nq, d)
    k = qkv[:, nq * d:(nq + nkv) * d].reshape(T, nkv, d)
    v = qkv[:, (nq + nkv) * d:].reshape(T, nkv, d)
    q_rot = rope(q, pos, theta)
    k_rot = rope(k, pos, theta)
    kp = np.array(k_pool, dtype=np.float64, copy=True)
    vp = np.array(v_pool, dtype=np.float64, copy=True)
    kv_append(kp, vp, k_rot, v, tok_req, pos, indptr, indices, S, pool_dtype)
    o = paged_attention(q_rot, kp, vp, q_start, q_len, pos, indptr, indices, S, nkv)
    attn = o.reshape(T, nq * d)
    x1 = x + attn @ w["w_o"].T

    # FFN branch
    h2 = rmsnorm(x1, w["ffn_norm"], eps)
    res = {"q_rot": q_rot, "attn": attn, "x1": x1, "k_pool": kp, "v_pool": vp}
    if E == 1:
        act, y = swiglu_ffn(h2, w["w_gate"][0], w["w_up"][0], w["w_down"][0])
        res["act"] = act
        res["out"] = x1 + y
    else:
        idx, gw, perm, offsets = moe_route(np.asarray(batch["router_logits"], dtype=np.float64), top_k)
        y = np.zeros_like(x1)
        for e in range(E):
            toks, slots = np.nonzero(idx == e)
            if len(toks) == 0:
                continue
            _, ye = swiglu_ffn(h2[toks], w["w_gate"][e], w["w_up"][e], w["w_down"][e])
            y[toks] += gw[toks, slots][:, None] * ye
        res["route"] = {"idx": idx, "w": gw, "perm": perm, "offsets": offsets}
        res["out"] = x1 + y
    return res


def layer_step_split(shape, w, batch, k_pool, v_pool, sizes, pool_dtype=None):
    """The same step run as consecutive nano-batches of ``sizes`` tokens, each
    a full pass of the layer over its rows, the pool carried from one to the
    next.  Requests may be cut between nano-batches; each piece keeps its
    positions and page table."""
    assert sum(sizes) == len(batch["pos"])
    q_start = np.asarray(batch["req_q_start"])
    q_len = np.asarray(batch["req_q_len"])
    kp, vp = k_pool, v_pool
    outs = []
    t0 = 0
    for n in sizes:
        t1 = t0 + n
        reqs, qs, ql, p0 = [], [], [], []
        for r in range(len(q_len)):
            a, b = max(t0, q_start[r]), min(t1, q_start[r] + q_len[r])
            if a < b:
                reqs.append(r)
                qs.append(a - t0)
                ql.append(b - a)
                p0.append(int(batch["pos"][a]))
        ip = np.asarray(batch["page_indptr"])
        pages = [np.asarray(batch["page_indices"])[ip[r]:ip[r + 1]] for r in reqs]
        sub = {
            "x": np.asarray(batch["x"])[t0:t1],
            "req_q_start": np.array(qs), "req_q_len": np.array(ql), "req_pos0": np.array(p0),
            "pos": np.asarray(batch["pos"])[t0:t1],
            "page_indptr": np.concatenate([[0], np.cumsum([len(p) for p in pages])]),
            "page_indices": np.concatenate(pages) if pages else np.zeros(0, np.int64),
        }
        if "router_logits" in batch:
            sub["router_logits"] = np.asarray(batch["router_logits"])[t0:t1]
        r = layer_step(shape, w, sub, kp, vp, pool_dtype)
        kp, vp = r["k_pool"], r["v_pool"]
        outs.append(r)
        t0 = t1
    merged = {key: np.concatenate([o[key] for o in outs]) for key in ("out", "x1", "q_rot", "attn")}
    merged["k_pool"], merged["v_pool"] = kp, vp
    return merged
