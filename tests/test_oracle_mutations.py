"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in the oracle (on the CPU, through monkeypatch:
the oracle's source is not touched) and checks that the whole-layer pin --
the scalar-loop layer written from the definition in test_oracle_pins -- no
longer agrees.  If a pin stopped discriminating (for example because a tiny
problem made some term vanish), the corresponding case here would fail.
"""
import numpy as np
import pytest

import oracle
import oracle.layer as OL
from tests.test_oracle_pins import _brute_force_layer, _tiny_problem

_orig = {name: getattr(OL, name) for name in
         ("rope", "rope_cos_sin", "rmsnorm", "attention_weights", "paged_attention", "silu", "swiglu_ffn",
          "kv_append", "page_slots", "moe_route")}


# ---------------------------------------------------------------- mutants

def rope_sin_sign(v, pos, theta):
    d = v.shape[-1]
    half = d // 2
    cos, sin = OL.rope_cos_sin(pos, d, theta)
    cos, sin = cos[:, None, :], sin[:, None, :]
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * cos + b * sin, -a * sin + b * cos], axis=-1)


def rope_interleaved(v, pos, theta):
    d = v.shape[-1]
    cos, sin = OL.rope_cos_sin(pos, d, theta)
    cos, sin = cos[:, None, :], sin[:, None, :]
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = a * sin + b * cos
    return out


def rope_cos_sin_half_frequency(pos, head_dim, theta):
    half = head_dim // 2
    inv_freq = theta ** (-1.0 * np.arange(half, dtype=np.float64) / head_dim)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang), np.sin(ang)


def rmsnorm_no_gain(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rmsnorm_eps_outside(x, g, eps):
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * g


def attention_no_scale(q, keys):
    s = q @ keys.T
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention_excludes_own_key(q, keys):
    """Causal window one short: the newest key is left out (when there is
    an older one)."""
    w = _orig["attention_weights"](q, keys)
    if keys.shape[0] > 1:
        w[:, -1] = 0.0
        w = w / w.sum(axis=-1, keepdims=True)
    return w


def paged_attention_gqa_modulo(q_rot, k_pool, v_pool, req_q_start, req_q_len, pos,
                               page_indptr, page_indices, page_size, n_kv_heads):
    """Query head h read from KV head h % nkv instead of h // G."""
    T, nq, d = q_rot.shape
    out = np.zeros_like(q_rot)
    for r in range(len(req_q_len)):
        t0, n = int(req_q_start[r]), int(req_q_len[r])
        last = int(pos[t0 + n - 1])
        pages, slots = OL.page_slots(page_indptr, page_indices, r, last + 1, page_size)
        for h in range(nq):
            kh = h % n_kv_heads
            K = k_pool[pages, kh, slots]
            V = v_pool[pages, kh, slots]
            for t in range(t0, t0 + n):
                p = int(pos[t])
                out[t, h] = OL.attention_weights(q_rot[t, h:h + 1], K[:p + 1])[0] @ V[:p + 1]
    return out


def silu_is_sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def swiglu_gate_up_swapped(h, w_gate, w_up, w_down):
    return _orig["swiglu_ffn"](h, w_up, w_gate, w_down)


def kv_append_next_slot(k_pool, v_pool, k_new, v_new, tok_req, pos, page_indptr, page_indices, page_size, dtype):
    for t in range(k_new.shape[0]):
        r, p = tok_req[t], int(pos[t])
        page = page_indices[page_indptr[r] + p // page_size]
        slot = (p + 1) % page_size
        k_pool[page, :, slot] = OL.store_round(k_new[t], dtype)
        v_pool[page, :, slot] = OL.store_round(v_new[t], dtype)


def kv_append_kv_swapped(k_pool, v_pool, k_new, v_new, tok_req, pos, page_indptr, page_indices, page_size, dtype):
    """Key and value written to each other's pool."""
    _orig["kv_append"](v_pool, k_pool, k_new, v_new, tok_req, pos, page_indptr, page_indices, page_size, dtype)


def page_slots_ignore_table(page_indptr, page_indices, r, n_keys, page_size):
    j = np.arange(n_keys)
    return page_indptr[r] + j // page_size, j % page_size


def moe_route_full_softmax(logits, top_k):
    idx, w, perm, offsets = _orig["moe_route"](logits, top_k)
    full = np.exp(logits - logits.max(axis=-1, keepdims=True))
    full /= full.sum(axis=-1, keepdims=True)
    return idx, np.take_along_axis(full, idx, axis=-1), perm, offsets


def moe_route_smallest(logits, top_k):
    return _orig["moe_route"](-logits, top_k)


DENSE = [
    ("rope", rope_sin_sign),
    ("rope", rope_interleaved),
    ("rope_cos_sin", rope_cos_sin_half_frequency),
    ("rmsnorm", rmsnorm_no_gain),
    ("rmsnorm", rmsnorm_eps_outside),
    ("attention_weights", attention_no_scale),
    ("attention_weights", attention_excludes_own_key),
    ("paged_attention", paged_attention_gqa_modulo),
    ("silu", silu_is_sigmoid),
    ("swiglu_ffn", swiglu_gate_up_swapped),
    ("kv_append", kv_append_next_slot),
    ("kv_append", kv_append_kv_swapped),
    ("page_slots", page_slots_ignore_table),
]
MOE = [
    ("moe_route", moe_route_full_softmax),
    ("moe_route", moe_route_smallest),
]


@pytest.fixture(scope="module")
def dense_case():
    rng = np.random.Generator(np.random.PCG64(21))
    shape, w, batch, kp, vp = _tiny_problem(rng)
    return (shape, w, batch, kp, vp), _brute_force_layer(shape, w, batch, kp, vp)[0]


@pytest.fixture(scope="module")
def moe_case():
    rng = np.random.Generator(np.random.PCG64(22))
    shape, w, batch, kp, vp = _tiny_problem(rng, E=4, top_k=2, pos0=(3, 1), qlen=(1, 3))
    return (shape, w, batch, kp, vp), _brute_force_layer(shape, w, batch, kp, vp)[0]


def _agrees(case):
    (shape, w, batch, kp, vp), want = case
    got = oracle.layer_step(shape, w, batch, kp, vp, pool_dtype="f64")["out"]
    return np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_unmutated_oracle_agrees(dense_case, moe_case):
    assert _agrees(dense_case) and _agrees(moe_case)


@pytest.mark.parametrize("name,mutant", DENSE, ids=[m.__name__ for _, m in DENSE])
def test_dense_mutant_is_caught(monkeypatch, dense_case, name, mutant):
    monkeypatch.setattr(OL, name, mutant)
    assert not _agrees(dense_case), f"pin did not catch {mutant.__name__}"


@pytest.mark.parametrize("name,mutant", MOE, ids=[m.__name__ for _, m in MOE])
def test_moe_mutant_is_caught(monkeypatch, moe_case, name, mutant):
    monkeypatch.setattr(OL, name, mutant)
    assert not _agrees(moe_case), f"pin did not catch {mutant.__name__}"
