"""Pins for the CPU oracle: closed forms, invariants, library routines and brute
force on tiny inputs, each chosen so that a plausible slip in the oracle (a
dropped term, a wrong sign or index, a transposed operand) fails one of them.
None of these re-types the oracle's own formula; the whole-layer check below is
a scalar-loop brute force written from the layer's definition."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import layer as L


RNG = np.random.Generator(np.random.PCG64(7))


# ---------------------------------------------------------------- rounding

def test_bf16_rounding_closed_forms():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -7), 3.0, 0.0,
                     2.0 ** -133, 2.0 ** -134, 2.0 ** -134 * 3])
    want = np.array([1.0, 1.0, 1 + 2 ** -6, -(1 + 2 ** -7), 3.0, 0.0,
                     2.0 ** -133, 0.0, 2.0 ** -132])
    assert np.array_equal(L.round_to_bf16(vals), want)
    assert np.isinf(L.round_to_bf16(np.array([3.4e38]))).all()


def test_f32_rounding_closed_forms():
    """fp32 keeps 24 significant bits, normals from 2^-126, subnormals in
    steps of 2^-149, largest finite (2 - 2^-23) 2^127."""
    u = 2.0 ** -23                       # ulp of [1, 2)
    big = (2 - u) * 2.0 ** 127
    vals = np.array([1.0, 1 + u / 2, 1 + 3 * u / 2, 1 + u / 2 + 2.0 ** -40, -(1 + u / 2),
                     2.0 ** -149, 2.0 ** -150, 3 * 2.0 ** -150, 2.0 ** -150 + 2.0 ** -170,
                     2.0 ** -126 * (1 + u / 2), big, big + 2.0 ** 103 * 0.999, big + 2.0 ** 103, 0.0, -0.0])
    want = np.array([1.0, 1.0, 1 + 2 * u, 1 + u, -1.0,
                     2.0 ** -149, 0.0, 2.0 ** -148, 2.0 ** -149,
                     2.0 ** -126, big, big, np.inf, 0.0, -0.0])
    got = L.round_to_f32(vals)
    assert np.array_equal(got, want)
    assert np.signbit(got[-1]) and not np.signbit(got[-2])
    # idempotent on fp32 values; monotone; result within half an ulp
    a = RNG.standard_normal(5000) * np.exp(RNG.uniform(-80, 80, 5000))
    r = L.round_to_f32(a)
    assert np.array_equal(L.round_to_f32(r), r)
    order = np.argsort(a)
    assert np.all(np.diff(r[order]) >= 0)
    m, e = np.frexp(a)
    half_ulp = np.ldexp(1.0, np.maximum(e - 24, -149) - 1)
    assert np.all(np.abs(r - a) <= half_ulp)


def test_bf16_rounding_matches_torch_on_fp32_values():
    a = (RNG.standard_normal(20000) * np.exp(RNG.uniform(-30, 30, 20000))).astype(np.float32)
    want = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(L.round_to_bf16(a.astype(np.float64)), want)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_row_closed_form():
    c, eps = 0.75, 1e-5
    g = RNG.uniform(0.5, 1.5, 16)
    out = oracle.rmsnorm(np.full((1, 16), c), g, eps)
    assert np.allclose(out[0], g * c / math.sqrt(c * c + eps), rtol=1e-14, atol=0)


def test_rmsnorm_scale_invariant_without_eps_and_unit_rms():
    x = RNG.standard_normal((3, 32))
    g = RNG.uniform(0.5, 1.5, 32)
    a = oracle.rmsnorm(x, g, 0.0)
    assert np.allclose(a, oracle.rmsnorm(7.5 * x, g, 0.0), rtol=1e-13)
    # with unit gain the output rows have root-mean-square exactly 1
    b = oracle.rmsnorm(x, np.ones(32), 0.0)
    assert np.allclose(np.sqrt((b * b).mean(axis=1)), 1.0, rtol=1e-14)


# ---------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity():
    v = RNG.standard_normal((1, 3, 16))
    assert np.array_equal(oracle.rope(v, np.array([0]), 1e4), v)


def test_rope_direction_closed_form():
    # d = 2: the pair (1, 0) at position p turns to (cos p, sin p) (frequency 1)
    for p in (1, 2, 5, 1000):
        out = oracle.rope(np.array([[[1.0, 0.0]]]), np.array([p]), 5e5)
        assert np.allclose(out[0, 0], [math.cos(p), math.sin(p)], rtol=0, atol=1e-15)


def test_rope_equals_complex_multiplication():
    d, theta = 32, 5e5
    pos = RNG.integers(0, 4096, 6)
    v = RNG.standard_normal((6, 2, d))
    z = v[..., :d // 2] + 1j * v[..., d // 2:]
    freq = np.array([theta ** (-2.0 * j / d) for j in range(d // 2)])
    zr = z * np.exp(1j * pos[:, None, None] * freq[None, None, :])
    got = oracle.rope(v, pos, theta)
    assert np.allclose(got[..., :d // 2], zr.real, atol=1e-12)
    assert np.allclose(got[..., d // 2:], zr.imag, atol=1e-12)


def test_rope_norm_and_relative_position():
    d, theta = 64, 1e4
    q, k = RNG.standard_normal((2, 1, 1, d))
    for p, s, delta in [(3, 10, 100), (900, 20, 7)]:
        rq = oracle.rope(q, np.array([p]), theta)
        rk = oracle.rope(k, np.array([s]), theta)
        rq2 = oracle.rope(q, np.array([p + delta]), theta)
        rk2 = oracle.rope(k, np.array([s + delta]), theta)
        assert abs(np.sum(rq * rk) - np.sum(rq2 * rk2)) < 1e-10
        assert abs(np.linalg.norm(rq) - np.linalg.norm(q)) < 1e-12


# ---------------------------------------------------------------- SwiGLU

def test_silu_special_values():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([40.0]))[0] - 40.0) < 1e-12
    assert abs(oracle.silu(np.array([-40.0]))[0]) < 1e-15
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15


def test_swiglu_ffn_matches_numpy_matmul_reading():
    h = RNG.standard_normal((3, 5))
    wg, wu = RNG.standard_normal((2, 4, 5))
    wd = RNG.standard_normal((5, 4))
    act, y = oracle.swiglu_ffn(h, wg, wu, wd)
    for t in range(3):
        for f in range(4):
            zg = sum(h[t, i] * wg[f, i] for i in range(5))
            zu = sum(h[t, i] * wu[f, i] for i in range(5))
            assert abs(act[t, f] - zg / (1 + math.exp(-zg)) * zu) < 1e-12
    assert np.allclose(y, act @ wd.T, rtol=1e-13)


# ---------------------------------------------------------------- paging

def _random_pages(lengths, page_size, rng, spare=3):
    need = [(n + page_size - 1) // page_size for n in lengths]
    P = sum(need) + spare
    perm = rng.permutation(P)
    indptr = np.concatenate([[0], np.cumsum(need)])
    return P, indptr, perm[:sum(need)]


def _contiguous_attention(q, K, V):
    """Brute force with scalar loops: q [d], K/V [L, d]."""
    d = len(q)
    s = [sum(q[i] * K[j, i] for i in range(d)) / math.sqrt(d) for j in range(len(K))]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = sum(e)
    return np.array([sum(e[j] * V[j, i] for j in range(len(K))) / z for i in range(d)])


def _fill_pool(P, nkv, S, d, rng):
    """Plain paged K and V pools [page][KV head][slot][dim]."""
    return rng.standard_normal((P, nkv, S, d)), rng.standard_normal((P, nkv, S, d))


def _kv(kp, vp, page, kh, slot, d):
    """Key and value vectors of one pool slot, read element by element."""
    return (np.array([kp[page, kh, slot, i] for i in range(d)]),
            np.array([vp[page, kh, slot, i] for i in range(d)]))


def test_paged_attention_equals_contiguous_brute_force():
    S, d, nkv, nq = 16, 32, 2, 4
    lengths = [1, 17, 40, 16]              # keys per decode request (position + 1)
    rng = np.random.Generator(np.random.PCG64(3))
    P, indptr, indices = _random_pages(lengths, S, rng)
    kp, vp = _fill_pool(P, nkv, S, d, rng)
    R = len(lengths)
    pos = np.array([n - 1 for n in lengths])
    q = rng.standard_normal((R, nq, d))
    got = oracle.paged_attention(q, kp, vp, np.arange(R), np.ones(R, int), pos, indptr, indices, S, nkv)
    for r, n in enumerate(lengths):
        pages = [indices[indptr[r] + j // S] for j in range(n)]
        for h in range(nq):
            kh = h // (nq // nkv)
            K = np.array([_kv(kp, vp, pages[j], kh, j % S, d)[0] for j in range(n)])
            V = np.array([_kv(kp, vp, pages[j], kh, j % S, d)[1] for j in range(n)])
            assert np.allclose(got[r, h], _contiguous_attention(q[r, h], K, V), rtol=1e-12, atol=1e-13)


def test_paged_attention_page_permutation_invariance_and_gqa():
    S, d, nkv, G = 16, 32, 2, 3
    nq = nkv * G
    lengths = [7, 45]
    rng = np.random.Generator(np.random.PCG64(5))
    P, indptr, indices = _random_pages(lengths, S, rng)
    kp, vp = _fill_pool(P, nkv, S, d, rng)
    pos = np.array([n - 1 for n in lengths])
    q = rng.standard_normal((2, nq, d))
    args = (np.arange(2), np.ones(2, int), pos, indptr)
    base = oracle.paged_attention(q, kp, vp, *args, indices, S, nkv)
    # move every page to a new pool index; the result must not change at all
    perm = rng.permutation(P)
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    assert np.array_equal(base, oracle.paged_attention(q, kp2, vp2, *args, perm[indices], S, nkv))
    # GQA == MHA over KV heads replicated G times (the matmul groups rows
    # differently, so equal up to fp64 summation order)
    kp3, vp3 = np.repeat(kp, G, axis=1), np.repeat(vp, G, axis=1)
    mha = oracle.paged_attention(q, kp3, vp3, *args, indices, S, nq)
    assert np.allclose(base, mha, rtol=1e-13, atol=1e-14)


def test_attention_special_cases():
    d = 16
    K = RNG.standard_normal((9, d))
    V = RNG.standard_normal((9, d))
    w = oracle.attention_weights(RNG.standard_normal((3, d)), K)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    # one key: output is that key's value exactly
    assert np.array_equal(oracle.attention_weights(RNG.standard_normal((1, d)), K[:1]) @ V[:1], V[:1])
    # q = 0: uniform weights -> mean of the values
    assert np.allclose(oracle.attention_weights(np.zeros((1, d)), K) @ V, V.mean(axis=0), atol=1e-14)


def test_kv_append_rebuild_and_sentinel():
    S, d, nkv = 16, 32, 2
    pos0 = [3, 0, 30]
    qlen = [1, 20, 2]
    lengths = [p + q for p, q in zip(pos0, qlen)]
    rng = np.random.Generator(np.random.PCG64(11))
    P, indptr, indices = _random_pages(lengths, S, rng)
    kp, vp = _fill_pool(P, nkv, S, d, rng)
    kp0, vp0 = kp.copy(), vp.copy()
    T = sum(qlen)
    tok_req = np.repeat(np.arange(3), qlen)
    pos = np.concatenate([np.arange(p, p + q) for p, q in zip(pos0, qlen)])
    kn, vn = rng.standard_normal((2, T, nkv, d))
    oracle.kv_append(kp, vp, kn, vn, tok_req, pos, indptr, indices, S, "bf16")
    touched = np.zeros((P, S), bool)
    for t in range(T):
        r, p = tok_req[t], pos[t]
        pg = indices[indptr[r] + p // S]
        touched[pg, p % S] = True
        for kh in range(nkv):
            kg, vg = _kv(kp, vp, pg, kh, p % S, d)
            assert np.array_equal(kg, oracle.round_to_bf16(kn[t, kh]))
            assert np.array_equal(vg, oracle.round_to_bf16(vn[t, kh]))
    # every slot no (page table, position) pair names is bit-identical
    for pg in range(P):
        for sl in range(S):
            if not touched[pg, sl]:
                assert np.array_equal(kp[pg, :, sl], kp0[pg, :, sl])
                assert np.array_equal(vp[pg, :, sl], vp0[pg, :, sl])


# ---------------------------------------------------------------- whole layer

def _tiny_problem(rng, nq=4, nkv=2, d=32, H=16, F=12, E=1, top_k=1, S=16,
                  pos0=(19, 0, 2), qlen=(1, 6, 1), dtype="f32", theta=1e4):
    shape = dict(hidden=H, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, ffn=F, n_experts=E,
                 top_k=top_k, dtype=dtype, rms_eps=1e-5, rope_theta=theta, page_size=S)
    w = dict(attn_norm=rng.uniform(0.5, 1.5, H), w_qkv=rng.standard_normal(((nq + 2 * nkv) * d, H)) * 0.3,
             w_o=rng.standard_normal((H, nq * d)) * 0.3, ffn_norm=rng.uniform(0.5, 1.5, H),
             w_gate=rng.standard_normal((E, F, H)) * 0.3, w_up=rng.standard_normal((E, F, H)) * 0.3,
             w_down=rng.standard_normal((E, H, F)) * 0.3)
    lengths = [p + q for p, q in zip(pos0, qlen)]
    P, indptr, indices = _random_pages(lengths, S, rng)
    kp, vp = _fill_pool(P, nkv, S, d, rng)
    T = sum(qlen)
    batch = dict(x=rng.standard_normal((T, H)), req_q_start=np.concatenate([[0], np.cumsum(qlen)[:-1]]),
                 req_q_len=np.array(qlen), req_pos0=np.array(pos0),
                 pos=np.concatenate([np.arange(p, p + q) for p, q in zip(pos0, qlen)]),
                 page_indptr=indptr, page_indices=indices)
    if E > 1:
        batch["router_logits"] = rng.standard_normal((T, E)).astype(np.float32).astype(np.float64)
    return shape, w, batch, kp, vp


def _brute_force_layer(shape, w, batch, kp, vp):
    """Scalar-loop decoder layer written from the definition (pool kept exact)."""
    H, nq, nkv, d, F = (shape[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn"))
    S, eps, theta = shape["page_size"], shape["rms_eps"], shape["rope_theta"]
    E, top_k = shape["n_experts"], shape["top_k"]
    G = nq // nkv
    x = batch["x"]
    T = x.shape[0]
    kp, vp = kp.copy(), vp.copy()
    req_of = []
    for r, n in enumerate(batch["req_q_len"]):
        req_of += [r] * int(n)

    def norm(row, g):
        ms = sum(v * v for v in row) / len(row)
        return [row[i] / math.sqrt(ms + eps) * g[i] for i in range(len(row))]

    def rot(vec, p):
        out = list(vec)
        for j in range(d // 2):
            ang = p * theta ** (-2.0 * j / d)
            a, b = vec[j], vec[j + d // 2]
            out[j] = a * math.cos(ang) - b * math.sin(ang)
            out[j + d // 2] = a * math.sin(ang) + b * math.cos(ang)
        return out

    qs = []
    for t in range(T):
        h = norm(x[t], w["attn_norm"])
        col = [sum(h[i] * w["w_qkv"][n, i] for i in range(H)) for n in range((nq + 2 * nkv) * d)]
        p = int(batch["pos"][t])
        r = req_of[t]
        pg = batch["page_indices"][batch["page_indptr"][r] + p // S]
        qs.append([rot(col[hq * d:(hq + 1) * d], p) for hq in range(nq)])
        for kh in range(nkv):
            kv = rot(col[(nq + kh) * d:(nq + kh + 1) * d], p)
            vv = col[(nq + nkv + kh) * d:(nq + nkv + kh + 1) * d]
            for i in range(d):
                kp[pg, kh, p % S, i] = kv[i]
                vp[pg, kh, p % S, i] = vv[i]
    out = np.zeros((T, H))
    for t in range(T):
        r, p = req_of[t], int(batch["pos"][t])
        att = []
        for hq in range(nq):
            kh = hq // G
            slots = [(batch["page_indices"][batch["page_indptr"][r] + j // S], j % S) for j in range(p + 1)]
            keys = [_kv(kp, vp, pg_, kh, sl_, d)[0] for pg_, sl_ in slots]
            vals = [_kv(kp, vp, pg_, kh, sl_, d)[1] for pg_, sl_ in slots]
            att += list(_contiguous_attention(np.array(qs[t][hq]), np.array(keys), np.array(vals)))
        x1 = [x[t, j] + sum(att[c] * w["w_o"][j, c] for c in range(nq * d)) for j in range(H)]
        h2 = norm(x1, w["ffn_norm"])

        def ffn(e):
            act = []
            for f in range(F):
                zg = sum(h2[i] * w["w_gate"][e, f, i] for i in range(H))
                zu = sum(h2[i] * w["w_up"][e, f, i] for i in range(H))
                act.append(zg / (1 + math.exp(-zg)) * zu)
            return [sum(act[f] * w["w_down"][e, j, f] for f in range(F)) for j in range(H)]

        if E == 1:
            y = ffn(0)
        else:
            lg = list(batch["router_logits"][t])
            best = max(((a, b) for a in range(E) for b in range(E) if a != b),
                       key=lambda ab: (lg[ab[0]] + lg[ab[1]], lg[ab[0]] >= lg[ab[1]]))
            z = math.exp(lg[best[0]]) + math.exp(lg[best[1]])
            y = [0.0] * H
            for e in best:
                ye = ffn(e)
                y = [y[j] + math.exp(lg[e]) / z * ye[j] for j in range(H)]
        out[t] = [x1[j] + y[j] for j in range(H)]
    return out, kp, vp


def test_whole_layer_matches_scalar_brute_force():
    rng = np.random.Generator(np.random.PCG64(21))
    shape, w, batch, kp, vp = _tiny_problem(rng)
    res = oracle.layer_step(shape, w, batch, kp, vp, pool_dtype="f64")
    bf_out, bf_k, bf_v = _brute_force_layer(shape, w, batch, kp, vp)
    assert np.allclose(res["out"], bf_out, rtol=1e-12, atol=1e-12)
    assert np.allclose(res["k_pool"], bf_k, rtol=1e-12, atol=1e-12)
    assert np.allclose(res["v_pool"], bf_v, rtol=1e-12, atol=1e-12)


def test_whole_moe_layer_matches_scalar_brute_force():
    rng = np.random.Generator(np.random.PCG64(22))
    shape, w, batch, kp, vp = _tiny_problem(rng, E=4, top_k=2, pos0=(3, 1), qlen=(1, 3))
    res = oracle.layer_step(shape, w, batch, kp, vp, pool_dtype="f64")
    bf_out, _, _ = _brute_force_layer(shape, w, batch, kp, vp)
    assert np.allclose(res["out"], bf_out, rtol=1e-12, atol=1e-12)


def test_residual_wiring_zero_projections_return_x():
    rng = np.random.Generator(np.random.PCG64(23))
    shape, w, batch, kp, vp = _tiny_problem(rng)
    w["w_o"][:] = 0
    w["w_down"][:] = 0
    res = oracle.layer_step(shape, w, batch, kp, vp)
    assert np.array_equal(res["out"], batch["x"])
    assert np.array_equal(res["x1"], batch["x"])


def test_nano_batch_split_equals_unsplit():
    rng = np.random.Generator(np.random.PCG64(24))
    shape, w, batch, kp, vp = _tiny_problem(rng, pos0=(5, 0, 2, 9, 3), qlen=(1, 6, 1, 1, 4))
    full = oracle.layer_step(shape, w, batch, kp, vp)
    for sizes in ([13], [3, 10], [2, 4, 7], [1, 1, 5, 6]):   # cuts through requests too
        split = oracle.layer_step_split(shape, w, batch, kp, vp, sizes)
        for key in ("out", "x1", "q_rot", "attn", "k_pool", "v_pool"):
            assert np.allclose(split[key], full[key], rtol=1e-12, atol=1e-12), (sizes, key)


def test_chunked_prefill_equals_unchunked():
    rng = np.random.Generator(np.random.PCG64(25))
    shape, w, batch, kp, vp = _tiny_problem(rng, pos0=(0,), qlen=(16,))
    full = oracle.layer_step(shape, w, batch, kp, vp)
    # the same prompt as 4 sequential chunks of 4 tokens, each its own step
    kp_c, vp_c = kp, vp
    outs = []
    for c in range(4):
        sub = dict(batch)
        sub.update(x=batch["x"][4 * c:4 * c + 4], req_q_start=np.array([0]), req_q_len=np.array([4]),
                   req_pos0=np.array([4 * c]), pos=np.arange(4 * c, 4 * c + 4))
        r = oracle.layer_step(shape, w, sub, kp_c, vp_c)
        kp_c, vp_c = r["k_pool"], r["v_pool"]
        outs.append(r["out"])
    assert np.allclose(np.concatenate(outs), full["out"], rtol=1e-12, atol=1e-12)
    assert np.array_equal(kp_c, full["k_pool"]) and np.array_equal(vp_c, full["v_pool"])


# ---------------------------------------------------------------- MoE routing

def test_moe_route_brute_force_and_stable_perm():
    rng = np.random.Generator(np.random.PCG64(26))
    T, E = 40, 8
    logits = rng.standard_normal((T, E)).astype(np.float32).astype(np.float64)
    logits[3, 2] = logits[3, 5] = 9.0            # a tie: the lower index ranks first
    idx, w, perm, offsets = oracle.moe_route(logits, 2)
    assert list(idx[3]) == [2, 5]
    for t in range(T):
        best = max(((a, b) for a in range(E) for b in range(E) if a != b),
                   key=lambda ab: (logits[t, ab[0]] + logits[t, ab[1]], logits[t, ab[0]] > logits[t, ab[1]], -ab[0]))
        assert tuple(idx[t]) == best
        assert abs(w[t].sum() - 1) < 1e-15 and w[t, 0] >= w[t, 1]
        full = np.exp(logits[t] - logits[t].max())
        full /= full.sum()
        assert np.allclose(w[t], full[idx[t]] / full[idx[t]].sum(), rtol=1e-13)
    # perm lists assignment ids grouped by expert, ascending inside each group
    flat = idx.reshape(-1)
    assert sorted(perm.tolist()) == list(range(T * 2))
    want = sorted(range(T * 2), key=lambda a: (flat[a], a))
    assert perm.tolist() == want
    assert offsets[0] == 0 and offsets[-1] == T * 2
    for e in range(E):
        assert all(flat[a] == e for a in perm[offsets[e]:offsets[e + 1]])


def test_moe_identical_experts_equal_dense_ffn():
    rng = np.random.Generator(np.random.PCG64(27))
    shape, w, batch, kp, vp = _tiny_problem(rng, E=4, top_k=2)
    for k in ("w_gate", "w_up", "w_down"):
        w[k][:] = w[k][0]
    moe = oracle.layer_step(shape, w, batch, kp, vp)
    dense_shape = dict(shape, n_experts=1, top_k=1)
    dense_w = dict(w, w_gate=w["w_gate"][:1], w_up=w["w_up"][:1], w_down=w["w_down"][:1])
    dense = oracle.layer_step(dense_shape, dense_w, batch, kp, vp)
    assert np.allclose(moe["out"], dense["out"], rtol=1e-12, atol=1e-12)
