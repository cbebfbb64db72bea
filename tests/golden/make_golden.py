"""Writes tiny_layer.json: a seeded tiny decoder-layer problem and the
oracle's outputs for it.

The pages print no worked example (no input/output values for any step of
the layer), so this fixture is a regression guard on the oracle, not an
external pin: its expected values come from the oracle alone.  Any change to
them must name, in its commit message, the passage or reading that justifies
the oracle change.  Run from the repository root:

    python -m tests.golden.make_golden
"""
import json
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def problem():
    rng = np.random.Generator(np.random.PCG64(4242))
    H, nq, nkv, d, F, S = 16, 4, 2, 32, 24, 16
    shape = dict(hidden=H, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, ffn=F, n_experts=1, top_k=1,
                 dtype="bf16", rms_eps=1e-5, rope_theta=1e4, page_size=S)
    w = dict(attn_norm=rng.uniform(0.5, 1.5, H), w_qkv=rng.standard_normal(((nq + 2 * nkv) * d, H)) * 0.2,
             w_o=rng.standard_normal((H, nq * d)) * 0.2, ffn_norm=rng.uniform(0.5, 1.5, H),
             w_gate=rng.standard_normal((1, F, H)) * 0.2, w_up=rng.standard_normal((1, F, H)) * 0.2,
             w_down=rng.standard_normal((1, H, F)) * 0.2)
    # two decode requests (positions 20 and 3) and a 5-token prefill chunk at 16..20
    pos0, qlen = [20, 3, 16], [1, 1, 5]
    n_pages = [-(-(p + q) // S) for p, q in zip(pos0, qlen)]
    perm = rng.permutation(sum(n_pages) + 2)
    indptr = np.concatenate([[0], np.cumsum(n_pages)])
    indices = perm[:sum(n_pages)]
    P = len(perm)
    kp = oracle.round_to_bf16(rng.standard_normal((P, nkv, S, d)))
    vp = oracle.round_to_bf16(rng.standard_normal((P, nkv, S, d)))
    T = sum(qlen)
    batch = dict(x=oracle.round_to_bf16(rng.standard_normal((T, H))),
                 req_q_start=np.concatenate([[0], np.cumsum(qlen)[:-1]]), req_q_len=np.array(qlen),
                 req_pos0=np.array(pos0), pos=np.concatenate([np.arange(p, p + q) for p, q in zip(pos0, qlen)]),
                 page_indptr=indptr, page_indices=indices)
    return shape, w, batch, kp, vp


def main():
    shape, w, batch, kp, vp = problem()
    res = oracle.layer_step(shape, w, batch, kp, vp)
    out = {"note": "oracle outputs for tests/golden/make_golden.py:problem(); not values printed by the pages",
           "out": res["out"].tolist(), "x1": res["x1"].tolist(), "attn": res["attn"].tolist()}
    with open(os.path.join(HERE, "tiny_layer.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
