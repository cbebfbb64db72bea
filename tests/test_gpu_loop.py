"""The serving loop (nf_loop_*) through the C ABI.

Requests of random prompt and generation lengths go through a loop that
chunks prompts and decodes one token per iteration.  Some requests carry an
end marker in an input row past their prompt (first element 200), which makes
that position's output exceed the loop's threshold, so only the device's flag
tells the host where they end.
- The synchronous loop (flags read after every iteration) and the asynchronous
  one (iteration i + 1 launched before i's flags are read, retirement at i + 2)
  end every request at the same position and give the same output rows; the
  asynchronous loop runs exactly one wasted token per request that ended on a
  flag.
- Each request's output rows equal the fp64 oracle applied to its rows as one
  unchunked prefill from position 0 (rows are independent across requests and
  causal attention sees only the request's own positions), within the bf16
  tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from intra_operation_overlap_amd import binding as B
from intra_operation_overlap_amd import workload as W
from tests import gpu_harness as GH

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

SHAPE = W.Shape(hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=688, dtype="bf16", rope_theta=5e5)
MARK = 200.0


def _requests(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    reqs = []
    for i in range(n):
        prompt = int(rng.integers(1, 60))
        max_len = prompt + int(rng.integers(1, 24))
        g = torch.Generator(device="cuda")
        g.manual_seed(seed * 1000 + i)
        rows = torch.randn(max_len, SHAPE.hidden, generator=g, device="cuda").to(torch.bfloat16)
        end = None
        if i % 3 == 0 and max_len - prompt >= 2:
            end = int(rng.integers(prompt - 1, max_len - 1))       # a generated position before the last
            rows[end, 0] = MARK
        reqs.append((prompt, rows, end))
    return reqs


def _run(layer, pool, reqs, async_, max_tokens=96, max_prefill=48):
    loop = B.Loop(layer, pool, max_tokens, max_prefill, async_, MARK / 2)
    outs, ids = [], []
    for prompt, rows, _ in reqs:
        out = torch.full_like(rows, float("nan"))
        ids.append(loop.add(prompt, rows, out))
        outs.append(out)
    stats = loop.run(GH.stream())
    torch.cuda.synchronize()
    lengths = [loop.length(i) for i in ids]
    loop.close()
    return outs, lengths, stats


def test_async_loop_matches_sync_loop_and_the_oracle():
    wl = W.Workload("loop", SHAPE, n_decode=1, ctx_range=(1, 1), prefill=None, seed=95)
    weights = W.make_weights(wl, "cuda")
    layer = B.Layer(SHAPE, weights, 96, 128)
    n_pages = 64                                      # fewer than all requests need at once: admission waits
    kp = torch.zeros(n_pages, SHAPE.n_kv_heads, 16, SHAPE.head_dim, dtype=torch.bfloat16, device="cuda")
    pool = B.KVPool.from_plain(layer, kp, kp, GH.stream())
    reqs = _requests(30, 7)
    o_sync, len_sync, st_sync = _run(layer, pool, reqs, False)
    o_async, len_async, st_async = _run(layer, pool, reqs, True)
    GH.log(f"sync {st_sync}; async {st_async}")
    want = [(end + 1) if end is not None else rows.shape[0] for _, rows, end in reqs]
    assert len_sync == want and len_async == want
    flagged = sum(1 for _, _, end in reqs if end is not None)
    assert st_sync["wasted_tokens"] == 0 and st_async["wasted_tokens"] == flagged
    assert st_sync["finished"] == st_async["finished"] == len(reqs)
    assert st_async["tokens"] == st_sync["tokens"] + flagged
    for r, n in enumerate(want):
        e = GH.normwise(GH.f64(o_async[r][:n]), GH.f64(o_sync[r][:n]))
        assert e <= 1e-2, (r, e)
    # against the oracle: each request as one prefill of its rows 0..n-1
    w_np = {k: v.detach().to("cpu", torch.float32).numpy() for k, v in weights.items()}
    for r in (0, 1, 2, 5, 9, 29):
        prompt, rows, _ = reqs[r]
        n = want[r]
        pages = -(-n // 16)
        bd = dict(x=GH.f64(rows[:n]), req_q_start=np.array([0]), req_q_len=np.array([n]), req_pos0=np.array([0]),
                  pos=np.arange(n), page_indptr=np.array([0, pages]), page_indices=np.arange(pages))
        kz = np.zeros((pages, SHAPE.n_kv_heads, 16, SHAPE.head_dim))
        ref = oracle.layer_step(SHAPE.as_dict(), w_np, bd, kz, kz.copy())
        e = GH.normwise(GH.f64(o_async[r][:n]), ref["out"])
        GH.log(f"request {r}: {n} positions (prompt {prompt}), error {e:.2e}")
        assert e <= 2e-2, (r, e)
    pool.close()
    layer.close()


def test_loop_under_two_lanes_matches_the_unsplit_loop():
    """The loop spreads the layer's plan over every batch it forms: under the
    lanes order (two nano-batches, each on a stream of its own) every request
    ends at the same position and its rows match the unsplit loop's within the
    bf16 tolerance (the lanes pick GEMM tiles for half the chip)."""
    wl = W.Workload("loop_lanes", SHAPE, n_decode=1, ctx_range=(1, 1), prefill=None, seed=96)
    weights = W.make_weights(wl, "cuda")
    layer = B.Layer(SHAPE, weights, 96, 128)
    kp = torch.zeros(64, SHAPE.n_kv_heads, 16, SHAPE.head_dim, dtype=torch.bfloat16, device="cuda")
    pool = B.KVPool.from_plain(layer, kp, kp, GH.stream())
    reqs = _requests(20, 11)
    o_ref, len_ref, st_ref = _run(layer, pool, reqs, True)
    layer.set_plan(B.make_plan(2, [1, 1], order=B.NF_ORDER_LANES, n_streams=2))
    o_lanes, len_lanes, st_lanes = _run(layer, pool, reqs, True)
    GH.log(f"unsplit {st_ref}; lanes {st_lanes}")
    assert len_lanes == len_ref
    assert st_lanes["wasted_tokens"] == st_ref["wasted_tokens"]
    for r, n in enumerate(len_ref):
        e = GH.normwise(GH.f64(o_lanes[r][:n]), GH.f64(o_ref[r][:n]))
        assert e <= 2e-2, (r, e)
    pool.close()
    layer.close()
