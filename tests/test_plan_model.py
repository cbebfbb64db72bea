"""The plan search's step-time model (nf_plan_predict, host only) against
timelines worked out by hand: one stream adds every operation; two streams
follow the dependency chain F -> A -> O -> N of each nano-batch, pay the
cross-stream wait on A's and O's inputs, and progress at the co-run rates
while both run."""
import numpy as np
import pytest

from intra_operation_overlap_amd import binding as B
from intra_operation_overlap_amd import workload as W


def _profile(front=10.0, oproj=5.0, ffn=30.0, attn=50.0, gap=0.0, slow_g=1.0, slow_a=1.0, wait=0.0):
    p = B.nf_plan_profile()
    p.n_points = 2
    p.tokens[0], p.tokens[1] = 1.0, 100000.0
    for arr, v in ((p.front_us, front), (p.oproj_us, oproj), (p.ffn_us, ffn)):
        arr[0] = arr[1] = v            # flat in the nano-batch size
    p.attn_base_us, p.attn_us_per_page = attn, 0.0
    p.gap_us, p.slow_gemm, p.slow_attn, p.wait_us = gap, slow_g, slow_a, wait
    return p


def _setup():
    wl = W.WORKLOADS["c1"]
    batch = W.make_batch(wl)
    shape = B.make_shape(wl.shape, 64, 512)
    return batch, shape, B.HostBatch(batch, 0x1000, 0x2000)


def _predict(p, plan):
    _, shape, hb = _setup()
    return B.plan_predict(p, shape, plan, hb)


def test_one_stream_adds_every_operation():
    T = 16
    assert _predict(_profile(gap=1.0), B.make_plan(1, [T])) == pytest.approx(10 + 50 + 5 + 30 + 4)
    for order in (B.NF_ORDER_PIPELINED, B.NF_ORDER_SEQUENTIAL, B.NF_ORDER_DEEP):
        assert _predict(_profile(), B.make_plan(2, [8, 8], order=order)) == pytest.approx(2 * 95)
        assert _predict(_profile(), B.make_plan(4, [4, 4, 4, 4], order=order)) == pytest.approx(4 * 95)


def test_two_streams_pipelined_critical_path():
    plan = B.make_plan(2, [8, 8], n_streams=2)
    # F0 0-10; A0 10-60 beside F1 10-20; O0 60-65; N0 65-95; A1 60-110; O1 110-115; N1 115-145
    assert _predict(_profile(), plan) == pytest.approx(145)
    # a 3 us wait on each cross-stream edge: A0 13-63, O0 66-71, N0 71-101, A1 63-113, O1 116-121, N1 121-151
    assert _predict(_profile(wait=3.0), plan) == pytest.approx(151)


def test_two_streams_co_run_rates():
    # both sides at half speed while both run:
    # F0 0-10; F1 beside A0 10-30 (A0 has 40 left); A0 30-70; O0 beside A1 70-80 (A1 45 left);
    # N0 beside A1 80-140 (A1 15 left); A1 140-155; O1 155-160; N1 160-190
    plan = B.make_plan(2, [8, 8], n_streams=2)
    assert _predict(_profile(slow_g=2.0, slow_a=2.0), plan) == pytest.approx(190)


def test_budget_scales_apply_whether_or_not_the_other_side_runs():
    # one stream: every GEMM-side duration x2, attention x3
    p = _profile()
    p.scale_gemm, p.scale_attn = 2.0, 3.0
    assert _predict(p, B.make_plan(1, [16])) == pytest.approx(2 * (10 + 5 + 30) + 3 * 50)
    # two streams, GEMM side x2 (F 20, O 10, N 60), attention unscaled, no co-run slowdown:
    # F0 0-20; F1 20-40; A0 20-70; O0 70-80; N0 80-140; A1 70-120; O1 140-150; N1 150-210
    p = _profile()
    p.scale_gemm = 2.0
    assert _predict(p, B.make_plan(2, [8, 8], n_streams=2)) == pytest.approx(210)
    # zero reads as one
    p = _profile()
    p.scale_gemm = p.scale_attn = 0.0
    assert _predict(p, B.make_plan(1, [16])) == pytest.approx(95)


def test_deep_order_two_streams():
    # two: G issues F0 | F1 O0 | O1 N0 | N1
    # F0 0-10; F1 10-20; A0 10-60; O0 60-65; A1 60-110; O1 110-115; N0 115-145; N1 145-175
    plan = B.make_plan(2, [8, 8], order=B.NF_ORDER_DEEP, n_streams=2)
    assert _predict(_profile(), plan) == pytest.approx(175)
    # three: G issues F0 | F1 O0 | F2 O1 N0 | O2 N1 | N2 with A on its own stream
    # F0 0-10; F1 10-20; A0 10-60; O0 60-65; F2 65-75; A1 60-110; O1 110-115; N0 115-145;
    # A2 110-160; O2 160-165; N1 165-195; N2 195-225
    plan3 = B.make_plan(3, [6, 5, 5], order=B.NF_ORDER_DEEP, n_streams=2)
    assert _predict(_profile(), plan3) == pytest.approx(225)


def test_sizes_interpolate_and_attention_follows_page_units():
    batch, shape, hb = _setup()
    p = _profile()
    p.tokens[0], p.tokens[1] = 8.0, 16.0
    p.front_us[0], p.front_us[1] = 10.0, 30.0           # 20 us more per 8 tokens
    p.attn_base_us, p.attn_us_per_page = 0.0, 1.0
    # decode requests: one work item each, over the pages holding positions 0..pos0
    units = sum((int(batch.req_pos0[r]) + 16) // 16 for r in range(batch.n_requests))
    got = B.plan_predict(p, shape, B.make_plan(1, [16]), hb)
    assert got == pytest.approx(30 + units + 5 + 30)
    got12 = B.plan_predict(p, shape, B.make_plan(2, [12, 4]), hb)
    assert got12 == pytest.approx((20 + 5 + 30) + (0 + 5 + 30) + units)   # 4 tokens: extrapolated to 0, floored


def test_predict_rejects_bad_arguments():
    batch, shape, hb = _setup()
    p = _profile()
    p.n_points = 0
    with pytest.raises(B.NfError):
        B.plan_predict(p, shape, B.make_plan(1, [16]), hb)
    with pytest.raises(B.NfError):
        B.plan_predict(_profile(), shape, B.make_plan(2, [8, 9]), hb)


def test_lanes_share_the_chip_by_operation_class():
    plan = B.make_plan(2, [8, 8], order=B.NF_ORDER_LANES, n_streams=2)
    # F0 0-10; F1 beside A0 10-20; A0 beside A1 at half rate each 20-100 (A1 10 left);
    # O0 beside A1 100-105; N0 beside A1 105-110 (25 left); O1 beside N0 at half rate 110-120
    # (N0 20 left); N1 beside N0 at half rate 120-160 (N1 10 left); N1 alone 160-170
    assert _predict(_profile(), plan) == pytest.approx(170)
    # attention beside a GEMM-side operation at the calibrated rates (half here):
    # F1 beside A0 10-30 (A0 40 left); A0 beside A1 30-110 (A1 10 left); O0 beside A1 110-120;
    # N0 beside A1 120-130 (N0 25 left); O1 beside N0 130-140 (N0 20 left);
    # N1 beside N0 140-180 (N1 10 left); N1 alone 180-190
    assert _predict(_profile(slow_g=2.0, slow_a=2.0), plan) == pytest.approx(190)
    # a 7 us wait before lane 1 starts and before the caller joins it:
    # A0 alone 10-17 (43 left); F1 beside A0 17-27 (33 left); A0 beside A1 27-93 (A1 17 left);
    # O0 beside A1 93-98; N0 beside A1 98-110 (18 left); O1 beside N0 110-120 (13 left);
    # N1 beside N0 120-146 (N1 17 left); N1 alone 146-163; join 170
    assert _predict(_profile(wait=7.0), plan) == pytest.approx(170)
    # one nano-batch: one lane, no join
    assert _predict(_profile(wait=7.0), B.make_plan(1, [16], order=B.NF_ORDER_LANES, n_streams=2)) == \
        pytest.approx(95)


def test_lane_rate_sets_how_two_same_class_operations_share_the_chip():
    plan = B.make_plan(2, [8, 8], order=B.NF_ORDER_LANES, n_streams=2)
    # as the first lanes timeline, with same-class pairs at full rate each:
    # F0 0-10; F1 beside A0 10-20; A0 beside A1 20-60 (A1 10 left); O0 beside A1 60-65;
    # N0 beside A1 65-70 (25 left); O1 beside N0 70-75 (20 left); N1 beside N0 75-95 (N1 10 left);
    # N1 alone 95-105
    p = _profile()
    p.lane_rate = 1.0
    assert _predict(p, plan) == pytest.approx(105)
    # 0 means one half: the first lanes timeline
    p.lane_rate = 0.0
    assert _predict(p, plan) == pytest.approx(170)
    # the rate only matters for lanes: two streams pipelined are unchanged
    q = _profile()
    q.lane_rate = 1.0
    assert _predict(q, B.make_plan(2, [8, 8], n_streams=2)) == pytest.approx(145)
