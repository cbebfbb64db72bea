// Step-time model of a nano-batch plan (host only, no HIP): the event-graph
// prediction that ranks the plan search's candidates before the best of them
// are timed on the device.
//
// A plan's step is four operations per nano-batch j -- F_j (RMSNorm, QKV
// projection, RoPE/append), A_j (attention), O_j (O-projection with the FFN
// norm) and N_j (gate/up and down projections) -- on one stream, or on a GEMM
// stream and an attention stream, in the plan's issue order.  F_j -> A_j ->
// O_j -> N_j is each nano-batch's dependency chain; a dependency that crosses
// streams costs `wait_us` before the consumer may start.  Each operation's
// solo duration comes from per-kernel profiles of split steps run on one
// stream (piecewise linear in the nano-batch's tokens; attention linear in
// its KV pages).  While both streams run an operation, the GEMM side
// progresses at 1 / slow_gemm and attention at 1 / slow_attn of its solo
// rate: the co-run interference, calibrated per resource split from one
// overlapped run.  Under a CU budget a side is confined whether or not the
// other runs, so its durations are scaled by scale_gemm / scale_attn
// throughout.  The simulation advances from event to event (an operation
// finishing, or one becoming ready) and returns the makespan.
//
// With the lanes order each stream is a lane that runs whole nano-batches
// (j on lane j mod 2), lane 1 starting after F_0, and the caller waiting for
// both lanes.  The co-run rates then follow the classes of the two running
// operations: attention beside a GEMM-side operation as above; two
// operations of the same class share the chip, each at lane_rate of its solo
// rate (one half unless a two-lane calibration run fitted it: a lane's GEMMs
// take tiles for half the chip, and two lanes' GEMMs lose each other's L2
// reuse, so the whole-chip profiles only approximate the pair).
#include <algorithm>
#include <cmath>
#include <vector>

#include "nf_host.h"

namespace nf {
namespace {

double interp(const nf_plan_profile& p, const double* y, double tokens) {
  const int n = std::max(1, std::min(p.n_points, NF_PROFILE_POINTS));
  // points sorted by tokens (ascending) by the caller
  if (n == 1) return y[0] * tokens / std::max(1.0, p.tokens[0]);
  int i = 0;
  while (i + 2 < n && tokens > p.tokens[i + 1]) ++i;
  const double x0 = p.tokens[i], x1 = p.tokens[i + 1];
  const double t = (tokens - x0) / std::max(1e-9, x1 - x0);
  return std::max(0.0, y[i] + t * (y[i + 1] - y[i]));
}

struct Op {
  int stream;        // 0 GEMM side (or lane 0), 1 attention (or lane 1)
  bool attn;         // attention (else a GEMM-side operation)
  double work;       // solo microseconds left
  int dep = -1;      // index of the operation this one waits for (-1: none)
  double ready = 0;  // time its dependency (plus a cross-stream wait) allowed it
  double done = -1;
};

}  // namespace

void attn_page_units(const nf_shape& sh, const nf_batch& b, const nf_plan& plan, double* units) {
  const int k = std::max(1, std::min(plan.count, NF_MAX_NANO));
  const int G = std::max(1, sh.n_q_heads / std::max(1, sh.n_kv_heads));
  const int per_item = std::max(1, 16 / G);        // query tokens per attention work item
  int t0 = 0;
  for (int j = 0; j < k; ++j) {
    const int t1 = (plan.count == 1 && plan.sizes[0] == 0) ? b.n_tokens : t0 + plan.sizes[j];
    double u = 0;
    for (int r = 0; r < b.n_requests; ++r) {
      const int a = std::max(t0, b.req_q_start[r]), e = std::min(t1, b.req_q_start[r] + b.req_q_len[r]);
      if (a >= e) continue;
      const int last_pos = b.pos[e - 1];
      const int items = (e - a + per_item - 1) / per_item;
      u += (double)items * ((last_pos + 16) / 16);
    }
    units[j] = u;
    t0 = t1;
  }
}

double predict_plan_us(const nf_plan_profile& p, const nf_plan& plan, const double* tokens, const double* pages) {
  const int k = std::max(1, std::min(plan.count, NF_MAX_NANO));
  const bool two = plan.n_streams == 2;
  const bool lanes = two && plan.order == NF_ORDER_LANES;
  const double sc_g = p.scale_gemm > 0 ? p.scale_gemm : 1.0, sc_a = p.scale_attn > 0 ? p.scale_attn : 1.0;
  std::vector<Op> ops;
  std::vector<std::vector<int>> queue(2);
  int f[NF_MAX_NANO], a[NF_MAX_NANO], o[NF_MAX_NANO], nn[NF_MAX_NANO];
  for (int j = 0; j < k; ++j) {
    const double tj = tokens[j];
    auto add = [&](int stream, bool at, double us) {
      ops.push_back(Op{stream, at, std::max(0.0, us) + p.gap_us});
      return (int)ops.size() - 1;
    };
    const int ln = lanes ? j % 2 : 0;
    f[j] = add(ln, false, sc_g * interp(p, p.front_us, tj));
    a[j] = add(lanes ? ln : (two ? 1 : 0), true, sc_a * (p.attn_base_us + p.attn_us_per_page * pages[j]));
    o[j] = add(ln, false, sc_g * interp(p, p.oproj_us, tj));
    nn[j] = add(ln, false, sc_g * interp(p, p.ffn_us, tj));
    ops[a[j]].dep = f[j];
    ops[o[j]].dep = a[j];
  }
  // issue order of the GEMM stream (attention goes on its own stream with
  // two streams, else right after its front)
  std::vector<int>& g = queue[0];
  auto front = [&](int j) {
    g.push_back(f[j]);
    if (two) queue[1].push_back(a[j]);
    else g.push_back(a[j]);
  };
  if (lanes) {
    for (int j = 0; j < k; ++j)
      for (int op : {f[j], a[j], o[j], nn[j]}) queue[j % 2].push_back(op);
    if (k > 1) ops[f[1]].dep = f[0];
  } else if (plan.order == NF_ORDER_PIPELINED) {
    front(0);
    for (int j = 0; j < k; ++j) {
      if (j + 1 < k) front(j + 1);
      g.push_back(o[j]);
      g.push_back(nn[j]);
    }
  } else if (plan.order == NF_ORDER_DEEP) {
    for (int t = 0; t < k + 2; ++t) {
      if (t < k) front(t);
      if (t >= 1 && t - 1 < k) g.push_back(o[t - 1]);
      if (t >= 2) g.push_back(nn[t - 2]);
    }
  } else {
    for (int j = 0; j < k; ++j) {
      front(j);
      g.push_back(o[j]);
      g.push_back(nn[j]);
    }
  }
  size_t head[2] = {0, 0};
  int running[2] = {-1, -1};
  double now = 0;
  const double slow_g = std::max(1.0, p.slow_gemm), slow_a = std::max(1.0, p.slow_attn);
  for (int guard = 0; guard < 64 * (int)ops.size() + 64; ++guard) {
    // start what can start now
    for (int s = 0; s < 2; ++s) {
      if (running[s] >= 0 || head[s] >= queue[s].size()) continue;
      Op& op = ops[queue[s][head[s]]];
      if (op.dep >= 0) {
        const Op& d = ops[op.dep];
        if (d.done < 0) continue;
        op.ready = d.done + (d.stream != op.stream ? p.wait_us : 0.0);
      }
      if (op.ready <= now + 1e-9) {
        running[s] = queue[s][head[s]];
        ++head[s];
      }
    }
    if (running[0] < 0 && running[1] < 0) {
      // nothing runs: jump to the next ready time, or stop
      double next = INFINITY;
      for (int s = 0; s < 2; ++s) {
        if (head[s] >= queue[s].size()) continue;
        const Op& op = ops[queue[s][head[s]]];
        if (op.dep >= 0 && ops[op.dep].done < 0) continue;
        const double r = op.dep >= 0 ? ops[op.dep].done + (ops[op.dep].stream != op.stream ? p.wait_us : 0.0) : 0.0;
        next = std::min(next, r);
      }
      if (!std::isfinite(next)) break;
      now = std::max(now, next);
      continue;
    }
    const bool both = running[0] >= 0 && running[1] >= 0;
    double rate[2] = {1.0, 1.0};
    if (both) {
      const bool a0 = ops[running[0]].attn, a1 = ops[running[1]].attn;
      if (a0 == a1) {
        rate[0] = rate[1] = p.lane_rate > 0 ? p.lane_rate : 0.5;
      } else {
        rate[0] = a0 ? 1.0 / slow_a : 1.0 / slow_g;
        rate[1] = a1 ? 1.0 / slow_a : 1.0 / slow_g;
      }
    }
    // next event: a running op finishing, or a waiting op becoming ready
    double dt = INFINITY;
    for (int s = 0; s < 2; ++s)
      if (running[s] >= 0) dt = std::min(dt, ops[running[s]].work / rate[s]);
    for (int s = 0; s < 2; ++s) {
      if (running[s] >= 0 || head[s] >= queue[s].size()) continue;
      const Op& op = ops[queue[s][head[s]]];
      if (op.dep >= 0 && ops[op.dep].done >= 0) {
        const double r = ops[op.dep].done + (ops[op.dep].stream != op.stream ? p.wait_us : 0.0);
        if (r > now) dt = std::min(dt, r - now);
      }
    }
    if (!std::isfinite(dt)) break;
    now += dt;
    for (int s = 0; s < 2; ++s) {
      if (running[s] < 0) continue;
      Op& op = ops[running[s]];
      op.work -= dt * rate[s];
      if (op.work <= 1e-9) {
        op.work = 0;
        op.done = now;
        running[s] = -1;
      }
    }
  }
  double end = 0;
  for (const Op& op : ops) {
    if (op.done < 0) return INFINITY;    // cannot happen for a valid order
    end = std::max(end, op.done);
  }
  // the caller's stream joins lane 1
  return lanes && k > 1 ? end + p.wait_us : end;
}

}  // namespace nf
