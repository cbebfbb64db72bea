// A serving loop around nf_layer_step with the asynchronous CPU control flow
// the Nanoflow pages describe: the host forms iteration i + 1's batch and
// allocates its KV pages while iteration i runs on the device, launches it
// without reading i's end-of-request flags, and retires the requests that
// ended at i when it forms i + 2 (README "Introduction" on the ossradar page:
// batch formation, KV management and retirement cost over a tenth of the
// inference time when done in step with the device; "The failure modes the
// design accepts" on the hysenlabs page: a finished request then occupies
// one more iteration).  With async off the host reads every iteration's
// flags right after it and retires at i + 1, the synchronous baseline.
//
// Each request brings its input rows (prompt and then the rows fed back for
// every generated position) and receives the layer's output row for every
// position it processes.  A position ends its request when the first element
// of its output exceeds the loop's threshold (the device writes that flag to
// pinned host memory) or when it is the request's last row.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "nf_internal.h"

using namespace nf;

namespace {

nf_status fail(nf_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
nf_status fail(nf_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return nf::set_error(st, buf);
}

#define LOOP_HIP(expr)                                                                              \
  do {                                                                                              \
    hipError_t e_ = (expr);                                                                         \
    if (e_ != hipSuccess) {                                                                         \
      (void)hipGetLastError();                                                                      \
      return fail(NF_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));                       \
    }                                                                                               \
  } while (0)

enum State { WAITING, ACTIVE, DONE };

struct Request {
  int32_t prompt_len = 0, max_len = 0;
  const char* rows_in = nullptr;   // [max_len][H]
  char* rows_out = nullptr;        // [max_len][H]
  State state = WAITING;
  int32_t next_pos = 0;            // first position not yet scheduled
  int32_t length = 0;              // positions with a valid output once DONE
  std::vector<int32_t> pages;
};

// What one launched iteration scheduled: per token, its request and
// position; the flags the device writes for it.
struct Slot {
  std::vector<int32_t> tok_req, tok_pos;
  uint64_t* src = nullptr;         // pinned, mapped: input row address per token
  uint64_t* dst = nullptr;         // pinned, mapped: output row address per token
  int32_t* flag = nullptr;         // pinned, mapped: out[t][0] > threshold
  hipEvent_t done = nullptr;
  bool pending = false;
};

}  // namespace

struct nf_loop {
  nf_layer* L = nullptr;
  nf_kv_pool* P = nullptr;
  nf_loop_opts o{};
  nf_shape s{};
  int32_t n_pages = 0;
  int64_t row_bytes = 0;
  std::vector<Request> reqs;
  std::vector<int32_t> free_pages;
  Slot slot[2];
  void* x = nullptr;               // device [max_tokens][H]
  void* out = nullptr;
};

namespace {

// Processes the flags of a finished iteration: requests whose scheduled
// position ended them become DONE (their pages return to the free list).
// Tokens of requests already DONE count as wasted.
void retire(nf_loop* lp, Slot& sl, int64_t& wasted, int32_t& finished) {
  for (size_t t = 0; t < sl.tok_req.size(); ++t) {
    Request& r = lp->reqs[sl.tok_req[t]];
    const int32_t p = sl.tok_pos[t];
    if (r.state == DONE) {
      ++wasted;
      continue;
    }
    const bool generated = p >= r.prompt_len - 1;
    if ((generated && sl.flag[t]) || p == r.max_len - 1) {
      r.state = DONE;
      r.length = p + 1;
      ++finished;
      lp->free_pages.insert(lp->free_pages.end(), r.pages.begin(), r.pages.end());
      r.pages.clear();
    }
  }
  sl.pending = false;
}

}  // namespace

extern "C" {

nf_status nf_loop_create(nf_layer* L, nf_kv_pool* P, const nf_loop_opts* o, nf_loop** out) {
  if (!L || !P || !o || !out) return fail(NF_ERR_INVALID_ARG, "nf_loop_create: null argument");
  *out = nullptr;
  const nf_shape& s = *layer_shape(L);
  if (o->max_tokens < 1 || o->max_tokens > s.max_tokens || o->max_prefill_tokens < 0 || s.n_experts > 1)
    return fail(NF_ERR_INVALID_ARG, "nf_loop_create: max_tokens must be 1..%d, max_prefill_tokens >= 0, dense layer",
                s.max_tokens);
  const int64_t row_bytes = (int64_t)s.hidden * (s.dtype == NF_BF16 ? 2 : 4);
  if (row_bytes % 16) return fail(NF_ERR_UNSUPPORTED, "nf_loop_create: rows must be whole 16-byte units");
  nf_loop* lp = new nf_loop();
  lp->L = L;
  lp->P = P;
  lp->o = *o;
  lp->s = s;
  lp->n_pages = pool_pages(P);
  lp->row_bytes = row_bytes;
  for (int32_t pg = lp->n_pages - 1; pg >= 0; --pg) lp->free_pages.push_back(pg);
  auto bad = [&](hipError_t e) {
    nf_loop_destroy(lp);
    (void)hipGetLastError();
    return fail(NF_ERR_HIP, "nf_loop_create: %s", hipGetErrorString(e));
  };
  hipError_t e;
  if ((e = hipMalloc(&lp->x, (size_t)o->max_tokens * row_bytes)) != hipSuccess) return bad(e);
  if ((e = hipMalloc(&lp->out, (size_t)o->max_tokens * row_bytes)) != hipSuccess) return bad(e);
  for (Slot& sl : lp->slot) {
    const unsigned fl = hipHostMallocMapped | hipHostMallocCoherent;
    if ((e = hipHostMalloc((void**)&sl.src, (size_t)o->max_tokens * 8, fl)) != hipSuccess) return bad(e);
    if ((e = hipHostMalloc((void**)&sl.dst, (size_t)o->max_tokens * 8, fl)) != hipSuccess) return bad(e);
    if ((e = hipHostMalloc((void**)&sl.flag, (size_t)o->max_tokens * 4, fl)) != hipSuccess) return bad(e);
    if ((e = hipEventCreateWithFlags(&sl.done, hipEventDisableTiming)) != hipSuccess) return bad(e);
  }
  *out = lp;
  return NF_OK;
}

void nf_loop_destroy(nf_loop* lp) {
  if (!lp) return;
  (void)hipDeviceSynchronize();
  for (Slot& sl : lp->slot) {
    if (sl.src) (void)hipHostFree(sl.src);
    if (sl.dst) (void)hipHostFree(sl.dst);
    if (sl.flag) (void)hipHostFree(sl.flag);
    if (sl.done) (void)hipEventDestroy(sl.done);
  }
  if (lp->x) (void)hipFree(lp->x);
  if (lp->out) (void)hipFree(lp->out);
  delete lp;
}

nf_status nf_loop_add_request(nf_loop* lp, int32_t prompt_len, int32_t max_len, const void* rows_in, void* rows_out,
                              int32_t* id) {
  if (!lp || !rows_in || !rows_out || !id || prompt_len < 1 || max_len < prompt_len ||
      max_len > lp->s.max_pos)
    return fail(NF_ERR_INVALID_ARG, "nf_loop_add_request: bad argument (1 <= prompt_len <= max_len <= max_pos)");
  if ((((uintptr_t)rows_in) | ((uintptr_t)rows_out)) & 15)
    return fail(NF_ERR_INVALID_ARG, "nf_loop_add_request: rows must be 16-byte aligned");
  if ((max_len + 15) / 16 > lp->n_pages)
    return fail(NF_ERR_OUT_OF_RANGE, "nf_loop_add_request: %d positions need more pages than the pool holds", max_len);
  Request r;
  r.prompt_len = prompt_len;
  r.max_len = max_len;
  r.rows_in = (const char*)rows_in;
  r.rows_out = (char*)rows_out;
  lp->reqs.push_back(r);
  *id = (int32_t)lp->reqs.size() - 1;
  return NF_OK;
}

nf_status nf_loop_request_length(const nf_loop* lp, int32_t id, int32_t* length) {
  if (!lp || !length || id < 0 || id >= (int32_t)lp->reqs.size())
    return fail(NF_ERR_INVALID_ARG, "nf_loop_request_length: bad argument");
  *length = lp->reqs[id].state == DONE ? lp->reqs[id].length : -1;
  return NF_OK;
}

nf_status nf_loop_run(nf_loop* lp, void* stream, nf_loop_stats* stats) {
  if (!lp) return fail(NF_ERR_INVALID_ARG, "nf_loop_run: null loop");
  hipStream_t st = (hipStream_t)stream;
  const auto w0 = std::chrono::steady_clock::now();
  double host_us = 0;
  int64_t tokens = 0, wasted = 0;
  int32_t iters = 0, finished = 0;
  std::vector<int32_t> q_start, q_len, pos0, pos, indptr, indices;
  for (int it = 0;; ++it) {
    Slot& sl = lp->slot[it & 1];
    Slot& prev = lp->slot[(it + 1) & 1];
    // this slot's buffers were last used two iterations ago: retire it (in
    // async mode that is the first time its flags are read)
    if (sl.pending) LOOP_HIP(hipEventSynchronize(sl.done));
    const auto h0 = std::chrono::steady_clock::now();
    if (sl.pending) retire(lp, sl, wasted, finished);
    // admit waiting requests whose whole length fits in the free pages
    for (Request& r : lp->reqs) {
      if (r.state != WAITING) continue;
      const size_t need = (size_t)(r.max_len + 15) / 16;
      if (need > lp->free_pages.size()) break;
      r.pages.assign(lp->free_pages.end() - need, lp->free_pages.end());
      lp->free_pages.resize(lp->free_pages.size() - need);
      r.state = ACTIVE;
    }
    // form the batch: decode tokens first, then prefill chunks
    sl.tok_req.clear();
    sl.tok_pos.clear();
    q_start.clear(); q_len.clear(); pos0.clear(); pos.clear(); indptr.assign(1, 0); indices.clear();
    int budget = lp->o.max_tokens, pre_budget = lp->o.max_prefill_tokens;
    for (int pass = 0; pass < 2; ++pass)
      for (size_t id = 0; id < lp->reqs.size() && budget > 0; ++id) {
        Request& r = lp->reqs[id];
        if (r.state != ACTIVE || r.next_pos >= r.max_len) continue;
        const bool prefill = r.next_pos < r.prompt_len, decode = !prefill;
        if ((pass == 0 && !decode) || (pass == 1 && !prefill)) continue;
        int n = 1;
        if (prefill) {
          n = std::min({r.prompt_len - r.next_pos, budget, pre_budget});
          if (n <= 0) continue;
          pre_budget -= n;
        }
        budget -= n;
        q_start.push_back((int32_t)pos.size());
        q_len.push_back(n);
        pos0.push_back(r.next_pos);
        for (int i = 0; i < n; ++i) {
          const int32_t p = r.next_pos + i;
          sl.tok_req.push_back((int32_t)id);
          sl.tok_pos.push_back(p);
          pos.push_back(p);
        }
        const int np = (r.next_pos + n + 15) / 16;
        indices.insert(indices.end(), r.pages.begin(), r.pages.begin() + np);
        indptr.push_back((int32_t)indices.size());
        r.next_pos += n;
      }
    const int T = (int)pos.size();
    if (T == 0) {
      // nothing to schedule: finish the iteration still in flight, if any
      if (prev.pending) {
        LOOP_HIP(hipEventSynchronize(prev.done));
        retire(lp, prev, wasted, finished);
        continue;
      }
      bool waiting = false;
      for (const Request& r : lp->reqs) waiting = waiting || r.state != DONE;
      if (waiting) return fail(NF_ERR_OUT_OF_RANGE, "nf_loop_run: a waiting request does not fit in the pool");
      break;
    }
    for (int t = 0; t < T; ++t) {
      const Request& r = lp->reqs[sl.tok_req[t]];
      sl.src[t] = (uint64_t)(uintptr_t)(r.rows_in + (int64_t)sl.tok_pos[t] * lp->row_bytes);
      sl.dst[t] = (uint64_t)(uintptr_t)(r.rows_out + (int64_t)sl.tok_pos[t] * lp->row_bytes);
    }
    nf_batch b{};
    b.n_tokens = T;
    b.n_requests = (int32_t)q_len.size();
    b.x = lp->x;
    b.out = lp->out;
    b.req_q_start = q_start.data();
    b.req_q_len = q_len.data();
    b.req_pos0 = pos0.data();
    b.pos = pos.data();
    b.page_indptr = indptr.data();
    b.page_indices = indices.data();
    // the layer's plan with its nano-batch count spread over this batch
    nf_plan plan = layer_plan(lp->L);
    plan.count = std::max(1, std::min(plan.count, T));
    for (int j = 0; j < NF_MAX_NANO; ++j) plan.sizes[j] = j < plan.count ? T / plan.count + (j < T % plan.count) : 0;
    LOOP_HIP(loop_gather(sl.src, lp->x, T, lp->row_bytes, st));
    nf_status s1 = layer_step_with_plan(lp->L, lp->P, &b, st, plan);
    if (s1 != NF_OK) return s1;
    LOOP_HIP(loop_scatter(lp->s.dtype, lp->out, sl.dst, T, lp->s.hidden, lp->o.eos_threshold, sl.flag, st));
    LOOP_HIP(hipEventRecord(sl.done, st));
    sl.pending = true;
    host_us += std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - h0).count();
    tokens += T;
    ++iters;
    if (!lp->o.async) {          // synchronous control flow: read this iteration's flags now
      LOOP_HIP(hipEventSynchronize(sl.done));
      retire(lp, sl, wasted, finished);
    }
  }
  if (stats) {
    stats->iterations = iters;
    stats->finished = finished;
    stats->tokens = tokens;
    stats->wasted_tokens = wasted;
    stats->host_us = host_us;
    stats->wall_us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - w0).count();
  }
  return NF_OK;
}

}  // extern "C"
