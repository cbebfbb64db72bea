// Host-only validation of shapes, batches and plans, and the per-step work
// lists.  Nothing here calls HIP: every check runs before anything launches.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "nf_host.h"

namespace nf {
namespace {

nf_status fail(std::string& err, nf_status st, const char* fmt, ...) __attribute__((format(printf, 3, 4)));
nf_status fail(std::string& err, nf_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  err = buf;
  return st;
}

}  // namespace

nf_status check_shape(const nf_shape& s, std::string& err) {
  if (s.hidden <= 0 || s.n_q_heads <= 0 || s.n_kv_heads <= 0 || s.head_dim <= 0 || s.ffn <= 0 ||
      s.n_experts <= 0 || s.top_k <= 0 || s.max_tokens <= 0 || s.max_pos <= 0)
    return fail(err, NF_ERR_INVALID_ARG, "shape: every size must be positive");
  if (s.dtype != NF_F32 && s.dtype != NF_BF16)
    return fail(err, NF_ERR_UNSUPPORTED, "shape: dtype %d is not NF_F32 or NF_BF16", s.dtype);
  if (s.n_q_heads % s.n_kv_heads)
    return fail(err, NF_ERR_INVALID_ARG, "shape: n_q_heads %d not a multiple of n_kv_heads %d",
                s.n_q_heads, s.n_kv_heads);
  const int G = s.n_q_heads / s.n_kv_heads;
  if (G > 16)
    return fail(err, NF_ERR_UNSUPPORTED, "shape: more than 16 query heads per KV head (%d)", G);
  if (s.head_dim % 32 || s.head_dim > 256)
    return fail(err, NF_ERR_UNSUPPORTED, "shape: head_dim %d must be a multiple of 32, at most 256", s.head_dim);
  if (s.dtype == NF_BF16 && s.head_dim != 128)
    return fail(err, NF_ERR_UNSUPPORTED, "shape: bf16 layers need head_dim 128 (got %d)", s.head_dim);
  if (s.hidden % 8 || s.ffn % 8 || s.head_dim % 8)
    return fail(err, NF_ERR_UNSUPPORTED, "shape: hidden, ffn and head_dim must be multiples of 8");
  if (s.top_k > s.n_experts || s.n_experts > 64 || s.top_k > 8)
    return fail(err, NF_ERR_UNSUPPORTED, "shape: need top_k <= n_experts <= 64 and top_k <= 8");
  if (s.n_experts == 1 && s.top_k != 1)
    return fail(err, NF_ERR_INVALID_ARG, "shape: a dense layer has top_k 1");
  if (!(s.rms_eps >= 0.f) || !(s.rope_theta > 0.0))
    return fail(err, NF_ERR_INVALID_ARG, "shape: rms_eps must be >= 0 and rope_theta > 0");
  if ((int64_t)s.max_tokens * s.top_k > (1 << 24))
    return fail(err, NF_ERR_OUT_OF_RANGE, "shape: max_tokens too large");
  if (s.dtype == NF_BF16) {
    // the bf16 GEMMs address each operand with 32-bit byte offsets
    const int64_t rows = (int64_t)s.max_tokens * s.top_k;
    const int64_t qkv = (int64_t)(s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim;
    const int64_t qd = (int64_t)s.n_q_heads * s.head_dim;
    const int64_t widest = std::max(std::max((int64_t)s.hidden, (int64_t)s.ffn), std::max(qkv, qd));
    const int64_t weight = std::max(std::max(qkv, qd), (int64_t)s.ffn) * s.hidden;
    if (std::max(rows * widest, weight) * 2 >= (int64_t(1) << 32))
      return fail(err, NF_ERR_OUT_OF_RANGE, "shape: a GEMM operand would exceed 4 GiB");
  }
  return NF_OK;
}

nf_status check_batch(const nf_shape& s, int64_t n_pages, int page_size, const nf_batch& b,
                      std::string& err) {
  const int T = b.n_tokens, R = b.n_requests;
  if (T < 0 || R < 0) return fail(err, NF_ERR_INVALID_ARG, "batch: negative size");
  if (T > s.max_tokens)
    return fail(err, NF_ERR_OUT_OF_RANGE, "batch: %d tokens exceed max_tokens %d", T, s.max_tokens);
  if (T == 0) return NF_OK;
  if (R == 0) return fail(err, NF_ERR_INVALID_ARG, "batch: tokens without requests");
  if (!b.x || !b.out) return fail(err, NF_ERR_INVALID_ARG, "batch: x and out must be set");
  if (b.x == b.out) return fail(err, NF_ERR_INVALID_ARG, "batch: out must not alias x");
  if (!b.req_q_start || !b.req_q_len || !b.req_pos0 || !b.pos || !b.page_indptr || !b.page_indices)
    return fail(err, NF_ERR_INVALID_ARG, "batch: a host array is null");
  if (s.n_experts > 1 && !b.router_logits)
    return fail(err, NF_ERR_INVALID_ARG, "batch: router_logits required for a mixture-of-experts layer");
  if (b.page_indptr[0] != 0) return fail(err, NF_ERR_INVALID_ARG, "batch: page_indptr[0] must be 0");
  int64_t expect_start = 0;           // 64-bit: a huge q_len must not wrap past the bound check
  for (int r = 0; r < R; ++r) {
    const int qs = b.req_q_start[r], ql = b.req_q_len[r], p0 = b.req_pos0[r];
    if (ql < 0 || p0 < 0)
      return fail(err, NF_ERR_INVALID_ARG, "batch: request %d has negative q_len or pos0", r);
    if (qs != expect_start)
      return fail(err, NF_ERR_INVALID_ARG, "batch: request %d starts at token %d, expected %lld", r, qs,
                  (long long)expect_start);
    expect_start += ql;
    if (expect_start > T)
      return fail(err, NF_ERR_INVALID_ARG, "batch: requests cover more than %d tokens", T);
    if ((int64_t)p0 + ql > s.max_pos)
      return fail(err, NF_ERR_OUT_OF_RANGE, "batch: request %d reaches position %lld >= max_pos %d", r,
                  (long long)p0 + ql - 1, s.max_pos);
    for (int i = 0; i < ql; ++i)
      if (b.pos[qs + i] != p0 + i)
        return fail(err, NF_ERR_INVALID_ARG, "batch: pos[%d] = %d, expected pos0 + %d = %d", qs + i,
                    b.pos[qs + i], i, p0 + i);
    const int64_t have = (int64_t)b.page_indptr[r + 1] - b.page_indptr[r];
    if (have < 0) return fail(err, NF_ERR_INVALID_ARG, "batch: page_indptr decreases at request %d", r);
    const int64_t need = ((int64_t)p0 + ql + page_size - 1) / page_size;
    if (have < need)
      return fail(err, NF_ERR_OUT_OF_RANGE, "batch: request %d has %lld pages, needs %lld", r,
                  (long long)have, (long long)need);
  }
  if (expect_start != T)
    return fail(err, NF_ERR_INVALID_ARG, "batch: requests cover %lld tokens, batch has %d", (long long)expect_start,
                T);
  const int64_t nnz = b.page_indptr[R];
  std::vector<int32_t> owner((size_t)n_pages, -1);
  for (int r = 0; r < R; ++r) {
    for (int64_t i = b.page_indptr[r]; i < b.page_indptr[r + 1]; ++i) {
      const int32_t pg = b.page_indices[i];
      if (pg < 0 || pg >= n_pages)
        return fail(err, NF_ERR_OUT_OF_RANGE, "batch: page index %d (entry %lld) outside pool of %lld", pg,
                    (long long)i, (long long)n_pages);
      if (owner[pg] >= 0)
        return fail(err, NF_ERR_INVALID_ARG, "batch: page %d listed twice (requests %d and %d)", pg, owner[pg],
                    r);
      owner[pg] = r;
    }
  }
  (void)nnz;
  return NF_OK;
}

nf_status check_plan(const nf_plan& p, int cus_per_xcd, std::string& err) {
  if (p.count < 1 || p.count > NF_MAX_NANO)
    return fail(err, NF_ERR_INVALID_ARG, "plan: count %d outside 1..%d", p.count, NF_MAX_NANO);
  if (p.order != NF_ORDER_PIPELINED && p.order != NF_ORDER_SEQUENTIAL && p.order != NF_ORDER_DEEP &&
      p.order != NF_ORDER_LANES)
    return fail(err, NF_ERR_INVALID_ARG, "plan: unknown order %d", p.order);
  if (p.n_streams != 1 && p.n_streams != 2)
    return fail(err, NF_ERR_INVALID_ARG, "plan: n_streams must be 1 or 2");
  if (p.order == NF_ORDER_LANES && p.n_streams != 2)
    return fail(err, NF_ERR_INVALID_ARG, "plan: the lanes order needs two streams");
  if (p.gemm_cus_per_xcd < 0 || p.gemm_cus_per_xcd >= cus_per_xcd)
    return fail(err, NF_ERR_OUT_OF_RANGE, "plan: gemm_cus_per_xcd %d outside 0..%d", p.gemm_cus_per_xcd,
                cus_per_xcd - 1);
  if (p.attn_cus_per_xcd < 0 || p.attn_cus_per_xcd >= cus_per_xcd)
    return fail(err, NF_ERR_OUT_OF_RANGE, "plan: attn_cus_per_xcd %d outside 0..%d", p.attn_cus_per_xcd,
                cus_per_xcd - 1);
  if (p.attn_waves_per_cu < 0 || p.attn_waves_per_cu > 16)
    return fail(err, NF_ERR_OUT_OF_RANGE, "plan: attn_waves_per_cu %d outside 0..16", p.attn_waves_per_cu);
  if (p.n_streams == 1 && (p.gemm_cus_per_xcd != 0 || p.attn_cus_per_xcd != 0))
    return fail(err, NF_ERR_INVALID_ARG, "plan: a CU split needs two streams");
  for (int j = 0; j < p.count; ++j)
    if (p.sizes[j] < 0) return fail(err, NF_ERR_INVALID_ARG, "plan: negative nano-batch size");
  return NF_OK;
}

nf_status check_plan_batch(const nf_plan& p, int n_tokens, std::string& err) {
  if (p.count == 1 && p.sizes[0] == 0) return NF_OK;   // one nano-batch of whatever the batch holds
  int64_t sum = 0;
  for (int j = 0; j < p.count; ++j) {
    if (p.sizes[j] <= 0 && n_tokens > 0)
      return fail(err, NF_ERR_NO_PLAN, "plan: nano-batch %d is empty", j);
    sum += p.sizes[j];
  }
  if (sum != n_tokens)
    return fail(err, NF_ERR_NO_PLAN, "plan: sizes sum to %lld, batch has %d tokens", (long long)sum, n_tokens);
  return NF_OK;
}

void build_work(const nf_shape& s, const nf_batch& b, const nf_plan& p, int page_size, int target_items,
                int min_split_pages, int max_item_pages, StepWork& w) {
  const int T = b.n_tokens, R = b.n_requests;
  const int G = s.n_q_heads / s.n_kv_heads;
  const int qg = std::max(1, 16 / G);               // query tokens per item
  w.tok_req.assign(T, 0);
  for (int r = 0; r < R; ++r)
    for (int i = 0; i < b.req_q_len[r]; ++i) w.tok_req[b.req_q_start[r] + i] = r;
  w.items.clear();
  w.merges.clear();
  w.nanos.clear();
  w.n_partials = 0;

  const int count = (p.count == 1 && p.sizes[0] == 0) ? 1 : p.count;
  int t0 = 0;
  for (int j = 0; j < count; ++j) {
    NanoWork nw;
    nw.t0 = t0;
    nw.t1 = (count == 1 && p.sizes[0] == 0) ? T : t0 + p.sizes[j];
    // token groups of this nano-batch (never crossing a request)
    struct Group { int req, tok0, ntok, pages; };
    std::vector<Group> groups;
    int64_t total_pages = 0;
    for (int t = nw.t0; t < nw.t1;) {
      const int r = w.tok_req[t];
      const int req_end = std::min(nw.t1, b.req_q_start[r] + b.req_q_len[r]);
      const int n = std::min(qg, req_end - t);
      const int keys = b.pos[t + n - 1] + 1;
      const int pages = (keys + page_size - 1) / page_size;
      groups.push_back({r, t, n, pages});
      total_pages += pages;
      t += n;
    }
    // split page ranges when the groups cannot fill the attention CUs, and cap
    // the pages of one item
    int per = 1 << 30;
    const int64_t target_wg = std::max(1, target_items);
    if (min_split_pages > 0 && (int64_t)groups.size() * s.n_kv_heads < target_wg && total_pages > 0) {
      const int64_t want = (total_pages * s.n_kv_heads + target_wg - 1) / target_wg;
      per = (int)std::max<int64_t>(min_split_pages, want);
    }
    if (max_item_pages > 0) per = std::min(per, max_item_pages);
    // longest groups first so the long tails start early
    std::stable_sort(groups.begin(), groups.end(), [](const Group& x, const Group& y) { return x.pages > y.pages; });
    nw.item0 = (int)w.items.size();
    nw.merge0 = (int)w.merges.size();
    for (const Group& g : groups) {
      if (g.pages <= per) {
        w.items.push_back({g.req, g.tok0, g.ntok, 0, g.pages, -1, 0, 0});
        continue;
      }
      const int pieces = (g.pages + per - 1) / per;
      w.merges.push_back({g.tok0, g.ntok, w.n_partials, pieces});
      for (int k = 0; k < pieces; ++k) {
        const int pb = k * per, pe = std::min(g.pages, pb + per);
        w.items.push_back({g.req, g.tok0, g.ntok, pb, pe, w.n_partials + k, 0, 0});
      }
      w.n_partials += pieces;
    }
    nw.n_items = (int)w.items.size() - nw.item0;
    nw.n_merges = (int)w.merges.size() - nw.merge0;
    w.nanos.push_back(nw);
    t0 = nw.t1;
  }
}

}  // namespace nf
