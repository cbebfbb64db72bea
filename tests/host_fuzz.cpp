// Randomised checks of the step's host-side logic: batch, plan and shape
// validation, the attention work lists the kernels index with, and the plan
// step model.  Built with AddressSanitizer and UndefinedBehaviorSanitizer from
// the library's host-only sources (no HIP) by tests/test_host_sanitizers.py.
//
// Every generated batch either fails validation, or passes and then yields
// work lists whose every index the attention kernels use stays in range:
// requests, tokens, pages of the request, partial slots, merge items.
//
// usage: host_fuzz <cases> <seed>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <algorithm>
#include <random>
#include <string>
#include <vector>

#include "../intra_operation_overlap_amd/csrc/nf_host.h"

namespace nf {
nf_status set_error(nf_status st, const char*) { return st; }
}  // namespace nf

using namespace nf;

namespace {

std::mt19937_64 rng;

int uni(int lo, int hi) {   // inclusive
  return std::uniform_int_distribution<int>(lo, hi)(rng);
}
bool coin(double p) { return std::uniform_real_distribution<double>(0, 1)(rng) < p; }

[[noreturn]] void die(const char* what, int c) {
  std::fprintf(stderr, "case %d: %s\n", c, what);
  std::exit(1);
}

struct HostBatch {
  std::vector<int32_t> q_start, q_len, pos0, pos, indptr, indices;
  nf_batch b{};
  void bind(int T, int R) {
    b.n_tokens = T;
    b.n_requests = R;
    static char dummy_x, dummy_out;
    static float dummy_logits;
    b.x = &dummy_x;
    b.out = &dummy_out;
    b.router_logits = &dummy_logits;
    // one past each vector so an empty batch still has non-null arrays
    q_start.push_back(0);
    q_len.push_back(0);
    pos0.push_back(0);
    pos.push_back(0);
    indices.push_back(0);
    b.req_q_start = q_start.data();
    b.req_q_len = q_len.data();
    b.req_pos0 = pos0.data();
    b.pos = pos.data();
    b.page_indptr = indptr.data();
    b.page_indices = indices.data();
  }
};

nf_shape random_shape() {
  nf_shape s{};
  s.dtype = coin(0.8) ? NF_BF16 : NF_F32;
  s.n_kv_heads = uni(1, 8);
  const int gs[] = {1, 2, 4, 8, 16};
  s.n_q_heads = s.n_kv_heads * gs[uni(0, 4)];
  s.head_dim = s.dtype == NF_BF16 ? 128 : 32 * uni(1, 8);
  s.hidden = 8 * uni(8, 256);
  s.ffn = 8 * uni(8, 512);
  s.n_experts = coin(0.2) ? uni(2, 8) : 1;
  s.top_k = s.n_experts > 1 ? uni(1, s.n_experts) : 1;
  s.max_tokens = uni(1, 600);
  s.max_pos = uni(1, 40000);
  s.rms_eps = 1e-5f;
  s.rope_theta = 1e4f;
  if (coin(0.05)) s.hidden = uni(-3, 0);
  if (coin(0.05)) s.n_q_heads = s.n_kv_heads * 3 + 1;
  return s;
}

// A batch of decode requests and prefill chunks on a pool of n_pages pages,
// then, with some probability, one corruption.
void random_batch(const nf_shape& s, int& n_pages, HostBatch& h) {
  const int PS = 16;
  const int R = uni(0, 40);
  int T = 0;
  std::vector<int> need(R);
  for (int r = 0; r < R; ++r) {
    int ql = coin(0.7) ? 1 : uni(0, 70);
    if (T + ql > s.max_tokens) ql = std::max(0, std::min(ql, s.max_tokens - T));
    const int p0 = uni(0, std::max(0, std::min(s.max_pos, 20000) - std::max(ql, 1)));
    h.q_start.push_back(T);
    h.q_len.push_back(ql);
    h.pos0.push_back(p0);
    for (int i = 0; i < ql; ++i) h.pos.push_back(p0 + i);
    T += ql;
    need[r] = (p0 + ql + PS - 1) / PS + (coin(0.1) ? uni(0, 3) : 0);
  }
  int total = 0;
  for (int v : need) total += v;
  n_pages = std::max(1, coin(0.05) ? uni(1, total + 1) : total + uni(0, 200));
  std::vector<int32_t> perm(n_pages);
  for (int i = 0; i < n_pages; ++i) perm[i] = i;
  std::shuffle(perm.begin(), perm.end(), rng);
  int used = 0;
  h.indptr.assign(1, 0);
  for (int r = 0; r < R; ++r) {
    for (int i = 0; i < need[r]; ++i) h.indices.push_back(used < n_pages ? perm[used++] : uni(0, n_pages - 1));
    h.indptr.push_back((int32_t)h.indices.size());
  }
  if (coin(0.35)) {
    switch (uni(0, 11)) {
      case 0: if (R) h.q_len[uni(0, R - 1)] = std::numeric_limits<int32_t>::max(); break;
      case 1: if (R) h.q_len[uni(0, R - 1)] = -uni(1, 5); break;
      case 2: if (R) h.q_start[uni(0, R - 1)] += uni(-2, 2); break;
      case 3: if (R) h.pos0[uni(0, R - 1)] = std::numeric_limits<int32_t>::max() - uni(0, 3); break;
      case 4: if (!h.pos.empty()) h.pos[uni(0, (int)h.pos.size() - 1)] += uni(-3, 3); break;
      case 5: if (R) h.indptr[uni(1, R)] = uni(-5, (int)h.indices.size() + 5); break;
      case 6: if (!h.indices.empty()) h.indices[uni(0, (int)h.indices.size() - 1)] = uni(-3, n_pages + 3); break;
      case 7: if (h.indices.size() > 1) h.indices[1] = h.indices[0]; break;
      case 8: T += uni(-3, 3); break;
      case 9: T = std::numeric_limits<int32_t>::max(); break;
      case 10: if (R) h.pos0[uni(0, R - 1)] = -uni(1, 9); break;
      default: if (R) h.q_len[uni(0, R - 1)] = std::numeric_limits<int32_t>::max() / 2 + uni(0, 99); break;
    }
  }
  h.bind(T, R);
}

nf_plan random_plan(int T) {
  nf_plan p{};
  p.count = uni(1, NF_MAX_NANO);
  if (coin(0.05)) p.count = uni(-1, NF_MAX_NANO + 2);
  const int k = std::max(1, std::min(p.count, NF_MAX_NANO));
  int left = std::max(T, 0);
  for (int j = 0; j < k; ++j) {
    p.sizes[j] = j + 1 < k ? uni(0, left) : left;
    left -= p.sizes[j];
  }
  if (coin(0.1)) p.sizes[uni(0, k - 1)] += uni(-2, 2);
  if (p.count == 1 && coin(0.3)) p.sizes[0] = 0;          // "the whole batch"
  p.order = uni(0, 3);
  if (coin(0.05)) p.order = uni(-1, 5);
  p.n_streams = uni(1, 2);
  p.gemm_cus_per_xcd = coin(0.5) ? 0 : uni(0, 32);
  p.attn_cus_per_xcd = coin(0.5) ? 0 : uni(0, 32);
  p.attn_waves_per_cu = coin(0.6) ? 0 : uni(0, 12);
  return p;
}

// Every index the attention and merge kernels read from the work lists.
void check_work(const nf_shape& s, const nf_batch& b, const StepWork& w, int max_item_pages, int c) {
  const int T = b.n_tokens, R = b.n_requests;
  const int G = s.n_q_heads / s.n_kv_heads;
  const int qg = std::max(1, 16 / G);
  if ((int)w.tok_req.size() != T) die("tok_req size", c);
  for (int t = 0; t < T; ++t) {
    const int r = w.tok_req[t];
    if (r < 0 || r >= R || t < b.req_q_start[r] || t >= b.req_q_start[r] + b.req_q_len[r]) die("tok_req", c);
  }
  if (w.nanos.empty()) die("no nano-batch", c);
  int t0 = 0, item_end = 0, merge_end = 0;
  std::vector<int> partial_uses(std::max(0, w.n_partials), 0), item_of(std::max(0, w.n_partials), -1);
  for (int i = 0; i < (int)w.items.size(); ++i)
    if (w.items[i].partial >= 0 && w.items[i].partial < w.n_partials) item_of[w.items[i].partial] = i;
  for (const NanoWork& nw : w.nanos) {
    if (nw.t0 != t0 || nw.t1 < nw.t0 || nw.t1 > T) die("nano ranges", c);
    if (nw.item0 != item_end || nw.n_items < 0 || nw.item0 + nw.n_items > (int)w.items.size()) die("nano items", c);
    if (nw.merge0 != merge_end || nw.n_merges < 0 || nw.merge0 + nw.n_merges > (int)w.merges.size())
      die("nano merges", c);
    // each token of the nano-batch is covered by one group, each group by one
    // whole item or by split pieces that tile its pages
    std::vector<int> covered(nw.t1 - nw.t0, 0);
    for (int i = nw.item0; i < nw.item0 + nw.n_items; ++i) {
      const AttnItem& it = w.items[i];
      if (it.req < 0 || it.req >= R) die("item request", c);
      if (it.ntok < 1 || it.ntok > qg) die("item tokens", c);
      if (it.tok0 < nw.t0 || it.tok0 + it.ntok > nw.t1) die("item outside its nano-batch", c);
      const int rs = b.req_q_start[it.req], re = rs + b.req_q_len[it.req];
      if (it.tok0 < rs || it.tok0 + it.ntok > re) die("item outside its request", c);
      const int keys = b.pos[it.tok0 + it.ntok - 1] + 1;
      const int pages = (keys + 15) / 16;
      const int have = b.page_indptr[it.req + 1] - b.page_indptr[it.req];
      if (it.page_begin < 0 || it.page_end <= it.page_begin || it.page_end > pages || pages > have)
        die("item pages", c);
      if (max_item_pages > 0 && it.page_end - it.page_begin > max_item_pages) die("item longer than the cap", c);
      if (it.partial < 0) {
        if (it.page_begin != 0 || it.page_end != pages) die("whole item does not span its pages", c);
        for (int t = it.tok0; t < it.tok0 + it.ntok; ++t) covered[t - nw.t0]++;
      } else {
        if (it.partial >= w.n_partials) die("partial slot", c);
        partial_uses[it.partial]++;
      }
    }
    for (int m = nw.merge0; m < nw.merge0 + nw.n_merges; ++m) {
      const MergeItem& mi = w.merges[m];
      if (mi.n_partials < 2 || mi.first_partial < 0 || mi.first_partial + mi.n_partials > w.n_partials)
        die("merge partials", c);
      if (mi.ntok < 1 || mi.tok0 < nw.t0 || mi.tok0 + mi.ntok > nw.t1) die("merge tokens", c);
      // the pieces of this merge: items whose partial lies in its slots
      int next = 0, pages = -1;
      for (int q = 0; q < mi.n_partials; ++q) {
        const int i = item_of[mi.first_partial + q];
        const AttnItem* piece = i >= nw.item0 && i < nw.item0 + nw.n_items ? &w.items[i] : nullptr;
        if (!piece || piece->tok0 != mi.tok0 || piece->ntok != mi.ntok) die("merge piece", c);
        if (piece->page_begin != next) die("merge pieces do not tile the pages", c);
        next = piece->page_end;
        pages = (b.pos[piece->tok0 + piece->ntok - 1] + 16) / 16;
      }
      if (next != pages) die("merge pieces stop short", c);
      for (int t = mi.tok0; t < mi.tok0 + mi.ntok; ++t) covered[t - nw.t0]++;
    }
    for (int v : covered)
      if (v != 1) die("token not covered exactly once", c);
    t0 = nw.t1;
    item_end = nw.item0 + nw.n_items;
    merge_end = nw.merge0 + nw.n_merges;
  }
  if (t0 != T || item_end != (int)w.items.size() || merge_end != (int)w.merges.size()) die("lists not covered", c);
  for (int u : partial_uses)
    if (u != 1) die("partial slot used other than once", c);
}

void check_model(const nf_shape& s, const nf_batch& b, const nf_plan& plan, int c) {
  nf_plan_profile p{};
  p.n_points = uni(1, NF_PROFILE_POINTS);
  double tok = 0;
  for (int i = 0; i < p.n_points; ++i) {
    tok += uni(1, 512);
    p.tokens[i] = tok;
    p.front_us[i] = uni(1, 200);
    p.oproj_us[i] = uni(1, 200);
    p.ffn_us[i] = uni(1, 500);
  }
  p.attn_base_us = uni(0, 20);
  p.attn_us_per_page = 0.001 * uni(0, 50);
  p.gap_us = uni(0, 10);
  p.wait_us = uni(0, 30);
  p.slow_gemm = 1 + 0.1 * uni(0, 30);
  p.slow_attn = 1 + 0.1 * uni(0, 30);
  double units[NF_MAX_NANO] = {}, tokens[NF_MAX_NANO] = {};
  attn_page_units(s, b, plan, units);
  const int k = std::max(1, std::min(plan.count, NF_MAX_NANO));
  for (int j = 0; j < k; ++j) {
    if (!(units[j] >= 0) || !std::isfinite(units[j])) die("page units", c);
    tokens[j] = (plan.count == 1 && plan.sizes[0] == 0) ? b.n_tokens : plan.sizes[j];
  }
  const double us = predict_plan_us(p, plan, tokens, units);
  if (!(us >= 0) || !std::isfinite(us)) die("model prediction", c);
}

}  // namespace

int main(int argc, char** argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 2000;
  rng.seed(argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 1);
  int valid = 0, rejected = 0, work = 0;
  for (int c = 0; c < cases; ++c) {
    const nf_shape s = random_shape();
    std::string err;
    if (check_shape(s, err) != NF_OK) {
      ++rejected;
      if (std::getenv("HOST_FUZZ_VERBOSE")) std::fprintf(stderr, "%s\n", err.c_str());
      continue;
    }
    int n_pages = 0;
    HostBatch h;
    random_batch(s, n_pages, h);
    if (check_batch(s, n_pages, 16, h.b, err) != NF_OK) {
      ++rejected;
      if (std::getenv("HOST_FUZZ_VERBOSE")) std::fprintf(stderr, "%s\n", err.c_str());
      continue;
    }
    nf_plan plan = random_plan(h.b.n_tokens);
    if (check_plan(plan, 32, err) != NF_OK || check_plan_batch(plan, h.b.n_tokens, err) != NF_OK) {
      ++rejected;
      continue;
    }
    ++valid;
    if (h.b.n_tokens == 0) continue;
    // the step's calls: four-wave items (no cap) or one-wave items (32 pages)
    const int attn_cus = 8 * uni(1, 32);
    const bool wave_items = coin(0.5);
    StepWork w;
    const int cap = wave_items ? 32 : 0;
    build_work(s, h.b, plan, 16, wave_items ? 8 * attn_cus : 2 * attn_cus, 8, cap, w);
    check_work(s, h.b, w, cap, c);
    // and arbitrary splitting parameters
    const int cap2 = coin(0.5) ? 0 : uni(1, 64);
    build_work(s, h.b, plan, 16, uni(1, 5000), uni(0, 20), cap2, w);
    check_work(s, h.b, w, cap2, c);
    check_model(s, h.b, plan, c);
    ++work;
  }
  std::printf("ok: %d cases, %d rejected, %d valid, %d with work lists checked\n", cases, rejected, valid, work);
  return 0;
}
