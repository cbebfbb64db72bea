// Host-only logic of the step (no HIP calls): argument validation and the
// per-step work lists the kernels consume.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/nf.h"

namespace nf {

// Stores `msg` as the calling thread's nf_last_error() text; returns st.
nf_status set_error(nf_status st, const char* msg);

// One attention work item: query tokens tok0 .. tok0+ntok-1 of request `req`,
// keys of its logical pages page_begin .. page_end-1; the result goes straight
// to the attention output (partial < 0) or to partial slot `partial`.
struct AttnItem {
  int32_t req;
  int32_t tok0;
  int32_t ntok;
  int32_t page_begin;
  int32_t page_end;
  int32_t partial;
  int32_t pad0, pad1;
};

// A token group whose page range was split: partial slots first .. first+n-1.
struct MergeItem {
  int32_t tok0, ntok;
  int32_t first_partial, n_partials;
};

struct NanoWork {
  int t0 = 0, t1 = 0;              // token range
  int item0 = 0, n_items = 0;      // attention items
  int merge0 = 0, n_merges = 0;    // merge items
};

struct StepWork {
  std::vector<int32_t> tok_req;    // [T] request of each token
  std::vector<AttnItem> items;
  std::vector<MergeItem> merges;
  std::vector<NanoWork> nanos;
  int n_partials = 0;
};

nf_status check_shape(const nf_shape& s, std::string& err);
nf_status check_batch(const nf_shape& s, int64_t n_pages, int page_size, const nf_batch& b,
                      std::string& err);
// static plan checks (count, order, streams, CU split); cus_per_xcd = CUs in one XCD
nf_status check_plan(const nf_plan& p, int cus_per_xcd, std::string& err);
// plan against one batch: sizes must cover the batch's tokens
nf_status check_plan_batch(const nf_plan& p, int n_tokens, std::string& err);

// Splits the batch per the plan into nano-batches and builds the attention
// items.  A nano-batch with fewer (token group, KV head) items than
// `target_items` gets its page ranges split (min_split_pages pages at least
// per piece; 0 disables splitting); no item holds more than max_item_pages
// pages (0: no cap).  Split pieces write partials merged by a later kernel.
void build_work(const nf_shape& s, const nf_batch& b, const nf_plan& p, int page_size, int target_items,
                int min_split_pages, int max_item_pages, StepWork& w);

// Step-time model of a plan (plan_model.cpp).  tokens[j] / pages[j]: the
// tokens and the attention page units (work items x KV pages) of nano-batch j.
double predict_plan_us(const nf_plan_profile& p, const nf_plan& plan, const double* tokens, const double* pages);
// Attention page units of each nano-batch of `plan` on batch `b`.
void attn_page_units(const nf_shape& sh, const nf_batch& b, const nf_plan& plan, double* units);

}  // namespace nf
