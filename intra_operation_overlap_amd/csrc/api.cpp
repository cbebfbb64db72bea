// C ABI of the nano-batched decoder-layer step: objects, metadata upload and
// the overlap executor.
//
// Executor.  A plan splits the batch's tokens into nano-batches and duplicates
// every operation per nano-batch (nano-batching, README "Introduction" and
// "Abstract" on the ossradar Nanoflow page).  With two streams, the GEMM side
// (norm, QKV, RoPE/append, O-proj, norm, FFN) runs on stream G and attention
// on stream A; each stream may be restricted to a subset of every XCD's CUs
// (hipExtStreamCreateWithCUMask), which is the execution-unit partition of the
// device-level pipeline ("How it works" on the bytedragons Nanoflow page).
// Events carry the only cross-stream dependencies: attention(j) waits for the
// RoPE/append of nano-batch j, the O-projection of j waits for attention(j).
// In the pipelined order the GEMM stream issues the front half of nano-batch
// j+1 (norm, QKV, RoPE/append) before the back half of j (O-proj, FFN), so
// j's memory-bound attention runs beside j+1's compute-bound projections and
// compute stays on the critical path (README "Introduction").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "nf_internal.h"

using namespace nf;

namespace {

thread_local std::string g_err;

nf_status set_err(nf_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
nf_status set_err(nf_status st, const char* fmt, ...) {
  char buf[768];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

}  // namespace

nf_status nf::set_error(nf_status st, const char* msg) {
  g_err = msg;
  return st;
}

namespace {

// Host-side fault injection for tests of the error paths: with NF_FAULT set
// to "after:<n>" when nf_layer_step or nf_stack_step is called, the n-th
// (from 0) checked HIP call inside that call is not made and reports
// failure instead, once.  No device work is touched: the call is skipped.
thread_local int g_fault_at = -1;
thread_local int g_fault_seen = 0;

struct FaultScope {
  FaultScope() {
    g_fault_at = -1;
    g_fault_seen = 0;
    const char* v = std::getenv("NF_FAULT");
    if (v && std::strncmp(v, "after:", 6) == 0) g_fault_at = std::atoi(v + 6);
  }
  ~FaultScope() { g_fault_at = -1; }
};

bool fault_now() {
  if (g_fault_at < 0) return false;
  if (g_fault_seen++ != g_fault_at) return false;
  g_fault_at = -1;
  return true;
}

// On a HIP failure the runtime's last-error slot is cleared so that the
// caller's next unrelated HIP call does not report it again.
#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
    if (fault_now()) return set_err(NF_ERR_HIP, "%s not made: injected failure (NF_FAULT)", #expr); \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess) {                                                               \
      (void)hipGetLastError();                                                            \
      return set_err(NF_ERR_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_), \
                     __FILE__, __LINE__);                                                 \
    }                                                                                     \
  } while (0)

constexpr int PAGE_SIZE = 16;

struct DevBuf {
  void* p = nullptr;
  size_t bytes = 0;
  // buffers this one outgrew: kept until the layer is destroyed, so device
  // pointers captured in a graph stay valid (and growing needs no sync)
  std::vector<void*> old;
};

// Kinds of kernel launches, for the per-kernel timing facility.
enum Kind {
  K_NORM1, K_QKV, K_QKV_RED, K_ROPE, K_ATTN, K_MERGE, K_OPROJ, K_OPROJ_RED, K_NORM2,
  K_GATEUP, K_GATEUP_RED, K_DOWN, K_DOWN_RED, K_ROUTE, K_MOE_GATEUP, K_MOE_DOWN, K_COMBINE,
  K_COUNT
};
const char* kKindNames[K_COUNT] = {
  "rmsnorm_attn", "gemm_qkv", "gemm_qkv_splitk_reduce", "rope_kv_append", "attention",
  "attention_merge", "gemm_o_residual", "gemm_o_splitk_reduce", "rmsnorm_ffn", "gemm_gate_up_swiglu",
  "gemm_gate_up_splitk_reduce", "gemm_down_residual", "gemm_down_splitk_reduce", "moe_route",
  "moe_gemm_gate_up_swiglu", "moe_gemm_down", "moe_combine",
};

struct ProfRec {
  int kind;
  hipEvent_t a, b;
};

struct StreamPair {
  hipStream_t g = nullptr, a = nullptr;
};

size_t dtype_bytes(int dt) { return dt == NF_BF16 ? 2 : 4; }

}  // namespace

// a plan the last search timed: its predicted and measured ms per step
struct SearchEntry {
  nf_plan plan;
  double predicted_ms, measured_ms;
  bool calibration = false;     // a run the model's inputs were fitted to
};

struct nf_layer {
  nf_shape s{};
  nf_weights w{};
  int device = 0;
  int n_cus = 0, n_xcd = 8, cus_per_xcd = 32;
  std::vector<int> xcc_of_bit;                  // CU-mask bit -> XCD (measured; -1 unknown)
  nf_plan plan{};
  std::map<std::pair<int, int>, StreamPair> pairs;   // unmasked two-stream pair (masked ones: g_pairs)
  hipEvent_t ev_app[NF_MAX_NANO] = {}, ev_att[NF_MAX_NANO] = {};
  hipEvent_t ev_start = nullptr, ev_g = nullptr, ev_a = nullptr;
  hipEvent_t ev_lane = nullptr;                 // end of lane 1 (lanes order)
  // emulated tensor-parallel all-reduce of the O and down projections
  // (nf_layer_set_allreduce_emulation): mode 0 off, 1 copy engines, 2 a copy
  // kernel of ar_wgs workgroups; on stream sc, with these events
  int ar_mode = 0, ar_wgs = 16;
  hipStream_t sc = nullptr;
  hipStream_t sc2 = nullptr;                    // lane 1's collectives (lanes order)
  hipEvent_t ev_a2 = nullptr;
  hipEvent_t ev_o[NF_MAX_NANO] = {}, ev_co[NF_MAX_NANO] = {}, ev_d[NF_MAX_NANO] = {}, ev_cd[NF_MAX_NANO] = {};
  DevBuf x1r, ypre, ar_stage;   // the all-reduced x1, the down output before its all-reduce, the send leg
  DevBuf h, qkv, q_rot, attn, x1, h2, act, y;
  DevBuf r_idx, r_w, r_perm, r_inv, r_off;
  DevBuf splitk, part_o, part_ml, meta, cos_sin;
  DevBuf splitk_lane1;                          // lane 1's split-K partials (lanes order)
  DevBuf stack_out;                             // this layer's output inside a multi-layer step
  // expert weights in MFMA operand order for the weight-streaming kernels
  // (bf16 mixture-of-experts layers; empty otherwise)
  DevBuf wp_qkv, wp_o, wp_gu, wp_down;
  // bf16: the attention RMSNorm folded into the QKV projection.  w_qkv_g
  // holds W_qkv with the norm gain applied to its columns (made once), the
  // GEMM reads the layer input itself, and rs holds each row's 1 / RMS, which
  // RoPE/append applies to q, k and v
  bool fold_norm1 = false;
  DevBuf w_qkv_g, rs;
  void* stage[2] = {nullptr, nullptr};       // pinned, coherent host staging
  void* stage_dev[2] = {nullptr, nullptr};   // their device addresses
  size_t stage_bytes[2] = {0, 0};
  hipEvent_t stage_ev[2] = {nullptr, nullptr};
  bool stage_used[2] = {false, false};
  int stage_i = 0;
  bool prof = false;
  int prof_only = -1;                           // kind filter (-1: every kind)
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> ev_free;
  double prof_ms[K_COUNT] = {};
  int64_t prof_n[K_COUNT] = {};
  StepWork work;
  int last_T = 0;
  int attn_variant = -1;   // bf16 d=128 attention kernel: -1 chosen per step, 0 one-wave items, 1 four-wave items
  bool debug_capture = true;   // nf_layer_intermediate answers (nf_layer_debug_capture)
  std::vector<SearchEntry> search_report;   // the last plan search's timed plans
};

struct nf_kv_pool {
  const nf_layer* layer = nullptr;
  int device = 0;
  int32_t n_pages = 0, page_size = 0;
  int64_t block_bytes = 0;   // one page's K (or V) block: n_kv_heads x page_size x head_dim elements
  void* k = nullptr;
  void* v = nullptr;
  DevBuf offload;      // page list and gathered K / V blocks of nf_kv_offload
  DevBuf xfer;         // page list of nf_kv_pool_import / nf_kv_pool_export
};

namespace {

hipError_t ensure(DevBuf& b, size_t bytes) {
  if (bytes <= b.bytes) return hipSuccess;
  // at least doubling, so the buffers kept below stay under the final size
  const size_t want = std::max({bytes, 2 * b.bytes, (size_t)256});
  if (b.p) {                 // may still be in use by queued work or a graph
    b.old.push_back(b.p);
    b.p = nullptr;
    b.bytes = 0;
  }
  hipError_t e = hipMalloc(&b.p, want);
  if (e != hipSuccess) {
    b.p = nullptr;
    return e;
  }
  b.bytes = want;
  return hipSuccess;
}

void release(DevBuf& b) {
  if (b.p) (void)hipFree(b.p);
  for (void* q : b.old) (void)hipFree(q);
  b.old.clear();
  b.p = nullptr;
  b.bytes = 0;
}

// --------------------------------------------------------------- CU masks
struct CuMap {
  std::vector<int> xcc;   // CU-mask bit -> XCD, -1 unknown
  std::vector<int> cu;    // CU-mask bit -> hardware CU inside its XCD: HW_ID bits 15..8 (SE, SH, CU), -1 unknown
};
std::mutex g_map_mu;
std::map<int, CuMap> g_cu_maps;     // by device

// Runs the identity probe on a stream masked to `mask`; returns the distinct
// (XCC_ID, HW_ID CU field) pairs its workgroups reported.
nf_status probe_mask(const std::vector<uint32_t>& mask, std::vector<std::pair<int, int>>& seen) {
  constexpr int kBlocks = 512;
  seen.clear();
  uint32_t* d_id = nullptr;
  HIP_TRY(hipMalloc(&d_id, 2 * kBlocks * sizeof(uint32_t)));
  hipStream_t st = nullptr;
  std::vector<uint32_t> h_id(2 * kBlocks, 0xFFFFFFFFu);
  hipError_t e = hipExtStreamCreateWithCUMask(&st, (uint32_t)mask.size(), mask.data());
  if (e == hipSuccess) {
    e = probe_hwid(d_id, kBlocks, st);
    if (e == hipSuccess) e = hipMemcpyAsync(h_id.data(), d_id, h_id.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    (void)hipStreamDestroy(st);
  }
  (void)hipFree(d_id);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return set_err(NF_ERR_HIP, "CU-mask probe failed: %s", hipGetErrorString(e));
  }
  for (int b = 0; b < kBlocks; ++b) {
    const std::pair<int, int> id((int)(h_id[2 * b + 1] & 0xF), (int)((h_id[2 * b] >> 8) & 0xFF));
    if (std::find(seen.begin(), seen.end(), id) == seen.end()) seen.push_back(id);
  }
  std::sort(seen.begin(), seen.end());
  return NF_OK;
}

// Which XCD and which CU each CU-mask bit selects, measured.  The runtime
// deals mask bits to the XCDs in turn (bit i to XCD i % n_xcd), and every XCD
// must keep at least one CU of a mask, since workgroups are dealt to the XCDs
// round-robin whatever the mask.  So the probe masks are the aligned groups
// of n_xcd bits {n_xcd c .. n_xcd c + n_xcd - 1}, which hold one CU of every
// XCD under that rule: many single-wave workgroups run on each and report
// XCC_ID and the CU field of HW_ID (shader engine, array, CU).  The map is
// accepted when every group shows n_xcd distinct XCDs with one CU each and,
// per XCD, the groups select distinct CUs; bit n_xcd c + x is then CU c of
// XCD x.  Otherwise every bit stays -1 and budgets use the striping guess.
nf_status measure_cu_map(int device, int n_cus, int n_xcd, CuMap& out) {
  std::lock_guard<std::mutex> lk(g_map_mu);
  auto it = g_cu_maps.find(device);
  if (it != g_cu_maps.end()) {
    out = it->second;
    return NF_OK;
  }
  CuMap m;
  m.xcc.assign(n_cus, -1);
  m.cu.assign(n_cus, -1);
  const int words = (n_cus + 31) / 32, groups = n_cus / n_xcd;
  bool ok = n_cus % n_xcd == 0 && groups > 0;
  std::vector<std::vector<int>> per_xcd(n_xcd);
  std::vector<std::pair<int, int>> seen;
  for (int c = 0; ok && c < groups; ++c) {
    std::vector<uint32_t> mask(words, 0u);
    for (int x = 0; x < n_xcd; ++x) {
      const int bit = c * n_xcd + x;
      mask[bit / 32] |= 1u << (bit % 32);
    }
    nf_status st = probe_mask(mask, seen);
    if (st != NF_OK) return st;
    ok = (int)seen.size() == n_xcd;
    for (int x = 0; ok && x < n_xcd; ++x) {
      ok = seen[x].first == x;            // sorted: XCD x, exactly one CU
      if (ok) {
        m.xcc[c * n_xcd + x] = x;
        m.cu[c * n_xcd + x] = seen[x].second;
        per_xcd[x].push_back(seen[x].second);
      }
    }
  }
  for (int x = 0; ok && x < n_xcd; ++x) {
    std::vector<int> v = per_xcd[x];
    std::sort(v.begin(), v.end());
    ok = std::adjacent_find(v.begin(), v.end()) == v.end();
  }
  if (!ok) {
    m.xcc.assign(n_cus, -1);
    m.cu.assign(n_cus, -1);
  }
  g_cu_maps[device] = m;
  out = m;
  return NF_OK;
}

// CU budgets per XCD -> masks: the GEMM stream gets the first g CUs of each
// XCD, the attention stream the last a (g or a == 0: see nf_plan).  Whole-
// chip budgets use ordinary streams; a mask always leaves every XCD a CU.
int attn_budget(int g, int a, int per_xcd) { return a ? a : (g ? per_xcd - g : 0); }

void make_mask(const std::vector<int>& xcc, int n_xcd, int lo, int hi, std::vector<uint32_t>& m) {
  const int n = (int)xcc.size(), words = (n + 31) / 32;
  m.assign(words, 0u);
  std::vector<int> seen(std::max(n_xcd, 16), 0);
  for (int bit = 0; bit < n; ++bit) {
    const int x = xcc[bit] < 0 ? bit % n_xcd : xcc[bit];
    const int k = seen[x]++;                    // k-th CU of XCD x
    if (k >= lo && k < hi) m[bit / 32] |= 1u << (bit % 32);
  }
}

// CU-masked stream pairs are shared by every layer on a device, and at most
// kMaskedPairs of them stay alive (the least recently used is drained and
// destroyed when another is needed).  Each masked stream holds a hardware
// queue of its own; with a pair per layer and budget alive (a stack of
// layers that had each been given the plan), steps on masked streams stalled
// for milliseconds at a time: a traced attention launch and a GEMM launch on
// disjoint CU masks both took 11 ms against 0.5, and a four-layer two
// nano-batch step with 16 + 16 CUs per XCD averaged 1.81 ms per layer with
// every layer's pair alive against 1.37 with one.  A step holds its pair
// while it enqueues (`busy`), so a step on another host thread never
// destroys it underneath; when every pair is held, one more is made.
constexpr int kMaskedPairs = 2;

struct MaskedPair {
  int dev, g, ab;
  StreamPair p;
  uint64_t used;
  int busy;
};

std::mutex g_pairs_mu;
std::vector<MaskedPair> g_pairs;
uint64_t g_pairs_clock = 0;

// The pair for GEMM and attention budgets g and a (CUs per XCD, 0 = all),
// made on first use.  With `hold`, a masked pair stays held until
// release_pair.
nf_status get_pair(nf_layer* L, int g, int a, StreamPair& out, bool hold = false) {
  const int ab = attn_budget(g, a, L->cus_per_xcd);
  auto key = std::make_pair(g, ab);
  if (g == 0 && ab == 0) {
    auto it = L->pairs.find(key);
    if (it != L->pairs.end()) {
      out = it->second;
      return NF_OK;
    }
  } else {
    std::lock_guard<std::mutex> lk(g_pairs_mu);
    for (MaskedPair& e : g_pairs)
      if (e.dev == L->device && e.g == g && e.ab == ab) {
        e.used = ++g_pairs_clock;
        e.busy += hold;
        out = e.p;
        return NF_OK;
      }
  }
  if ((g || ab) && L->xcc_of_bit.empty()) {
    CuMap cm;
    nf_status st = measure_cu_map(L->device, L->n_cus, L->n_xcd, cm);
    if (st != NF_OK) return st;
    L->xcc_of_bit = cm.xcc;
  }
  StreamPair p;
  std::vector<uint32_t> m;
  if (g == 0) {
    HIP_TRY(hipStreamCreateWithFlags(&p.g, hipStreamNonBlocking));
  } else {
    make_mask(L->xcc_of_bit, L->n_xcd, 0, g, m);
    HIP_TRY(hipExtStreamCreateWithCUMask(&p.g, (uint32_t)m.size(), m.data()));
  }
  nf_status st = [&]() -> nf_status {
    if (ab == 0) {
      HIP_TRY(hipStreamCreateWithFlags(&p.a, hipStreamNonBlocking));
    } else {
      make_mask(L->xcc_of_bit, L->n_xcd, L->cus_per_xcd - ab, L->cus_per_xcd, m);
      HIP_TRY(hipExtStreamCreateWithCUMask(&p.a, (uint32_t)m.size(), m.data()));
    }
    return NF_OK;
  }();
  if (st != NF_OK) {            // the first stream is not kept: destroy it
    (void)hipStreamDestroy(p.g);
    return st;
  }
  if (g == 0 && ab == 0) {
    L->pairs[key] = p;
  } else {
    std::lock_guard<std::mutex> lk(g_pairs_mu);
    int on_dev = 0, lru = -1;
    for (int i = 0; i < (int)g_pairs.size(); ++i)
      if (g_pairs[i].dev == L->device) {
        ++on_dev;
        if (g_pairs[i].busy == 0 && (lru < 0 || g_pairs[i].used < g_pairs[lru].used)) lru = i;
      }
    if (on_dev >= kMaskedPairs && lru >= 0) {
      const StreamPair old = g_pairs[lru].p;
      (void)hipStreamSynchronize(old.g);
      (void)hipStreamSynchronize(old.a);
      (void)hipStreamDestroy(old.g);
      (void)hipStreamDestroy(old.a);
      g_pairs.erase(g_pairs.begin() + lru);
    }
    g_pairs.push_back({L->device, g, ab, p, ++g_pairs_clock, hold ? 1 : 0});
  }
  out = p;
  return NF_OK;
}

void release_pair(int dev, hipStream_t g) {
  std::lock_guard<std::mutex> lk(g_pairs_mu);
  for (MaskedPair& e : g_pairs)
    if (e.dev == dev && e.p.g == g && e.busy > 0) {
      --e.busy;
      return;
    }
}

// --------------------------------------------------------------- profiling
struct Prof {
  nf_layer* L;
  int kind;
  hipStream_t s;
};

void prof_begin(nf_layer* L, int kind, hipStream_t s) {
  if (!L->prof || (L->prof_only >= 0 && kind != L->prof_only)) return;
  ProfRec r{kind, nullptr, nullptr};
  for (hipEvent_t* e : {&r.a, &r.b}) {
    if (!L->ev_free.empty()) {
      *e = L->ev_free.back();
      L->ev_free.pop_back();
    } else if (hipEventCreate(e) != hipSuccess) {
      *e = nullptr;
    }
  }
  if (r.a && r.b) {
    // the next launch on this thread records its own start and end
    kernel_timer() = KernelTimer{r.a, r.b};
    L->recs.push_back(r);
  }
  (void)s;
}

void prof_end(nf_layer* L, int kind, hipStream_t s) {
  (void)s;
  if (!L->prof || L->recs.empty() || L->recs.back().kind != kind) return;
  KernelTimer& t = kernel_timer();
  if (t.start) {          // nothing was launched for this kind: drop the record
    L->ev_free.push_back(L->recs.back().a);
    L->ev_free.push_back(L->recs.back().b);
    L->recs.pop_back();
    t = KernelTimer{};
  }
}

void prof_hook_fn(void* ctx, int phase) {
  Prof* p = (Prof*)ctx;
  (void)phase;
  prof_end(p->L, p->kind, p->s);
  prof_begin(p->L, p->kind + 1, p->s);     // the reduce kind follows its GEMM kind
  p->kind += 1;
}

// --------------------------------------------------------------- step pieces
struct StepCtx {
  nf_layer* L;
  nf_kv_pool* P;
  const nf_batch* b;
  // device metadata
  const int32_t *tok_req, *pos, *indptr, *indices;
  const AttnItem* items;
  const MergeItem* merges;
  int gemm_cus, attn_cus;
  // lanes order: nano-batch j runs on lane j % 2, whose GEMMs choose tiles
  // for lane_cus[j % 2] CUs and keep their split-K partials apart
  bool lanes;
  int lane;                // lane of the nano-batch being issued
  int lane_cus[2];
  int attn_waves_per_cu;
  int attn_variant;        // 0: one-wave work items (any grid), 1: four-wave workgroups
  // the step's metadata copy rides on the first front's RMSNorm; the event
  // marks the end of its reads from the pinned staging buffer
  MetaCopy mc;
  bool mc_pending;
  hipEvent_t mc_event;
};

char* ptr(const DevBuf& b, int64_t elems, int dt) { return (char*)b.p + elems * (int64_t)dtype_bytes(dt); }

// CUs the GEMMs of the nano-batch being issued choose their tiles for, and
// the split-K workspace they write
int gemm_cus_of(const StepCtx& c) { return c.lanes ? c.lane_cus[c.lane] : c.gemm_cus; }
// GEMM tiles that fit beside a bounded attention grid on the same CUs (not
// for lanes: there the other lane's attention takes the CUs a GEMM leaves)
bool coresident(const StepCtx& c) { return c.attn_waves_per_cu > 0 && !c.lanes; }
DevBuf& splitk_of(const StepCtx& c) { return c.lanes && c.lane ? c.L->splitk_lane1 : c.L->splitk; }

// `partials` != nullptr: when the GEMM splits K, its reduce is left to the
// consumer, and *partials receives the slice count (1: C was written).
hipError_t run_gemm(StepCtx& c, GemmArgs& g, int kind, hipStream_t s, int* partials = nullptr) {
  nf_layer* L = c.L;
  if (partials) *partials = 1;
  if (L->s.dtype == NF_F32) {
    prof_begin(L, kind, s);
    hipError_t e = gemm_f32(g, s);
    prof_end(L, kind, s);
    return e;
  }
  GemmPlan gp = gemm_choose(g, gemm_cus_of(c), coresident(c));
  if (partials) {
    *partials = gemm_partials(g, gp);
    g.defer_reduce = *partials > 1;
  }
  Prof pctx{L, kind, s};
  LaunchHook hook{prof_hook_fn, &pctx};
  prof_begin(L, kind, s);
  hipError_t e = gemm_bf16(g, gp, splitk_of(c).p, s, L->prof ? &hook : nullptr);
  prof_end(L, pctx.kind, s);
  return e;
}

size_t gemm_ws_need(const StepCtx& c, GemmArgs g) {
  if (c.L->s.dtype == NF_F32) return 0;
  return gemm_workspace_bytes(g, gemm_choose(g, gemm_cus_of(c), coresident(c)));
}

// GEMM descriptors of nano-batch [t0, t1)
struct NanoGemms {
  GemmArgs qkv, o, gu, down, moe_gu, moe_down;
};

NanoGemms nano_gemms(const StepCtx& c, int j, int t0, int t1) {
  nf_layer* L = c.L;
  const nf_shape& s = L->s;
  const int dt = s.dtype;
  const int H = s.hidden, F = s.ffn, nqd = s.n_q_heads * s.head_dim;
  const int Nqkv = (s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim;
  const int Tj = t1 - t0, k = s.top_k;
  NanoGemms n;
  GemmArgs& q = n.qkv;
  if (L->fold_norm1) {
    q.A = (const char*)c.b->x + (int64_t)t0 * H * dtype_bytes(dt);
    q.B = L->w_qkv_g.p;
  } else {
    q.A = ptr(L->h, (int64_t)t0 * H, dt);
    q.B = L->w.w_qkv;
  }
  q.lda = H; q.ldb = H; q.Bp = L->wp_qkv.p;
  q.C = ptr(L->qkv, (int64_t)t0 * Nqkv, dt); q.ldc = Nqkv;
  q.M = Tj; q.N = Nqkv; q.K = H; q.mode = GEMM_STORE;
  GemmArgs& o = n.o;
  o.A = ptr(L->attn, (int64_t)t0 * nqd, dt); o.lda = nqd;
  o.B = L->w.w_o; o.ldb = nqd; o.Bp = L->wp_o.p;
  o.C = ptr(L->x1, (int64_t)t0 * H, dt); o.ldc = H;
  o.R = (const char*)c.b->x + (int64_t)t0 * H * dtype_bytes(dt); o.ldr = H;
  o.M = Tj; o.N = H; o.K = nqd; o.mode = GEMM_RESIDUAL;
  if (s.n_experts == 1) {
    GemmArgs& g = n.gu;
    g.A = ptr(L->h2, (int64_t)t0 * H, dt); g.lda = H;
    g.B = L->w.w_gate; g.B2 = L->w.w_up; g.ldb = H; g.Bp = L->wp_gu.p;
    g.C = ptr(L->act, (int64_t)t0 * F, dt); g.ldc = F;
    g.M = Tj; g.N = F; g.K = H; g.mode = GEMM_SWIGLU;
    GemmArgs& d = n.down;
    d.A = ptr(L->act, (int64_t)t0 * F, dt); d.lda = F;
    d.B = L->w.w_down; d.ldb = F; d.Bp = L->wp_down.p;
    d.C = L->ar_mode ? ptr(L->ypre, (int64_t)t0 * H, dt) : (char*)c.b->out + (int64_t)t0 * H * dtype_bytes(dt);
    d.ldc = H;
    d.R = ptr(L->ar_mode ? L->x1r : L->x1, (int64_t)t0 * H, dt); d.ldr = H;
    d.M = Tj; d.N = H; d.K = F; d.mode = GEMM_RESIDUAL;
  } else {
    const int32_t* off = (const int32_t*)L->r_off.p + j * (s.n_experts + 1);
    GemmArgs& g = n.moe_gu;
    g.A = ptr(L->h2, (int64_t)t0 * H, dt); g.lda = H;
    g.a_rows = (const int32_t*)L->r_perm.p + (int64_t)t0 * k; g.a_row_div = k;
    g.group_off = off; g.n_groups = s.n_experts; g.max_group_rows = Tj * k;
    g.B = L->w.w_gate; g.B2 = L->w.w_up; g.ldb = H; g.b_group_stride = (int64_t)F * H;
    g.Bp = L->wp_gu.p; g.bp_group_stride = 2 * (int64_t)F * H;
    g.C = ptr(L->act, (int64_t)t0 * k * F, dt); g.ldc = F;
    g.M = Tj * k; g.N = F; g.K = H; g.mode = GEMM_SWIGLU;
    GemmArgs& d = n.moe_down;
    d.A = ptr(L->act, (int64_t)t0 * k * F, dt); d.lda = F;
    d.group_off = off; d.n_groups = s.n_experts; d.max_group_rows = Tj * k;
    d.B = L->w.w_down; d.ldb = F; d.b_group_stride = (int64_t)H * F;
    d.Bp = L->wp_down.p; d.bp_group_stride = (int64_t)H * F;
    d.C = (float*)L->y.p + (int64_t)t0 * k * H; d.ldc = H;
    d.M = Tj * k; d.N = H; d.K = F; d.mode = GEMM_F32OUT;
  }
  return n;
}

#define HIP_STEP(expr)                                                                      \
  do {                                                                                      \
    if (fault_now()) return set_err(NF_ERR_HIP, "%s not made: injected failure (NF_FAULT)", #expr); \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess)                                                                   \
      return set_err(NF_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));           \
  } while (0)

nf_status issue_front(StepCtx& c, int j, hipStream_t s) {
  nf_layer* L = c.L;
  const nf_shape& sh = L->s;
  const NanoWork& nw = L->work.nanos[j];
  const int t0 = nw.t0, Tj = nw.t1 - nw.t0, dt = sh.dtype, H = sh.hidden;
  if (Tj == 0) return NF_OK;
  NanoGemms g = nano_gemms(c, j, nw.t0, nw.t1);
  // The step's metadata (first reader: RoPE/append, after the QKV GEMM)
  // crosses PCIe from the pinned staging buffer in extra blocks of a kernel.
  // Above 64 KB (page tables of hundreds of requests: ~12 us at c4) those
  // ride on the QKV GEMM when it takes the LDS-pipelined path, beside its
  // tiles; otherwise on the RMSNorm before it.
  const bool meta_in_gemm = c.mc_pending && dt == NF_BF16 && c.mc.n16 * 16 > (64 << 10) && [&] {
    const int cfg = gemm_choose(g.qkv, gemm_cus_of(c), coresident(c)).cfg;
    return cfg >= 10 && cfg <= 30 && g.qkv.K % 64 == 0;
  }();
  prof_begin(L, K_NORM1, s);
  const char* x = (const char*)c.b->x + (int64_t)t0 * H * dtype_bytes(dt);
  const MetaCopy* mc = c.mc_pending && !meta_in_gemm ? &c.mc : nullptr;
  if (L->fold_norm1)
    HIP_STEP(row_rms_scale(x, (float*)L->rs.p + t0, Tj, H, sh.rms_eps, s, mc));
  else
    HIP_STEP(rmsnorm(dt, x, L->w.attn_norm, ptr(L->h, (int64_t)t0 * H, dt), Tj, H, sh.rms_eps, s, mc));
  prof_end(L, K_NORM1, s);
  if (meta_in_gemm) g.qkv.meta = c.mc;
  int qkv_parts = 1;
  HIP_STEP(run_gemm(c, g.qkv, K_QKV, s, &qkv_parts));
  if (c.mc_pending) {
    HIP_TRY(hipEventRecord(c.mc_event, s));     // the copy's reads of the staging buffer are done
    c.mc_pending = false;
  }
  RopeAppendArgs r;
  const int Nqkv = (sh.n_q_heads + 2 * sh.n_kv_heads) * sh.head_dim;
  if (qkv_parts > 1) {          // RoPE reduces the split-K partials itself
    r.part = (const float*)splitk_of(c).p;
    r.part_ld = Nqkv;
    r.zstride = (int64_t)Tj * Nqkv;
    r.splits = qkv_parts;
  }
  r.qkv = ptr(L->qkv, (int64_t)t0 * Nqkv, dt);
  r.q_rot = ptr(L->q_rot, (int64_t)t0 * sh.n_q_heads * sh.head_dim, dt);
  r.k_pool = c.P->k;
  r.v_pool = c.P->v;
  r.pos = c.pos + t0;
  r.tok_req = c.tok_req + t0;
  r.page_indptr = c.indptr;
  r.page_indices = c.indices;
  r.cos_sin = (const float*)L->cos_sin.p;
  if (L->fold_norm1) r.row_scale = (const float*)L->rs.p + t0;
  r.T = Tj; r.nq = sh.n_q_heads; r.nkv = sh.n_kv_heads; r.d = sh.head_dim; r.page_size = c.P->page_size;
  prof_begin(L, K_ROPE, s);
  HIP_STEP(rope_append(dt, r, s));
  prof_end(L, K_ROPE, s);
  return NF_OK;
}

nf_status issue_attention(StepCtx& c, int j, hipStream_t s) {
  nf_layer* L = c.L;
  const nf_shape& sh = L->s;
  const NanoWork& nw = L->work.nanos[j];
  if (nw.t1 == nw.t0) return NF_OK;
  AttnArgs a;
  a.q_rot = L->q_rot.p;
  a.k_pool = c.P->k;
  a.v_pool = c.P->v;
  a.attn = L->attn.p;
  a.part_o = (float*)L->part_o.p;
  a.part_ml = (float*)L->part_ml.p;
  a.items = c.items + nw.item0;
  a.n_items = nw.n_items;
  a.merges = c.merges + nw.merge0;
  a.n_merges = nw.n_merges;
  a.pos = c.pos;
  a.page_indptr = c.indptr;
  a.page_indices = c.indices;
  a.nq = sh.n_q_heads; a.nkv = sh.n_kv_heads; a.d = sh.head_dim; a.page_size = c.P->page_size;
  a.scale = (float)(1.0 / std::sqrt((double)sh.head_dim));
  a.variant = c.attn_variant;
  a.max_blocks = c.attn_waves_per_cu > 0 ? c.attn_waves_per_cu * c.attn_cus / (c.attn_variant == 1 ? 4 : 1) : 0;
  prof_begin(L, K_ATTN, s);
  HIP_STEP(attention(sh.dtype, a, s));
  prof_end(L, K_ATTN, s);
  if (nw.n_merges) {
    prof_begin(L, K_MERGE, s);
    HIP_STEP(attention_merge(sh.dtype, a, s));
    prof_end(L, K_MERGE, s);
  }
  return NF_OK;
}

// Emulated all-reduce of rows [t0, t0 + Tj) of a [T][H] buffer: a send leg
// (src -> the staging buffer) and a receive leg (staging -> dst) on stream
// sc, on the copy engines (mode 1) or a copy kernel of ar_wgs workgroups
// (mode 2).  On one GPU the tensor-parallel all-reduce is the identity, so
// dst receives src's bits.
nf_status issue_allreduce(nf_layer* L, const void* src, void* dst, int64_t t0, int64_t Tj, hipStream_t sc) {
  const size_t eb = dtype_bytes(L->s.dtype);
  const size_t off = (size_t)t0 * L->s.hidden * eb, bytes = (size_t)Tj * L->s.hidden * eb;
  char* stage = (char*)L->ar_stage.p + off;
  if (L->ar_mode == 1) {
    HIP_TRY(hipMemcpyAsync(stage, (const char*)src + off, bytes, hipMemcpyDeviceToDeviceNoCU, sc));
    HIP_TRY(hipMemcpyAsync((char*)dst + off, stage, bytes, hipMemcpyDeviceToDeviceNoCU, sc));
  } else {
    HIP_TRY(copy_rows((const char*)src + off, stage, bytes, L->ar_wgs, sc));
    HIP_TRY(copy_rows(stage, (char*)dst + off, bytes, L->ar_wgs, sc));
  }
  return NF_OK;
}

// O-projection of nano-batch j on stream s: x1 = x + attn W_o^T and, where
// the split-K reduce fuses with it, h2 = RMSNorm(x1) (*normed = true).  With
// the all-reduce emulation the reduce is not fused: x1 then goes through the
// all-reduce to x1r, which the FFN half reads.
nf_status issue_oproj(StepCtx& c, int j, hipStream_t s, bool* normed) {
  nf_layer* L = c.L;
  const nf_shape& sh = L->s;
  const NanoWork& nw = L->work.nanos[j];
  const int t0 = nw.t0, Tj = nw.t1 - nw.t0, dt = sh.dtype, H = sh.hidden;
  *normed = false;
  if (Tj == 0) return NF_OK;
  NanoGemms g = nano_gemms(c, j, nw.t0, nw.t1);
  const bool fuse = dt == NF_BF16 && H % 8 == 0 && !L->ar_mode;
  int o_parts = 1;
  HIP_STEP(run_gemm(c, g.o, K_OPROJ, s, fuse ? &o_parts : nullptr));
  if (o_parts > 1) {            // O-projection split-K reduce + residual + FFN norm in one kernel
    prof_begin(L, K_NORM2, s);
    HIP_STEP(residual_rmsnorm_partials((const float*)splitk_of(c).p, H, (int64_t)Tj * H, o_parts, g.o.R, g.o.ldr,
                                       g.o.C, g.o.ldc, L->w.ffn_norm, ptr(L->h2, (int64_t)t0 * H, dt), Tj, H,
                                       sh.rms_eps, s));
    prof_end(L, K_NORM2, s);
    *normed = true;
  }
  return NF_OK;
}

// FFN half of nano-batch j on stream s: h2 = RMSNorm(x1) unless the O half
// fused it, then the SwiGLU FFN or the experts, out = x1 + FFN(h2) (with the
// all-reduce emulation: x1r in, ypre out).
nf_status issue_ffn(StepCtx& c, int j, hipStream_t s, bool normed) {
  nf_layer* L = c.L;
  const nf_shape& sh = L->s;
  const NanoWork& nw = L->work.nanos[j];
  const int t0 = nw.t0, Tj = nw.t1 - nw.t0, dt = sh.dtype, H = sh.hidden;
  if (Tj == 0) return NF_OK;
  NanoGemms g = nano_gemms(c, j, nw.t0, nw.t1);
  const DevBuf& x1 = L->ar_mode ? L->x1r : L->x1;
  if (!normed) {
    prof_begin(L, K_NORM2, s);
    HIP_STEP(rmsnorm(dt, ptr(x1, (int64_t)t0 * H, dt), L->w.ffn_norm, ptr(L->h2, (int64_t)t0 * H, dt), Tj, H,
                     sh.rms_eps, s));
    prof_end(L, K_NORM2, s);
  }
  if (sh.n_experts == 1) {
    HIP_STEP(run_gemm(c, g.gu, K_GATEUP, s));
    HIP_STEP(run_gemm(c, g.down, K_DOWN, s));
    return NF_OK;
  }
  const int k = sh.top_k, E = sh.n_experts;
  RouteArgs r;
  r.logits = c.b->router_logits + (int64_t)t0 * E;
  r.idx = (int32_t*)L->r_idx.p + (int64_t)t0 * k;
  r.w = (float*)L->r_w.p + (int64_t)t0 * k;
  r.perm = (int32_t*)L->r_perm.p + (int64_t)t0 * k;
  r.inv = (int32_t*)L->r_inv.p + (int64_t)t0 * k;
  r.offsets = (int32_t*)L->r_off.p + j * (E + 1);
  r.T = Tj; r.E = E; r.k = k;
  prof_begin(L, K_ROUTE, s);
  HIP_STEP(moe_route(r, s));
  prof_end(L, K_ROUTE, s);
  // grouped: the tile choice depends on the mean rows per expert; the
  // streaming kernels may split K (partials in the split-K workspace)
  prof_begin(L, K_MOE_GATEUP, s);
  HIP_STEP(gemm_bf16(g.moe_gu, gemm_choose(g.moe_gu, gemm_cus_of(c)), splitk_of(c).p, s));
  prof_end(L, K_MOE_GATEUP, s);
  prof_begin(L, K_MOE_DOWN, s);
  HIP_STEP(gemm_bf16(g.moe_down, gemm_choose(g.moe_down, gemm_cus_of(c)), splitk_of(c).p, s));
  prof_end(L, K_MOE_DOWN, s);
  void* dst = L->ar_mode ? (void*)ptr(L->ypre, (int64_t)t0 * H, dt)
                         : (void*)((char*)c.b->out + (int64_t)t0 * H * dtype_bytes(dt));
  prof_begin(L, K_COMBINE, s);
  HIP_STEP(moe_combine(dt, ptr(x1, (int64_t)t0 * H, dt), (const float*)L->y.p + (int64_t)t0 * k * H, r.w, r.inv,
                       dst, Tj, H, k, s));
  prof_end(L, K_COMBINE, s);
  return NF_OK;
}

size_t align_words(size_t w) { return (w + 63) & ~(size_t)63; }

// Copies of the expert weights in MFMA operand order for the weight-streaming
// expert GEMMs (made once; the caller's weights must not change after
// nf_layer_create).  Dense layers keep only the caller's copy: their GEMMs use
// the LDS-tiled kernels, which measured faster there.  Expert matrices whose
// output features are not a multiple of 32 or whose K is not a multiple of 16
// get no copy either.
hipError_t pack_weights(nf_layer* L) {
  const nf_shape& s = L->s;
  const int64_t H = s.hidden, F = s.ffn, E = s.n_experts;
  hipError_t e;
  if (E == 1 || F % 32 || H % 32) return hipSuccess;
  if ((e = ensure(L->wp_gu, E * 2 * F * H * 2)) != hipSuccess) return e;
  if ((e = pack_b(L->w.w_gate, H, F * H, (int)F, (int)H, (int)E, L->wp_gu.p, 2, 0, 2 * F * H, nullptr)) != hipSuccess)
    return e;
  if ((e = pack_b(L->w.w_up, H, F * H, (int)F, (int)H, (int)E, L->wp_gu.p, 2, 1, 2 * F * H, nullptr)) != hipSuccess)
    return e;
  if ((e = ensure(L->wp_down, E * H * F * 2)) != hipSuccess) return e;
  if ((e = pack_b(L->w.w_down, F, H * F, (int)H, (int)F, (int)E, L->wp_down.p, 1, 0, H * F, nullptr)) != hipSuccess)
    return e;
  return hipDeviceSynchronize();
}

// One layer's step as prepared for launch: its batch (the caller's, with this
// layer's input and output rows), its context and nano-batch count.
struct LayerRun {
  nf_layer* L = nullptr;
  nf_batch b{};
  StepCtx c{};
  int count = 0;
  bool normed[NF_MAX_NANO] = {};   // the O half of nano-batch j also wrote h2
};

// Everything of one layer's step before its launches: the checks, the
// attention work items, the workspace and the metadata image.  With
// fixed_meta == nullptr the metadata goes through the layer's pinned staging
// buffer and the first front's RMSNorm copies it on the device; otherwise it
// is copied now, synchronously, into *fixed_meta (a buffer the caller owns,
// grown here), so that launches captured in a graph read it there.
nf_status prepare_layer(nf_layer* L, nf_kv_pool* P, const nf_batch* b, const nf_plan& plan, DevBuf* fixed_meta,
                        LayerRun& r) {
  std::string err;
  nf_status st = check_batch(L->s, P->n_pages, P->page_size, *b, err);
  if (st != NF_OK) return set_err(st, "%s", err.c_str());
  st = check_plan_batch(plan, b->n_tokens, err);
  if (st != NF_OK) return set_err(st, "%s", err.c_str());
  const int T = b->n_tokens, R = b->n_requests;
  L->last_T = T;
  r.L = L;
  r.b = *b;
  r.count = 0;
  if (T == 0) return NF_OK;
  HIP_TRY(hipSetDevice(L->device));

  const bool two = plan.n_streams == 2;
  const int gsplit = two ? plan.gemm_cus_per_xcd : 0;
  const int asplit = two ? attn_budget(plan.gemm_cus_per_xcd, plan.attn_cus_per_xcd, L->cus_per_xcd) : 0;
  StepCtx& c = r.c;
  c = StepCtx{};
  c.L = L;
  c.P = P;
  c.b = &r.b;
  c.gemm_cus = gsplit ? gsplit * L->n_xcd : L->n_cus;
  c.attn_cus = asplit ? asplit * L->n_xcd : L->n_cus;
  c.lanes = two && plan.order == NF_ORDER_LANES;
  c.lane = 0;
  c.lane_cus[0] = gsplit ? c.gemm_cus : std::max(1, L->n_cus / 2);
  c.lane_cus[1] = asplit ? c.attn_cus : std::max(1, L->n_cus / 2);
  c.attn_waves_per_cu = two ? plan.attn_waves_per_cu : 0;
  // attention work items: a four-wave workgroup each (fastest when attention
  // has the whole chip), or one wave each (many short items) when the plan
  // asks for a persistent attention grid that leaves room for GEMM waves
  // bounded residency: multiples of four waves per CU run as persistent
  // four-wave workgroups, other counts as persistent single waves
  c.attn_variant = L->attn_variant >= 0 ? L->attn_variant : (c.attn_waves_per_cu % 4 == 0 ? 1 : 0);
  const bool wave_items = L->s.dtype == NF_BF16 && L->s.head_dim == 128 && c.attn_variant == 0;
  build_work(L->s, *b, plan, P->page_size, wave_items ? 8 * c.attn_cus : 2 * c.attn_cus, 8,
             wave_items ? 32 : 0, L->work);
  const StepWork& w = L->work;
  r.count = (int)w.nanos.size();

  // workspace the GEMMs and the split attention items need (before any launch)
  size_t ws[2] = {0, 0};
  for (int j = 0; j < r.count; ++j) {
    c.lane = c.lanes ? j % 2 : 0;
    NanoGemms g = nano_gemms(c, j, w.nanos[j].t0, w.nanos[j].t1);
    size_t& need = ws[c.lane];
    if (L->s.n_experts == 1)
      for (const GemmArgs* a : {&g.qkv, &g.o, &g.gu, &g.down}) need = std::max(need, gemm_ws_need(c, *a));
    else
      for (const GemmArgs* a : {&g.qkv, &g.o, &g.moe_gu, &g.moe_down}) need = std::max(need, gemm_ws_need(c, *a));
  }
  c.lane = 0;
  HIP_TRY(ensure(L->splitk, ws[0]));
  if (ws[1]) HIP_TRY(ensure(L->splitk_lane1, ws[1]));
  const size_t n_part = (size_t)std::max(1, w.n_partials) * L->s.n_kv_heads * 16;
  HIP_TRY(ensure(L->part_o, n_part * L->s.head_dim * sizeof(float)));
  HIP_TRY(ensure(L->part_ml, n_part * 2 * sizeof(float)));

  // metadata: tok_req | pos | indptr | indices | items | merges (int32 words)
  const int64_t nnz = b->page_indptr[R];
  const size_t o_tok = 0, o_pos = align_words(T), o_ip = o_pos + align_words(T), o_ix = o_ip + align_words(R + 1),
               o_it = o_ix + align_words(nnz), o_mg = o_it + align_words(w.items.size() * 8),
               words = o_mg + align_words(w.merges.size() * 4);
  const size_t bytes = words * 4;
  auto fill = [&](int32_t* hs) {
    std::memcpy(hs + o_tok, w.tok_req.data(), (size_t)T * 4);
    std::memcpy(hs + o_pos, b->pos, (size_t)T * 4);
    std::memcpy(hs + o_ip, b->page_indptr, (size_t)(R + 1) * 4);
    std::memcpy(hs + o_ix, b->page_indices, (size_t)nnz * 4);
    if (!w.items.empty()) std::memcpy(hs + o_it, w.items.data(), w.items.size() * sizeof(AttnItem));
    if (!w.merges.empty()) std::memcpy(hs + o_mg, w.merges.data(), w.merges.size() * sizeof(MergeItem));
  };
  const int32_t* dm = nullptr;
  if (fixed_meta) {
    HIP_TRY(ensure(*fixed_meta, bytes));
    std::vector<int32_t> img(words, 0);
    fill(img.data());
    HIP_TRY(hipMemcpy(fixed_meta->p, img.data(), bytes, hipMemcpyHostToDevice));
    c.mc_pending = false;
    dm = (const int32_t*)fixed_meta->p;
  } else {
    const int si = L->stage_i;
    L->stage_i ^= 1;
    if (L->stage_used[si]) HIP_TRY(hipEventSynchronize(L->stage_ev[si]));  // previous copy from it done
    if (L->stage_bytes[si] < bytes) {
      if (L->stage[si]) HIP_TRY(hipHostFree(L->stage[si]));
      L->stage[si] = nullptr;
      L->stage_bytes[si] = 0;
      HIP_TRY(hipHostMalloc(&L->stage[si], bytes * 2, hipHostMallocMapped | hipHostMallocCoherent));
      HIP_TRY(hipHostGetDevicePointer(&L->stage_dev[si], L->stage[si], 0));
      L->stage_bytes[si] = bytes * 2;
    }
    if (L->meta.bytes < bytes) HIP_TRY(ensure(L->meta, bytes * 2));
    fill((int32_t*)L->stage[si]);
    // copied on the device by extra blocks of the first front's RMSNorm, which
    // precedes every reader of the metadata on its stream
    c.mc.src = L->stage_dev[si];
    c.mc.dst = L->meta.p;
    c.mc.n16 = (int64_t)(bytes / 16);
    c.mc_pending = true;
    c.mc_event = L->stage_ev[si];
    L->stage_used[si] = true;
    dm = (const int32_t*)L->meta.p;
  }
  c.tok_req = dm + o_tok;
  c.pos = dm + o_pos;
  c.indptr = dm + o_ip;
  c.indices = dm + o_ix;
  c.items = (const AttnItem*)(dm + o_it);
  c.merges = (const MergeItem*)(dm + o_mg);
  return NF_OK;
}

// Streams of a step (or of every layer of a multi-layer step): the GEMM side
// runs on the caller's stream unless it is CU-masked; attention runs on the
// pair's attention stream.  Cross-stream waits cost ~20 us each on this
// runtime, so only the necessary ones are issued: attention(j) waits for
// RoPE/append(j), the O-projection of j waits for attention(j).  The last of
// those also orders every attention kernel before the end of the step on the
// GEMM stream.  With the all-reduce emulation a third stream carries the
// collectives: the all-reduce of nano-batch j's O-projection waits for that
// GEMM and its FFN half waits for the all-reduce; the caller's stream waits
// for the last collective.
struct Streams {
  bool two = false, comm = false;
  bool lanes = false;            // nano-batch j on lane j % 2 (sg, sa)
  hipStream_t caller = nullptr, sg = nullptr, sa = nullptr, sc = nullptr;
  hipStream_t sc2 = nullptr;     // lane 1's collectives (sc unless lanes)
  int held_dev = -1;             // a held masked pair (released here)
  hipStream_t held = nullptr;
  Streams() = default;
  Streams(const Streams&) = delete;
  Streams& operator=(const Streams&) = delete;
  ~Streams() {
    if (held) release_pair(held_dev, held);
  }
};

nf_status open_streams(nf_layer* L, const nf_plan& plan, hipStream_t caller, Streams& S) {
  S.two = plan.n_streams == 2;
  S.lanes = S.two && plan.order == NF_ORDER_LANES;
  S.caller = S.sg = S.sa = caller;
  S.comm = L->ar_mode != 0;
  if (S.comm) {
    if (!L->sc) HIP_TRY(hipStreamCreateWithFlags(&L->sc, hipStreamNonBlocking));
    S.sc = S.sc2 = L->sc;
    // with lanes each lane's collectives go on a stream of their own: on one
    // stream, in issue order, lane 1's would queue behind all of lane 0's
    if (S.lanes) {
      if (!L->sc2) HIP_TRY(hipStreamCreateWithFlags(&L->sc2, hipStreamNonBlocking));
      if (!L->ev_a2) HIP_TRY(hipEventCreateWithFlags(&L->ev_a2, hipEventDisableTiming));
      S.sc2 = L->sc2;
    }
  }
  if (!S.two) return NF_OK;
  StreamPair pr;
  const bool masked = plan.gemm_cus_per_xcd || plan.attn_cus_per_xcd;
  nf_status st = get_pair(L, plan.gemm_cus_per_xcd, plan.attn_cus_per_xcd, pr, masked);
  if (st != NF_OK) return st;
  if (masked) {
    S.held_dev = L->device;
    S.held = pr.g;
  }
  S.sa = pr.a;
  // CU-masked streams are blocking streams, which the null stream
  // synchronises with implicitly: GEMM work left on a null caller stream
  // would wait for the attention stream's earlier launches and hold back its
  // later ones, serialising the two sides.  The GEMM side then runs on the
  // pair's own (non-blocking, or masked) stream, as under a GEMM budget.
  if (plan.gemm_cus_per_xcd || caller == nullptr) {
    S.sg = pr.g;
    HIP_TRY(hipEventRecord(L->ev_start, caller));
    HIP_TRY(hipStreamWaitEvent(S.sg, L->ev_start, 0));
  }
  return NF_OK;
}

// After a failure partway through enqueuing a step: wait for what was
// enqueued (each launch went out with its dependencies in place), so that no
// kernel of the failed step still reads the metadata staging or the
// workspace when the caller goes on.  Errors here are ignored: the step's own
// error is the one reported.
void drain_after_error(const Streams& S) {
  const hipStream_t all[5] = {S.caller, S.sg, S.sa, S.sc, S.sc2};
  for (int i = 0; i < 5; ++i) {
    bool seen = false;
    for (int k = 0; k < i; ++k) seen = seen || all[k] == all[i];
    if (!seen && (i == 0 || all[i])) (void)hipStreamSynchronize(all[i]);
  }
  (void)hipGetLastError();
}

nf_status close_streams(nf_layer* L, const Streams& S) {
  if (S.lanes) {                 // lane 1 joins the caller (lane 0 below)
    HIP_TRY(hipEventRecord(L->ev_lane, S.sa));
    HIP_TRY(hipStreamWaitEvent(S.caller, L->ev_lane, 0));
  }
  if (S.two && S.sg != S.caller) {
    HIP_TRY(hipEventRecord(L->ev_g, S.sg));
    HIP_TRY(hipStreamWaitEvent(S.caller, L->ev_g, 0));
  }
  if (S.comm) {
    HIP_TRY(hipEventRecord(L->ev_a, S.sc));
    HIP_TRY(hipStreamWaitEvent(S.caller, L->ev_a, 0));
    if (S.sc2 != S.sc) {
      HIP_TRY(hipEventRecord(L->ev_a2, S.sc2));
      HIP_TRY(hipStreamWaitEvent(S.caller, L->ev_a2, 0));
    }
  }
  return NF_OK;
}

// The stream of nano-batch j's collectives
hipStream_t comm_stream(const Streams& S, int j) { return S.lanes && j % 2 ? S.sc2 : S.sc; }

// The stream the GEMM side of nano-batch j goes to, and that of its
// attention; with lanes both are lane j % 2 and the context is set to it.
hipStream_t gemm_stream(LayerRun& r, const Streams& S, int j) {
  r.c.lane = S.lanes ? j % 2 : 0;
  return S.lanes && j % 2 ? S.sa : S.sg;
}

// front (norm, QKV, RoPE/append) of nano-batch j and its attention
nf_status issue_front_attn(LayerRun& r, const Streams& S, int j) {
  nf_layer* L = r.L;
  if (S.lanes) {                 // the whole nano-batch on its lane
    const hipStream_t s = gemm_stream(r, S, j);
    // lane 1 starts after nano-batch 0's front, whose RMSNorm also carries
    // the step's metadata copy that every lane reads
    if (j == 1) HIP_TRY(hipStreamWaitEvent(s, L->ev_app[0], 0));
    nf_status st = issue_front(r.c, j, s);
    if (st != NF_OK) return st;
    if (j + 1 < r.count) HIP_TRY(hipEventRecord(L->ev_app[j], s));
    // A request whose tokens began in an earlier nano-batch (a prefill chunk
    // cut by the plan) attends to keys that the fronts before j appended; the
    // last of them ran on the other lane (earlier ones on either lane are
    // ordered before it or before this launch)
    const NanoWork& nw = L->work.nanos[j];
    if (j >= 2 && nw.t1 > nw.t0 && r.b.req_q_start[L->work.tok_req[nw.t0]] < nw.t0)
      HIP_TRY(hipStreamWaitEvent(s, L->ev_app[j - 1], 0));
    return issue_attention(r.c, j, s);
  }
  nf_status st = issue_front(r.c, j, S.sg);
  if (st != NF_OK) return st;
  if (S.two) {
    HIP_TRY(hipEventRecord(L->ev_app[j], S.sg));
    HIP_TRY(hipStreamWaitEvent(S.sa, L->ev_app[j], 0));
  }
  st = issue_attention(r.c, j, S.sa);
  if (st != NF_OK) return st;
  if (S.two) HIP_TRY(hipEventRecord(L->ev_att[j], S.sa));
  return NF_OK;
}

// O half of nano-batch j once its attention is done; with the all-reduce
// emulation its x1 rows then go through the collective on the third stream.
nf_status issue_o_after_attn(LayerRun& r, const Streams& S, int j) {
  nf_layer* L = r.L;
  const hipStream_t sg = gemm_stream(r, S, j);
  if (S.two && !S.lanes) HIP_TRY(hipStreamWaitEvent(sg, L->ev_att[j], 0));
  nf_status st = issue_oproj(r.c, j, sg, &r.normed[j]);
  if (st != NF_OK || !L->ar_mode) return st;
  const NanoWork& nw = L->work.nanos[j];
  if (nw.t1 == nw.t0) return NF_OK;
  const hipStream_t sc = comm_stream(S, j);
  HIP_TRY(hipEventRecord(L->ev_o[j], sg));
  HIP_TRY(hipStreamWaitEvent(sc, L->ev_o[j], 0));
  if ((st = issue_allreduce(L, L->x1.p, L->x1r.p, nw.t0, nw.t1 - nw.t0, sc)) != NF_OK) return st;
  HIP_TRY(hipEventRecord(L->ev_co[j], sc));
  return NF_OK;
}

// FFN half of nano-batch j (after its O half on the same stream); with the
// all-reduce emulation it first waits for the O-projection's collective and
// its output rows go through the collective into the batch's out.
nf_status issue_ffn_after_o(LayerRun& r, const Streams& S, int j) {
  nf_layer* L = r.L;
  const NanoWork& nw = L->work.nanos[j];
  const bool live = nw.t1 > nw.t0;
  const hipStream_t sg = gemm_stream(r, S, j);
  if (L->ar_mode && live) HIP_TRY(hipStreamWaitEvent(sg, L->ev_co[j], 0));
  nf_status st = issue_ffn(r.c, j, sg, r.normed[j]);
  if (st != NF_OK || !L->ar_mode || !live) return st;
  const hipStream_t sc = comm_stream(S, j);
  HIP_TRY(hipEventRecord(L->ev_d[j], sg));
  HIP_TRY(hipStreamWaitEvent(sc, L->ev_d[j], 0));
  if ((st = issue_allreduce(L, L->ypre.p, r.c.b->out, nw.t0, nw.t1 - nw.t0, sc)) != NF_OK) return st;
  HIP_TRY(hipEventRecord(L->ev_cd[j], sc));
  return NF_OK;
}

// back (O-projection, norm, FFN or experts) of nano-batch j
nf_status issue_back_after_attn(LayerRun& r, const Streams& S, int j) {
  nf_status st = issue_o_after_attn(r, S, j);
  if (st != NF_OK) return st;
  return issue_ffn_after_o(r, S, j);
}

// one layer's launches in the plan's order
nf_status issue_layer(LayerRun& r, const Streams& S, int order) {
  nf_status st;
  if (S.lanes) {
    // in nano-batch order, each on its lane: every event a launch waits for
    // (the front of the nano-batch before it) is recorded before the wait
    for (int j = 0; j < r.count; ++j) {
      if ((st = issue_front_attn(r, S, j)) != NF_OK) return st;
      if ((st = issue_back_after_attn(r, S, j)) != NF_OK) return st;
    }
    return NF_OK;
  }
  if (order == NF_ORDER_PIPELINED) {
    if ((st = issue_front_attn(r, S, 0)) != NF_OK) return st;
    for (int j = 0; j < r.count; ++j) {
      if (j + 1 < r.count && (st = issue_front_attn(r, S, j + 1)) != NF_OK) return st;
      if ((st = issue_back_after_attn(r, S, j)) != NF_OK) return st;
    }
  } else if (order == NF_ORDER_DEEP) {
    // round t: front of t, O half of t - 1, FFN half of t - 2
    for (int t = 0; t < r.count + 2; ++t) {
      if (t < r.count && (st = issue_front_attn(r, S, t)) != NF_OK) return st;
      if (t >= 1 && t - 1 < r.count && (st = issue_o_after_attn(r, S, t - 1)) != NF_OK) return st;
      if (t >= 2 && (st = issue_ffn_after_o(r, S, t - 2)) != NF_OK) return st;
    }
  } else {
    for (int j = 0; j < r.count; ++j) {
      if ((st = issue_front_attn(r, S, j)) != NF_OK) return st;
      if ((st = issue_back_after_attn(r, S, j)) != NF_OK) return st;
    }
  }
  return NF_OK;
}

// The launches of a prepared multi-layer step.  With two streams, several
// nano-batches and the pipelined order, nano-batches are pipelined across
// layers: nano-batch j's front of layer l + 1 is issued right after its back
// of layer l, before nano-batch j + 1's back of layer l, so j's next
// attention overlaps j + 1's remaining GEMMs and no layer boundary drains the
// pipeline.  Otherwise the layers run one after another in the plan's order.
nf_status issue_stack(std::vector<LayerRun>& runs, const Streams& S, int order) {
  nf_status st;
  const int n = (int)runs.size(), count = runs[0].count;
  if (!S.two || count < 2 || order != NF_ORDER_PIPELINED) {
    for (LayerRun& r : runs)
      if ((st = issue_layer(r, S, order)) != NF_OK) return st;
    return NF_OK;
  }
  if ((st = issue_front_attn(runs[0], S, 0)) != NF_OK) return st;
  for (int l = 0; l < n; ++l)
    for (int j = 0; j < count; ++j) {
      if (l == 0 && j + 1 < count && (st = issue_front_attn(runs[0], S, j + 1)) != NF_OK) return st;
      if ((st = issue_back_after_attn(runs[l], S, j)) != NF_OK) return st;
      if (l + 1 < n && (st = issue_front_attn(runs[l + 1], S, j)) != NF_OK) return st;
    }
  return NF_OK;
}

nf_status step_impl(nf_layer* L, nf_kv_pool* P, const nf_batch* b, hipStream_t caller, const nf_plan& plan) {
  LayerRun r;
  nf_status st = prepare_layer(L, P, b, plan, nullptr, r);
  if (st != NF_OK || r.count == 0) return st;
  Streams S;
  if ((st = open_streams(L, plan, caller, S)) == NF_OK && (st = issue_layer(r, S, plan.order)) == NF_OK &&
      (st = close_streams(L, S)) == NF_OK)
    return NF_OK;
  drain_after_error(S);
  return st;
}

// Checks of a multi-layer step's arguments (no HIP call).
nf_status check_stack(nf_layer* const* layers, nf_kv_pool* const* pools, int n, const nf_batch* b) {
  if (!layers || !pools || !b) return set_err(NF_ERR_INVALID_ARG, "stack: null argument");
  if (n < 1) return set_err(NF_ERR_INVALID_ARG, "stack: n_layers %d must be positive", n);
  for (int l = 0; l < n; ++l) {
    if (!layers[l] || !pools[l]) return set_err(NF_ERR_INVALID_ARG, "stack: layer or pool %d is null", l);
    if (pools[l]->layer != layers[l]) return set_err(NF_ERR_INVALID_ARG, "stack: pool %d belongs to another layer", l);
    for (int m = 0; m < l; ++m)
      if (layers[m] == layers[l]) return set_err(NF_ERR_INVALID_ARG, "stack: layer %d appears twice", l);
    const nf_shape &s0 = layers[0]->s, &sl = layers[l]->s;
    if (sl.hidden != s0.hidden || sl.dtype != s0.dtype || sl.max_tokens != s0.max_tokens ||
        sl.n_experts != s0.n_experts || layers[l]->device != layers[0]->device ||
        layers[l]->ar_mode != layers[0]->ar_mode)
      return set_err(NF_ERR_INVALID_ARG, "stack: layer %d differs from layer 0 in hidden size, dtype, "
                     "max_tokens, experts, device or all-reduce emulation", l);
  }
  return NF_OK;
}

// Prepares every layer of a multi-layer step (layer 0's plan for all); layer
// l writes its own stack_out buffer, which layer l + 1 reads.
nf_status prepare_stack(nf_layer* const* layers, nf_kv_pool* const* pools, int n, const nf_batch* b,
                        std::vector<DevBuf>* fixed_meta, std::vector<LayerRun>& runs) {
  const nf_plan& plan = layers[0]->plan;
  const nf_shape& s = layers[0]->s;
  runs.assign(n, LayerRun{});
  HIP_TRY(hipSetDevice(layers[0]->device));
  const size_t io = (size_t)std::max(0, b->n_tokens) * s.hidden * dtype_bytes(s.dtype);
  for (int l = 0; l + 1 < n; ++l) HIP_TRY(ensure(layers[l]->stack_out, io));
  for (int l = 0; l < n; ++l) {
    nf_batch bl = *b;
    if (l > 0) bl.x = layers[l - 1]->stack_out.p;
    if (l + 1 < n) bl.out = layers[l]->stack_out.p;
    nf_status st = prepare_layer(layers[l], pools[l], &bl, plan, fixed_meta ? &(*fixed_meta)[l] : nullptr, runs[l]);
    if (st != NF_OK) return st;
  }
  return NF_OK;
}

nf_status stack_impl(nf_layer* const* layers, nf_kv_pool* const* pools, int n, const nf_batch* b,
                     hipStream_t caller) {
  std::vector<LayerRun> runs;
  nf_status st = prepare_stack(layers, pools, n, b, nullptr, runs);
  if (st != NF_OK || runs[0].count == 0) return st;
  Streams S;
  if ((st = open_streams(layers[0], layers[0]->plan, caller, S)) == NF_OK &&
      (st = issue_stack(runs, S, layers[0]->plan.order)) == NF_OK && (st = close_streams(layers[0], S)) == NF_OK)
    return NF_OK;
  drain_after_error(S);
  return st;
}

}  // namespace

// =============================================================== C ABI
extern "C" {

const char* nf_last_error(void) { return g_err.c_str(); }

const char* nf_status_string(nf_status s) {
  switch (s) {
    case NF_OK: return "ok";
    case NF_ERR_INVALID_ARG: return "invalid argument";
    case NF_ERR_OUT_OF_RANGE: return "out of range";
    case NF_ERR_UNSUPPORTED: return "unsupported";
    case NF_ERR_NO_PLAN: return "no plan";
    case NF_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

nf_status nf_kv_pool_bytes(const nf_shape* s, int32_t n_pages, int32_t page_size, size_t* k_bytes,
                           size_t* v_bytes) {
  if (!s || !k_bytes || !v_bytes) return set_err(NF_ERR_INVALID_ARG, "nf_kv_pool_bytes: null argument");
  std::string err;
  nf_status st = check_shape(*s, err);
  if (st != NF_OK) return set_err(st, "%s", err.c_str());
  if (page_size != PAGE_SIZE) return set_err(NF_ERR_UNSUPPORTED, "page_size %d: only 16 is supported", page_size);
  if (n_pages <= 0) return set_err(NF_ERR_INVALID_ARG, "n_pages must be positive");
  const size_t b = (size_t)n_pages * s->n_kv_heads * page_size * s->head_dim * dtype_bytes(s->dtype);
  *k_bytes = b;
  *v_bytes = b;
  return NF_OK;
}

nf_status nf_batch_validate(const nf_shape* s, int32_t n_pages, int32_t page_size, const nf_batch* b,
                            const nf_plan* p) {
  if (!s || !b) return set_err(NF_ERR_INVALID_ARG, "nf_batch_validate: null argument");
  std::string err;
  nf_status st = check_shape(*s, err);
  if (st == NF_OK && page_size != PAGE_SIZE) {
    err = "page_size: only 16 is supported";
    st = NF_ERR_UNSUPPORTED;
  }
  if (st == NF_OK) st = check_batch(*s, n_pages, page_size, *b, err);
  if (st == NF_OK && p) st = check_plan(*p, 32, err);
  if (st == NF_OK && p) st = check_plan_batch(*p, b->n_tokens, err);
  if (st != NF_OK) return set_err(st, "%s", err.c_str());
  return NF_OK;
}

nf_status nf_layer_create(const nf_shape* s, const nf_weights* w, nf_layer** out) {
  if (!s || !w || !out) return set_err(NF_ERR_INVALID_ARG, "nf_layer_create: null argument");
  *out = nullptr;
  std::string err;
  nf_status st = check_shape(*s, err);
  if (st != NF_OK) return set_err(st, "%s", err.c_str());
  if (s->n_experts > 1 && s->dtype != NF_BF16)
    return set_err(NF_ERR_UNSUPPORTED, "mixture-of-experts layers need dtype bf16");
  if (!w->attn_norm || !w->w_qkv || !w->w_o || !w->ffn_norm || !w->w_gate || !w->w_up || !w->w_down)
    return set_err(NF_ERR_INVALID_ARG, "nf_layer_create: a weight pointer is null");
  nf_layer* L = new nf_layer();
  L->s = *s;
  L->w = *w;
  auto fail = [&](nf_status st2) {
    nf_layer_destroy(L);
    return st2;
  };
  if (hipGetDevice(&L->device) != hipSuccess) return fail(set_err(NF_ERR_HIP, "hipGetDevice failed"));
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, L->device) != hipSuccess)
    return fail(set_err(NF_ERR_HIP, "hipGetDeviceProperties failed"));
  L->n_cus = prop.multiProcessorCount;
  L->n_xcd = 8;
  L->cus_per_xcd = std::max(1, L->n_cus / L->n_xcd);
  L->plan = nf_plan{1, {0, 0, 0, 0}, NF_ORDER_PIPELINED, 1, 0, 0, 0};
  if (const char* v = std::getenv("NF_ATTN_VARIANT")) L->attn_variant = std::atoi(v);
  L->fold_norm1 = s->dtype == NF_BF16 && s->hidden % 8 == 0;
  if (const char* v = std::getenv("NF_NORM_FOLD")) L->fold_norm1 = L->fold_norm1 && std::atoi(v) != 0;

  const int dt = s->dtype;
  const size_t eb = dtype_bytes(dt);
  const int64_t Tm = s->max_tokens, H = s->hidden, F = s->ffn, k = s->top_k;
  const int64_t nqd = (int64_t)s->n_q_heads * s->head_dim;
  const int64_t Nqkv = (int64_t)(s->n_q_heads + 2 * s->n_kv_heads) * s->head_dim;
  struct {
    DevBuf* b;
    size_t bytes;
  } allocs[] = {
      {&L->h, L->fold_norm1 ? 0 : Tm * H * eb}, {&L->rs, L->fold_norm1 ? (size_t)Tm * 4 : 0},
      {&L->qkv, Tm * Nqkv * eb},     {&L->q_rot, Tm * nqd * eb},
      {&L->attn, Tm * nqd * eb},     {&L->x1, Tm * H * eb},     {&L->h2, Tm * H * eb},
      {&L->act, Tm * k * F * eb},
  };
  for (auto& a : allocs)
    if (ensure(*a.b, a.bytes) != hipSuccess) return fail(set_err(NF_ERR_HIP, "workspace allocation failed"));
  if (s->n_experts > 1) {
    if (ensure(L->y, Tm * k * H * 4) != hipSuccess || ensure(L->r_idx, Tm * k * 4) != hipSuccess ||
        ensure(L->r_w, Tm * k * 4) != hipSuccess || ensure(L->r_perm, Tm * k * 4) != hipSuccess ||
        ensure(L->r_inv, Tm * k * 4) != hipSuccess ||
        ensure(L->r_off, (size_t)NF_MAX_NANO * (s->n_experts + 1) * 4) != hipSuccess)
      return fail(set_err(NF_ERR_HIP, "router workspace allocation failed"));
  }
  // fp32 (cos, sin) of p * theta^(-2j/d), angles in fp64
  const int half = s->head_dim / 2;
  std::vector<float> cs((size_t)s->max_pos * half * 2);
  for (int64_t p = 0; p < s->max_pos; ++p)
    for (int j = 0; j < half; ++j) {
      const double ang = (double)p * std::pow(s->rope_theta, -2.0 * j / s->head_dim);
      cs[(p * half + j) * 2] = (float)std::cos(ang);
      cs[(p * half + j) * 2 + 1] = (float)std::sin(ang);
    }
  if (dt == NF_BF16 && pack_weights(L) != hipSuccess)
    return fail(set_err(NF_ERR_HIP, "weight packing failed"));
  if (L->fold_norm1 && (ensure(L->w_qkv_g, Nqkv * H * eb) != hipSuccess ||
                        scale_cols_bf16(L->w.w_qkv, L->w.attn_norm, L->w_qkv_g.p, Nqkv, (int)H, nullptr) != hipSuccess ||
                        hipDeviceSynchronize() != hipSuccess))
    return fail(set_err(NF_ERR_HIP, "gain-scaled QKV weight failed"));
  if (ensure(L->cos_sin, cs.size() * 4) != hipSuccess ||
      hipMemcpy(L->cos_sin.p, cs.data(), cs.size() * 4, hipMemcpyHostToDevice) != hipSuccess)
    return fail(set_err(NF_ERR_HIP, "cos/sin table upload failed"));
  for (int j = 0; j < NF_MAX_NANO; ++j)
    if (hipEventCreateWithFlags(&L->ev_app[j], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&L->ev_att[j], hipEventDisableTiming) != hipSuccess)
      return fail(set_err(NF_ERR_HIP, "event creation failed"));
  if (hipEventCreateWithFlags(&L->ev_start, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&L->ev_g, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&L->ev_a, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&L->ev_lane, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&L->stage_ev[0], hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&L->stage_ev[1], hipEventDisableTiming) != hipSuccess)
    return fail(set_err(NF_ERR_HIP, "event creation failed"));
  *out = L;
  return NF_OK;
}

void nf_layer_destroy(nf_layer* L) {
  if (!L) return;
  (void)hipSetDevice(L->device);
  (void)hipDeviceSynchronize();
  for (auto& kv : L->pairs) {
    if (kv.second.g) (void)hipStreamDestroy(kv.second.g);
    if (kv.second.a) (void)hipStreamDestroy(kv.second.a);
  }
  for (DevBuf* b : {&L->h, &L->qkv, &L->q_rot, &L->attn, &L->x1, &L->h2, &L->act, &L->y, &L->r_idx, &L->r_w,
                    &L->r_perm, &L->r_inv, &L->r_off, &L->splitk, &L->splitk_lane1, &L->part_o, &L->part_ml, &L->meta, &L->cos_sin,
                    &L->wp_qkv, &L->wp_o, &L->wp_gu, &L->wp_down, &L->w_qkv_g, &L->rs, &L->stack_out})
    release(*b);
  for (int i = 0; i < 2; ++i) {
    if (L->stage[i]) (void)hipHostFree(L->stage[i]);
    if (L->stage_ev[i]) (void)hipEventDestroy(L->stage_ev[i]);
  }
  for (int j = 0; j < NF_MAX_NANO; ++j) {
    if (L->ev_app[j]) (void)hipEventDestroy(L->ev_app[j]);
    if (L->ev_att[j]) (void)hipEventDestroy(L->ev_att[j]);
  }
  for (hipEvent_t e : {L->ev_start, L->ev_g, L->ev_a, L->ev_lane})
    if (e) (void)hipEventDestroy(e);
  for (int j = 0; j < NF_MAX_NANO; ++j)
    for (hipEvent_t e : {L->ev_o[j], L->ev_co[j], L->ev_d[j], L->ev_cd[j]})
      if (e) (void)hipEventDestroy(e);
  if (L->sc) (void)hipStreamDestroy(L->sc);
  if (L->sc2) (void)hipStreamDestroy(L->sc2);
  if (L->ev_a2) (void)hipEventDestroy(L->ev_a2);
  for (DevBuf* b : {&L->x1r, &L->ypre, &L->ar_stage}) release(*b);
  for (auto& r : L->recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (hipEvent_t e : L->ev_free) (void)hipEventDestroy(e);
  delete L;
}

nf_status nf_kv_pool_create(const nf_layer* L, int32_t n_pages, int32_t page_size, void* k_dev, void* v_dev,
                            nf_kv_pool** out) {
  if (!L || !k_dev || !v_dev || !out) return set_err(NF_ERR_INVALID_ARG, "nf_kv_pool_create: null argument");
  *out = nullptr;
  if (page_size != PAGE_SIZE) return set_err(NF_ERR_UNSUPPORTED, "page_size %d: only 16 is supported", page_size);
  if (n_pages <= 0) return set_err(NF_ERR_INVALID_ARG, "n_pages must be positive");
  nf_kv_pool* p = new nf_kv_pool();
  p->layer = L;
  p->device = L->device;
  p->n_pages = n_pages;
  p->page_size = page_size;
  p->k = k_dev;
  p->v = v_dev;
  p->block_bytes = (int64_t)L->s.n_kv_heads * page_size * L->s.head_dim * (int64_t)dtype_bytes(L->s.dtype);
  *out = p;
  return NF_OK;
}

void nf_kv_pool_destroy(nf_kv_pool* p) {
  if (!p) return;
  if (p->offload.p || !p->offload.old.empty() || p->xfer.p || !p->xfer.old.empty()) {   // the layer may be gone
    (void)hipSetDevice(p->device);
    (void)hipDeviceSynchronize();
    release(p->offload);
    release(p->xfer);
  }
  delete p;
}

}  // extern "C"

namespace {

// Shared part of nf_kv_pool_import / nf_kv_pool_export: checks, the page list
// on the device, the conversion kernel.
nf_status kv_transfer(nf_kv_pool* P, const int32_t* pages, int32_t n, void* k_rm, void* v_rm, bool to_pool,
                      void* stream, const char* who) {
  if (!P || n < 0 || (n > 0 && (!k_rm || !v_rm)))
    return set_err(NF_ERR_INVALID_ARG, "%s: null argument or negative count", who);
  if (!pages && n > P->n_pages)
    return set_err(NF_ERR_OUT_OF_RANGE, "%s: %d pages requested from a pool of %d", who, n, P->n_pages);
  if (pages)
    for (int i = 0; i < n; ++i)
      if (pages[i] < 0 || pages[i] >= P->n_pages)
        return set_err(NF_ERR_OUT_OF_RANGE, "%s: page %d at %d is outside the pool's %d pages", who, pages[i], i,
                       P->n_pages);
  const nf_shape& sh = P->layer->s;
  if ((int64_t)n * sh.n_kv_heads * 2 >= (int64_t(1) << 31))
    return set_err(NF_ERR_OUT_OF_RANGE, "%s: %d pages exceed one launch", who, n);
  if (n == 0) return NF_OK;
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(P->device));
  const int32_t* d_pages = nullptr;
  if (pages) {
    HIP_TRY(ensure(P->xfer, (size_t)n * 4));
    HIP_TRY(hipMemcpyAsync(P->xfer.p, pages, (size_t)n * 4, hipMemcpyHostToDevice, st));
    d_pages = (const int32_t*)P->xfer.p;
  }
  HIP_TRY(kv_convert(sh.dtype, P->k, P->v, d_pages, n, sh.n_kv_heads, sh.head_dim, k_rm, v_rm, to_pool, st));
  return NF_OK;
}

}  // namespace

extern "C" {

nf_status nf_kv_pool_import(nf_kv_pool* P, const int32_t* pages, int32_t n, const void* k_src, const void* v_src,
                            void* stream) {
  return kv_transfer(P, pages, n, const_cast<void*>(k_src), const_cast<void*>(v_src), true, stream,
                     "nf_kv_pool_import");
}

nf_status nf_kv_pool_export(nf_kv_pool* P, const int32_t* pages, int32_t n, void* k_dst, void* v_dst, void* stream) {
  return kv_transfer(P, pages, n, k_dst, v_dst, false, stream, "nf_kv_pool_export");
}

nf_status nf_kv_offload(nf_kv_pool* P, const int32_t* pages, int32_t n, void* host_k, void* host_v,
                        void* stream) {
  if (!P || n < 0 || (n > 0 && (!pages || !host_k || !host_v)))
    return set_err(NF_ERR_INVALID_ARG, "nf_kv_offload: null argument or negative count");
  for (int i = 0; i < n; ++i)
    if (pages[i] < 0 || pages[i] >= P->n_pages)
      return set_err(NF_ERR_OUT_OF_RANGE, "nf_kv_offload: page %d at %d is outside the pool's %d pages", pages[i],
                     i, P->n_pages);
  if (n == 0) return NF_OK;
  const int64_t blk = P->block_bytes;
  const size_t idx_bytes = ((size_t)n * 4 + 255) & ~(size_t)255;
  hipStream_t st = (hipStream_t)stream;
  HIP_TRY(hipSetDevice(P->device));
  HIP_TRY(ensure(P->offload, idx_bytes + 2 * (size_t)n * blk));
  char* base = (char*)P->offload.p;
  int32_t* d_pages = (int32_t*)base;
  char* gk = base + idx_bytes;
  char* gv = gk + (size_t)n * blk;
  HIP_TRY(hipMemcpyAsync(d_pages, pages, (size_t)n * 4, hipMemcpyHostToDevice, st));
  HIP_TRY(kv_gather(P->k, P->v, d_pages, n, blk, gk, gv, st));
  HIP_TRY(hipMemcpyAsync(host_k, gk, (size_t)n * blk, hipMemcpyDeviceToHost, st));
  HIP_TRY(hipMemcpyAsync(host_v, gv, (size_t)n * blk, hipMemcpyDeviceToHost, st));
  return NF_OK;
}

nf_status nf_plan_set(nf_layer* L, const nf_plan* p) {
  if (!L || !p) return set_err(NF_ERR_INVALID_ARG, "nf_plan_set: null argument");
  std::string err;
  nf_status st = check_plan(*p, L->cus_per_xcd, err);
  if (st != NF_OK) return set_err(st, "%s", err.c_str());
  if (p->n_streams == 2) {
    HIP_TRY(hipSetDevice(L->device));
    StreamPair pr;
    st = get_pair(L, p->gemm_cus_per_xcd, p->attn_cus_per_xcd, pr);
    if (st != NF_OK) return st;
  }
  L->plan = *p;
  return NF_OK;
}

nf_status nf_plan_get(const nf_layer* L, nf_plan* p) {
  if (!L || !p) return set_err(NF_ERR_INVALID_ARG, "nf_plan_get: null argument");
  *p = L->plan;
  return NF_OK;
}

nf_status nf_layer_set_allreduce_emulation(nf_layer* L, int32_t mode, int32_t copy_workgroups) {
  if (!L || mode < 0 || mode > 2 || (mode == 2 && (copy_workgroups < 1 || copy_workgroups > 4096)))
    return set_err(NF_ERR_INVALID_ARG, "nf_layer_set_allreduce_emulation: bad argument");
  if (mode == 0) {
    L->ar_mode = 0;
    return NF_OK;
  }
  if (L->s.dtype == NF_F32 ? L->s.hidden % 4 : L->s.hidden % 8)
    return set_err(NF_ERR_UNSUPPORTED, "nf_layer_set_allreduce_emulation: rows must be whole 16-byte units");
  HIP_TRY(hipSetDevice(L->device));
  const size_t bytes = (size_t)L->s.max_tokens * L->s.hidden * dtype_bytes(L->s.dtype);
  for (DevBuf* b : {&L->x1r, &L->ypre, &L->ar_stage}) HIP_TRY(ensure(*b, bytes));
  for (int j = 0; j < NF_MAX_NANO; ++j)
    for (hipEvent_t* e : {&L->ev_o[j], &L->ev_co[j], &L->ev_d[j], &L->ev_cd[j]})
      if (!*e) HIP_TRY(hipEventCreateWithFlags(e, hipEventDisableTiming));
  if (!L->sc) HIP_TRY(hipStreamCreateWithFlags(&L->sc, hipStreamNonBlocking));
  L->ar_mode = mode;
  L->ar_wgs = mode == 2 ? copy_workgroups : L->ar_wgs;
  return NF_OK;
}

}  // extern "C"

const nf_shape* nf::layer_shape(const nf_layer* L) { return &L->s; }
nf_plan nf::layer_plan(const nf_layer* L) { return L->plan; }
int32_t nf::pool_pages(const nf_kv_pool* P) { return P->n_pages; }
nf_status nf::layer_step_with_plan(nf_layer* L, nf_kv_pool* P, const nf_batch* b, hipStream_t s, const nf_plan& plan) {
  if (P->layer != L) return set_err(NF_ERR_INVALID_ARG, "step: pool belongs to another layer");
  std::string err;
  nf_status st = check_plan(plan, L->cus_per_xcd, err);
  if (st != NF_OK) return set_err(st, "%s", err.c_str());
  return step_impl(L, P, b, s, plan);
}

extern "C" {

nf_status nf_layer_step(nf_layer* L, nf_kv_pool* P, const nf_batch* b, void* stream) {
  if (!L || !P || !b) return set_err(NF_ERR_INVALID_ARG, "nf_layer_step: null argument");
  if (P->layer != L) return set_err(NF_ERR_INVALID_ARG, "nf_layer_step: pool belongs to another layer");
  FaultScope fault;
  return step_impl(L, P, b, (hipStream_t)stream, L->plan);
}

nf_status nf_stack_step(nf_layer* const* layers, nf_kv_pool* const* pools, int32_t n_layers, const nf_batch* batch,
                        void* stream) {
  nf_status st = check_stack(layers, pools, n_layers, batch);
  if (st != NF_OK) return st;
  FaultScope fault;
  return stack_impl(layers, pools, n_layers, batch, (hipStream_t)stream);
}

struct nf_graph {
  int device = 0;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  std::vector<DevBuf> meta;      // each layer's step metadata, read by the captured launches
};

void nf_graph_destroy(nf_graph* g) {
  if (!g) return;
  (void)hipSetDevice(g->device);
  (void)hipDeviceSynchronize();
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  for (DevBuf& b : g->meta) release(b);
  delete g;
}

nf_status nf_stack_graph_create(nf_layer* const* layers, nf_kv_pool* const* pools, int32_t n_layers,
                                const nf_batch* batch, void* stream, nf_graph** out) {
  if (!out) return set_err(NF_ERR_INVALID_ARG, "nf_stack_graph_create: null argument");
  *out = nullptr;
  nf_status st = check_stack(layers, pools, n_layers, batch);
  if (st != NF_OK) return st;
  const nf_plan& plan = layers[0]->plan;
  if (plan.n_streams == 2 && (plan.gemm_cus_per_xcd || plan.attn_cus_per_xcd))
    return set_err(NF_ERR_UNSUPPORTED, "nf_stack_graph_create: a graph does not keep a stream's CU mask; "
                   "use a plan without a CU split");
  for (int l = 0; l < n_layers; ++l) {
    if (layers[l]->prof) return set_err(NF_ERR_UNSUPPORTED, "nf_stack_graph_create: per-kernel timing is on");
    if (layers[l]->ar_mode)
      return set_err(NF_ERR_UNSUPPORTED, "nf_stack_graph_create: the all-reduce emulation is on");
  }
  if (batch->n_tokens == 0) return set_err(NF_ERR_INVALID_ARG, "nf_stack_graph_create: empty batch");
  hipStream_t s = (hipStream_t)stream;
  // one eager step first: every buffer, stream and event the step needs
  // exists before the capture, which must not allocate
  if ((st = stack_impl(layers, pools, n_layers, batch, s)) != NF_OK) return st;
  HIP_TRY(hipStreamSynchronize(s));
  nf_graph* g = new nf_graph();
  g->device = layers[0]->device;
  g->meta.resize(n_layers);
  std::vector<LayerRun> runs;
  st = prepare_stack(layers, pools, n_layers, batch, &g->meta, runs);
  if (st != NF_OK) {
    nf_graph_destroy(g);
    return st;
  }
  // captured on a stream of its own (the caller's may be the null stream,
  // which cannot be captured); the caller's stream is idle after the warm-up
  hipStream_t cap = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&cap, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipStreamBeginCapture(cap, hipStreamCaptureModeRelaxed);
  if (e != hipSuccess) {
    if (cap) (void)hipStreamDestroy(cap);
    nf_graph_destroy(g);
    return set_err(NF_ERR_HIP, "stream capture could not start: %s", hipGetErrorString(e));
  }
  Streams S;
  st = open_streams(layers[0], plan, cap, S);
  if (st == NF_OK) st = issue_stack(runs, S, plan.order);
  if (st == NF_OK) st = close_streams(layers[0], S);
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(cap, &graph);
  (void)hipStreamDestroy(cap);
  if (st != NF_OK || e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    nf_graph_destroy(g);
    return st != NF_OK ? st : set_err(NF_ERR_HIP, "hipStreamEndCapture failed: %s", hipGetErrorString(e));
  }
  g->graph = graph;
  e = hipGraphInstantiate(&g->exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    g->exec = nullptr;
    nf_graph_destroy(g);
    return set_err(NF_ERR_HIP, "hipGraphInstantiate failed: %s", hipGetErrorString(e));
  }
  *out = g;
  return NF_OK;
}

nf_status nf_graph_launch(nf_graph* g, void* stream) {
  if (!g) return set_err(NF_ERR_INVALID_ARG, "nf_graph_launch: null argument");
  HIP_TRY(hipSetDevice(g->device));
  HIP_TRY(hipGraphLaunch(g->exec, (hipStream_t)stream));
  return NF_OK;
}

nf_status nf_layer_intermediate(const nf_layer* L, int32_t which, const void** dev, int64_t* stride) {
  if (!L || !dev || !stride) return set_err(NF_ERR_INVALID_ARG, "nf_layer_intermediate: null argument");
  if (!L->debug_capture)
    return set_err(NF_ERR_UNSUPPORTED, "nf_layer_intermediate: capture is off (nf_layer_debug_capture)");
  const nf_shape& s = L->s;
  const int64_t nqd = (int64_t)s.n_q_heads * s.head_dim;
  switch (which) {
    case 0: *dev = L->q_rot.p; *stride = nqd; break;
    case 1: *dev = L->attn.p; *stride = nqd; break;
    case 2: *dev = L->x1.p; *stride = s.hidden; break;
    case 3: *dev = L->act.p; *stride = s.ffn; break;
    case 4: *dev = L->qkv.p; *stride = (int64_t)(s.n_q_heads + 2 * s.n_kv_heads) * s.head_dim; break;
    case 5: *dev = L->r_idx.p; *stride = s.top_k; break;
    case 6: *dev = L->r_w.p; *stride = s.top_k; break;
    case 7: *dev = L->r_perm.p; *stride = 1; break;
    case 8: *dev = L->r_off.p; *stride = s.n_experts + 1; break;
    default: return set_err(NF_ERR_INVALID_ARG, "nf_layer_intermediate: unknown index %d", which);
  }
  if (!*dev) return set_err(NF_ERR_INVALID_ARG, "nf_layer_intermediate: %d not held by this layer", which);
  return NF_OK;
}

nf_status nf_layer_debug_capture(nf_layer* L, int32_t on) {
  if (!L) return set_err(NF_ERR_INVALID_ARG, "nf_layer_debug_capture: null layer");
  L->debug_capture = on != 0;
  return NF_OK;
}

nf_status nf_profile_enable(nf_layer* L, int32_t on, const char* only_kind) {
  if (!L) return set_err(NF_ERR_INVALID_ARG, "nf_profile_enable: null layer");
  L->prof_only = -1;
  if (only_kind) {
    for (int k = 0; k < K_COUNT; ++k)
      if (std::strcmp(kKindNames[k], only_kind) == 0) L->prof_only = k;
    if (L->prof_only < 0) return set_err(NF_ERR_INVALID_ARG, "nf_profile_enable: unknown kind %s", only_kind);
  }
  L->prof = on != 0;
  for (auto& r : L->recs) {
    L->ev_free.push_back(r.a);
    L->ev_free.push_back(r.b);
  }
  L->recs.clear();
  for (int k = 0; k < K_COUNT; ++k) {
    L->prof_ms[k] = 0;
    L->prof_n[k] = 0;
  }
  return NF_OK;
}

nf_status nf_profile_read(nf_layer* L, int32_t max_kinds, const char** names, int64_t* launches,
                          double* total_ms, int32_t* n_kinds) {
  if (!L || !n_kinds) return set_err(NF_ERR_INVALID_ARG, "nf_profile_read: null argument");
  for (auto& r : L->recs) {
    HIP_TRY(hipEventSynchronize(r.b));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, r.a, r.b));
    L->prof_ms[r.kind] += ms;
    L->prof_n[r.kind] += 1;
    L->ev_free.push_back(r.a);
    L->ev_free.push_back(r.b);
  }
  L->recs.clear();
  int n = 0;
  for (int k = 0; k < K_COUNT; ++k) {
    if (!L->prof_n[k]) continue;
    if (n < max_kinds) {
      if (names) names[n] = kKindNames[k];
      if (launches) launches[n] = L->prof_n[k];
      if (total_ms) total_ms[n] = L->prof_ms[k];
    }
    ++n;
  }
  *n_kinds = n;
  return NF_OK;
}

nf_status nf_probe_cu_map(int32_t* xcc, int32_t* cu, int32_t n) {
  if (!xcc || n <= 0) return set_err(NF_ERR_INVALID_ARG, "nf_probe_cu_map: bad argument");
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, dev));
  CuMap map;
  nf_status st = measure_cu_map(dev, prop.multiProcessorCount, 8, map);
  if (st != NF_OK) return st;
  for (int i = 0; i < n; ++i) {
    xcc[i] = i < (int)map.xcc.size() ? map.xcc[i] : -1;
    if (cu) cu[i] = i < (int)map.cu.size() ? map.cu[i] : -1;
  }
  return NF_OK;
}

nf_status nf_probe_budget_cus(int32_t first, int32_t count, int32_t* xcc_cu, int32_t max, int32_t* n_out) {
  if (!xcc_cu || !n_out || max <= 0 || first < 0 || count <= 0)
    return set_err(NF_ERR_INVALID_ARG, "nf_probe_budget_cus: bad argument");
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, dev));
  const int n_cus = prop.multiProcessorCount, n_xcd = 8, per = std::max(1, n_cus / n_xcd);
  if (first + count > per)
    return set_err(NF_ERR_OUT_OF_RANGE, "nf_probe_budget_cus: CUs %d..%d of an XCD with %d", first, first + count - 1,
                   per);
  CuMap map;
  nf_status st = measure_cu_map(dev, n_cus, n_xcd, map);
  if (st != NF_OK) return st;
  std::vector<uint32_t> mask;
  make_mask(map.xcc, n_xcd, first, first + count, mask);
  std::vector<std::pair<int, int>> seen;
  if ((st = probe_mask(mask, seen)) != NF_OK) return st;
  *n_out = (int32_t)seen.size();
  for (int i = 0; i < (int)seen.size() && i < max; ++i) xcc_cu[i] = (seen[i].first << 16) | seen[i].second;
  return NF_OK;
}

// Device buffers and events of a probe, released on every return path.
struct ProbeRes {
  void* buf = nullptr;
  float* sink = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  ~ProbeRes() {
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (buf) (void)hipFree(buf);
    if (sink) (void)hipFree(sink);
  }
};

nf_status nf_probe_mfma_bf16_tflops(double* tflops) {
  if (!tflops) return set_err(NF_ERR_INVALID_ARG, "nf_probe_mfma_bf16_tflops: null argument");
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, dev));
  ProbeRes r;
  HIP_TRY(hipMalloc(&r.sink, 1024 * sizeof(float)));
  HIP_TRY(hipEventCreate(&r.e0));
  HIP_TRY(hipEventCreate(&r.e1));
  const int blocks = prop.multiProcessorCount * 4, iters = 4096;
  double best = 0;
  for (int shape = 0; shape < 2; ++shape) {
    double best_shape = 0;
    for (int rep = 0; rep < 4; ++rep) {
      HIP_TRY(hipEventRecord(r.e0, nullptr));
      HIP_TRY(probe_mfma(shape, blocks, iters, r.sink, nullptr));
      HIP_TRY(hipEventRecord(r.e1, nullptr));
      HIP_TRY(hipEventSynchronize(r.e1));
      float ms = 0;
      HIP_TRY(hipEventElapsedTime(&ms, r.e0, r.e1));
      // per wave and iteration: 8 x 16x16x32 or 4 x 32x32x16, both 131072 FLOP
      const double flops = (double)blocks * 4 /*waves*/ * iters * 131072.0;
      if (rep > 0) best_shape = std::max(best_shape, flops / (ms * 1e-3) / 1e12);
    }
    if (std::getenv("NF_PROBE_VERBOSE"))
      std::fprintf(stderr, "nf probe: mfma %s %.1f TFLOP/s\n", shape ? "32x32x16" : "16x16x32", best_shape);
    best = std::max(best, best_shape);
  }
  *tflops = best;
  return NF_OK;
}

nf_status nf_probe_hbm_read_gbps(size_t bytes, double* gbps) {
  if (!gbps || bytes < (1u << 20)) return set_err(NF_ERR_INVALID_ARG, "nf_probe_hbm_read_gbps: bad argument");
  bytes &= ~(size_t)15;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, dev));
  ProbeRes r;
  HIP_TRY(hipMalloc(&r.buf, bytes));
  HIP_TRY(hipMalloc(&r.sink, 1024 * sizeof(float)));
  HIP_TRY(hipMemset(r.buf, 1, bytes));
  HIP_TRY(hipEventCreate(&r.e0));
  HIP_TRY(hipEventCreate(&r.e1));
  // best of a few occupancies (workgroups per CU) of a streaming read
  double best = 0;
  for (int per_cu : {2, 4, 8}) {
    for (int rep = 0; rep < 4; ++rep) {
      HIP_TRY(hipEventRecord(r.e0, nullptr));
      HIP_TRY(probe_read(r.buf, bytes, r.sink, prop.multiProcessorCount * per_cu, nullptr));
      HIP_TRY(hipEventRecord(r.e1, nullptr));
      HIP_TRY(hipEventSynchronize(r.e1));
      float ms = 0;
      HIP_TRY(hipEventElapsedTime(&ms, r.e0, r.e1));
      if (rep > 0) best = std::max(best, (double)bytes / (ms * 1e-3) / 1e9);
    }
  }
  *gbps = best;
  return NF_OK;
}

nf_status nf_plan_search(nf_layer* L, nf_kv_pool* P, const nf_batch* b, const nf_search_opts* o, nf_plan* out,
                         double* times_ms, void* stream);

}  // extern "C"

// =============================================================== plan search
// Profile-driven search over the four plan dimensions (count, sizes, order,
// resource split) for one batch; it replaces the pages' MILP-based parameter
// search ("Search Space 4D" card on the do-not-panic NanoFlow page; Gurobi
// note on the ossradar page) and, like it, weighs the interference of
// concurrent operations (abstract on the codewithpapers page).
//  1. Solo profiles: the batch split into 1..max_count equal nano-batches on
//     one stream, every kernel timed; per nano-batch size, the front (norm,
//     QKV, RoPE), O-projection and FFN durations, and attention as a linear
//     function of its KV page units.
//  2. Interference: per two-stream resource split (GEMM / attention CUs per
//     XCD, attention residency), one overlapped run of two equal nano-batches
//     gives the co-run slowdown of each side and the cost of a cross-stream
//     wait.
//  3. The event-graph model (plan_model.cpp) predicts every candidate: counts
//     1..max_count; sizes equal, attention-balanced, 64-token steps for two,
//     quarter / half / quarter for three, decode requests apart from a
//     prefill chunk; pipelined and deep orders; each resource split, and one
//     stream.
//  4. The top_k predictions and the unsplit plan are timed on the device;
//     the fastest is kept.
namespace {

// Nano-batch boundaries that balance attention work (KV pages) plus GEMM rows.
void balanced_sizes(const nf_batch* b, int count, int32_t* sizes) {
  const int T = b->n_tokens;
  std::vector<double> cost(T, 0.0);
  double total = 0;
  for (int r = 0; r < b->n_requests; ++r)
    for (int i = 0; i < b->req_q_len[r]; ++i) {
      const int t = b->req_q_start[r] + i;
      const double pages = (b->pos[t] + 1) / 16.0;
      cost[t] = pages + 8.0;             // KV pages read + a row of GEMM work
      total += cost[t];
    }
  int t = 0;
  double acc = 0;
  for (int j = 0; j < count; ++j) {
    const int start = t;
    const double goal = total * (j + 1) / count;
    while (t < T - (count - 1 - j) && (acc + cost[t] <= goal || t == start)) acc += cost[t++];
    if (j == count - 1) t = T;
    sizes[j] = t - start;
  }
}

// operation class of a kernel kind: 0 front, 1 attention, 2 O half, 3 FFN
int kind_class(int k) {
  switch (k) {
    case K_NORM1: case K_QKV: case K_QKV_RED: case K_ROPE: return 0;
    case K_ATTN: case K_MERGE: return 1;
    case K_OPROJ: case K_OPROJ_RED: case K_NORM2: return 2;
    default: return 3;
  }
}

nf_plan make_plan(int count, const int32_t* sizes, int order, int streams, int g, int a, int w) {
  nf_plan p{};
  p.count = count;
  for (int j = 0; j < count; ++j) p.sizes[j] = sizes[j];
  p.order = order;
  p.n_streams = streams;
  p.gemm_cus_per_xcd = g;
  p.attn_cus_per_xcd = a;
  p.attn_waves_per_cu = w;
  return p;
}

bool same_plan(const nf_plan& x, const nf_plan& y) {
  if (x.count != y.count || x.order != y.order || x.n_streams != y.n_streams ||
      x.gemm_cus_per_xcd != y.gemm_cus_per_xcd || x.attn_cus_per_xcd != y.attn_cus_per_xcd ||
      x.attn_waves_per_cu != y.attn_waves_per_cu)
    return false;
  for (int j = 0; j < x.count; ++j)
    if (x.sizes[j] != y.sizes[j]) return false;
  return true;
}

struct Split {
  int g, a, w;
};
// two-stream resource splits: every CU to both sides; attention held to 8 or
// 4 waves per CU (persistent four-wave workgroups, GEMM tiles that fit beside
// them); CU partitions per XCD from 28 + 4 to 8 + 24
const Split kSplits[] = {{0, 0, 0}, {0, 0, 8}, {0, 0, 4}, {28, 4, 0}, {24, 8, 0}, {20, 12, 0},
                         {16, 16, 0}, {12, 20, 0}, {8, 24, 0}};
constexpr int kNSplits = sizeof(kSplits) / sizeof(kSplits[0]);

}  // namespace


extern "C" nf_status nf_plan_search(nf_layer* L, nf_kv_pool* P, const nf_batch* b, const nf_search_opts* o,
                                    nf_plan* out, double* times_ms, void* stream) {
  if (!L || !P || !b || !out) return set_err(NF_ERR_INVALID_ARG, "nf_plan_search: null argument");
  nf_search_opts opts{4, 2, 5, 8};
  if (o) opts = *o;
  opts.max_count = std::max(1, std::min(opts.max_count, NF_MAX_NANO));
  opts.reps = std::max(1, opts.reps);
  opts.top_k = std::max(1, opts.top_k);
  hipStream_t s = (hipStream_t)stream;
  const int T = b->n_tokens;
  const nf_plan unsplit = make_plan(1, &T, NF_ORDER_PIPELINED, 1, 0, 0, 0);
  if (T == 0) {
    *out = nf_plan{1, {0, 0, 0, 0}, NF_ORDER_PIPELINED, 1, 0, 0, 0};
    L->plan = *out;
    return NF_OK;
  }
  if (L->prof) return set_err(NF_ERR_UNSUPPORTED, "nf_plan_search: per-kernel timing is on");

  // The candidates are timed on this batch, whose steps write K/V into the
  // pool pages holding its new positions.  Those pages are saved first and
  // put back before returning, so the caller's pool ends bit-identical.
  std::string err;
  nf_status st0 = check_batch(L->s, P->n_pages, P->page_size, *b, err);
  if (st0 != NF_OK) return set_err(st0, "%s", err.c_str());
  std::vector<int32_t> saved;
  {
    std::vector<char> mark(P->n_pages, 0);
    for (int r = 0; r < b->n_requests; ++r)
      for (int i = 0; i < b->req_q_len[r]; ++i) {
        const int32_t pg = b->page_indices[b->page_indptr[r] + (b->req_pos0[r] + i) / P->page_size];
        if (!mark[pg]) {
          mark[pg] = 1;
          saved.push_back(pg);
        }
      }
  }
  const size_t list_bytes = ((saved.size() * 4) + 255) & ~(size_t)255;
  struct Backup {
    void* p = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    ~Backup() {
      if (p) (void)hipFree(p);
      if (e0) (void)hipEventDestroy(e0);
      if (e1) (void)hipEventDestroy(e1);
    }
  } bk;
  HIP_TRY(hipSetDevice(L->device));
  HIP_TRY(hipMalloc(&bk.p, list_bytes + 2 * saved.size() * (size_t)P->block_bytes));
  int32_t* d_saved = (int32_t*)bk.p;
  char* bkk = (char*)bk.p + list_bytes;
  char* bkv = bkk + saved.size() * (size_t)P->block_bytes;
  HIP_TRY(hipMemcpyAsync(d_saved, saved.data(), saved.size() * 4, hipMemcpyHostToDevice, s));
  HIP_TRY(kv_gather(P->k, P->v, d_saved, (int)saved.size(), P->block_bytes, bkk, bkv, s));
  HIP_TRY(hipEventCreate(&bk.e0));
  HIP_TRY(hipEventCreate(&bk.e1));
  const bool verbose = std::getenv("NF_SEARCH_VERBOSE") != nullptr;

  // ms per step of `plan`: `warm` untimed steps, then `reps` between events
  auto measure = [&](const nf_plan& plan, int warm, int reps, double& ms, const nf_batch* bb = nullptr) -> nf_status {
    if (!bb) bb = b;
    nf_status st = NF_OK;
    for (int w = 0; w < warm && st == NF_OK; ++w) st = step_impl(L, P, bb, s, plan);
    if (st != NF_OK) return st;
    HIP_TRY(hipEventRecord(bk.e0, s));
    for (int r = 0; r < reps && st == NF_OK; ++r) st = step_impl(L, P, bb, s, plan);
    HIP_TRY(hipEventRecord(bk.e1, s));
    HIP_TRY(hipEventSynchronize(bk.e1));
    if (st != NF_OK) return st;
    float t = 0;
    HIP_TRY(hipEventElapsedTime(&t, bk.e0, bk.e1));
    ms = t / reps;
    return NF_OK;
  };
  // per-step microseconds of each operation class over `reps` profiled steps
  auto classes = [&](const nf_plan& plan, int reps, double* cls, const nf_batch* bb = nullptr) -> nf_status {
    if (!bb) bb = b;
    nf_status st = nf_profile_enable(L, 1, nullptr);
    for (int r = 0; r < reps && st == NF_OK; ++r) st = step_impl(L, P, bb, s, plan);
    if (st != NF_OK) {
      (void)nf_profile_enable(L, 0, nullptr);
      return st;
    }
    for (auto& rec : L->recs) {
      HIP_TRY(hipEventSynchronize(rec.b));
      float ms = 0;
      HIP_TRY(hipEventElapsedTime(&ms, rec.a, rec.b));
      L->prof_ms[rec.kind] += ms;
    }
    for (int c = 0; c < 4; ++c) cls[c] = 0;
    for (int k = 0; k < K_COUNT; ++k) cls[kind_class(k)] += L->prof_ms[k] * 1e3 / reps;
    return nf_profile_enable(L, 0, nullptr);
  };

  // Per-kernel timing adds event packets around every kernel, so a profiled
  // step's class times can sum past the same step timed plainly; they are
  // scaled down to the plain step time (one stream: the step is their sum
  // plus the gaps between launches).
  auto fit_classes = [](double* cls, double ms) {
    const double total = cls[0] + cls[1] + cls[2] + cls[3];
    if (total > ms * 1e3 && total > 0)
      for (int c = 0; c < 4; ++c) cls[c] *= ms * 1e3 / total;
  };

  nf_status st = NF_OK;
  nf_plan_profile prof{};
  std::vector<SearchEntry> report, timed;      // calibration runs; candidates timed in step 4
  std::vector<std::pair<nf_plan, double>> preds;
  do {
    // the device settles first (clocks, caches): the first steps after idle
    // run slower than the ones the candidates are timed with later
    {
      double ms = 0;
      if ((st = measure(unsplit, 10, 1, ms)) != NF_OK) break;
    }
    // 1. solo profiles on one stream
    double gap_sum = 0;
    int gap_n = 0;
    std::vector<std::pair<double, double>> att;     // (page units per nano-batch, us per launch)
    const int kmax = std::min(opts.max_count, T);
    // a prefix of the batch's requests of about T/8 tokens adds the profile
    // point below the smallest equal split, where weight-bound GEMMs stop
    // scaling with the tokens
    nf_batch pre = *b;
    pre.n_requests = 0;
    pre.n_tokens = 0;
    for (int r = 0; r < b->n_requests && pre.n_tokens < T / 8; ++r) {
      pre.n_requests = r + 1;
      pre.n_tokens = b->req_q_start[r] + b->req_q_len[r];
    }
    const bool small = kmax >= 2 && pre.n_tokens > 0 && 2 * pre.n_tokens <= T / kmax;
    const int base = small ? 1 : 0;
    prof.n_points = kmax + base;
    double solo2[4] = {0, 0, 0, 0};
    for (int k = 1; k <= kmax && st == NF_OK; ++k) {
      int32_t sz[NF_MAX_NANO];
      for (int j = 0; j < k; ++j) sz[j] = T / k + (j < T % k ? 1 : 0);
      const nf_plan pl = make_plan(k, sz, NF_ORDER_SEQUENTIAL, 1, 0, 0, 0);
      double ms = 0, cls[4];
      if ((st = measure(pl, k == 1 ? 3 : 1, 3, ms)) != NF_OK) break;
      if ((st = classes(pl, 2, cls)) != NF_OK) break;
      // the co-run ratios below compare profiled runs with profiled runs
      if (k == 2) std::copy(cls, cls + 4, solo2);
      fit_classes(cls, ms);
      const int i = base + kmax - k;           // ascending nano-batch size
      prof.tokens[i] = (double)T / k;
      prof.front_us[i] = cls[0] / k;
      prof.oproj_us[i] = cls[2] / k;
      prof.ffn_us[i] = cls[3] / k;
      double units[NF_MAX_NANO];
      attn_page_units(L->s, *b, pl, units);
      double u = 0;
      for (int j = 0; j < k; ++j) u += units[j];
      att.push_back({u / k, cls[1] / k});
      gap_sum += std::max(0.0, ms * 1e3 - (cls[0] + cls[1] + cls[2] + cls[3])) / (4.0 * k);
      ++gap_n;
    }
    if (st != NF_OK) break;
    if (small) {
      const int32_t one = pre.n_tokens;
      const nf_plan pl = make_plan(1, &one, NF_ORDER_SEQUENTIAL, 1, 0, 0, 0);
      double ms = 0, cls[4];
      if ((st = measure(pl, 1, 3, ms, &pre)) != NF_OK) break;
      if ((st = classes(pl, 2, cls, &pre)) != NF_OK) break;
      fit_classes(cls, ms);
      prof.tokens[0] = pre.n_tokens;
      prof.front_us[0] = cls[0];
      prof.oproj_us[0] = cls[2];
      prof.ffn_us[0] = cls[3];
      double units[NF_MAX_NANO];
      attn_page_units(L->s, pre, pl, units);
      att.push_back({units[0], cls[1]});
    }
    prof.gap_us = gap_n ? gap_sum / gap_n : 0;
    if (att.size() >= 2) {          // least squares: us = base + slope * units
      double sx = 0, sy = 0, sxx = 0, sxy = 0;
      for (auto& q : att) {
        sx += q.first;
        sy += q.second;
        sxx += q.first * q.first;
        sxy += q.first * q.second;
      }
      const double n = (double)att.size(), den = n * sxx - sx * sx;
      prof.attn_us_per_page = den > 0 ? std::max(0.0, (n * sxy - sx * sy) / den) : 0;
      prof.attn_base_us = std::max(0.0, (sy - prof.attn_us_per_page * sx) / n);
    } else {
      prof.attn_base_us = 0;
      prof.attn_us_per_page = att[0].first > 0 ? att[0].second / att[0].first : 0;
    }
    prof.slow_gemm = prof.slow_attn = 1;
    prof.wait_us = 0;
    if (verbose)
      std::fprintf(stderr, "nf search: solo fronts %.1f..%.1f us, attention %.2f + %.5f us/page unit, gap %.1f us\n",
                   prof.front_us[0], prof.front_us[prof.n_points - 1], prof.attn_base_us, prof.attn_us_per_page,
                   prof.gap_us);

    // 2. interference per two-stream resource split
    nf_plan_profile calib[kNSplits];
    bool calib_ok[kNSplits] = {};
    if (kmax >= 2) {
      int32_t sz2[2] = {T - T / 2, T / 2};
      for (int c = 0; c < kNSplits && st == NF_OK; ++c) {
        const Split& sp = kSplits[c];
        if (sp.g >= L->cus_per_xcd || sp.a >= L->cus_per_xcd) continue;
        const nf_plan pl = make_plan(2, sz2, NF_ORDER_PIPELINED, 2, sp.g, sp.a, sp.w);
        double ms = 0, cls[4];
        if ((st = measure(pl, 1, 3, ms)) != NF_OK) break;
        if ((st = classes(pl, 2, cls)) != NF_OK) break;
        nf_plan_profile q = prof;
        const double g_ov = cls[0] + cls[2] + cls[3], g_solo = solo2[0] + solo2[2] + solo2[3];
        if (sp.g || sp.a) {
          // a CU budget confines each side also while it runs alone: its
          // durations scale throughout, with no further co-run slowdown
          q.scale_gemm = g_solo > 0 ? std::max(0.5, g_ov / g_solo) : 1.0;
          q.scale_attn = solo2[1] > 0 ? std::max(0.5, cls[1] / solo2[1]) : 1.0;
        } else {
          // unmasked, the sides slow each other only while both run
          q.slow_attn = std::max(1.0, solo2[1] > 0 ? cls[1] / solo2[1] : 1.0);
          const double frac = cls[1] > 0 ? std::min(0.95, std::max(0.0, (g_ov - g_solo) / cls[1])) : 0.0;
          q.slow_gemm = 1.0 / (1.0 - frac);
        }
        double tok[2] = {(double)sz2[0], (double)sz2[1]}, units[NF_MAX_NANO];
        attn_page_units(L->s, *b, pl, units);
        // the cross-stream wait that makes the model meet the measured step
        // (the prediction grows with the wait; bisection over 0..500 us)
        double lo = 0, hi = 500;
        q.wait_us = 0;
        if (predict_plan_us(q, pl, tok, units) < ms * 1e3) {
          for (int it = 0; it < 40; ++it) {
            q.wait_us = 0.5 * (lo + hi);
            (predict_plan_us(q, pl, tok, units) < ms * 1e3 ? lo : hi) = q.wait_us;
          }
          q.wait_us = 0.5 * (lo + hi);
        }
        calib[c] = q;
        calib_ok[c] = true;
        report.push_back({pl, predict_plan_us(q, pl, tok, units) * 1e-3, ms, true});
        if (verbose)
          std::fprintf(stderr, "nf search: split gemm %d attn %d waves %d: slowdown gemm %.2f attn %.2f, scale gemm %.2f "
                       "attn %.2f, wait %.1f us (two nano-batches %.3f ms)\n", sp.g, sp.a, sp.w, q.slow_gemm,
                       q.slow_attn, q.scale_gemm, q.scale_attn, q.wait_us, ms);
      }
    }
    if (st != NF_OK) break;
    // Two lanes of the same two nano-batches, once: the rate at which two
    // operations of one class share the chip is fitted so that the model meets
    // the run (bisection; the prediction falls as the rate rises), on top of
    // the unmasked split's co-run slowdowns.
    nf_plan_profile calib_lanes{};
    bool lanes_ok = false;
    if (kmax >= 2 && calib_ok[0]) {
      int32_t sz2[2] = {T - T / 2, T / 2};
      const nf_plan pl = make_plan(2, sz2, NF_ORDER_LANES, 2, 0, 0, 0);
      double ms = 0;
      if ((st = measure(pl, 1, 3, ms)) != NF_OK) break;
      nf_plan_profile q = calib[0];
      double tok[2] = {(double)sz2[0], (double)sz2[1]}, units[NF_MAX_NANO];
      attn_page_units(L->s, *b, pl, units);
      double lo = 0.25, hi = 1.0;
      auto pred = [&](double rate) {
        q.lane_rate = rate;
        return predict_plan_us(q, pl, tok, units);
      };
      if (pred(lo) <= ms * 1e3) {
        // slower than the slowest rate explains: the cross-stream wait takes
        // the rest, fitted as for the splits
        q.lane_rate = lo;
        double wlo = q.wait_us, whi = q.wait_us + 500;
        for (int it = 0; it < 40; ++it) {
          q.wait_us = 0.5 * (wlo + whi);
          (predict_plan_us(q, pl, tok, units) < ms * 1e3 ? wlo : whi) = q.wait_us;
        }
        q.wait_us = whi;
      } else if (pred(hi) >= ms * 1e3) {
        q.lane_rate = hi;
      } else {
        for (int it = 0; it < 40; ++it) {
          const double mid = 0.5 * (lo + hi);
          (pred(mid) > ms * 1e3 ? lo : hi) = mid;
        }
        q.lane_rate = 0.5 * (lo + hi);
      }
      calib_lanes = q;
      lanes_ok = true;
      report.push_back({pl, predict_plan_us(q, pl, tok, units) * 1e-3, ms, true});
      if (verbose)
        std::fprintf(stderr, "nf search: two lanes: same-class rate %.3f (two nano-batches %.3f ms)\n", q.lane_rate,
                     ms);
    }

    // 3. candidates, predicted
    std::vector<std::vector<int32_t>> sizes;
    auto add_sizes = [&](std::vector<int32_t> v) {
      int64_t sum = 0;
      for (int32_t x : v) {
        if (x <= 0) return;
        sum += x;
      }
      if (sum != T || (int)v.size() > kmax) return;
      for (auto& w : sizes)
        if (w == v) return;
      sizes.push_back(v);
    };
    add_sizes({T});
    // the decode requests apart from a trailing prefill chunk
    int dec = 0;
    for (int r = 0; r < b->n_requests; ++r)
      if (b->req_q_len[r] == 1) dec = b->req_q_start[r] + 1;
    const bool chunk_last = b->n_requests > 0 && b->req_q_len[b->n_requests - 1] > 1 && dec > 0 &&
                            dec == b->req_q_start[b->n_requests - 1];
    for (int k = 2; k <= kmax; ++k) {
      std::vector<int32_t> eq(k), bal(k);
      for (int j = 0; j < k; ++j) eq[j] = T / k + (j < T % k ? 1 : 0);
      balanced_sizes(b, k, bal.data());
      add_sizes(eq);
      add_sizes(bal);
      if (chunk_last) {
        std::vector<int32_t> v(k);
        const int nd = k - 1;
        for (int j = 0; j < nd; ++j) v[j] = dec / nd + (j < dec % nd ? 1 : 0);
        v[k - 1] = T - dec;
        add_sizes(v);
      }
    }
    if (kmax >= 2)
      for (int f = 64; f < T; f += 64) add_sizes({f, T - f});
    if (kmax >= 3) {
      const int q = std::max(64, 64 * ((T / 4 + 32) / 64));
      add_sizes({q, T - 2 * q, q});
    }
    for (auto& v : sizes) {
      const int k = (int)v.size();
      double tok[NF_MAX_NANO], units[NF_MAX_NANO];
      for (int j = 0; j < k; ++j) tok[j] = v[j];
      const nf_plan one = make_plan(k, v.data(), NF_ORDER_SEQUENTIAL, 1, 0, 0, 0);
      attn_page_units(L->s, *b, one, units);
      preds.push_back({k == 1 ? unsplit : one, predict_plan_us(prof, one, tok, units)});
      if (k == 1) continue;
      for (int c = 0; c < kNSplits; ++c) {
        if (!calib_ok[c]) continue;
        for (int order : {NF_ORDER_PIPELINED, NF_ORDER_DEEP}) {
          const nf_plan pl = make_plan(k, v.data(), order, 2, kSplits[c].g, kSplits[c].a, kSplits[c].w);
          preds.push_back({pl, predict_plan_us(calib[c], pl, tok, units)});
        }
      }
      // two lanes without CU masks, with the co-run rates of the unmasked
      // calibration (kSplits[0]) and the fitted lane rate
      if (lanes_ok) {
        const nf_plan pl = make_plan(k, v.data(), NF_ORDER_LANES, 2, 0, 0, 0);
        preds.push_back({pl, predict_plan_us(calib_lanes, pl, tok, units)});
      }
    }
    std::stable_sort(preds.begin(), preds.end(), [](const std::pair<nf_plan, double>& x,
                                                    const std::pair<nf_plan, double>& y) { return x.second < y.second; });

    // 4. the best predictions and the unsplit plan, timed
    std::vector<std::pair<nf_plan, double>> top;
    for (auto& pr : preds) {
      if ((int)top.size() >= opts.top_k) break;
      top.push_back(pr);
    }
    bool has_unsplit = false;
    for (auto& t : top) has_unsplit = has_unsplit || same_plan(t.first, unsplit);
    if (!has_unsplit)
      for (auto& pr : preds)
        if (same_plan(pr.first, unsplit)) top.push_back(pr);
    for (auto& t : top) {
      double ms = 0;
      if ((st = measure(t.first, opts.warmup, opts.reps, ms)) != NF_OK) break;
      timed.push_back({t.first, t.second * 1e-3, ms});
      if (verbose) {
        const nf_plan& q = t.first;
        std::fprintf(stderr, "nf search: count %d sizes %d/%d/%d/%d order %d streams %d cus/xcd gemm %2d attn %2d "
                     "waves %d: predicted %.3f ms, measured %.3f ms\n", q.count, q.sizes[0], q.sizes[1], q.sizes[2],
                     q.sizes[3], q.order, q.n_streams, q.gemm_cus_per_xcd, q.attn_cus_per_xcd, q.attn_waves_per_cu,
                     t.second * 1e-3, ms);
      }
    }
  } while (false);

  {
    const std::string step_err = g_err;
    hipError_t re = kv_scatter(P->k, P->v, d_saved, (int)saved.size(), P->block_bytes, bkk, bkv, s);
    if (re == hipSuccess) re = hipStreamSynchronize(s);
    if (re != hipSuccess) {
      (void)hipGetLastError();
      return set_err(NF_ERR_HIP, "nf_plan_search: restoring the pool's pages failed: %s", hipGetErrorString(re));
    }
    g_err = step_err;
  }
  if (st != NF_OK) return st;
  // the fastest of the timed candidates (the calibration runs used fewer steps)
  int best = -1;
  for (size_t i = 0; i < timed.size(); ++i)
    if (best < 0 || timed[i].measured_ms < timed[best].measured_ms) best = (int)i;
  if (best < 0) return set_err(NF_ERR_NO_PLAN, "nf_plan_search: no candidate was timed");
  if (times_ms) {
    times_ms[0] = timed[best].measured_ms;
    times_ms[1] = (double)preds.size();
  }
  L->plan = timed[best].plan;
  *out = timed[best].plan;
  report.insert(report.end(), timed.begin(), timed.end());
  L->search_report = report;
  return NF_OK;
}

extern "C" nf_status nf_plan_search_report(const nf_layer* L, int32_t max, nf_plan* plans, double* predicted_ms,
                                           double* measured_ms, int32_t* calibration, int32_t* n) {
  if (!L || !n || max < 0) return set_err(NF_ERR_INVALID_ARG, "nf_plan_search_report: bad argument");
  const std::vector<SearchEntry>& r = L->search_report;
  *n = (int32_t)r.size();
  for (int i = 0; i < (int)r.size() && i < max; ++i) {
    if (plans) plans[i] = r[i].plan;
    if (predicted_ms) predicted_ms[i] = r[i].predicted_ms;
    if (measured_ms) measured_ms[i] = r[i].measured_ms;
    if (calibration) calibration[i] = r[i].calibration ? 1 : 0;
  }
  return NF_OK;
}

extern "C" nf_status nf_plan_predict(const nf_plan_profile* prof, const nf_shape* shape, const nf_plan* plan,
                                     const nf_batch* batch, double* us) {
  if (!prof || !shape || !plan || !batch || !us || prof->n_points < 1 || prof->n_points > NF_PROFILE_POINTS)
    return set_err(NF_ERR_INVALID_ARG, "nf_plan_predict: bad argument");
  std::string err;
  nf_status st = check_plan(*plan, 32, err);
  if (st == NF_OK) st = check_plan_batch(*plan, batch->n_tokens, err);
  if (st != NF_OK) return set_err(st, "%s", err.c_str());
  double tok[NF_MAX_NANO], units[NF_MAX_NANO];
  const int k = plan->count;
  for (int j = 0; j < k; ++j) tok[j] = (k == 1 && plan->sizes[0] == 0) ? batch->n_tokens : plan->sizes[j];
  attn_page_units(*shape, *batch, *plan, units);
  *us = predict_plan_us(*prof, *plan, tok, units);
  return NF_OK;
}

extern "C" nf_status nf_gemm_bf16(int32_t M, int32_t N, int32_t K, int32_t mode, const void* A, int64_t lda,
                                  const void* Bw, const void* B2, int64_t ldb, const void* R, int64_t ldr, void* C,
                                  int64_t ldc, int32_t tile_cfg, int32_t k_splits, int32_t cus, void* stream,
                                  int32_t* out_cfg, int32_t* out_splits) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 8 || N % 8 || mode < 0 || mode > 2 || !A || !Bw || !C ||
      (mode == GEMM_RESIDUAL && !R) || (mode == GEMM_SWIGLU && !B2) || lda < K || ldb < K || ldc < N ||
      (mode == GEMM_RESIDUAL && ldr < N))
    return set_err(NF_ERR_INVALID_ARG, "nf_gemm_bf16: bad argument");
  const bool streaming = tile_cfg >= 40;
  if (tile_cfg >= 0 && !((tile_cfg <= 6) || (tile_cfg >= 10 && tile_cfg <= 30 && K % 64 == 0) ||
                         (streaming && stream_kc(tile_cfg) > 0 && N % 32 == 0 && K % (16 * stream_kc(tile_cfg)) == 0 &&
                          stream_nbw(tile_cfg) == (mode == GEMM_SWIGLU ? 2 : 1))))
    return set_err(NF_ERR_INVALID_ARG, "nf_gemm_bf16: tile_cfg %d not available for N %d K %d mode %d", tile_cfg, N, K,
                   mode);
  if ((int64_t)M * lda * 2 >= (int64_t(1) << 32) || (int64_t)N * ldb * 2 >= (int64_t(1) << 32))
    return set_err(NF_ERR_OUT_OF_RANGE, "nf_gemm_bf16: an operand would exceed 4 GiB");
  GemmArgs g;
  g.A = A; g.lda = lda;
  g.B = Bw; g.B2 = B2; g.ldb = ldb;
  g.C = C; g.ldc = ldc; g.R = R; g.ldr = ldr;
  g.M = M; g.N = N; g.K = K; g.mode = mode;
  GemmPlan p = gemm_choose(g, cus > 0 ? cus : 256);
  if (tile_cfg >= 0) p.cfg = tile_cfg;
  if (k_splits > 0) p.k_splits = k_splits;
  hipStream_t s = (hipStream_t)stream;
  void* Bp = nullptr;
  if (streaming) {              // the weight-streaming kernels read an operand-order copy of B
    const int nb = mode == GEMM_SWIGLU ? 2 : 1;
    HIP_TRY(hipMalloc(&Bp, (size_t)nb * N * K * 2));
    hipError_t pe = pack_b(Bw, ldb, 0, N, K, 1, Bp, nb, 0, 0, s);
    if (pe == hipSuccess && nb == 2) pe = pack_b(B2, ldb, 0, N, K, 1, Bp, 2, 1, 0, s);
    if (pe != hipSuccess) {
      (void)hipFree(Bp);
      return set_err(NF_ERR_HIP, "nf_gemm_bf16: packing B: %s", hipGetErrorString(pe));
    }
    g.Bp = Bp;
  }
  void* ws = nullptr;
  const size_t wsb = gemm_workspace_bytes(g, p);
  hipError_t e = wsb ? hipMalloc(&ws, wsb) : hipSuccess;
  if (e == hipSuccess) e = gemm_bf16(g, p, ws, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (ws) (void)hipFree(ws);
  if (Bp) (void)hipFree(Bp);
  if (e != hipSuccess) return set_err(NF_ERR_HIP, "nf_gemm_bf16: %s", hipGetErrorString(e));
  if (out_cfg) *out_cfg = p.cfg;
  if (out_splits) *out_splits = p.k_splits;
  return NF_OK;
}

extern "C" nf_status nf_probe_gemm_bf16_ms(int32_t M, int32_t N, int32_t K, int32_t mode, int32_t tile_cfg,
                                           int32_t k_splits, int32_t cus, int32_t reps, double* ms,
                                           int32_t* out_cfg, int32_t* out_splits) {
  if (!ms || M <= 0 || N <= 0 || K <= 0 || K % 8 || N % 8 || mode < 0 || mode > 2 || reps <= 0)
    return set_err(NF_ERR_INVALID_ARG, "nf_probe_gemm_bf16_ms: bad argument");
  if (tile_cfg >= 0 && !((tile_cfg <= 6) || (tile_cfg >= 10 && tile_cfg <= 30 && K % 64 == 0) ||
                         (tile_cfg >= 40 && stream_kc(tile_cfg) > 0 && N % 32 == 0 &&
                          K % (16 * stream_kc(tile_cfg)) == 0 && stream_nbw(tile_cfg) == (mode == GEMM_SWIGLU ? 2 : 1))))
    return set_err(NF_ERR_INVALID_ARG, "nf_probe_gemm_bf16_ms: tile_cfg %d not available for N %d K %d mode %d",
                   tile_cfg, N, K, mode);
  if ((int64_t)std::max(M, N) * K * 2 >= (int64_t(1) << 32))
    return set_err(NF_ERR_OUT_OF_RANGE, "nf_probe_gemm_bf16_ms: an operand would exceed 4 GiB");
  const int64_t nb = mode == GEMM_SWIGLU ? 2 : 1;
  // device buffers and events, released on every return path
  struct Res {
    void *A = nullptr, *Bm = nullptr, *C = nullptr, *R = nullptr, *Bp = nullptr, *ws = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    ~Res() {
      if (e0) (void)hipEventDestroy(e0);
      if (e1) (void)hipEventDestroy(e1);
      for (void* q : {A, Bm, C, R, ws, Bp})
        if (q) (void)hipFree(q);
    }
  } r;
  HIP_TRY(hipMalloc(&r.A, (size_t)M * K * 2));
  HIP_TRY(hipMalloc(&r.Bm, (size_t)nb * N * K * 2));
  HIP_TRY(hipMalloc(&r.C, (size_t)M * N * 2));
  HIP_TRY(hipMalloc(&r.R, (size_t)M * N * 2));
  // activations ~ unit scale, weights uniform with standard deviation 0.02
  HIP_TRY(probe_fill_bf16(r.A, (int64_t)M * K, 1u, 1.0f, nullptr));
  HIP_TRY(probe_fill_bf16(r.Bm, nb * N * K, 2u, 0.0346f, nullptr));
  HIP_TRY(hipMemset(r.R, 0, (size_t)M * N * 2));
  GemmArgs g;
  g.A = r.A; g.lda = K;
  g.B = r.Bm; g.B2 = (char*)r.Bm + (size_t)N * K * 2; g.ldb = K;
  g.C = r.C; g.ldc = N; g.R = r.R; g.ldr = N;
  g.M = M; g.N = N; g.K = K; g.mode = mode;
  if (N % 32 == 0 && K % 16 == 0) {             // operand-order copy for the streaming kernels
    HIP_TRY(hipMalloc(&r.Bp, (size_t)nb * N * K * 2));
    HIP_TRY(pack_b(g.B, K, 0, N, K, 1, r.Bp, (int)nb, 0, 0, nullptr));
    if (nb == 2) HIP_TRY(pack_b(g.B2, K, 0, N, K, 1, r.Bp, 2, 1, 0, nullptr));
    g.Bp = r.Bp;
  }
  GemmPlan p = gemm_choose(g, cus);
  if (tile_cfg >= 0) p.cfg = tile_cfg;
  if (k_splits > 0) p.k_splits = k_splits;
  const size_t wsb = gemm_workspace_bytes(g, p);
  if (wsb) HIP_TRY(hipMalloc(&r.ws, wsb));
  HIP_TRY(hipEventCreate(&r.e0));
  HIP_TRY(hipEventCreate(&r.e1));
  for (int i = 0; i < 3; ++i) HIP_TRY(gemm_bf16(g, p, r.ws, nullptr));
  HIP_TRY(hipEventRecord(r.e0, nullptr));
  for (int i = 0; i < reps; ++i) HIP_TRY(gemm_bf16(g, p, r.ws, nullptr));
  HIP_TRY(hipEventRecord(r.e1, nullptr));
  HIP_TRY(hipEventSynchronize(r.e1));
  float t = 0;
  HIP_TRY(hipEventElapsedTime(&t, r.e0, r.e1));
  *ms = t / reps;
  if (out_cfg) *out_cfg = p.cfg;
  if (out_splits) *out_splits = p.k_splits;
  return NF_OK;
}
