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

// On a HIP failure the runtime's last-error slot is cleared so that the
// caller's next unrelated HIP call does not report it again.
#define HIP_TRY(expr)                                                                     \
  do {                                                                                    \
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

struct nf_layer {
  nf_shape s{};
  nf_weights w{};
  int device = 0;
  int n_cus = 0, n_xcd = 8, cus_per_xcd = 32;
  std::vector<int> xcc_of_bit;                  // CU-mask bit -> XCD (measured)
  nf_plan plan{};
  std::map<std::pair<int, int>, StreamPair> pairs;   // by (GEMM CUs, attention CUs) per XCD
  hipEvent_t ev_app[NF_MAX_NANO] = {}, ev_att[NF_MAX_NANO] = {};
  hipEvent_t ev_start = nullptr, ev_g = nullptr, ev_a = nullptr;
  DevBuf h, qkv, q_rot, attn, x1, h2, act, y;
  DevBuf r_idx, r_w, r_perm, r_inv, r_off;
  DevBuf splitk, part_o, part_ml, meta, cos_sin;
  DevBuf stack_out;                             // this layer's output inside a multi-layer step
  // expert weights in MFMA operand order for the weight-streaming kernels
  // (bf16 mixture-of-experts layers; empty otherwise)
  DevBuf wp_qkv, wp_o, wp_gu, wp_down;
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
};

struct nf_kv_pool {
  const nf_layer* layer = nullptr;
  int device = 0;
  int32_t n_pages = 0, page_size = 0;
  int64_t block_bytes = 0;   // one page's K (or V) block: n_kv_heads x page_size x head_dim elements
  void* k = nullptr;
  void* v = nullptr;
  DevBuf offload;      // page list and gathered K / V blocks of nf_kv_offload
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
std::mutex g_map_mu;
std::map<int, std::vector<int>> g_xcc_maps;     // device -> bit -> XCD

// Which XCD each CU-mask bit lands on.  The driver stripes mask bits over
// the XCDs (bit i -> XCD i % n_xcd, CU i / n_xcd within it), and a mask must
// leave every XCD at least one CU (workgroups are dealt to XCDs round-robin
// whatever the mask).  The striping is checked with a stream masked to bits
// 0 .. n_xcd-1 -- one CU per XCD if striped -- running many single-wave
// workgroups that report their XCC_ID: every XCD must show up.  If it does
// not, the bits stay -1 (unknown) and splits still use the striped guess.
nf_status measure_cu_map(int device, int n_cus, int n_xcd, std::vector<int>& out) {
  std::lock_guard<std::mutex> lk(g_map_mu);
  auto it = g_xcc_maps.find(device);
  if (it != g_xcc_maps.end()) {
    out = it->second;
    return NF_OK;
  }
  constexpr int kBlocks = 256;
  std::vector<int> map(n_cus, -1);
  const int words = (n_cus + 31) / 32;
  std::vector<uint32_t> mask(words, 0u);
  for (int bit = 0; bit < n_xcd && bit < n_cus; ++bit) mask[bit / 32] |= 1u << (bit % 32);
  uint32_t* d_id = nullptr;
  HIP_TRY(hipMalloc(&d_id, 2 * kBlocks * sizeof(uint32_t)));
  hipStream_t st = nullptr;
  hipError_t e = hipExtStreamCreateWithCUMask(&st, words, mask.data());
  std::vector<uint32_t> h_id(2 * kBlocks, 0xFFFFFFFFu);
  if (e == hipSuccess) {
    e = probe_hwid(d_id, kBlocks, st);
    if (e == hipSuccess) e = hipMemcpyAsync(h_id.data(), d_id, h_id.size() * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    (void)hipStreamDestroy(st);
  }
  (void)hipGetLastError();
  (void)hipFree(d_id);
  if (e == hipSuccess) {
    std::vector<int> seen(16, 0);
    for (int b = 0; b < kBlocks; ++b) seen[h_id[2 * b + 1] & 0xF] = 1;
    int n_seen = 0;
    for (int x = 0; x < 16; ++x) n_seen += seen[x];
    if (n_seen == n_xcd)
      for (int bit = 0; bit < n_cus; ++bit) map[bit] = bit % n_xcd;
  }
  g_xcc_maps[device] = map;
  out = map;
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

nf_status get_pair(nf_layer* L, int g, int a, StreamPair& out) {
  const int ab = attn_budget(g, a, L->cus_per_xcd);
  auto key = std::make_pair(g, ab);
  auto it = L->pairs.find(key);
  if (it != L->pairs.end()) {
    out = it->second;
    return NF_OK;
  }
  if ((g || ab) && L->xcc_of_bit.empty()) {
    nf_status st = measure_cu_map(L->device, L->n_cus, L->n_xcd, L->xcc_of_bit);
    if (st != NF_OK) return st;
  }
  StreamPair p;
  std::vector<uint32_t> m;
  if (g == 0) {
    HIP_TRY(hipStreamCreateWithFlags(&p.g, hipStreamNonBlocking));
  } else {
    make_mask(L->xcc_of_bit, L->n_xcd, 0, g, m);
    HIP_TRY(hipExtStreamCreateWithCUMask(&p.g, (uint32_t)m.size(), m.data()));
  }
  if (ab == 0) {
    HIP_TRY(hipStreamCreateWithFlags(&p.a, hipStreamNonBlocking));
  } else {
    make_mask(L->xcc_of_bit, L->n_xcd, L->cus_per_xcd - ab, L->cus_per_xcd, m);
    HIP_TRY(hipExtStreamCreateWithCUMask(&p.a, (uint32_t)m.size(), m.data()));
  }
  L->pairs[key] = p;
  out = p;
  return NF_OK;
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
  int attn_waves_per_cu;
  int attn_variant;        // 0: one-wave work items (any grid), 1: four-wave workgroups
  // the step's metadata copy rides on the first front's RMSNorm; the event
  // marks the end of its reads from the pinned staging buffer
  MetaCopy mc;
  bool mc_pending;
  hipEvent_t mc_event;
};

char* ptr(const DevBuf& b, int64_t elems, int dt) { return (char*)b.p + elems * (int64_t)dtype_bytes(dt); }

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
  GemmPlan gp = gemm_choose(g, c.gemm_cus);
  if (partials) {
    *partials = gemm_partials(g, gp);
    g.defer_reduce = *partials > 1;
  }
  Prof pctx{L, kind, s};
  LaunchHook hook{prof_hook_fn, &pctx};
  prof_begin(L, kind, s);
  hipError_t e = gemm_bf16(g, gp, L->splitk.p, s, L->prof ? &hook : nullptr);
  prof_end(L, pctx.kind, s);
  return e;
}

size_t gemm_ws_need(const StepCtx& c, GemmArgs g) {
  if (c.L->s.dtype == NF_F32) return 0;
  return gemm_workspace_bytes(g, gemm_choose(g, c.gemm_cus));
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
  q.A = ptr(L->h, (int64_t)t0 * H, dt); q.lda = H;
  q.B = L->w.w_qkv; q.ldb = H; q.Bp = L->wp_qkv.p;
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
    d.C = (char*)c.b->out + (int64_t)t0 * H * dtype_bytes(dt); d.ldc = H;
    d.R = ptr(L->x1, (int64_t)t0 * H, dt); d.ldr = H;
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
    const int cfg = gemm_choose(g.qkv, c.gemm_cus).cfg;
    return cfg >= 10 && cfg <= 30 && g.qkv.K % 64 == 0;
  }();
  prof_begin(L, K_NORM1, s);
  HIP_STEP(rmsnorm(dt, (const char*)c.b->x + (int64_t)t0 * H * dtype_bytes(dt), L->w.attn_norm,
                   ptr(L->h, (int64_t)t0 * H, dt), Tj, H, sh.rms_eps, s,
                   c.mc_pending && !meta_in_gemm ? &c.mc : nullptr));
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
    r.part = (const float*)L->splitk.p;
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
  a.max_blocks = c.attn_waves_per_cu > 0 ? c.attn_waves_per_cu * c.attn_cus : 0;
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

nf_status issue_back(StepCtx& c, int j, hipStream_t s) {
  nf_layer* L = c.L;
  const nf_shape& sh = L->s;
  const NanoWork& nw = L->work.nanos[j];
  const int t0 = nw.t0, Tj = nw.t1 - nw.t0, dt = sh.dtype, H = sh.hidden;
  if (Tj == 0) return NF_OK;
  NanoGemms g = nano_gemms(c, j, nw.t0, nw.t1);
  const bool fuse = dt == NF_BF16 && H % 8 == 0;
  int o_parts = 1;
  HIP_STEP(run_gemm(c, g.o, K_OPROJ, s, fuse ? &o_parts : nullptr));
  prof_begin(L, K_NORM2, s);
  if (o_parts > 1)              // O-projection split-K reduce + residual + FFN norm in one kernel
    HIP_STEP(residual_rmsnorm_partials((const float*)L->splitk.p, H, (int64_t)Tj * H, o_parts, g.o.R, g.o.ldr,
                                       g.o.C, g.o.ldc, L->w.ffn_norm, ptr(L->h2, (int64_t)t0 * H, dt), Tj, H,
                                       sh.rms_eps, s));
  else
    HIP_STEP(rmsnorm(dt, ptr(L->x1, (int64_t)t0 * H, dt), L->w.ffn_norm, ptr(L->h2, (int64_t)t0 * H, dt), Tj, H,
                     sh.rms_eps, s));
  prof_end(L, K_NORM2, s);
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
  HIP_STEP(gemm_bf16(g.moe_gu, gemm_choose(g.moe_gu, c.gemm_cus), L->splitk.p, s));
  prof_end(L, K_MOE_GATEUP, s);
  prof_begin(L, K_MOE_DOWN, s);
  HIP_STEP(gemm_bf16(g.moe_down, gemm_choose(g.moe_down, c.gemm_cus), L->splitk.p, s));
  prof_end(L, K_MOE_DOWN, s);
  prof_begin(L, K_COMBINE, s);
  HIP_STEP(moe_combine(dt, ptr(L->x1, (int64_t)t0 * H, dt), (const float*)L->y.p + (int64_t)t0 * k * H,
                       r.w, r.inv, (char*)c.b->out + (int64_t)t0 * H * dtype_bytes(dt), Tj, H, k, s));
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
  c.attn_waves_per_cu = two ? plan.attn_waves_per_cu : 0;
  // attention work items: a four-wave workgroup each (fastest when attention
  // has the whole chip), or one wave each (many short items) when the plan
  // asks for a persistent attention grid that leaves room for GEMM waves
  c.attn_variant = L->attn_variant >= 0 ? L->attn_variant : (c.attn_waves_per_cu > 0 ? 0 : 1);
  if (c.attn_waves_per_cu > 0) c.attn_variant = 0;
  const bool wave_items = L->s.dtype == NF_BF16 && L->s.head_dim == 128 && c.attn_variant == 0;
  build_work(L->s, *b, plan, P->page_size, wave_items ? 8 * c.attn_cus : 2 * c.attn_cus, 8,
             wave_items ? 32 : 0, L->work);
  const StepWork& w = L->work;
  r.count = (int)w.nanos.size();

  // workspace the GEMMs and the split attention items need (before any launch)
  size_t ws = 0;
  for (int j = 0; j < r.count; ++j) {
    NanoGemms g = nano_gemms(c, j, w.nanos[j].t0, w.nanos[j].t1);
    if (L->s.n_experts == 1)
      for (const GemmArgs* a : {&g.qkv, &g.o, &g.gu, &g.down}) ws = std::max(ws, gemm_ws_need(c, *a));
    else
      for (const GemmArgs* a : {&g.qkv, &g.o, &g.moe_gu, &g.moe_down}) ws = std::max(ws, gemm_ws_need(c, *a));
  }
  HIP_TRY(ensure(L->splitk, ws));
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
// GEMM stream.
struct Streams {
  bool two = false;
  hipStream_t caller = nullptr, sg = nullptr, sa = nullptr;
};

nf_status open_streams(nf_layer* L, const nf_plan& plan, hipStream_t caller, Streams& S) {
  S.two = plan.n_streams == 2;
  S.caller = S.sg = S.sa = caller;
  if (!S.two) return NF_OK;
  StreamPair pr;
  nf_status st = get_pair(L, plan.gemm_cus_per_xcd, plan.attn_cus_per_xcd, pr);
  if (st != NF_OK) return st;
  S.sa = pr.a;
  if (plan.gemm_cus_per_xcd) {
    S.sg = pr.g;
    HIP_TRY(hipEventRecord(L->ev_start, caller));
    HIP_TRY(hipStreamWaitEvent(S.sg, L->ev_start, 0));
  }
  return NF_OK;
}

nf_status close_streams(nf_layer* L, const Streams& S) {
  if (S.two && S.sg != S.caller) {
    HIP_TRY(hipEventRecord(L->ev_g, S.sg));
    HIP_TRY(hipStreamWaitEvent(S.caller, L->ev_g, 0));
  }
  return NF_OK;
}

// front (norm, QKV, RoPE/append) of nano-batch j and its attention
nf_status issue_front_attn(LayerRun& r, const Streams& S, int j) {
  nf_layer* L = r.L;
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

// back (O-projection, norm, FFN or experts) of nano-batch j
nf_status issue_back_after_attn(LayerRun& r, const Streams& S, int j) {
  if (S.two) HIP_TRY(hipStreamWaitEvent(S.sg, r.L->ev_att[j], 0));
  return issue_back(r.c, j, S.sg);
}

// one layer's launches in the plan's order
nf_status issue_layer(LayerRun& r, const Streams& S, int order) {
  nf_status st;
  if (order == NF_ORDER_PIPELINED) {
    if ((st = issue_front_attn(r, S, 0)) != NF_OK) return st;
    for (int j = 0; j < r.count; ++j) {
      if (j + 1 < r.count && (st = issue_front_attn(r, S, j + 1)) != NF_OK) return st;
      if ((st = issue_back_after_attn(r, S, j)) != NF_OK) return st;
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
  if ((st = open_streams(L, plan, caller, S)) != NF_OK) return st;
  if ((st = issue_layer(r, S, plan.order)) != NF_OK) return st;
  return close_streams(L, S);
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
        sl.n_experts != s0.n_experts || layers[l]->device != layers[0]->device)
      return set_err(NF_ERR_INVALID_ARG, "stack: layer %d differs from layer 0 in hidden size, dtype, "
                     "max_tokens, experts or device", l);
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
  if ((st = open_streams(layers[0], layers[0]->plan, caller, S)) != NF_OK) return st;
  if ((st = issue_stack(runs, S, layers[0]->plan.order)) != NF_OK) return st;
  return close_streams(layers[0], S);
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

  const int dt = s->dtype;
  const size_t eb = dtype_bytes(dt);
  const int64_t Tm = s->max_tokens, H = s->hidden, F = s->ffn, k = s->top_k;
  const int64_t nqd = (int64_t)s->n_q_heads * s->head_dim;
  const int64_t Nqkv = (int64_t)(s->n_q_heads + 2 * s->n_kv_heads) * s->head_dim;
  struct {
    DevBuf* b;
    size_t bytes;
  } allocs[] = {
      {&L->h, Tm * H * eb},          {&L->qkv, Tm * Nqkv * eb}, {&L->q_rot, Tm * nqd * eb},
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
                    &L->r_perm, &L->r_inv, &L->r_off, &L->splitk, &L->part_o, &L->part_ml, &L->meta, &L->cos_sin,
                    &L->wp_qkv, &L->wp_o, &L->wp_gu, &L->wp_down, &L->stack_out})
    release(*b);
  for (int i = 0; i < 2; ++i) {
    if (L->stage[i]) (void)hipHostFree(L->stage[i]);
    if (L->stage_ev[i]) (void)hipEventDestroy(L->stage_ev[i]);
  }
  for (int j = 0; j < NF_MAX_NANO; ++j) {
    if (L->ev_app[j]) (void)hipEventDestroy(L->ev_app[j]);
    if (L->ev_att[j]) (void)hipEventDestroy(L->ev_att[j]);
  }
  for (hipEvent_t e : {L->ev_start, L->ev_g, L->ev_a})
    if (e) (void)hipEventDestroy(e);
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
  if (p->offload.p || !p->offload.old.empty()) {   // the layer may be gone already
    (void)hipSetDevice(p->device);
    (void)hipDeviceSynchronize();
    release(p->offload);
  }
  delete p;
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

nf_status nf_layer_step(nf_layer* L, nf_kv_pool* P, const nf_batch* b, void* stream) {
  if (!L || !P || !b) return set_err(NF_ERR_INVALID_ARG, "nf_layer_step: null argument");
  if (P->layer != L) return set_err(NF_ERR_INVALID_ARG, "nf_layer_step: pool belongs to another layer");
  return step_impl(L, P, b, (hipStream_t)stream, L->plan);
}

nf_status nf_stack_step(nf_layer* const* layers, nf_kv_pool* const* pools, int32_t n_layers, const nf_batch* batch,
                        void* stream) {
  nf_status st = check_stack(layers, pools, n_layers, batch);
  if (st != NF_OK) return st;
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
  for (int l = 0; l < n_layers; ++l)
    if (layers[l]->prof) return set_err(NF_ERR_UNSUPPORTED, "nf_stack_graph_create: per-kernel timing is on");
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

nf_status nf_probe_cu_map(int32_t* xcc, int32_t n) {
  if (!xcc || n <= 0) return set_err(NF_ERR_INVALID_ARG, "nf_probe_cu_map: bad argument");
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, dev));
  std::vector<int> map;
  nf_status st = measure_cu_map(dev, prop.multiProcessorCount, 8, map);
  if (st != NF_OK) return st;
  for (int i = 0; i < n; ++i) xcc[i] = i < (int)map.size() ? map[i] : -1;
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
// CU split) for one batch; replaces the pages' MILP-based parameter search
// ("Search Space 4D" card on the do-not-panic NanoFlow page; Gurobi note on
// the ossradar page).  Every candidate is timed on the device with this batch.
namespace {

struct Cand {
  nf_plan plan;
  double ms = 0;
};

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
  if (T == 0) {
    *out = nf_plan{1, {0, 0, 0, 0}, NF_ORDER_PIPELINED, 1, 0, 0, 0};
    L->plan = *out;
    return NF_OK;
  }

  // candidate grid over the four plan dimensions
  std::vector<Cand> cands;
  const nf_plan base{1, {T, 0, 0, 0}, NF_ORDER_PIPELINED, 1, 0, 0, 0};
  cands.push_back({base});
  struct Split { int g, a, w; };
  const Split splits[] = {{0, 0, 0}, {0, 0, 4}, {0, 24, 0}, {16, 16, 0}, {20, 12, 0}, {24, 8, 0}};
  for (int k = 2; k <= opts.max_count && k <= T; ++k) {
    nf_plan eq = base, bal = base;
    eq.count = bal.count = k;
    for (int j = 0; j < k; ++j) eq.sizes[j] = T / k + (j < T % k ? 1 : 0);
    balanced_sizes(b, k, bal.sizes);
    for (const nf_plan& pz : {eq, bal}) {
      cands.push_back({pz});                      // split, one stream
      for (const Split& sp : splits) {
        if (sp.g >= L->cus_per_xcd || sp.a >= L->cus_per_xcd) continue;
        nf_plan c = pz;
        c.n_streams = 2;
        c.gemm_cus_per_xcd = sp.g;
        c.attn_cus_per_xcd = sp.a;
        c.attn_waves_per_cu = sp.w;
        cands.push_back({c});
      }
    }
  }

  hipEvent_t e0, e1;
  HIP_TRY(hipEventCreate(&e0));
  HIP_TRY(hipEventCreate(&e1));
  auto measure = [&](Cand& c, int warm, int reps) -> nf_status {
    nf_status st = NF_OK;
    for (int w = 0; w < warm && st == NF_OK; ++w) st = step_impl(L, P, b, s, c.plan);
    if (st != NF_OK) return st;
    HIP_TRY(hipEventRecord(e0, s));
    for (int r = 0; r < reps && st == NF_OK; ++r) st = step_impl(L, P, b, s, c.plan);
    HIP_TRY(hipEventRecord(e1, s));
    HIP_TRY(hipEventSynchronize(e1));
    if (st != NF_OK) return st;
    float ms = 0;
    HIP_TRY(hipEventElapsedTime(&ms, e0, e1));
    c.ms = ms / reps;
    return NF_OK;
  };
  // stage 1: every candidate, briefly (after a few steps of the unsplit plan,
  // so that the first candidate does not pay for clocks ramping up or
  // first-use allocations); stage 2: the top_k and the unsplit plan again,
  // longer
  nf_status st = NF_OK;
  {
    Cand warm{base};
    st = measure(warm, 3, 1);
  }
  for (Cand& c : cands) {
    if (st != NF_OK) break;
    st = measure(c, 1, 2);
  }
  std::vector<Cand> top;
  if (st == NF_OK) {
    const Cand unsplit = cands[0];
    std::stable_sort(cands.begin(), cands.end(), [](const Cand& x, const Cand& y) { return x.ms < y.ms; });
    top.assign(cands.begin(), cands.begin() + std::min<size_t>(cands.size(), opts.top_k));
    bool has_unsplit = false;
    for (const Cand& c : top) has_unsplit = has_unsplit || (c.plan.count == 1 && c.plan.n_streams == 1);
    if (!has_unsplit) top.push_back(unsplit);
    for (Cand& c : top) {
      const double quick = c.ms;
      if ((st = measure(c, opts.warmup, opts.reps)) != NF_OK) break;
      if (std::getenv("NF_SEARCH_VERBOSE")) {
        const nf_plan& q = c.plan;
        std::fprintf(stderr,
                     "nf search: count %d sizes %d/%d/%d/%d streams %d cus/xcd gemm %2d attn %2d waves %d -> %.3f ms "
                     "(first pass %.3f)\n",
                     q.count, q.sizes[0], q.sizes[1], q.sizes[2], q.sizes[3], q.n_streams, q.gemm_cus_per_xcd,
                     q.attn_cus_per_xcd, q.attn_waves_per_cu, c.ms, quick);
      }
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != NF_OK) return st;
  int best = 0;
  for (size_t i = 1; i < top.size(); ++i)
    if (top[i].ms < top[best].ms) best = (int)i;
  if (times_ms) {
    times_ms[0] = top[best].ms;
    times_ms[1] = cands.empty() ? 0 : (double)cands.size();
  }
  L->plan = top[best].plan;
  *out = top[best].plan;
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
