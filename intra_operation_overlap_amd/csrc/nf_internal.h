// Host-side internal interfaces between the C ABI and the kernel launchers.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf_host.h"

namespace nf {

// Kernel timing without marker packets: when the calling thread's timer holds
// two events, the next kernel launched through launch() records its own start
// and end into them (hipExtLaunchKernel), and the timer is cleared.
struct KernelTimer {
  hipEvent_t start = nullptr, stop = nullptr;
};
inline KernelTimer& kernel_timer() {
  static thread_local KernelTimer t;
  return t;
}
template <typename... KArgs, typename... Args>
inline void launch(void (*k)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
  KernelTimer& t = kernel_timer();
  if (t.start) {
    const KernelTimer use = t;
    t = KernelTimer{};
    hipExtLaunchKernelGGL(k, grid, block, shmem, s, use.start, use.stop, 0u, args...);
  } else {
    k<<<grid, block, shmem, s>>>(args...);
  }
}

// Accessors for the serving loop (api.cpp).
const nf_shape* layer_shape(const nf_layer* L);
nf_plan layer_plan(const nf_layer* L);
int32_t pool_pages(const nf_kv_pool* P);
// nf_layer_step with an explicit plan (validated against the batch)
nf_status layer_step_with_plan(nf_layer* L, nf_kv_pool* P, const nf_batch* b, hipStream_t s, const nf_plan& plan);

// ---------------------------------------------------------------- GEMM
// C[M][N] = epilogue(A[M][K] . B[N][K]^T): both operands K-contiguous.
enum GemmMode : int {
  GEMM_STORE = 0,     // C (layer dtype) = acc
  GEMM_RESIDUAL = 1,  // C = R + acc
  GEMM_SWIGLU = 2,    // C[:, n] = silu(A.Bg[n]) * (A.Bu[n]); N counts act columns
  GEMM_F32OUT = 3,    // C (fp32) = acc
};

// A copy of the step's metadata (pinned host staging -> device) done by extra
// blocks of a kernel that runs anyway: n16 16-byte units.
struct MetaCopy {
  const void* src = nullptr;
  void* dst = nullptr;
  int64_t n16 = 0;
};

struct GemmArgs {
  const void* A = nullptr; int64_t lda = 0;
  const void* B = nullptr; const void* B2 = nullptr; int64_t ldb = 0;  // B2: up rows (SWIGLU)
  void* C = nullptr; int64_t ldc = 0;
  const void* R = nullptr; int64_t ldr = 0;
  int M = 0, N = 0, K = 0;
  int mode = GEMM_STORE;
  // grouped GEMM (mixture of experts): group g owns rows group_off[g] ..
  // group_off[g+1]-1 (device array); its B is B + g * b_group_stride.
  const int32_t* group_off = nullptr; int n_groups = 1; int64_t b_group_stride = 0;
  int max_group_rows = 0;                 // bound on any group's rows (grid sizing)
  // optional row gather: A row of output row i is a_rows[i] / a_row_div
  const int32_t* a_rows = nullptr; int a_row_div = 1;
  // split-K only: leave the fp32 partials for the consumer to reduce (no
  // reduce kernel); see gemm_partials
  bool defer_reduce = false;
  // B (B2 interleaved for SWIGLU) packed in MFMA operand order by pack_b
  // (optional; enables the weight-streaming kernels), group stride in elements
  const void* Bp = nullptr; int64_t bp_group_stride = 0;
  // LDS-pipelined configurations (10..31) only: extra blocks after the tiles
  // also do this copy (meta.n16 == 0: none)
  MetaCopy meta;
};

struct GemmPlan {
  int cfg = 0;        // tile configuration id
  int k_splits = 1;   // split-K factor (fp32 partials + reduce)
};

// Chooses a tile configuration and split-K for a problem given the number of
// CUs its stream may use.  `coresident`: attention waves share every CU with
// the GEMM, so only tiles that leave registers and LDS for them are chosen
// (128 x 128 tiles, two workgroups per CU: 146 registers per lane and 64 KB
// of LDS each, against the 512 registers per SIMD lane and 160 KB of a CU).
GemmPlan gemm_choose(const GemmArgs& a, int cus, bool coresident = false);
// Workspace bytes the split-K path needs for this problem/plan.
size_t gemm_workspace_bytes(const GemmArgs& a, const GemmPlan& p);
// Called between the main kernel and the split-K reduce (phase 1) so callers
// can bracket each kernel on its stream.
struct LaunchHook {
  void (*fn)(void* ctx, int phase) = nullptr;
  void* ctx = nullptr;
};
// Launches (1 kernel, or 2 with split-K).  `ws` must hold gemm_workspace_bytes.
hipError_t gemm_bf16(const GemmArgs& a, const GemmPlan& p, void* ws, hipStream_t s,
                     const LaunchHook* hook = nullptr);
hipError_t gemm_f32(const GemmArgs& a, hipStream_t s);
// Sum of `splits` fp32 partial slices (M x part_ld each) plus the mode's
// epilogue, written to C.
hipError_t splitk_reduce(const GemmArgs& a, const float* part, int64_t part_ld, int splits, hipStream_t s);
// Weight-streaming kernels (tile configurations 40..51; need a.Bp).
hipError_t gemm_stream(const GemmArgs& a, const GemmPlan& p, void* ws, hipStream_t s, const LaunchHook* hook);
int stream_kc(int cfg);   // k-steps (of 16) per A chunk of a streaming configuration, 0 if none
int stream_nbw(int cfg);  // packed n-blocks per wave (2: SwiGLU gate + up), 0 if none
// Packs W [groups][N][K] (row stride ldw, group stride group_stride; N % 32 ==
// 0, K % 16 == 0) into 1 KB operand blocks (32 rows x 16 k); source n-block b
// becomes packed n-block b * nb_stride + nb_offset (gate/up interleave: 2, 0/1).
hipError_t pack_b(const void* W, int64_t ldw, int64_t group_stride, int N, int K, int groups, void* P,
                  int nb_stride, int nb_offset, int64_t packed_group_stride, hipStream_t s);
// Number of fp32 partial slices a split-K launch of this problem writes to
// its workspace (1: no split, the epilogue writes C).  Slice z starts at
// z * M * part_ld floats; rows have stride part_ld = N (2N for SWIGLU).
int gemm_partials(const GemmArgs& a, const GemmPlan& p);

// ---------------------------------------------------------------- row ops
// Copy of a step's metadata (16-byte units) from device-visible pinned host
// memory, done by extra blocks of the first kernel of a step.
hipError_t rmsnorm(int dtype, const void* x, const void* g, void* y, int T, int H, float eps, hipStream_t s,
                   const MetaCopy* mc = nullptr);

struct RopeAppendArgs {
  const void* qkv;          // [T][(nq+2nkv)d]
  void* q_rot;              // [T][nq*d]
  void* k_pool; void* v_pool;
  const int32_t* pos;       // device [T]
  const int32_t* tok_req;   // device [T]
  const int32_t* page_indptr; const int32_t* page_indices;
  const float* cos_sin;     // [max_pos][d/2][2]
  int T, nq, nkv, d, page_size;
  // splits > 1: qkv is not written yet; each value is the rounded sum of
  // `splits` fp32 partial slices (zstride floats apart, row stride part_ld),
  // which this kernel also stores to qkv
  const float* part = nullptr; int64_t part_ld = 0, zstride = 0; int splits = 1;
  // bf16: the attention RMSNorm folded in.  The QKV GEMM ran on x against
  // weights with the norm gain applied to their columns; each token's q, k
  // and v are multiplied by its 1 / RMS (row_scale[t]) before the rotation
  const float* row_scale = nullptr;
};
hipError_t rope_append(int dtype, const RopeAppendArgs& a, hipStream_t s);
// bf16, H % 8 == 0: s[t] = 1 / sqrt(mean(x[t]^2) + eps), with the sum of
// squares of rmsnorm (same threads, chunks and order); carries `mc` like rmsnorm
hipError_t row_rms_scale(const void* x, float* s, int T, int H, float eps, hipStream_t st, const MetaCopy* mc);
// bf16 [N][K] (K % 8 == 0): out[n][k] = round(w[n][k] * g[k])
hipError_t scale_cols_bf16(const void* w, const void* g, void* out, int64_t N, int K, hipStream_t s);
// bf16, H % 8 == 0: x1 = round(sum of `splits` split-K partial slices + x),
// then y = RMSNorm(x1) * g, in one kernel; bit-identical to the split-K
// reduce (residual epilogue) followed by rmsnorm.
hipError_t residual_rmsnorm_partials(const float* part, int64_t part_ld, int64_t zstride, int splits,
                                     const void* x, int64_t ldx, void* x1, int64_t ldx1, const void* g, void* y,
                                     int T, int H, float eps, hipStream_t s);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  const void* q_rot;        // [T][nq*d]
  const void* k_pool; const void* v_pool;
  void* attn;               // [T][nq*d]
  float* part_o;            // [n_partials][nkv][16][d]   (unnormalised)
  float* part_ml;           // [n_partials][nkv][16][2]   (max, sum)
  const AttnItem* items; int n_items;
  const MergeItem* merges; int n_merges;
  const int32_t* pos;       // device [T]
  const int32_t* page_indptr; const int32_t* page_indices;
  int nq, nkv, d, page_size;
  float scale;
  int variant = 0;          // bf16 d=128: 0 one wave per item, 1 four waves per item
  int max_blocks = 0;       // > 0 caps the grid (workgroups); each then loops over items
};
hipError_t attention(int dtype, const AttnArgs& a, hipStream_t s);
hipError_t attention_merge(int dtype, const AttnArgs& a, hipStream_t s);

// ---------------------------------------------------------------- MoE
struct RouteArgs {
  const float* logits;      // [T][E]
  int32_t* idx;             // [T][k]
  float* w;                 // [T][k]
  int32_t* perm;            // [T*k] assignment ids sorted by expert
  int32_t* inv;             // [T*k] position of assignment a in perm
  int32_t* offsets;         // [E+1]
  int T, E, k;
};
hipError_t moe_route(const RouteArgs& a, hipStream_t s);
// out[t] = x1[t] + sum_s w[t][s] * y[inv[t*k+s]]
hipError_t moe_combine(int dtype, const void* x1, const float* y, const float* w,
                       const int32_t* inv, void* out, int T, int H, int k, hipStream_t s);

// pool pages pages[0..n) (pages null: 0..n-1) <-> row-major [n][nkv][16][d]
// buffers k_rm / v_rm (to_pool: row-major -> pool); dtype 1 bf16, 0 fp32
hipError_t kv_convert(int dtype, void* k_pool, void* v_pool, const int32_t* pages, int n, int nkv, int d, void* k_rm,
                      void* v_rm, bool to_pool, hipStream_t s);
// copies pool pages pages[0..n) (K and V, block_bytes each) to dst_k / dst_v in list order
hipError_t kv_gather(const void* k_pool, const void* v_pool, const int32_t* pages, int n, int64_t block_bytes,
                     void* dst_k, void* dst_v, hipStream_t s);
// serving loop: x[t] = row at src[t]; then *dst[t] = out[t] and flag[t] =
// (out[t][0] > thr) (src, dst, flag: host-mapped pinned memory)
hipError_t loop_gather(const uint64_t* src, void* x, int T, int64_t row_bytes, hipStream_t s);
hipError_t loop_scatter(int dtype, const void* out, const uint64_t* dst, int T, int H, float thr, int32_t* flag,
                        hipStream_t s);
// copy of `bytes` (multiple of 16, 16-byte aligned) by a kernel of `wgs` workgroups
hipError_t copy_rows(const void* src, void* dst, size_t bytes, int wgs, hipStream_t s);
// the inverse: block i of src_k / src_v to pool page pages[i] (pages distinct)
hipError_t kv_scatter(void* k_pool, void* v_pool, const int32_t* pages, int n, int64_t block_bytes, const void* src_k,
                      const void* src_v, hipStream_t s);

// ---------------------------------------------------------------- probes
// shape 0: v_mfma_f32_16x16x32_bf16 (8 chains), 1: v_mfma_f32_32x32x16_bf16 (4 chains)
hipError_t probe_mfma(int shape, int n_blocks, int iters, float* sink, hipStream_t s);
hipError_t probe_read(const void* buf, size_t bytes, float* sink, int n_blocks, hipStream_t s);
// out[2*b] = HW_ID, out[2*b+1] = XCC_ID of workgroup b
hipError_t probe_hwid(uint32_t* out, int n_blocks, hipStream_t s);
hipError_t probe_fill_bf16(void* p, int64_t n, uint32_t seed, float scale, hipStream_t s);

}  // namespace nf
