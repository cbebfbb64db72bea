// Row-wise operations of the decoder layer: RMSNorm, rotary embedding fused
// with the paged KV-cache append, and the mixture-of-experts router and
// combine.  All are HBM-bound and small next to the GEMMs and attention.
#include "nf_device.h"
#include "nf_internal.h"

namespace nf {
namespace {

// ---------------------------------------------------------------- RMSNorm
// y = x / sqrt(mean(x^2) + eps) * g, one 256-thread block per row, fp32 math.
// Blocks past the last row copy the step's metadata instead (see MetaCopy).
__device__ __forceinline__ bool meta_copy_block(const MetaCopy& mc, int rows) {
  if ((int)blockIdx.x < rows) return false;
  const u32x4* src = (const u32x4*)mc.src;
  u32x4* dst = (u32x4*)mc.dst;
  const int64_t nb = gridDim.x - rows;
  for (int64_t i = (int64_t)(blockIdx.x - rows) * blockDim.x + threadIdx.x; i < mc.n16; i += nb * blockDim.x)
    dst[i] = src[i];
  return true;
}

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* __restrict__ x, const T* __restrict__ g,
                                                      T* __restrict__ y, int H, float eps, MetaCopy mc, int rows) {
  if (meta_copy_block(mc, rows)) return;
  const int64_t row = blockIdx.x;
  const T* xr = x + row * H;
  T* yr = y + row * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += 256) {
    const float v = to_f32(xr[i]);
    ss += v * v;
  }
  __shared__ float red[4];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float total = red[0] + red[1] + red[2] + red[3];
  const float inv = rsqrtf(total / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += 256)
    yr[i] = from_f32<T>(to_f32(xr[i]) * inv * to_f32(g[i]));
}

// bf16 rows, 8 elements (16 bytes) per access; requires H % 8 == 0.
// bf16 RMSNorms run one row per block of RN_THREADS threads.  A decode batch
// has few rows (one block each) and the fused norm below reads all of a row's
// split-K slices, so twice the usual threads keep twice the loads in flight per
// CU.  Both kernels share the size, the thread-to-chunk mapping and the order
// of the sum of squares, and the size does not depend on the batch, so every
// plan rounds the norm alike.
constexpr int RN_THREADS = 512;

// Sum of squares of a block's threads, added wave by wave in a fixed order.
__device__ __forceinline__ float block_sum_sq(float ss) {
  constexpr int NW = RN_THREADS / 64;
  __shared__ float red[NW];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) tot += red[w];
  return tot;
}

__global__ __launch_bounds__(RN_THREADS) void rmsnorm_bf16x8_kernel(const bf16* __restrict__ x,
                                                             const bf16* __restrict__ g,
                                                             bf16* __restrict__ y, int H, float eps, MetaCopy mc,
                                                             int rows) {
  if (meta_copy_block(mc, rows)) return;
  const int64_t row = blockIdx.x;
  const bf16x8* xr = (const bf16x8*)(x + row * H);
  const bf16x8* gr = (const bf16x8*)g;
  bf16x8* yr = (bf16x8*)(y + row * H);
  const int n8 = H / 8;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n8; i += RN_THREADS) {
    const bf16x8 v = xr[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += (float)v[e] * (float)v[e];
  }
  const float inv = rsqrtf(block_sum_sq(ss) / (float)H + eps);
  for (int i = threadIdx.x; i < n8; i += RN_THREADS) {
    const bf16x8 v = xr[i], w = gr[i];
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)v[e] * inv * (float)w[e]);
    yr[i] = o;
  }
}

// Split-K reduce of the O-projection (residual epilogue) fused with the FFN
// RMSNorm: x1 = round(sum_z partial_z + x) is stored, then y = RMSNorm(x1) * g.
// Same thread-to-chunk mapping and summation order as splitk_reduce_kernel
// followed by rmsnorm_bf16x8_kernel, so the result is bit-identical.
__global__ __launch_bounds__(RN_THREADS) void residual_rmsnorm_partials_kernel(
    const float* __restrict__ part, int64_t part_ld, int64_t zstride, int splits, const bf16* __restrict__ x,
    int64_t ldx, bf16* __restrict__ x1, int64_t ldx1, const bf16* __restrict__ g, bf16* __restrict__ y, int H,
    float eps) {
  const int64_t row = blockIdx.x;
  const int n8 = H / 8;
  const float* P = part + row * part_ld;
  const bf16x8* xr = (const bf16x8*)(x + row * ldx);
  bf16x8* x1r = (bf16x8*)(x1 + row * ldx1);
  float ss = 0.f;
  for (int i = threadIdx.x; i < n8; i += RN_THREADS) {
    const f32x4 lo = sum_slices<f32x4>(P + 8 * i, zstride, splits);
    const f32x4 hi = sum_slices<f32x4>(P + 8 * i + 4, zstride, splits);
    const bf16x8 r = xr[i];
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a0 = lo[e], a1 = hi[e];
      a0 += (float)r[e];
      a1 += (float)r[e + 4];
      o[e] = (bf16)a0;
      o[e + 4] = (bf16)a1;
    }
    x1r[i] = o;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += (float)o[e] * (float)o[e];
  }
  const float inv = rsqrtf(block_sum_sq(ss) / (float)H + eps);
  const bf16x8* gr = (const bf16x8*)g;
  bf16x8* yr = (bf16x8*)(y + row * H);
  for (int i = threadIdx.x; i < n8; i += RN_THREADS) {
    const bf16x8 v = x1r[i], w = gr[i];
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)v[e] * inv * (float)w[e]);
    yr[i] = o;
  }
}

// ---------------------------------------------------------------- RoPE + append
// Grid (token, head group): each block takes 256 / (d/2) heads of one token,
// one thread per rotation pair (j, j + d/2).  Q heads are rotated into q_rot;
// K heads are rotated and written to the K pool at (page of the position,
// slot); V heads are copied to the V pool (both pools in the attention
// kernel's MFMA-operand block order).  Pair j turns by p * theta^(-2j/d).
template <typename T>
__global__ __launch_bounds__(256) void rope_append_kernel(RopeAppendArgs a) {
  const int t = blockIdx.x;
  const int d = a.d, half = d / 2;
  const int hpb = 256 / half;
  const int head = blockIdx.y * hpb + threadIdx.x / half;
  const int j = threadIdx.x % half;
  if (threadIdx.x >= hpb * half || head >= a.nq + 2 * a.nkv) return;
  const int p = a.pos[t];
  const int r = a.tok_req[t];
  const int ncols = (a.nq + 2 * a.nkv) * d;
  T v0, v1;
  if (a.splits > 1) {           // reduce the QKV GEMM's split-K partials here
    const float* P = a.part + (int64_t)t * a.part_ld + (int64_t)head * d + j;
    const float s0 = sum_slices<float>(P, a.zstride, a.splits);
    const float s1 = sum_slices<float>(P + half, a.zstride, a.splits);
    v0 = from_f32<T>(s0);
    v1 = from_f32<T>(s1);
    T* out = (T*)a.qkv + (int64_t)t * ncols + (int64_t)head * d;
    out[j] = v0;
    out[j + half] = v1;
  } else {
    const T* row = (const T*)a.qkv + (int64_t)t * ncols + (int64_t)head * d;
    v0 = row[j];
    v1 = row[j + half];
  }
  if (head < a.nq + a.nkv) {
    const float2 c = ((const float2*)a.cos_sin)[(int64_t)p * half + j];
    const float x0 = to_f32(v0), x1 = to_f32(v1);
    const float y0 = x0 * c.x - x1 * c.y;
    const float y1 = x0 * c.y + x1 * c.x;
    if (head < a.nq) {
      T* q = (T*)a.q_rot + (int64_t)t * a.nq * d + (int64_t)head * d;
      q[j] = from_f32<T>(y0);
      q[j + half] = from_f32<T>(y1);
      return;
    }
    const int page = a.page_indices[a.page_indptr[r] + p / a.page_size];
    const int slot = p % a.page_size;
    T* k = (T*)a.k_pool + ((int64_t)page * a.nkv + (head - a.nq)) * a.page_size * d;
    k[kv_k_off(slot, j)] = from_f32<T>(y0);
    k[kv_k_off(slot, j + half)] = from_f32<T>(y1);
    return;
  }
  const int page = a.page_indices[a.page_indptr[r] + p / a.page_size];
  const int slot = p % a.page_size;
  T* v = (T*)a.v_pool + ((int64_t)page * a.nkv + (head - a.nq - a.nkv)) * a.page_size * d;
  v[kv_v_off(slot, j)] = v0;
  v[kv_v_off(slot, j + half)] = v1;
}

// ---------------------------------------------------------------- MoE router
// Single 256-thread block.  Top-k per token (larger logit first; equal logits
// keep the lower expert index first), gate weights = softmax over the chosen
// logits, then a stable counting sort of assignment ids t*k+s by expert:
// per-thread contiguous ranges are counted, scanned per expert across threads,
// then scattered in order, so perm is deterministic.
constexpr int ROUTE_THREADS = 256;
constexpr int ROUTE_MAX_E = 64;

__global__ __launch_bounds__(ROUTE_THREADS) void moe_route_kernel(RouteArgs a) {
  __shared__ int cnt[ROUTE_THREADS][ROUTE_MAX_E + 1];
  __shared__ int off[ROUTE_MAX_E + 1];
  const int tid = threadIdx.x;
  const int E = a.E, k = a.k;
  for (int t = tid; t < a.T; t += ROUTE_THREADS) {
    const float* lg = a.logits + (int64_t)t * E;
    uint64_t taken = 0;
    float sel[8];
    for (int s = 0; s < k; ++s) {
      int best = -1;
      float bv = 0.f;
      for (int e = 0; e < E; ++e) {
        if (taken & (1ull << e)) continue;
        const float v = lg[e];
        if (best < 0 || v > bv) { best = e; bv = v; }
      }
      taken |= 1ull << best;
      a.idx[t * k + s] = best;
      sel[s] = bv;
    }
    float z = 0.f;
    for (int s = 0; s < k; ++s) z += expf(sel[s] - sel[0]);
    for (int s = 0; s < k; ++s) a.w[t * k + s] = expf(sel[s] - sel[0]) / z;
  }
  __syncthreads();
  const int A = a.T * k;
  const int per = (A + ROUTE_THREADS - 1) / ROUTE_THREADS;
  const int lo = min(A, tid * per), hi = min(A, lo + per);
  for (int e = 0; e < E; ++e) cnt[tid][e] = 0;
  for (int i = lo; i < hi; ++i) cnt[tid][a.idx[i]]++;
  __syncthreads();
  if (tid < E) {                       // exclusive scan over threads, per expert
    int run = 0;
    for (int u = 0; u < ROUTE_THREADS; ++u) {
      const int c = cnt[u][tid];
      cnt[u][tid] = run;
      run += c;
    }
    off[tid] = run;                    // total for expert tid (scanned below)
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      const int c = off[e];
      off[e] = run;
      a.offsets[e] = run;
      run += c;
    }
    off[E] = run;
    a.offsets[E] = run;
  }
  __syncthreads();
  int local[ROUTE_MAX_E];
  for (int e = 0; e < E; ++e) local[e] = 0;
  for (int i = lo; i < hi; ++i) {
    const int e = a.idx[i];
    const int dst = off[e] + cnt[tid][e] + local[e]++;
    a.perm[dst] = i;
    a.inv[i] = dst;
  }
}

// out[t] = x1[t] + sum_s w[t][s] * y[inv[t*k + s]] (fp32 sum, one block per token)
template <typename T>
__global__ __launch_bounds__(256) void moe_combine_kernel(const T* __restrict__ x1, const float* __restrict__ y,
                                                          const float* __restrict__ w,
                                                          const int32_t* __restrict__ inv, T* __restrict__ out,
                                                          int H, int k) {
  const int64_t t = blockIdx.x;
  for (int i = threadIdx.x; i < H; i += 256) {
    float v = to_f32(x1[t * H + i]);
    for (int s = 0; s < k; ++s) v += w[t * k + s] * y[(int64_t)inv[t * k + s] * H + i];
    out[t * H + i] = from_f32<T>(v);
  }
}

// Gathers whole pool pages: block b < n copies page pages[b] of K into
// dst_k + b * blk16 (16-byte units); blocks n .. 2n - 1 do V.
__global__ __launch_bounds__(256) void kv_gather_kernel(const u32x4* __restrict__ k_pool,
                                                        const u32x4* __restrict__ v_pool,
                                                        const int32_t* __restrict__ pages, int n, int64_t blk16,
                                                        u32x4* __restrict__ dst_k, u32x4* __restrict__ dst_v) {
  const bool is_v = blockIdx.x >= (unsigned)n;
  const int b = is_v ? blockIdx.x - n : blockIdx.x;
  const u32x4* src = (is_v ? v_pool : k_pool) + (int64_t)pages[b] * blk16;
  u32x4* dst = (is_v ? dst_v : dst_k) + (int64_t)b * blk16;
  for (int64_t i = threadIdx.x; i < blk16; i += 256) dst[i] = __builtin_nontemporal_load(src + i);
}

}  // namespace

hipError_t kv_gather(const void* k_pool, const void* v_pool, const int32_t* pages, int n, int64_t block_bytes,
                     void* dst_k, void* dst_v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (block_bytes % 16) return hipErrorInvalidValue;
  launch(kv_gather_kernel, 2 * n, 256, 0, s, (const u32x4*)k_pool, (const u32x4*)v_pool, pages, n,
         block_bytes / 16, (u32x4*)dst_k, (u32x4*)dst_v);
  return hipGetLastError();
}

hipError_t rmsnorm(int dtype, const void* x, const void* g, void* y, int T, int H, float eps, hipStream_t s,
                   const MetaCopy* mc) {
  if (T == 0) return hipSuccess;
  MetaCopy m;
  if (mc) m = *mc;
  const int extra = m.n16 > 0 ? (int)std::min<int64_t>((m.n16 + 255) / 256, 64) : 0;
  const int grid = T + extra;
  if (dtype == 1 && H % 8 == 0)
    launch(rmsnorm_bf16x8_kernel, grid, RN_THREADS, 0, s, (const bf16*)x, (const bf16*)g, (bf16*)y, H, eps, m, T);
  else if (dtype == 1)
    launch(rmsnorm_kernel<bf16>, grid, 256, 0, s, (const bf16*)x, (const bf16*)g, (bf16*)y, H, eps, m, T);
  else
    launch(rmsnorm_kernel<float>, grid, 256, 0, s, (const float*)x, (const float*)g, (float*)y, H, eps, m, T);
  return hipGetLastError();
}

hipError_t residual_rmsnorm_partials(const float* part, int64_t part_ld, int64_t zstride, int splits,
                                     const void* x, int64_t ldx, void* x1, int64_t ldx1, const void* g, void* y,
                                     int T, int H, float eps, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (H % 8 != 0) return hipErrorInvalidValue;
  launch(residual_rmsnorm_partials_kernel, T, RN_THREADS, 0, s, part, part_ld, zstride, splits, (const bf16*)x, ldx,
         (bf16*)x1, ldx1, (const bf16*)g, (bf16*)y, H, eps);
  return hipGetLastError();
}

hipError_t rope_append(int dtype, const RopeAppendArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int hpb = 256 / (a.d / 2);                      // head_dim in [32, 256]: 2..16 heads per block
  const dim3 grid(a.T, (a.nq + 2 * a.nkv + hpb - 1) / hpb);
  if (dtype == 1)
    launch(rope_append_kernel<bf16>, grid, 256, 0, s, a);
  else
    launch(rope_append_kernel<float>, grid, 256, 0, s, a);
  return hipGetLastError();
}

hipError_t moe_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.E > ROUTE_MAX_E || a.k > 8) return hipErrorInvalidValue;
  launch(moe_route_kernel, 1, ROUTE_THREADS, 0, s, a);
  return hipGetLastError();
}

hipError_t moe_combine(int dtype, const void* x1, const float* y, const float* w, const int32_t* inv,
                       void* out, int T, int H, int k, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 1)
    launch(moe_combine_kernel<bf16>, T, 256, 0, s, (const bf16*)x1, y, w, inv, (bf16*)out, H, k);
  else
    launch(moe_combine_kernel<float>, T, 256, 0, s, (const float*)x1, y, w, inv, (float*)out, H, k);
  return hipGetLastError();
}


}  // namespace nf
