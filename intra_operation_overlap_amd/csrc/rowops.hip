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

// 16-byte chunks a thread keeps in registers between the sum of squares and
// the output (rows up to RN_HELD * RN_THREADS * 8 elements); longer rows read
// their chunks again.  The order of the sum is the same either way.
constexpr int RN_HELD = 4;

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
  if (n8 <= RN_HELD * RN_THREADS) {
    // every chunk of the row is loaded once, all loads issued before the sum
    bf16x8 v[RN_HELD];
#pragma unroll
    for (int k = 0; k < RN_HELD; ++k) {
      const int i = threadIdx.x + k * RN_THREADS;
      if (i < n8) v[k] = xr[i];
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < RN_HELD; ++k)
      if (threadIdx.x + k * RN_THREADS < n8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += (float)v[k][e] * (float)v[k][e];
      }
    const float inv = rsqrtf(block_sum_sq(ss) / (float)H + eps);
#pragma unroll
    for (int k = 0; k < RN_HELD; ++k) {
      const int i = threadIdx.x + k * RN_THREADS;
      if (i >= n8) break;
      const bf16x8 w = gr[i];
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)v[k][e] * inv * (float)w[e]);
      yr[i] = o;
    }
    return;
  }
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

// Each row's 1 / RMS only: the sum of squares exactly as rmsnorm_bf16x8_kernel
// forms it (same threads, chunks and order), one read of the row.
__global__ __launch_bounds__(RN_THREADS) void row_rms_scale_kernel(const bf16* __restrict__ x, float* __restrict__ s,
                                                                   int H, float eps, MetaCopy mc, int rows) {
  if (meta_copy_block(mc, rows)) return;
  const int64_t row = blockIdx.x;
  const bf16x8* xr = (const bf16x8*)(x + row * H);
  const int n8 = H / 8;
  float ss = 0.f;
  if (n8 <= RN_HELD * RN_THREADS) {
    bf16x8 v[RN_HELD];
#pragma unroll
    for (int k = 0; k < RN_HELD; ++k) {
      const int i = threadIdx.x + k * RN_THREADS;
      if (i < n8) v[k] = xr[i];
    }
#pragma unroll
    for (int k = 0; k < RN_HELD; ++k)
      if (threadIdx.x + k * RN_THREADS < n8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += (float)v[k][e] * (float)v[k][e];
      }
  } else {
    for (int i = threadIdx.x; i < n8; i += RN_THREADS) {
      const bf16x8 v = xr[i];
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += (float)v[e] * (float)v[e];
    }
  }
  const float inv = rsqrtf(block_sum_sq(ss) / (float)H + eps);
  if (threadIdx.x == 0) s[row] = inv;
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
  if (n8 <= RN_HELD * RN_THREADS) {
    // x1 stays in registers for the norm (same sums, same order)
    bf16x8 o[RN_HELD];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < RN_HELD; ++k) {
      const int i = threadIdx.x + k * RN_THREADS;
      if (i >= n8) break;
      const f32x4 lo = sum_slices<f32x4>(P + 8 * i, zstride, splits);
      const f32x4 hi = sum_slices<f32x4>(P + 8 * i + 4, zstride, splits);
      const bf16x8 r = xr[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float a0 = lo[e], a1 = hi[e];
        a0 += (float)r[e];
        a1 += (float)r[e + 4];
        o[k][e] = (bf16)a0;
        o[k][e + 4] = (bf16)a1;
      }
      x1r[i] = o[k];
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += (float)o[k][e] * (float)o[k][e];
    }
    const float inv = rsqrtf(block_sum_sq(ss) / (float)H + eps);
    const bf16x8* gr = (const bf16x8*)g;
    bf16x8* yr = (bf16x8*)(y + row * H);
#pragma unroll
    for (int k = 0; k < RN_HELD; ++k) {
      const int i = threadIdx.x + k * RN_THREADS;
      if (i >= n8) break;
      const bf16x8 w = gr[i];
      bf16x8 q;
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = (bf16)((float)o[k][e] * inv * (float)w[e]);
      yr[i] = q;
    }
    return;
  }
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

// bf16 form with four rotation pairs per thread (j .. j+3 and their partners
// j+d/2 ..): 16-byte partial loads, 8-byte stores, and one block of
// 2048 / d heads per token, so a token's heads go out in one round of loads
// rather than one 4-byte load per thread.  Same arithmetic per element as
// rope_append_kernel (partials summed in slice order, then the rotation).
__global__ __launch_bounds__(256) void rope_append_bf16x4_kernel(RopeAppendArgs a) {
  const int t = blockIdx.x;
  const int d = a.d, half = d / 2, tph = half / 4;       // threads per head
  const int head = blockIdx.y * (256 / tph) + threadIdx.x / tph;
  const int j = 4 * (threadIdx.x % tph);
  if (head >= a.nq + 2 * a.nkv) return;
  const int p = a.pos[t];
  const int r = a.tok_req[t];
  const int ncols = (a.nq + 2 * a.nkv) * d;
  // K and V heads: the pool page of this position, looked up before any
  // store (the compiler would otherwise keep these loads behind the stores
  // below, which it cannot tell apart from the page table)
  const int page = head >= a.nq ? a.page_indices[a.page_indptr[r] + p / a.page_size] : 0;
  float x0[4], x1[4];
  bf16x4 v0, v1;
  const float sc = a.row_scale ? a.row_scale[t] : 1.f;
  if (a.splits > 1) {
    const float* P = a.part + (int64_t)t * a.part_ld + (int64_t)head * d + j;
    const f32x4 s0 = sum_slices<f32x4>(P, a.zstride, a.splits);
    const f32x4 s1 = sum_slices<f32x4>(P + half, a.zstride, a.splits);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v0[e] = (bf16)(s0[e] * sc);
      v1[e] = (bf16)(s1[e] * sc);
    }
    bf16* out = (bf16*)a.qkv + (int64_t)t * ncols + (int64_t)head * d;
    *(bf16x4*)(out + j) = v0;
    *(bf16x4*)(out + j + half) = v1;
  } else {
    const bf16* row = (const bf16*)a.qkv + (int64_t)t * ncols + (int64_t)head * d;
    v0 = *(const bf16x4*)(row + j);
    v1 = *(const bf16x4*)(row + j + half);
    if (a.row_scale)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v0[e] = (bf16)((float)v0[e] * sc);
        v1[e] = (bf16)((float)v1[e] * sc);
      }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x0[e] = (float)v0[e];
    x1[e] = (float)v1[e];
  }
  if (head < a.nq + a.nkv) {
    const f32x4* cs = (const f32x4*)((const float2*)a.cos_sin + (int64_t)p * half + j);
    const f32x4 c01 = cs[0], c23 = cs[1];
    const float cx[4] = {c01[0], c01[2], c23[0], c23[2]}, cy[4] = {c01[1], c01[3], c23[1], c23[3]};
    bf16x4 y0, y1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y0[e] = (bf16)(x0[e] * cx[e] - x1[e] * cy[e]);
      y1[e] = (bf16)(x0[e] * cy[e] + x1[e] * cx[e]);
    }
    if (head < a.nq) {
      bf16* q = (bf16*)a.q_rot + (int64_t)t * a.nq * d + (int64_t)head * d;
      *(bf16x4*)(q + j) = y0;
      *(bf16x4*)(q + j + half) = y1;
      return;
    }
    const int slot = p % a.page_size;
    bf16* k = (bf16*)a.k_pool + ((int64_t)page * a.nkv + (head - a.nq)) * a.page_size * d;
    // dims j .. j+3 lie in one run of 8 of the K block order, so contiguously
    *(bf16x4*)(k + kv_k_off(slot, j)) = y0;
    *(bf16x4*)(k + kv_k_off(slot, j + half)) = y1;
    return;
  }
  const int slot = p % a.page_size;
  bf16* v = (bf16*)a.v_pool + ((int64_t)page * a.nkv + (head - a.nq - a.nkv)) * a.page_size * d;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[kv_v_off(slot, j + e)] = v0[e];
    v[kv_v_off(slot, j + half + e)] = v1[e];
  }
}

// ---------------------------------------------------------------- MoE router
// Single 256-thread block.  Top-k per token (larger logit first; equal logits
// keep the lower expert index first), gate weights = softmax over the chosen
// logits, then a stable counting sort of assignment ids t*k+s by expert:
// per-thread contiguous ranges are counted, scanned per expert across threads
// (shuffle scans within each wave, then the totals of the earlier waves), then
// scattered in order, each thread advancing its own row of the table, so perm
// is deterministic.
constexpr int ROUTE_THREADS = 256;
constexpr int ROUTE_MAX_E = 64;
constexpr int ROUTE_REG_E = 8;        // up to this many experts a token's logits are held in registers
constexpr int ROUTE_LDS_IDX = 8192;   // up to this many assignments the sort reads them from LDS

__global__ __launch_bounds__(ROUTE_THREADS) void moe_route_kernel(RouteArgs a) {
  __shared__ int cnt[ROUTE_THREADS][ROUTE_MAX_E + 1];
  __shared__ int off[ROUTE_MAX_E + 1];
  __shared__ int s_idx[ROUTE_LDS_IDX];
  const int tid = threadIdx.x;
  const int E = a.E, k = a.k;
  const int A = a.T * k;
  const bool lds_idx = A <= ROUTE_LDS_IDX;
  for (int t = tid; t < a.T; t += ROUTE_THREADS) {
    const float* lg = a.logits + (int64_t)t * E;
    uint64_t taken = 0;
    float sel[8];
    if (E <= ROUTE_REG_E) {
      // every logit of the token loaded before the selection
      float v[ROUTE_REG_E];
#pragma unroll
      for (int e = 0; e < ROUTE_REG_E; ++e) v[e] = e < E ? lg[e] : 0.f;
      for (int s = 0; s < k; ++s) {
        int best = -1;
        float bv = 0.f;
#pragma unroll
        for (int e = 0; e < ROUTE_REG_E; ++e) {
          if (e >= E || (taken & (1ull << e))) continue;
          if (best < 0 || v[e] > bv) { best = e; bv = v[e]; }
        }
        taken |= 1ull << best;
        a.idx[t * k + s] = best;
        if (lds_idx) s_idx[t * k + s] = best;
        sel[s] = bv;
      }
    } else {
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
        if (lds_idx) s_idx[t * k + s] = best;
        sel[s] = bv;
      }
    }
    float z = 0.f;
    for (int s = 0; s < k; ++s) z += expf(sel[s] - sel[0]);
    for (int s = 0; s < k; ++s) a.w[t * k + s] = expf(sel[s] - sel[0]) / z;
  }
  __syncthreads();
  auto idx_of = [&](int i) { return lds_idx ? s_idx[i] : a.idx[i]; };
  const int per = (A + ROUTE_THREADS - 1) / ROUTE_THREADS;
  const int lo = min(A, tid * per), hi = min(A, lo + per);
  for (int e = 0; e < E; ++e) cnt[tid][e] = 0;
  for (int i = lo; i < hi; ++i) cnt[tid][idx_of(i)]++;
  __syncthreads();
  // exclusive scan over threads of every expert's column: within each wave by
  // shuffles, then the totals of the waves before it
  constexpr int NWAVE = ROUTE_THREADS / 64;
  __shared__ int wsum[NWAVE][ROUTE_MAX_E];
  const int lane = tid & 63, wv = tid >> 6;
  for (int e = 0; e < E; ++e) {
    const int c = cnt[tid][e];
    int v = c;
    for (int d = 1; d < 64; d *= 2) {
      const int u = __shfl_up(v, d, 64);
      if (lane >= d) v += u;
    }
    cnt[tid][e] = v - c;
    if (lane == 63) wsum[wv][e] = v;
  }
  __syncthreads();
  for (int e = 0; e < E; ++e) {
    int base = 0;
    for (int q = 0; q < wv; ++q) base += wsum[q][e];
    cnt[tid][e] += base;
  }
  if (tid < E) {                       // total for expert tid (scanned below)
    int tot = 0;
    for (int q = 0; q < NWAVE; ++q) tot += wsum[q][tid];
    off[tid] = tot;
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
  for (int i = lo; i < hi; ++i) {
    const int e = idx_of(i);
    const int dst = off[e] + cnt[tid][e]++;
    a.perm[dst] = i;
    a.inv[i] = dst;
  }
}

// bf16, H % 8 == 0: the same sums over 8-element chunks, every load of a
// chunk issued before its sum (k <= 8)
__global__ __launch_bounds__(256) void moe_combine_bf16x8_kernel(const bf16* __restrict__ x1,
                                                                 const float* __restrict__ y,
                                                                 const float* __restrict__ w,
                                                                 const int32_t* __restrict__ inv,
                                                                 bf16* __restrict__ out, int H, int k) {
  const int64_t t = blockIdx.x;
  float ws[8];
  int64_t rows[8];
  for (int s = 0; s < k; ++s) {
    ws[s] = w[t * k + s];
    rows[s] = (int64_t)inv[t * k + s] * H;
  }
  for (int c = threadIdx.x; c < H / 8; c += 256) {
    const int i = 8 * c;
    const bf16x8 xv = *(const bf16x8*)(x1 + t * H + i);
    f32x4 lo[8], hi[8];
    for (int s = 0; s < k; ++s) {
      lo[s] = *(const f32x4*)(y + rows[s] + i);
      hi[s] = *(const f32x4*)(y + rows[s] + i + 4);
    }
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v0 = (float)xv[e], v1 = (float)xv[e + 4];
      for (int s = 0; s < k; ++s) {
        v0 += ws[s] * lo[s][e];
        v1 += ws[s] * hi[s][e];
      }
      o[e] = (bf16)v0;
      o[e + 4] = (bf16)v1;
    }
    *(bf16x8*)(out + t * H + i) = o;
  }
}

// out[n][k] = round(w[n][k] * g[k]) for a bf16 [N][K] matrix, 16 bytes per
// thread and step (K % 8 == 0): weights with a norm gain folded in
__global__ __launch_bounds__(256) void scale_cols_bf16x8_kernel(const bf16x8* __restrict__ w,
                                                                const bf16x8* __restrict__ g,
                                                                bf16x8* __restrict__ out, int64_t n16, int k8) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    const bf16x8 v = w[i], s = g[i % k8];
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)v[e] * (float)s[e]);
    out[i] = o;
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

// Plain copy of n16 16-byte units with a grid of few workgroups (the copy
// kernel of the emulated all-reduce).
__global__ __launch_bounds__(256) void copy_rows_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// Serving loop: row t of x comes from the device address src[t] (rows of
// `row16` 16-byte units); row t of `out` goes to dst[t]; flag[t] = 1 when
// out[t][0] > thr.  src, dst and flag are host-mapped pinned memory.
__global__ __launch_bounds__(256) void loop_gather_kernel(const uint64_t* __restrict__ src, u32x4* __restrict__ x,
                                                          int row16) {
  const u32x4* s = (const u32x4*)src[blockIdx.x];
  u32x4* d = x + (int64_t)blockIdx.x * row16;
  for (int i = threadIdx.x; i < row16; i += 256) d[i] = s[i];
}

template <typename T>
__global__ __launch_bounds__(256) void loop_scatter_kernel(const u32x4* __restrict__ out, const uint64_t* __restrict__ dst,
                                                           int row16, int H, float thr, int32_t* __restrict__ flag) {
  const u32x4* s = out + (int64_t)blockIdx.x * row16;
  u32x4* d = (u32x4*)dst[blockIdx.x];
  for (int i = threadIdx.x; i < row16; i += 256) d[i] = s[i];
  if (threadIdx.x == 0) flag[blockIdx.x] = to_f32(((const T*)s)[0]) > thr ? 1 : 0;
  (void)H;
}

// Inverse of kv_gather_kernel: block i of src_k / src_v back to pool page
// pages[i] (pages distinct).
__global__ __launch_bounds__(256) void kv_scatter_kernel(u32x4* __restrict__ k_pool, u32x4* __restrict__ v_pool,
                                                         const int32_t* __restrict__ pages, int n, int64_t blk16,
                                                         const u32x4* __restrict__ src_k,
                                                         const u32x4* __restrict__ src_v) {
  const bool is_v = blockIdx.x >= (unsigned)n;
  const int b = is_v ? blockIdx.x - n : blockIdx.x;
  u32x4* dst = (is_v ? v_pool : k_pool) + (int64_t)pages[b] * blk16;
  const u32x4* src = (is_v ? src_v : src_k) + (int64_t)b * blk16;
  for (int64_t i = threadIdx.x; i < blk16; i += 256) dst[i] = src[i];
}

// Pool pages <-> the plain paged layout [n][nkv][16][d] (element type E: the
// storage bits of one element).  Block b < n * nkv is K, the rest V; list
// entry i = (b % (n * nkv)) / nkv names pool page pages[i] (or i when pages
// is null).  Each thread moves single elements; this runs once per import or
// export, not per step.
template <typename E>
__global__ __launch_bounds__(256) void kv_convert_kernel(E* __restrict__ k_pool, E* __restrict__ v_pool,
                                                         const int32_t* __restrict__ pages, int n, int nkv, int d,
                                                         E* __restrict__ k_rm, E* __restrict__ v_rm, int to_pool) {
  const int64_t nb = (int64_t)n * nkv;
  const bool is_v = blockIdx.x >= nb;
  const int64_t b = is_v ? blockIdx.x - nb : blockIdx.x;
  const int i = (int)(b / nkv), kh = (int)(b % nkv);
  const int64_t page = pages ? pages[i] : i;
  const int blk = 16 * d;
  E* pool = (is_v ? v_pool : k_pool) + (page * nkv + kh) * blk;
  E* rm = (is_v ? v_rm : k_rm) + b * blk;
  for (int e = threadIdx.x; e < blk; e += 256) {
    const int slot = e / d, dim = e % d;
    const int off = is_v ? kv_v_off(slot, dim) : kv_k_off(slot, dim);
    if (to_pool)
      pool[off] = rm[e];
    else
      rm[e] = pool[off];
  }
}

}  // namespace

hipError_t kv_convert(int dtype, void* k_pool, void* v_pool, const int32_t* pages, int n, int nkv, int d, void* k_rm,
                      void* v_rm, bool to_pool, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (d % 32 || nkv <= 0) return hipErrorInvalidValue;
  const int64_t grid = 2 * (int64_t)n * nkv;
  if (dtype == 1)
    launch(kv_convert_kernel<uint16_t>, dim3((unsigned)grid), 256, 0, s, (uint16_t*)k_pool, (uint16_t*)v_pool, pages,
           n, nkv, d, (uint16_t*)k_rm, (uint16_t*)v_rm, to_pool ? 1 : 0);
  else
    launch(kv_convert_kernel<uint32_t>, dim3((unsigned)grid), 256, 0, s, (uint32_t*)k_pool, (uint32_t*)v_pool, pages,
           n, nkv, d, (uint32_t*)k_rm, (uint32_t*)v_rm, to_pool ? 1 : 0);
  return hipGetLastError();
}

hipError_t copy_rows(const void* src, void* dst, size_t bytes, int wgs, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  if (bytes % 16 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15) || wgs <= 0) return hipErrorInvalidValue;
  launch(copy_rows_kernel, wgs, 256, 0, s, (const u32x4*)src, (u32x4*)dst, (int64_t)(bytes / 16));
  return hipGetLastError();
}

hipError_t loop_gather(const uint64_t* src, void* x, int T, int64_t row_bytes, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (row_bytes % 16) return hipErrorInvalidValue;
  launch(loop_gather_kernel, T, 256, 0, s, src, (u32x4*)x, (int)(row_bytes / 16));
  return hipGetLastError();
}

hipError_t loop_scatter(int dtype, const void* out, const uint64_t* dst, int T, int H, float thr, int32_t* flag,
                        hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int64_t row_bytes = (int64_t)H * (dtype == 1 ? 2 : 4);
  if (row_bytes % 16) return hipErrorInvalidValue;
  if (dtype == 1)
    launch(loop_scatter_kernel<bf16>, T, 256, 0, s, (const u32x4*)out, dst, (int)(row_bytes / 16), H, thr, flag);
  else
    launch(loop_scatter_kernel<float>, T, 256, 0, s, (const u32x4*)out, dst, (int)(row_bytes / 16), H, thr, flag);
  return hipGetLastError();
}

hipError_t kv_scatter(void* k_pool, void* v_pool, const int32_t* pages, int n, int64_t block_bytes, const void* src_k,
                      const void* src_v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (block_bytes % 16) return hipErrorInvalidValue;
  launch(kv_scatter_kernel, 2 * n, 256, 0, s, (u32x4*)k_pool, (u32x4*)v_pool, pages, n, block_bytes / 16,
         (const u32x4*)src_k, (const u32x4*)src_v);
  return hipGetLastError();
}

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
  if (dtype == 1) {
    const int hpb4 = 2048 / a.d;                         // four pairs per thread: 8..64 heads per block
    launch(rope_append_bf16x4_kernel, dim3(a.T, (a.nq + 2 * a.nkv + hpb4 - 1) / hpb4), 256, 0, s, a);
  } else {
    launch(rope_append_kernel<float>, grid, 256, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t moe_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.E > ROUTE_MAX_E || a.k > 8) return hipErrorInvalidValue;
  launch(moe_route_kernel, 1, ROUTE_THREADS, 0, s, a);
  return hipGetLastError();
}

hipError_t row_rms_scale(const void* x, float* s, int T, int H, float eps, hipStream_t st, const MetaCopy* mc) {
  if (T == 0) return hipSuccess;
  if (H % 8) return hipErrorInvalidValue;
  MetaCopy m;
  if (mc) m = *mc;
  const int extra = m.n16 > 0 ? (int)std::min<int64_t>((m.n16 + 255) / 256, 64) : 0;
  launch(row_rms_scale_kernel, T + extra, RN_THREADS, 0, st, (const bf16*)x, s, H, eps, m, T);
  return hipGetLastError();
}

hipError_t scale_cols_bf16(const void* w, const void* g, void* out, int64_t N, int K, hipStream_t s) {
  if (N == 0) return hipSuccess;
  if (K % 8) return hipErrorInvalidValue;
  const int64_t n16 = N * K / 8;
  launch(scale_cols_bf16x8_kernel, (int)std::min<int64_t>((n16 + 255) / 256, 4096), 256, 0, s, (const bf16x8*)w,
         (const bf16x8*)g, (bf16x8*)out, n16, K / 8);
  return hipGetLastError();
}

hipError_t moe_combine(int dtype, const void* x1, const float* y, const float* w, const int32_t* inv,
                       void* out, int T, int H, int k, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 1)
    launch(H % 8 == 0 && k <= 8 ? moe_combine_bf16x8_kernel : moe_combine_kernel<bf16>, T, 256, 0, s,
           (const bf16*)x1, y, w, inv, (bf16*)out, H, k);
  else
    launch(moe_combine_kernel<float>, T, 256, 0, s, (const float*)x1, y, w, inv, (float*)out, H, k);
  return hipGetLastError();
}


}  // namespace nf
