// Row-wise operations of the decoder layer: RMSNorm, rotary embedding fused
// with the paged KV-cache append, and the mixture-of-experts router and
// combine.  All are HBM-bound and small next to the GEMMs and attention.
#include "nf_device.h"
#include "nf_internal.h"

namespace nf {
namespace {

// ---------------------------------------------------------------- RMSNorm
// y = x / sqrt(mean(x^2) + eps) * g, one 256-thread block per row, fp32 math.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* __restrict__ x, const T* __restrict__ g,
                                                      T* __restrict__ y, int H, float eps) {
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
__global__ __launch_bounds__(256) void rmsnorm_bf16x8_kernel(const bf16* __restrict__ x,
                                                             const bf16* __restrict__ g,
                                                             bf16* __restrict__ y, int H, float eps) {
  const int64_t row = blockIdx.x;
  const bf16x8* xr = (const bf16x8*)(x + row * H);
  const bf16x8* gr = (const bf16x8*)g;
  bf16x8* yr = (bf16x8*)(y + row * H);
  const int n8 = H / 8;
  float ss = 0.f;
  for (int i = threadIdx.x; i < n8; i += 256) {
    const bf16x8 v = xr[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += (float)v[e] * (float)v[e];
  }
  __shared__ float red[4];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float inv = rsqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
  for (int i = threadIdx.x; i < n8; i += 256) {
    const bf16x8 v = xr[i], w = gr[i];
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (bf16)((float)v[e] * inv * (float)w[e]);
    yr[i] = o;
  }
}

// ---------------------------------------------------------------- RoPE + append
// One block per token.  Q heads: rotate-half rotation by the token's angle
// table row, written to q_rot.  K heads: rotated and written to the K pool at
// (page of the position, slot); V heads written to the V pool (both in the
// pool's MFMA-operand block order).  Pairs (j, j + d/2) turn by the angle p * theta^(-2j/d).
template <typename T>
__global__ __launch_bounds__(256) void rope_append_kernel(RopeAppendArgs a) {
  const int t = blockIdx.x;
  const int d = a.d, half = d / 2;
  const int p = a.pos[t];
  const int r = a.tok_req[t];
  const int page = a.page_indices[a.page_indptr[r] + p / a.page_size];
  const int slot = p % a.page_size;
  const int ncols = (a.nq + 2 * a.nkv) * d;
  const T* row = (const T*)a.qkv + (int64_t)t * ncols;
  const float2* cs = (const float2*)a.cos_sin + (int64_t)p * half;
  const int rot_pairs = (a.nq + a.nkv) * half;
  for (int i = threadIdx.x; i < rot_pairs; i += blockDim.x) {
    const int head = i / half, j = i % half;
    const float x0 = to_f32(row[head * d + j]), x1 = to_f32(row[head * d + j + half]);
    const float2 c = cs[j];
    const float y0 = x0 * c.x - x1 * c.y;
    const float y1 = x0 * c.y + x1 * c.x;
    if (head < a.nq) {
      T* q = (T*)a.q_rot + (int64_t)t * a.nq * d + head * d;
      q[j] = from_f32<T>(y0);
      q[j + half] = from_f32<T>(y1);
    } else {
      const int kh = head - a.nq;
      T* k = (T*)a.k_pool + ((int64_t)page * a.nkv + kh) * a.page_size * d;
      k[kv_k_off(slot, j)] = from_f32<T>(y0);
      k[kv_k_off(slot, j + half)] = from_f32<T>(y1);
    }
  }
  const T* vrow = row + (a.nq + a.nkv) * d;
  for (int i = threadIdx.x; i < a.nkv * d; i += blockDim.x) {
    const int kh = i / d, e = i % d;
    T* v = (T*)a.v_pool + ((int64_t)page * a.nkv + kh) * a.page_size * d;
    v[kv_v_off(slot, e)] = vrow[i];
  }
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

}  // namespace

hipError_t rmsnorm(int dtype, const void* x, const void* g, void* y, int T, int H, float eps,
                   hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 1 && H % 8 == 0)
    rmsnorm_bf16x8_kernel<<<T, 256, 0, s>>>((const bf16*)x, (const bf16*)g, (bf16*)y, H, eps);
  else if (dtype == 1)
    rmsnorm_kernel<bf16><<<T, 256, 0, s>>>((const bf16*)x, (const bf16*)g, (bf16*)y, H, eps);
  else
    rmsnorm_kernel<float><<<T, 256, 0, s>>>((const float*)x, (const float*)g, (float*)y, H, eps);
  return hipGetLastError();
}

hipError_t rope_append(int dtype, const RopeAppendArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (dtype == 1)
    rope_append_kernel<bf16><<<a.T, 256, 0, s>>>(a);
  else
    rope_append_kernel<float><<<a.T, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t moe_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.E > ROUTE_MAX_E || a.k > 8) return hipErrorInvalidValue;
  moe_route_kernel<<<1, ROUTE_THREADS, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t moe_combine(int dtype, const void* x1, const float* y, const float* w, const int32_t* inv,
                       void* out, int T, int H, int k, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 1)
    moe_combine_kernel<bf16><<<T, 256, 0, s>>>((const bf16*)x1, y, w, inv, (bf16*)out, H, k);
  else
    moe_combine_kernel<float><<<T, 256, 0, s>>>((const float*)x1, y, w, inv, (float*)out, H, k);
  return hipGetLastError();
}

}  // namespace nf
