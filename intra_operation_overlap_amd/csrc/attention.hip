// Causal GQA attention over the paged KV cache, for decode tokens and for a
// chunk of prefill tokens alike.
//
// Work item = (a request's run of up to 16/G consecutive query tokens, one KV
// head, a range of the request's logical pages).  Its 16 "rows" are the
// (token, query head) pairs that share the KV head, so a decode token fills G
// rows and a prefill item packs 16/G tokens.  Each row r has its own causal
// limit: keys 0..pos(row).  A 256-thread workgroup (four wave64s) takes the
// item's pages round-robin across its waves; each wave keeps an online
// softmax (running max, running sum, unnormalised output) and the four are
// combined through LDS at the end.  Items whose page range was split write
// unnormalised partials + (max, sum) for a merge kernel.
//
// bf16, d = 128 path on matrix cores, per 16-key page:
//   S^T[key][row] = K_page[key][:] . Q[row][:]   4 x v_mfma_f32_16x16x32_bf16
//       (A = K page rows straight from the pool, B = Q held in registers)
//   the C layout of S^T puts keys 4*(lane/16)+i of row lane%16 in each lane,
//   which is exactly the B-operand layout of the next product, so the softmax
//   probabilities never leave registers:
//   O^T[dim][row] += V^T_page[dim][key] . P^T[key][row]
//                                       8 x v_mfma_f32_16x16x16_bf16
//       (A = V page, stored dimension-major in the pool, 8 contiguous bytes
//        per lane, each 16-dim block a contiguous 512-byte run)
// The running max and sum are per row, i.e. per lane%16 column in both
// products, so the rescale needs no data movement; row maxima are reduced
// over the four lanes that share a column with two xor-shuffles.
#include "nf_device.h"
#include "nf_internal.h"

namespace nf {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr int ROWS = 16;

__device__ __forceinline__ void row_info(const AttnArgs& a, const AttnItem& it, int row, int G, int kh,
                                         int& limit, int64_t& qoff) {
  const int tok = row / G;
  if (tok < it.ntok && row < (ROWS / G) * G) {
    const int t = it.tok0 + tok;
    limit = a.pos[t] + 1;
    qoff = (int64_t)t * a.nq * a.d + (int64_t)(kh * G + row % G) * a.d;
  } else {
    limit = 0;
    qoff = -1;
  }
}

// Final combine of (m, l, O) per row from the four waves, then either the
// normalised output or a partial for the merge kernel.  O_s is [4][16][d].
template <typename T>
__device__ void finish_item(const AttnArgs& a, const AttnItem& it, int G, int kh, float* m_s, float* l_s,
                            float* O_s) {
  const int tid = threadIdx.x;
  const int d = a.d;
  const int row = tid / 16;                 // 16 threads per row
  const int valid_rows = min(ROWS / G, it.ntok) * G;
  if (row >= valid_rows) return;
  float M = -INFINITY;
  for (int w = 0; w < 4; ++w) M = fmaxf(M, m_s[w * ROWS + row]);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float f[4], L = 0.f;
  for (int w = 0; w < 4; ++w) {
    f[w] = exp2f(m_s[w * ROWS + row] - Mu);
    L += f[w] * l_s[w * ROWS + row];
  }
  const int t = it.tok0 + row / G;
  const int head = kh * G + row % G;
  if (it.partial < 0) {
    const float invL = L > 0.f ? 1.f / L : 0.f;
    T* o = (T*)a.attn + (int64_t)t * a.nq * d + (int64_t)head * d;
    for (int e = tid % 16; e < d; e += 16) {
      float v = 0.f;
      for (int w = 0; w < 4; ++w) v += f[w] * O_s[(w * ROWS + row) * d + e];
      o[e] = from_f32<T>(v * invL);
    }
  } else {
    const int64_t base = ((int64_t)it.partial * a.nkv + kh) * ROWS + row;
    float* po = a.part_o + base * d;
    for (int e = tid % 16; e < d; e += 16) {
      float v = 0.f;
      for (int w = 0; w < 4; ++w) v += f[w] * O_s[(w * ROWS + row) * d + e];
      po[e] = v;
    }
    if (tid % 16 == 0) {
      a.part_ml[base * 2 + 0] = M;
      a.part_ml[base * 2 + 1] = L;
    }
  }
}

// ---------------------------------------------------------------- bf16, d = 128
__global__ __launch_bounds__(256) void attn_bf16_d128_kernel(AttnArgs a) {
  constexpr int D = 128;
  __shared__ float m_s[4 * ROWS], l_s[4 * ROWS];
  __shared__ float O_s[4 * ROWS * D];

  const AttnItem it = a.items[blockIdx.x];
  const int kh = blockIdx.y;
  const int G = a.nq / a.nkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15;        // row index of the S^T / O^T column this lane holds
  const int grp = lane >> 4;        // which 4-key (or 8-dim) group

  int limit;
  int64_t qoff;
  row_info(a, it, col, G, kh, limit, qoff);
  int max_limit = 0;                // largest causal limit over the item's rows
  for (int t = 0; t < it.ntok; ++t) max_limit = max(max_limit, a.pos[it.tok0 + t] + 1);

  // Q^T fragments (B operand of S^T = K Q^T): row `col`, dims 32c + 8*grp .. +7
  bf16x8 qf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (qoff >= 0)
      qf[c] = *(const bf16x8*)((const bf16*)a.q_rot + qoff + 32 * c + 8 * grp);
    else
      qf[c] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }

  const float sl2 = a.scale * LOG2E;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) oacc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* ptab = a.page_indices + a.page_indptr[it.req];
  const bf16* kpool = (const bf16*)a.k_pool;
  const bf16* vpool = (const bf16*)a.v_pool;

  for (int lp = it.page_begin + wave; lp < it.page_end; lp += 4) {
    const int64_t blk = (int64_t)ptab[lp] * a.nkv + kh;     // (page, kv head) block
    const bf16* kb = kpool + blk * (16 * D);
    const bf16* vb = vpool + blk * (16 * D);
    bf16x8 kf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) kf[c] = *(const bf16x8*)(kb + col * D + 32 * c + 8 * grp);
    s16x4 vf[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) vf[b] = *(const s16x4*)(vb + (16 * b + col) * 16 + 4 * grp);

    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], qf[c], s, 0, 0, 0);

    const int key0 = lp * 16 + 4 * grp;   // keys key0 .. key0+3 in this lane
    float sv[4];
    float pm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = (key0 + i < limit) ? s[i] * sl2 : -INFINITY;
      pm = fmaxf(pm, sv[i]);
    }
    pm = fmaxf(pm, __shfl_xor(pm, 16, 64));
    pm = fmaxf(pm, __shfl_xor(pm, 32, 64));
    const float m_new = fmaxf(m_run, pm);
    const float mu = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - mu);
    float ps = 0.f;
    bf16x4 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = exp2f(sv[i] - mu);
      ps += pv;
      pb[i] = (bf16)pv;
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int b = 0; b < 8; ++b) oacc[b] *= alpha;
    if (lp * 16 + 16 > max_limit) {
      // keys past every row's limit may be unwritten (or being written):
      // zero them so 0 * garbage cannot reach the sum
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (key0 + i >= max_limit)
#pragma unroll
          for (int b = 0; b < 8; ++b) vf[b][i] = 0;
    }
    const s16x4 pbs = __builtin_bit_cast(s16x4, pb);
#pragma unroll
    for (int b = 0; b < 8; ++b) oacc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[b], pbs, oacc[b], 0, 0, 0);
  }

  // this wave's (m, l, O^T) -> LDS; O^T lane layout: dim 16b + 4*grp + i, row col
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (grp == 0) {
    m_s[wave * ROWS + col] = m_run;
    l_s[wave * ROWS + col] = l_run;
  }
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) O_s[(wave * ROWS + col) * D + 16 * b + 4 * grp + i] = oacc[b][i];
  __syncthreads();
  finish_item<bf16>(a, it, G, kh, m_s, l_s, O_s);
}

// ---------------------------------------------------------------- generic
// Any dtype, any even d <= 256: one wave per row at a time, keys walked one
// by one with an online softmax; lanes split the head dimension.
template <typename T>
__global__ __launch_bounds__(256) void attn_generic_kernel(AttnArgs a) {
  constexpr int DMAX = 256;
  __shared__ float m_s[4 * ROWS], l_s[4 * ROWS];
  __shared__ float O_s[4 * ROWS * DMAX];
  const AttnItem it = a.items[blockIdx.x];
  const int kh = blockIdx.y;
  const int G = a.nq / a.nkv;
  const int d = a.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t* ptab = a.page_indices + a.page_indptr[it.req];
  const int S = a.page_size;
  // every wave owns all 16 rows for a quarter of the pages
  for (int row = 0; row < ROWS; ++row) {
    int limit;
    int64_t qoff;
    row_info(a, it, row, G, kh, limit, qoff);
    float q[DMAX / 64];
    float o[DMAX / 64];
    for (int u = 0; u < DMAX / 64; ++u) {
      const int e = lane + 64 * u;
      q[u] = (qoff >= 0 && e < d) ? to_f32(((const T*)a.q_rot)[qoff + e]) : 0.f;
      o[u] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int lp = it.page_begin + wave; lp < it.page_end; lp += 4) {
      const int64_t blk = (int64_t)ptab[lp] * a.nkv + kh;
      for (int sl = 0; sl < S; ++sl) {
        const int key = lp * S + sl;
        if (key >= limit) break;
        const T* kr = (const T*)a.k_pool + (blk * S + sl) * d;
        float part = 0.f;
        for (int u = 0; u < DMAX / 64; ++u) {
          const int e = lane + 64 * u;
          if (e < d) part += q[u] * to_f32(kr[e]);
        }
        const float sc = wave_sum(part) * a.scale;
        const float mn = fmaxf(m, sc);
        const float al = expf(m - mn);
        const float p = expf(sc - mn);
        l = l * al + p;
        for (int u = 0; u < DMAX / 64; ++u) {
          const int e = lane + 64 * u;
          const float v = e < d ? to_f32(((const T*)a.v_pool)[(blk * d + e) * S + sl]) : 0.f;
          o[u] = o[u] * al + p * v;
        }
        m = mn;
      }
    }
    // store in the base-2 convention finish_item uses
    if (lane == 0) {
      m_s[wave * ROWS + row] = m * LOG2E;
      l_s[wave * ROWS + row] = l;
    }
    for (int u = 0; u < DMAX / 64; ++u) {
      const int e = lane + 64 * u;
      if (e < d) O_s[(wave * ROWS + row) * d + e] = o[u];
    }
  }
  __syncthreads();
  finish_item<T>(a, it, G, kh, m_s, l_s, O_s);
}

// ---------------------------------------------------------------- merge
// Combines the partials of split items: one block per (merge item, KV head),
// 16 threads per row.
template <typename T>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs a) {
  const MergeItem mi = a.merges[blockIdx.x];
  const int kh = blockIdx.y;
  const int G = a.nq / a.nkv;
  const int d = a.d;
  const int row = threadIdx.x / 16;
  const int valid_rows = min(ROWS / G, mi.ntok) * G;
  if (row >= valid_rows) return;
  float M = -INFINITY;
  for (int s = 0; s < mi.n_partials; ++s) {
    const int64_t base = ((int64_t)(mi.first_partial + s) * a.nkv + kh) * ROWS + row;
    M = fmaxf(M, a.part_ml[base * 2]);
  }
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float L = 0.f;
  for (int s = 0; s < mi.n_partials; ++s) {
    const int64_t base = ((int64_t)(mi.first_partial + s) * a.nkv + kh) * ROWS + row;
    L += exp2f(a.part_ml[base * 2] - Mu) * a.part_ml[base * 2 + 1];
  }
  const float invL = L > 0.f ? 1.f / L : 0.f;
  const int t = mi.tok0 + row / G;
  const int head = kh * G + row % G;
  T* o = (T*)a.attn + (int64_t)t * a.nq * d + (int64_t)head * d;
  for (int e = threadIdx.x % 16; e < d; e += 16) {
    float v = 0.f;
    for (int s = 0; s < mi.n_partials; ++s) {
      const int64_t base = ((int64_t)(mi.first_partial + s) * a.nkv + kh) * ROWS + row;
      v += exp2f(a.part_ml[base * 2] - Mu) * a.part_o[base * d + e];
    }
    o[e] = from_f32<T>(v * invL);
  }
}

}  // namespace

hipError_t attention(int dtype, const AttnArgs& a, hipStream_t s) {
  if (a.n_items == 0) return hipSuccess;
  dim3 grid(a.n_items, a.nkv);
  if (dtype == 1 && a.d == 128 && a.page_size == 16)
    attn_bf16_d128_kernel<<<grid, 256, 0, s>>>(a);
  else if (dtype == 1)
    attn_generic_kernel<bf16><<<grid, 256, 0, s>>>(a);
  else
    attn_generic_kernel<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t attention_merge(int dtype, const AttnArgs& a, hipStream_t s) {
  if (a.n_merges == 0) return hipSuccess;
  dim3 grid(a.n_merges, a.nkv);
  if (dtype == 1)
    attn_merge_kernel<bf16><<<grid, 256, 0, s>>>(a);
  else
    attn_merge_kernel<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace nf
