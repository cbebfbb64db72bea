// Causal GQA attention over the paged KV cache, for decode tokens and for a
// chunk of prefill tokens alike.
//
// Work item = (a request's run of up to 16/G consecutive query tokens, one KV
// head, a range of the request's logical pages).  Its 16 "rows" are the
// (token, query head) pairs that share the KV head, so a decode token fills G
// rows and a prefill item packs 16/G tokens.  Each row r has its own causal
// limit: keys 0..pos(row).  Items whose page range was split write
// unnormalised partials + (max, sum) for a merge kernel.
//
// bf16, d = 128 path on matrix cores, per 16-key page:
//   S^T[key][row] = K_page[key][:] . Q[row][:]   4 x v_mfma_f32_16x16x32_bf16
//       (A = K page straight from the pool, B = Q held in registers)
//   the C layout of S^T puts keys 4*(lane/16)+i of row lane%16 in each lane,
//   which is exactly the B-operand layout of the next product, so the softmax
//   probabilities never leave registers:
//   O^T[dim][row] += V^T_page[dim][key] . P^T[key][row]
//                                       8 x v_mfma_f32_16x16x16_bf16
// The pool stores every (page, KV head) block in exactly these operand
// layouts (kv_k_off / kv_v_off), so a page arrives with eight linear
// 16-byte-per-lane loads (1 KB per instruction), the access pattern that lets
// one CU draw the most HBM bandwidth.  The running max and sum are per row,
// i.e. per lane%16 column in both products, so the rescale needs no data
// movement; row maxima are reduced over the four lanes that share a column
// with two xor-shuffles.
#include "nf_device.h"
#include "nf_internal.h"

namespace nf {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr int ROWS = 16;
constexpr int DH = 128;
constexpr int BLOCK = 16 * DH;                 // elements of one (page, KV head) block

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

// One page's operand fragments for this lane.
struct PageRegs {
  bf16x8 k[4];      // K operand fragments, dims 32c .. 32c+31 (c = 0..3)
  s16x8 v[4];       // V operand fragments of dim blocks 2c (first 4) and 2c+1 (last 4)
};

__device__ __forceinline__ void load_page(const bf16* kb, const bf16* vb, int lane, PageRegs& r) {
#pragma unroll
  for (int c = 0; c < 4; ++c) r.k[c] = __builtin_nontemporal_load((const bf16x8*)(kb + c * 512 + lane * 8));
#pragma unroll
  for (int c = 0; c < 4; ++c) r.v[c] = __builtin_nontemporal_load((const s16x8*)(vb + c * 512 + lane * 8));
}

struct RowState {
  float m = -INFINITY, l = 0.f;
  f32x4 o[8];
};

// One 16-key page: scores, online softmax, P.V.  `key0` is this lane's first
// key, `limit` its row's causal limit, `max_limit` the largest limit of the
// item (keys at or past it may be unwritten, so their V values are zeroed).
__device__ __forceinline__ void page_step(const bf16x8 (&qf)[4], PageRegs& r, int key0, int limit, int max_limit,
                                          bool tail, float sl2, RowState& st) {
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.k[c], qf[c], s, 0, 0, 0);
  float sv[4];
  float pm = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sv[i] = (key0 + i < limit) ? s[i] * sl2 : -INFINITY;
    pm = fmaxf(pm, sv[i]);
  }
  pm = fmaxf(pm, __shfl_xor(pm, 16, 64));
  pm = fmaxf(pm, __shfl_xor(pm, 32, 64));
  const float m_new = fmaxf(st.m, pm);
  const float mu = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = exp2f(st.m - mu);
  float ps = 0.f;
  bf16x4 pb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float pv = exp2f(sv[i] - mu);
    ps += pv;
    pb[i] = (bf16)pv;
  }
  st.l = st.l * alpha + ps;
  st.m = m_new;
#pragma unroll
  for (int b = 0; b < 8; ++b) st.o[b] *= alpha;
  if (tail) {
    // keys past every row's limit may be unwritten (or being written):
    // zero them so 0 * garbage cannot reach the sum
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (key0 + i >= max_limit)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          r.v[c][i] = 0;
          r.v[c][4 + i] = 0;
        }
  }
  const s16x4 pbs = __builtin_bit_cast(s16x4, pb);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const s16x4 lo = {r.v[c][0], r.v[c][1], r.v[c][2], r.v[c][3]};
    const s16x4 hi = {r.v[c][4], r.v[c][5], r.v[c][6], r.v[c][7]};
    st.o[2 * c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, pbs, st.o[2 * c], 0, 0, 0);
    st.o[2 * c + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, pbs, st.o[2 * c + 1], 0, 0, 0);
  }
}

// Walks n pages of request `req` (logical pages first, first + stride, ...)
// with the next page's K and V in flight while the current one feeds the
// matrix cores.  The pool page numbers of up to 64 pages are fetched at once,
// one per lane, and read back with readlane: a page-table load issued behind
// the K/V loads would otherwise make every next-page address wait for them.
__device__ __forceinline__ void walk_pages(const AttnArgs& a, int req, int first, int stride, int n, int kh,
                                           int lane, int grp, const bf16x8 (&qf)[4], int limit, int max_limit,
                                           float sl2, RowState& st) {
  const int32_t* ptab = a.page_indices + a.page_indptr[req];
  const bf16* kpool = (const bf16*)a.k_pool;
  const bf16* vpool = (const bf16*)a.v_pool;
  PageRegs r[2];
  for (int cb = 0; cb < n; cb += 64) {
    const int cn = min(64, n - cb);
    const int mine = lane < cn ? ptab[first + stride * (cb + lane)] : 0;
    auto load = [&](int j, int set) {
      const int64_t blk = (int64_t)__builtin_amdgcn_readlane(mine, j) * a.nkv + kh;
      load_page(kpool + blk * BLOCK, vpool + blk * BLOCK, lane, r[set]);
    };
    auto step = [&](int j, int set) {
      const int lp = first + stride * (cb + j);
      page_step(qf, r[set], lp * 16 + 4 * grp, limit, max_limit, lp * 16 + 16 > max_limit, sl2, st);
    };
    int j = 0;
    load(0, 0);
    for (; j + 1 < cn; j += 2) {
      load(j + 1, 1);
      step(j, 0);
      if (j + 2 < cn) load(j + 2, 0);
      step(j + 1, 1);
    }
    if (j < cn) step(j, 0);
  }
}

__device__ __forceinline__ void load_q(const AttnArgs& a, int64_t qoff, int grp, bf16x8 (&qf)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (qoff >= 0)
      qf[c] = *(const bf16x8*)((const bf16*)a.q_rot + qoff + 32 * c + 8 * grp);
    else
      qf[c] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

// ---------------------------------------------------------------- four waves per item
// A 256-thread workgroup takes the item's pages round-robin across its four
// waves and merges the four online-softmax states through LDS.
// Held to three waves per SIMD (160 registers, no spills; uncapped it takes
// 192 and fits two): long-context grids of thousands of items keep a third
// wave's page loads in flight per SIMD.
__device__ __forceinline__ void item4(const AttnArgs& a, int w, float* m_s, float* l_s, float* O_s) {
  // work w takes KV head w % nkv of item w / nkv: the heads of one item (the
  // same pages, adjacent blocks in the pool) are dispatched together, and the
  // longest items' heads all go first
  const AttnItem it = a.items[w / a.nkv];
  const int kh = w % a.nkv;
  const int G = a.nq / a.nkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15;        // row index of the S^T / O^T column this lane holds
  const int grp = lane >> 4;        // which 4-key (or 8-dim) group

  int limit;
  int64_t qoff;
  row_info(a, it, col, G, kh, limit, qoff);
  int max_limit = 0;                // largest causal limit over the item's rows
  for (int t = 0; t < it.ntok; ++t) max_limit = max(max_limit, a.pos[it.tok0 + t] + 1);
  bf16x8 qf[4];
  load_q(a, qoff, grp, qf);
  const float sl2 = a.scale * LOG2E;
  RowState st;
#pragma unroll
  for (int b = 0; b < 8; ++b) st.o[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this wave's pages: page_begin + wave, + 4, ...
  const int first = it.page_begin + wave;
  const int n = first < it.page_end ? (it.page_end - first + 3) / 4 : 0;
  walk_pages(a, it.req, first, 4, n, kh, lane, grp, qf, limit, max_limit, sl2, st);

  // this wave's (m, l, O^T) -> LDS; O^T lane layout: dim 16b + 4*grp + i, row col
  st.l += __shfl_xor(st.l, 16, 64);
  st.l += __shfl_xor(st.l, 32, 64);
  if (grp == 0) {
    m_s[wave * ROWS + col] = st.m;
    l_s[wave * ROWS + col] = st.l;
  }
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) O_s[(wave * ROWS + col) * DH + 16 * b + 4 * grp + i] = st.o[b][i];
  __syncthreads();
  finish_item<bf16>(a, it, G, kh, m_s, l_s, O_s);
}

// One workgroup per work item.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void attn_bf16_d128_kernel(AttnArgs a) {
  __shared__ float m_s[4 * ROWS], l_s[4 * ROWS];
  __shared__ float O_s[4 * ROWS * DH];
  item4(a, blockIdx.x, m_s, l_s, O_s);
}

// A capped grid: each workgroup walks the work list with a stride of the grid
// (a persistent grid that holds a fixed number of workgroups per CU and so
// leaves the rest of the CU's LDS and registers to a concurrent GEMM).  The
// loop keeps its bounds and the item index live across the item, which needs
// 172 registers: held to three waves per SIMD it spilled to scratch, so it
// runs at two (plans bound it to one or two workgroups per CU anyway).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_bf16_d128_loop_kernel(AttnArgs a) {
  __shared__ float m_s[4 * ROWS], l_s[4 * ROWS];
  __shared__ float O_s[4 * ROWS * DH];
  const int n_work = a.n_items * a.nkv;
  for (int w = blockIdx.x; w < n_work; w += gridDim.x) {
    item4(a, w, m_s, l_s, O_s);
    __syncthreads();                 // the next item reuses the LDS
  }
}

// ---------------------------------------------------------------- one wave per item
// One wave64 per work item, no LDS and no barrier: the wave walks its page
// range with the next page's K and V already in flight while the current one
// feeds the matrix cores, and writes either the normalised output or an
// unnormalised partial.  Small and LDS-free, these waves also fit beside the
// GEMM's LDS-heavy workgroups on a CU.
__device__ __forceinline__ void wave_item(const AttnArgs& a, const AttnItem& it, int kh) {
  const int G = a.nq / a.nkv;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;

  int limit;
  int64_t qoff;
  row_info(a, it, col, G, kh, limit, qoff);
  int max_limit = 0;
  for (int t = 0; t < it.ntok; ++t) max_limit = max(max_limit, a.pos[it.tok0 + t] + 1);
  bf16x8 qf[4];
  load_q(a, qoff, grp, qf);
  const float sl2 = a.scale * LOG2E;
  RowState st;
#pragma unroll
  for (int b = 0; b < 8; ++b) st.o[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  walk_pages(a, it.req, it.page_begin, 1, it.page_end - it.page_begin, kh, lane, grp, qf, limit, max_limit, sl2,
             st);

  // row totals: sum the four lane groups that share a column
  st.l += __shfl_xor(st.l, 16, 64);
  st.l += __shfl_xor(st.l, 32, 64);
  const int valid_rows = min(ROWS / G, it.ntok) * G;
  if (col >= valid_rows) return;
  const int t = it.tok0 + col / G;
  const int head = kh * G + col % G;
  // O^T lane layout: dim 16 b + 4 grp + i of row `col`
  if (it.partial < 0) {
    const float invL = st.l > 0.f ? 1.f / st.l : 0.f;
    bf16* o = (bf16*)a.attn + (int64_t)t * a.nq * DH + (int64_t)head * DH;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      bf16x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = (bf16)(st.o[b][q] * invL);
      *(bf16x4*)(o + 16 * b + 4 * grp) = v;
    }
  } else {
    const int64_t base = ((int64_t)it.partial * a.nkv + kh) * ROWS + col;
    float* po = a.part_o + base * DH;
#pragma unroll
    for (int b = 0; b < 8; ++b) *(f32x4*)(po + 16 * b + 4 * grp) = st.o[b];
    if (grp == 0) {
      a.part_ml[base * 2 + 0] = st.m;
      a.part_ml[base * 2 + 1] = st.l;
    }
  }
}

// Work index w = item * nkv + kv head; with a capped grid each wave strides
// over the work list (items are longest first, so the stride balances).
__global__ __launch_bounds__(64) void attn_bf16_d128_wave_kernel(AttnArgs a) {
  const int n_work = a.n_items * a.nkv;
  for (int w = blockIdx.x; w < n_work; w += gridDim.x) wave_item(a, a.items[w / a.nkv], w % a.nkv);
}

// ---------------------------------------------------------------- generic
// Any dtype, any head_dim multiple of 32 up to 256: one wave per row at a
// time, keys walked one by one with an online softmax; lanes split the head
// dimension.
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
      const T* kb = (const T*)a.k_pool + blk * S * d;
      const T* vb = (const T*)a.v_pool + blk * S * d;
      for (int sl = 0; sl < S; ++sl) {
        const int key = lp * S + sl;
        if (key >= limit) break;
        float part = 0.f;
        for (int u = 0; u < DMAX / 64; ++u) {
          const int e = lane + 64 * u;
          if (e < d) part += q[u] * to_f32(kb[kv_k_off(sl, e)]);
        }
        const float sc = wave_sum(part) * a.scale;
        const float mn = fmaxf(m, sc);
        const float al = expf(m - mn);
        const float p = expf(sc - mn);
        l = l * al + p;
        for (int u = 0; u < DMAX / 64; ++u) {
          const int e = lane + 64 * u;
          const float v = e < d ? to_f32(vb[kv_v_off(sl, e)]) : 0.f;
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
  if (dtype == 1 && a.d == 128 && a.page_size == 16) {
    if (a.variant == 1) {
      const int blocks = a.n_items * a.nkv;
      if (a.max_blocks > 0 && blocks > a.max_blocks)
        launch(attn_bf16_d128_loop_kernel, a.max_blocks, 256, 0, s, a);
      else
        launch(attn_bf16_d128_kernel, blocks, 256, 0, s, a);
    } else {
      int blocks = a.n_items * a.nkv;
      if (a.max_blocks > 0 && blocks > a.max_blocks) blocks = a.max_blocks;
      launch(attn_bf16_d128_wave_kernel, blocks, 64, 0, s, a);
    }
  } else if (dtype == 1) {
    launch(attn_generic_kernel<bf16>, grid, 256, 0, s, a);
  } else {
    launch(attn_generic_kernel<float>, grid, 256, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t attention_merge(int dtype, const AttnArgs& a, hipStream_t s) {
  if (a.n_merges == 0) return hipSuccess;
  dim3 grid(a.n_merges, a.nkv);
  if (dtype == 1)
    launch(attn_merge_kernel<bf16>, grid, 256, 0, s, a);
  else
    launch(attn_merge_kernel<float>, grid, 256, 0, s, a);
  return hipGetLastError();
}

}  // namespace nf
