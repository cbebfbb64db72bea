// bf16 GEMMs of the decoder layer on CDNA4 matrix cores (gfx950).
//
// C[M][N] = epilogue(A[M][K] . B[N][K]^T) with both operands K-contiguous
// (activations row-major, weights stored output-feature-major), fp32
// accumulation in v_mfma_f32_16x16x32_bf16.  One 256-thread workgroup (four
// wave64s) owns a BM x BN output tile; K is walked in 64-wide slabs staged
// through LDS, double-buffered, with the next slab's global loads in flight
// while the current slab feeds the matrix cores.  Epilogues fuse the layer's
// elementwise work into the producing GEMM: residual add (O and down
// projections), SwiGLU (gate and up rows of one tile come from the two weight
// matrices so each output column gets both dot products in registers), fp32
// output for the expert path.  Small-M problems (decode-heavy nano-batches)
// use split-K with fp32 partials and a reduce kernel that applies the same
// epilogue.  Workgroups are mapped to tiles XCD-aware: the dispatcher deals
// workgroups round-robin over the 8 XCDs, so each XCD is handed a contiguous
// range of tiles (M fastest) and the weight rows of one N tile stay in one
// XCD's L2.
#include "nf_device.h"
#include "nf_internal.h"

namespace nf {
namespace {

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;   // bf16 elements per LDS row (144 B: breaks bank aliasing)
constexpr int NXCD = 8;

template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static constexpr int A_LOADS = BM * 8 / 256, B_LOADS = BN * 8 / 256;
  static_assert(WM * WN == 4, "four waves");
  static_assert(FM >= 1 && FN >= 2 && FN % 2 == 0, "wave tile");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "loads");
};

using Cfg0 = Cfg<128, 128, 2, 2>;
using Cfg1 = Cfg<64, 128, 1, 4>;
using Cfg2 = Cfg<256, 128, 2, 2>;
using Cfg3 = Cfg<32, 128, 1, 4>;
using Cfg4 = Cfg<128, 256, 2, 2>;

struct KParams {
  GemmArgs a;
  int m_tiles, n_tiles, z_count;   // z: k split or group
  int k_per;                        // K per split (multiple of BK)
  float* part;                      // split-K partials
  int64_t part_ld;                  // row stride of partials
};

__device__ __forceinline__ int xcd_logical(int L, int total) {
  const int xcd = L % NXCD, slot = L / NXCD;
  const int q = total / NXCD, r = total % NXCD;
  return xcd * q + min(xcd, r) + slot;
}

template <class C, int MODE, bool PARTIAL>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(KParams p) {
  __shared__ __attribute__((aligned(16))) bf16 As[2][C::BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][C::BN * LDS_STRIDE];

  const GemmArgs& a = p.a;
  const int total = p.m_tiles * p.n_tiles * p.z_count;
  const int logical = xcd_logical(blockIdx.x, total);
  const int m_tile = logical % p.m_tiles;
  const int rest = logical / p.m_tiles;
  const int n_tile = rest % p.n_tiles;
  const int z = rest / p.n_tiles;

  int m_begin = 0, rows = a.M;
  if (a.group_off) {
    m_begin = a.group_off[z];
    rows = a.group_off[z + 1] - m_begin;
  }
  const int m0 = m_tile * C::BM;
  if (m0 >= rows) return;                       // whole workgroup exits together

  int k_lo = 0, k_hi = a.K;
  if (PARTIAL) {
    k_lo = z * p.k_per;
    k_hi = min(a.K, k_lo + p.k_per);
  }
  const bf16* Bbase = (const bf16*)a.B;
  const bf16* B2base = (const bf16*)a.B2;
  if (a.group_off) {
    Bbase += (int64_t)z * a.b_group_stride;
    if (B2base) B2base += (int64_t)z * a.b_group_stride;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;

  // per-thread global source rows for the A and B slabs
  const bf16* pa[C::A_LOADS];
  bool va[C::A_LOADS];
  const bf16* pb[C::B_LOADS];
  bool vb[C::B_LOADS];
  const int col8 = (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int row = (tid + 256 * i) >> 3;
    const int local = m0 + row;
    va[i] = local < rows;
    int src = m_begin + (va[i] ? local : 0);
    if (a.a_rows) src = a.a_rows[src] / a.a_row_div;
    pa[i] = (const bf16*)a.A + (int64_t)src * a.lda + col8;
  }
#pragma unroll
  for (int i = 0; i < C::B_LOADS; ++i) {
    const int row = (tid + 256 * i) >> 3;
    int n;
    const bf16* base;
    if (MODE == GEMM_SWIGLU) {
      const int half = C::BN / 2;
      n = n_tile * half + (row < half ? row : row - half);
      base = row < half ? Bbase : B2base;
    } else {
      n = n_tile * C::BN + row;
      base = Bbase;
    }
    vb[i] = n < a.N;
    pb[i] = base + (int64_t)(vb[i] ? n : 0) * a.ldb + col8;
  }

  u32x4 ra[C::A_LOADS], rb[C::B_LOADS];
  auto load_slab = [&](int k0) {
    const bool kin = k0 + col8 < k_hi;
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i)
      ra[i] = (va[i] && kin) ? *(const u32x4*)(pa[i] + k0) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i)
      rb[i] = (vb[i] && kin) ? *(const u32x4*)(pb[i] + k0) : u32x4{0, 0, 0, 0};
  };
  auto store_slab = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
      const int row = (tid + 256 * i) >> 3;
      *(u32x4*)&As[buf][row * LDS_STRIDE + col8] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
      const int row = (tid + 256 * i) >> 3;
      *(u32x4*)&Bs[buf][row * LDS_STRIDE + col8] = rb[i];
    }
  };

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS row of B fragment j for this wave
  auto b_row = [&](int j) {
    if (MODE == GEMM_SWIGLU) {
      constexpr int HF = C::FN / 2;
      return j < HF ? wn * (C::WTN / 2) + j * 16 : C::BN / 2 + wn * (C::WTN / 2) + (j - HF) * 16;
    }
    return wn * C::WTN + j * 16;
  };

  const int nk = (k_hi - k_lo + BK - 1) / BK;
  load_slab(k_lo);
  store_slab(0);
  __syncthreads();
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_slab(k_lo + (kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        af[i] = *(const bf16x8*)&As[buf][(wm * C::WTM + i * 16 + fr) * LDS_STRIDE + s * 32 + fk];
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        bfr[j] = *(const bf16x8*)&Bs[buf][(b_row(j) + fr) * LDS_STRIDE + s * 32 + fk];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_slab(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds D[m = 4*(lane/16) + r][n = lane % 16] of each 16x16 block
  const int er = (lane >> 4) * 4, ec = lane & 15;
  constexpr int NJ = (MODE == GEMM_SWIGLU) ? C::FN / 2 : C::FN;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int local = m0 + wm * C::WTM + i * 16 + er + r;
      if (local >= rows) continue;
      const int64_t orow = m_begin + local;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (MODE == GEMM_SWIGLU) {
          const int col = n_tile * (C::BN / 2) + wn * (C::WTN / 2) + j * 16 + ec;
          if (col >= a.N) continue;
          const float g = acc[i][j][r], u = acc[i][j + C::FN / 2][r];
          if (PARTIAL) {
            float* P = p.part + (int64_t)z * a.M * p.part_ld + orow * p.part_ld;
            P[col] = g;
            P[a.N + col] = u;
          } else {
            ((bf16*)a.C)[orow * a.ldc + col] = (bf16)(silu_f(g) * u);
          }
        } else {
          const int col = n_tile * C::BN + wn * C::WTN + j * 16 + ec;
          if (col >= a.N) continue;
          const float v = acc[i][j][r];
          if (PARTIAL) {
            p.part[(int64_t)z * a.M * p.part_ld + orow * p.part_ld + col] = v;
          } else if (MODE == GEMM_STORE) {
            ((bf16*)a.C)[orow * a.ldc + col] = (bf16)v;
          } else if (MODE == GEMM_RESIDUAL) {
            const float res = (float)((const bf16*)a.R)[orow * a.ldr + col];
            ((bf16*)a.C)[orow * a.ldc + col] = (bf16)(v + res);
          } else {
            ((float*)a.C)[orow * a.ldc + col] = v;
          }
        }
      }
    }
  }
}

// Sum of split-K partials + the mode's epilogue; 4 consecutive columns per thread.
template <int MODE>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs a, const float* part,
                                                            int64_t part_ld, int splits) {
  const int cols4 = (a.N + 3) / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.M * cols4) return;
  const int row = (int)(idx / cols4);
  const int c0 = (int)(idx % cols4) * 4;
  for (int c = c0; c < min(c0 + 4, a.N); ++c) {
    float v = 0.f, u = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float* P = part + (int64_t)s * a.M * part_ld + (int64_t)row * part_ld;
      v += P[c];
      if (MODE == GEMM_SWIGLU) u += P[a.N + c];
    }
    if (MODE == GEMM_SWIGLU) {
      ((bf16*)a.C)[(int64_t)row * a.ldc + c] = (bf16)(silu_f(v) * u);
    } else if (MODE == GEMM_STORE) {
      ((bf16*)a.C)[(int64_t)row * a.ldc + c] = (bf16)v;
    } else if (MODE == GEMM_RESIDUAL) {
      const float res = (float)((const bf16*)a.R)[(int64_t)row * a.ldr + c];
      ((bf16*)a.C)[(int64_t)row * a.ldc + c] = (bf16)(v + res);
    } else {
      ((float*)a.C)[(int64_t)row * a.ldc + c] = v;
    }
  }
}

template <class C>
int tiles_n(const GemmArgs& a) {
  const int bn = a.mode == GEMM_SWIGLU ? C::BN / 2 : C::BN;
  return (a.N + bn - 1) / bn;
}

template <class C>
hipError_t launch_cfg(const GemmArgs& a, const GemmPlan& pl, void* ws, hipStream_t s,
                      const LaunchHook* hook) {
  KParams p;
  p.a = a;
  const int rows = a.group_off ? a.max_group_rows : a.M;
  p.m_tiles = (rows + C::BM - 1) / C::BM;
  p.n_tiles = tiles_n<C>(a);
  p.part = (float*)ws;
  p.part_ld = a.mode == GEMM_SWIGLU ? 2 * (int64_t)a.N : a.N;
  const bool split = pl.k_splits > 1 && !a.group_off;
  if (split) {
    const int kb = (a.K + BK - 1) / BK;
    p.k_per = ((kb + pl.k_splits - 1) / pl.k_splits) * BK;
    p.z_count = (a.K + p.k_per - 1) / p.k_per;
  } else {
    p.k_per = a.K;
    p.z_count = a.group_off ? a.n_groups : 1;
  }
  const int total = p.m_tiles * p.n_tiles * p.z_count;
  if (total == 0) return hipSuccess;
  if (!split) {
    switch (a.mode) {
      case GEMM_STORE: gemm_bf16_kernel<C, GEMM_STORE, false><<<total, 256, 0, s>>>(p); break;
      case GEMM_RESIDUAL: gemm_bf16_kernel<C, GEMM_RESIDUAL, false><<<total, 256, 0, s>>>(p); break;
      case GEMM_SWIGLU: gemm_bf16_kernel<C, GEMM_SWIGLU, false><<<total, 256, 0, s>>>(p); break;
      default: gemm_bf16_kernel<C, GEMM_F32OUT, false><<<total, 256, 0, s>>>(p); break;
    }
    return hipGetLastError();
  }
  if (a.mode == GEMM_SWIGLU)
    gemm_bf16_kernel<C, GEMM_SWIGLU, true><<<total, 256, 0, s>>>(p);
  else
    gemm_bf16_kernel<C, GEMM_STORE, true><<<total, 256, 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (hook && hook->fn) hook->fn(hook->ctx, 1);
  const int64_t work = (int64_t)a.M * ((a.N + 3) / 4);
  const int blocks = (int)((work + 255) / 256);
  switch (a.mode) {
    case GEMM_STORE: splitk_reduce_kernel<GEMM_STORE><<<blocks, 256, 0, s>>>(a, p.part, p.part_ld, p.z_count); break;
    case GEMM_RESIDUAL: splitk_reduce_kernel<GEMM_RESIDUAL><<<blocks, 256, 0, s>>>(a, p.part, p.part_ld, p.z_count); break;
    case GEMM_SWIGLU: splitk_reduce_kernel<GEMM_SWIGLU><<<blocks, 256, 0, s>>>(a, p.part, p.part_ld, p.z_count); break;
    default: splitk_reduce_kernel<GEMM_F32OUT><<<blocks, 256, 0, s>>>(a, p.part, p.part_ld, p.z_count); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- fp32 path
// Plain LDS-tiled fp32 GEMM (64x64 tiles, 4x4 outputs per thread) for fp32
// layers; same operand layouts and epilogues as the bf16 path.
template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int T = 64, TK = 16;
  __shared__ float As[TK][T + 1];
  __shared__ float Bs[TK][T + 1];
  const int n_tile = blockIdx.x, m_tile = blockIdx.y;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  float acc2[4][4] = {};
  const float* A = (const float*)a.A;
  const float* B = (const float*)a.B;
  const float* B2 = (const float*)a.B2;
  const int nb = n_tile * T;
  for (int k0 = 0; k0 < a.K; k0 += TK) {
    for (int e = threadIdx.x; e < T * TK; e += 256) {
      const int r = e / TK, k = e % TK;
      const int m = m_tile * T + r, n = nb + r;
      As[k][r] = (m < a.M && k0 + k < a.K) ? A[(int64_t)m * a.lda + k0 + k] : 0.f;
      Bs[k][r] = (n < a.N && k0 + k < a.K) ? B[(int64_t)n * a.ldb + k0 + k] : 0.f;
    }
    __syncthreads();
    for (int k = 0; k < TK; ++k)
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] += As[k][ty * 4 + i] * Bs[k][tx * 4 + j];
    __syncthreads();
    if (MODE == GEMM_SWIGLU) {
      for (int e = threadIdx.x; e < T * TK; e += 256) {
        const int r = e / TK, k = e % TK;
        const int n = nb + r;
        Bs[k][r] = (n < a.N && k0 + k < a.K) ? B2[(int64_t)n * a.ldb + k0 + k] : 0.f;
      }
      __syncthreads();
      for (int k = 0; k < TK; ++k)
        for (int i = 0; i < 4; ++i)
          for (int j = 0; j < 4; ++j) acc2[i][j] += As[k][ty * 4 + i] * Bs[k][tx * 4 + j];
      __syncthreads();
    }
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int m = m_tile * T + ty * 4 + i, n = nb + tx * 4 + j;
      if (m >= a.M || n >= a.N) continue;
      float v = acc[i][j];
      if (MODE == GEMM_SWIGLU) v = (v / (1.0f + expf(-v))) * acc2[i][j];
      if (MODE == GEMM_RESIDUAL) v += ((const float*)a.R)[(int64_t)m * a.ldr + n];
      ((float*)a.C)[(int64_t)m * a.ldc + n] = v;
    }
}

}  // namespace

GemmPlan gemm_choose(const GemmArgs& a, int cus) {
  GemmPlan p;
  if (cus <= 0) cus = 256;
  if (a.group_off) {            // grouped (experts): rows per group ~ tokens*k/E
    p.cfg = 0;
    return p;
  }
  const int M = a.M;
  auto ntile = [&](int bn) { return (a.N + (a.mode == GEMM_SWIGLU ? bn / 2 : bn) - 1) / (a.mode == GEMM_SWIGLU ? bn / 2 : bn); };
  int bm;
  if (M <= 32) { p.cfg = 3; bm = 32; }
  else if (M <= 64) { p.cfg = 1; bm = 64; }
  else if (M >= 1024 && ((M + 255) / 256) * ntile(128) >= cus) { p.cfg = 2; bm = 256; }
  else { p.cfg = 0; bm = 128; }
  const int tiles = ((M + bm - 1) / bm) * ntile(128);
  if (tiles < cus) {
    int ks = (cus + tiles - 1) / tiles;
    const int max_ks = a.K / 512;           // keep >= 512 of K per split
    if (ks > max_ks) ks = max_ks;
    if (ks > 8) ks = 8;
    if (ks > 1) p.k_splits = ks;
  }
  return p;
}

size_t gemm_workspace_bytes(const GemmArgs& a, const GemmPlan& p) {
  if (p.k_splits <= 1 || a.group_off) return 0;
  const int64_t ld = a.mode == GEMM_SWIGLU ? 2 * (int64_t)a.N : a.N;
  return (size_t)p.k_splits * a.M * ld * sizeof(float);
}

hipError_t gemm_bf16(const GemmArgs& a, const GemmPlan& p, void* ws, hipStream_t s, const LaunchHook* hook) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  switch (p.cfg) {
    case 1: return launch_cfg<Cfg1>(a, p, ws, s, hook);
    case 2: return launch_cfg<Cfg2>(a, p, ws, s, hook);
    case 3: return launch_cfg<Cfg3>(a, p, ws, s, hook);
    case 4: return launch_cfg<Cfg4>(a, p, ws, s, hook);
    default: return launch_cfg<Cfg0>(a, p, ws, s, hook);
  }
}

hipError_t gemm_f32(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
  switch (a.mode) {
    case GEMM_RESIDUAL: gemm_f32_kernel<GEMM_RESIDUAL><<<grid, 256, 0, s>>>(a); break;
    case GEMM_SWIGLU: gemm_f32_kernel<GEMM_SWIGLU><<<grid, 256, 0, s>>>(a); break;
    default: gemm_f32_kernel<GEMM_STORE><<<grid, 256, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace nf
