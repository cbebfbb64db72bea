// bf16 GEMMs of the decoder layer on CDNA4 matrix cores (gfx950).
//
// C[M][N] = epilogue(A[M][K] . B[N][K]^T) with both operands K-contiguous
// (activations row-major, weights stored output-feature-major), fp32
// accumulation in v_mfma_f32_32x32x16_bf16 (large tiles) or
// v_mfma_f32_16x16x32_bf16 (decode-sized tiles).  One 256-thread workgroup
// (four wave64s) owns a BM x BN output tile; K is walked in slabs that the
// buffer unit writes straight into LDS (buffer_load ... lds), several slabs
// in flight, while the current slab feeds the matrix cores.  Epilogues fuse
// the layer's elementwise work into the producing GEMM: residual add (O and
// down projections), SwiGLU (gate and up rows of one tile come from the two
// weight matrices so each output column gets both dot products in
// registers), fp32 output for the expert path.  Small-M problems
// (decode-heavy nano-batches) use split-K with fp32 partials and a reduce
// kernel that applies the same epilogue.  Workgroups are mapped to tiles
// XCD-aware: the dispatcher deals workgroups round-robin over the 8 XCDs, so
// each XCD is handed a contiguous range of tiles (M fastest) and the weight
// rows of one N tile stay in one XCD's L2.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <type_traits>
#include <vector>

#include "nf_device.h"
#include "nf_internal.h"

namespace nf {
namespace {

constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;   // bf16 elements per LDS row (144 B: breaks bank aliasing)

template <int BM_, int BN_, int WM_, int WN_, int MS_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int MS = MS_;                    // MFMA block: 16x16x32 or 32x32x16
  static constexpr int KSTEP = MS == 16 ? 32 : 16;  // K per MFMA
  static constexpr int NACC = MS == 16 ? 4 : 16;    // accumulators per lane per block
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / MS, FN = WTN / MS;
  static constexpr int A_LOADS = BM * 8 / 256, B_LOADS = BN * 8 / 256;
  static_assert(WM * WN == 4, "four waves");
  static_assert(MS == 16 || MS == 32, "mfma shape");
  static_assert(FM >= 1 && FN >= 2 && FN % 2 == 0, "wave tile");
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "loads");
};

// 16x16x32 configs for decode-sized M (weight-streaming); 32x32x16 configs,
// which run at twice the rate on gfx950, for compute-bound M.
using Cfg0 = Cfg<128, 128, 2, 2, 32>;
using Cfg1 = Cfg<64, 128, 1, 4, 16>;
using Cfg2 = Cfg<256, 128, 2, 2, 32>;
using Cfg3 = Cfg<32, 128, 1, 4, 16>;
using Cfg4 = Cfg<128, 256, 2, 2, 32>;
using Cfg5 = Cfg<256, 256, 2, 2, 32>;
using Cfg6 = Cfg<64, 128, 2, 2, 32>;

template <int MS> struct Acc;
template <> struct Acc<16> { typedef f32x4 T; };
template <> struct Acc<32> { typedef f32x16 T; };

template <int MS>
__device__ __forceinline__ typename Acc<MS>::T mfma(const bf16x8& a, const bf16x8& b, const typename Acc<MS>::T& c) {
  if constexpr (MS == 16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of accumulator element r (within an MS x MS block) held by `lane`;
// the column is lane % MS.
template <int MS>
__device__ __forceinline__ int acc_row(int lane, int r) {
  if constexpr (MS == 16)
    return 4 * (lane >> 4) + r;
  else
    return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

struct KParams {
  GemmArgs a;
  int m_tiles, n_tiles, z_count;   // z: k split or group
  int k_per;                        // K per split (multiple of BK)
  float* part;                      // split-K partials
  int64_t part_ld;                  // row stride of partials
  int vec_epi = 0;                  // C (and R) rows 16-byte aligned, N % 8 == 0
};




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

  typedef typename Acc<C::MS>::T AccT;
  AccT acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int e = 0; e < C::NACC; ++e) acc[i][j][e] = 0.f;

  // LDS row of B fragment j for this wave
  auto b_row = [&](int j) {
    if (MODE == GEMM_SWIGLU) {
      constexpr int HF = C::FN / 2;
      return j < HF ? wn * (C::WTN / 2) + j * C::MS : C::BN / 2 + wn * (C::WTN / 2) + (j - HF) * C::MS;
    }
    return wn * C::WTN + j * C::MS;
  };

  const int nk = (k_hi - k_lo + BK - 1) / BK;
  load_slab(k_lo);
  store_slab(0);
  __syncthreads();
  // fragment of lane: row lane % MS of the block, 8 consecutive k at 8 * (lane / MS)
  const int fr = lane % C::MS, fk = (lane / C::MS) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_slab(k_lo + (kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < BK / C::KSTEP; ++s) {
      bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        af[i] = *(const bf16x8*)&As[buf][(wm * C::WTM + i * C::MS + fr) * LDS_STRIDE + s * C::KSTEP + fk];
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        bfr[j] = *(const bf16x8*)&Bs[buf][(b_row(j) + fr) * LDS_STRIDE + s * C::KSTEP + fk];
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma<C::MS>(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) store_slab(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds D[acc_row(lane, r)][lane % MS] of each block
  const int ec = lane % C::MS;
  constexpr int NJ = (MODE == GEMM_SWIGLU) ? C::FN / 2 : C::FN;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int r = 0; r < C::NACC; ++r) {
      const int local = m0 + wm * C::WTM + i * C::MS + acc_row<C::MS>(lane, r);
      if (local >= rows) continue;
      const int64_t orow = m_begin + local;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (MODE == GEMM_SWIGLU) {
          const int col = n_tile * (C::BN / 2) + wn * (C::WTN / 2) + j * C::MS + ec;
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
          const int col = n_tile * C::BN + wn * C::WTN + j * C::MS + ec;
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

// Sum of split-K partials + the mode's epilogue; 4 consecutive columns per
// thread, 16-byte partial loads (N % 4 == 0: hidden, ffn and head_dim are
// multiples of 8).
template <int MODE>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs a, const float* __restrict__ part,
                                                            int64_t part_ld, int splits) {
  const int cols4 = a.N / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)a.M * cols4) return;
  const int row = (int)(idx / cols4);
  const int c = (int)(idx % cols4) * 4;
  const int64_t zstride = (int64_t)a.M * part_ld;
  const float* P = part + (int64_t)row * part_ld + c;
  const f32x4 v = sum_slices<f32x4>(P, zstride, splits);
  f32x4 u = {0.f, 0.f, 0.f, 0.f};
  if (MODE == GEMM_SWIGLU) u = sum_slices<f32x4>(P + a.N, zstride, splits);
  const int64_t o = (int64_t)row * a.ldc + c;
  if (MODE == GEMM_F32OUT) {
    *(f32x4*)((float*)a.C + o) = v;
    return;
  }
  bf16x4 out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float r = v[q];
    if (MODE == GEMM_SWIGLU) r = silu_f(v[q]) * u[q];
    if (MODE == GEMM_RESIDUAL) r += (float)((const bf16*)a.R)[(int64_t)row * a.ldr + c + q];
    out[q] = (bf16)r;
  }
  *(bf16x4*)((bf16*)a.C + o) = out;
}

hipError_t splitk_reduce_impl(const GemmArgs& a, const float* part, int64_t part_ld, int splits, hipStream_t s) {
  const int64_t work = (int64_t)a.M * (a.N / 4);
  const int blocks = (int)((work + 255) / 256);
  switch (a.mode) {
    case GEMM_STORE: launch(splitk_reduce_kernel<GEMM_STORE>, blocks, 256, 0, s, a, part, part_ld, splits); break;
    case GEMM_RESIDUAL: launch(splitk_reduce_kernel<GEMM_RESIDUAL>, blocks, 256, 0, s, a, part, part_ld, splits); break;
    case GEMM_SWIGLU: launch(splitk_reduce_kernel<GEMM_SWIGLU>, blocks, 256, 0, s, a, part, part_ld, splits); break;
    default: launch(splitk_reduce_kernel<GEMM_F32OUT>, blocks, 256, 0, s, a, part, part_ld, splits); break;
  }
  return hipGetLastError();
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
  p.part_ld = a.mode == GEMM_SWIGLU ? 2 * (int64_t)a.N : a.N;
  bool split = pl.k_splits > 1 && !a.group_off;
  if (split) {
    const int kb = (a.K + BK - 1) / BK;
    p.k_per = ((kb + pl.k_splits - 1) / pl.k_splits) * BK;
    p.z_count = (a.K + p.k_per - 1) / p.k_per;
    split = p.z_count > 1;
  }
  if (!split) {
    p.k_per = a.K;
    p.z_count = a.group_off ? a.n_groups : 1;
  }
  p.part = split ? (float*)ws : nullptr;
  if (split && !ws) return hipErrorInvalidValue;            // split-K needs the workspace
  const int total = p.m_tiles * p.n_tiles * p.z_count;
  if (total == 0) return hipSuccess;
  if (!split) {
    switch (a.mode) {
      case GEMM_STORE: launch(gemm_bf16_kernel<C, GEMM_STORE, false>, total, 256, 0, s, p); break;
      case GEMM_RESIDUAL: launch(gemm_bf16_kernel<C, GEMM_RESIDUAL, false>, total, 256, 0, s, p); break;
      case GEMM_SWIGLU: launch(gemm_bf16_kernel<C, GEMM_SWIGLU, false>, total, 256, 0, s, p); break;
      default: launch(gemm_bf16_kernel<C, GEMM_F32OUT, false>, total, 256, 0, s, p); break;
    }
    return hipGetLastError();
  }
  if (a.mode == GEMM_SWIGLU)
    launch(gemm_bf16_kernel<C, GEMM_SWIGLU, true>, total, 256, 0, s, p);
  else
    launch(gemm_bf16_kernel<C, GEMM_STORE, true>, total, 256, 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.defer_reduce) return e;
  if (hook && hook->fn) hook->fn(hook->ctx, 1);
  return splitk_reduce(a, p.part, p.part_ld, p.z_count, s);
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

// ---------------------------------------------------------------- pipelined path
// For K % 64 == 0.  Slabs go global -> LDS with gfx950's direct 16-byte loads
// (global_load_lds_dwordx4), with no VGPR staging, so STAGES-1 slabs are in
// flight while the matrix cores work on the oldest; the wait is an explicit
// vmcnt on this wave's own loads followed by a workgroup barrier.  LDS rows
// are 128 bytes (64 bf16) with their 16-byte chunks XOR-swizzled by
// (row / 2) % 8: a DMA instruction still writes 8 whole rows (1 KB,
// contiguous), and the 16 lanes of a fragment read (16 rows, one chunk) hit 64
// distinct banks.  Split-K stores fp32 partials; a vectorised reduce kernel
// applies the epilogue (a last-arriving-workgroup reduction would need
// device-scope fences, which on a multi-XCD part write back the L2).
template <int BM_, int BN_, int WM_, int WN_, int MS_, int ST_, int BK_ = 64>
struct PCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, MS = MS_, STAGES = ST_, BK = BK_;
  static constexpr int KSTEP = MS == 16 ? 32 : 16;
  static constexpr int KS = BK / KSTEP;                  // MFMA k-steps per slab
  static constexpr int NACC = MS == 16 ? 4 : 16;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / MS, FN = WTN / MS;
  static constexpr int ROWB = BK * 2;                    // LDS bytes per slab row
  static constexpr int CPR = ROWB / 16;                  // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROWB;                // rows one DMA instruction fills
  static constexpr int A_IN = BM / (4 * RPI), B_IN = BN / (4 * RPI);   // DMA instructions per thread per slab
  static constexpr int X = A_IN + B_IN;
  static constexpr int SLAB = (BM + BN) * ROWB;          // LDS bytes per stage
  static_assert(BK == 64 || BK == 32, "slab K");
  static_assert(WM * WN == 4 && FM >= 1 && FN >= 2 && FN % 2 == 0 && A_IN >= 1 && B_IN >= 1 && KS >= 1, "cfg");
  static_assert(STAGES >= 2 && STAGES <= 10 && (STAGES - 1) * X <= 63, "vmcnt range");
  static_assert(STAGES * SLAB <= 160 * 1024, "LDS");
  // Slab refills spread over the MFMAs (else issued in one burst): for tiles
  // that run one workgroup per CU, whose single wave per SIMD would leave the
  // matrix unit idle while it waits to issue a burst.  With two workgroups
  // per CU the other one's MFMAs fill that time, and decode-sized tiles gain
  // more from the earlier issue.
  static constexpr bool SPREAD = (160 * 1024) / (STAGES * SLAB) == 1 && BM >= 128;
};

using P10 = PCfg<256, 256, 2, 2, 32, 2>;
using P11 = PCfg<256, 128, 2, 2, 32, 3>;
using P12 = PCfg<128, 256, 2, 2, 32, 3>;
using P13 = PCfg<128, 128, 2, 2, 32, 3>;
using P14 = PCfg<128, 128, 2, 2, 32, 2>;
using P15 = PCfg<64, 128, 1, 4, 16, 4>;
using P16 = PCfg<32, 128, 1, 4, 16, 4>;
using P17 = PCfg<64, 256, 1, 4, 16, 3>;
using P18 = PCfg<64, 128, 1, 4, 16, 6>;
using P19 = PCfg<32, 128, 1, 4, 16, 6>;
using P20 = PCfg<32, 128, 1, 4, 16, 8>;
// 32-wide K slabs (more slabs in flight for the same LDS; measured slower
// than P14 on the large shapes, kept as a probe configuration)
using P21 = PCfg<256, 256, 2, 2, 32, 4, 32>;
using P22 = PCfg<128, 128, 2, 2, 32, 4, 32>;
using P23 = PCfg<128, 128, 2, 2, 32, 5, 32>;
using P24 = PCfg<256, 128, 2, 2, 32, 4, 32>;
using P25 = PCfg<128, 256, 2, 2, 32, 4, 32>;
using P26 = PCfg<256, 256, 2, 2, 32, 3, 32>;
using P27 = PCfg<256, 256, 2, 2, 32, 5, 32>;
using P28 = PCfg<256, 128, 2, 2, 32, 5, 32>;
using P29 = PCfg<128, 128, 2, 2, 32, 9, 32>;
// expert groups of up to 160 rows: one m-tile per group, three 52 KB stages
using P30 = PCfg<160, 256, 1, 4, 32, 3>;


// Output rows staged through LDS per epilogue pass: the whole tile if it
// fits, else the largest power of two (>= 32, so fragment blocks never
// straddle passes) that fits and divides the tile.
constexpr int stage_rows(int bm, int fit) {
  if (fit >= bm) return bm;
  for (int p = 128; p >= 32; p /= 2)
    if (p <= fit && bm % p == 0) return p;
  return 0;
}

// f(integral_constant<int, U>) for U = B .. N - 1, in order
template <int B, int N, class F>
__device__ __forceinline__ void unroll_n(F&& f) {
  if constexpr (B < N) {
    f(std::integral_constant<int, B>{});
    unroll_n<B + 1, N>(f);
  }
}

// wait until at most `after` slabs issued after the current one are pending
// (each slab is X loads of this thread, and loads retire in order)
template <class C, int A = C::STAGES - 2>
__device__ __forceinline__ void wait_slab(int after) {
  if constexpr (A > 0) {
    if (after >= A) {
      wait_vmcnt<A * C::X>();
      return;
    }
    wait_slab<C, A - 1>(after);
  } else {
    wait_vmcnt<0>();
  }
}

// XOR swizzle of a row's 16-byte chunks: the 16 rows of a fragment read land
// on 16 distinct 16-byte bank groups (2 rows per 256-byte bank window for
// 128-byte rows, 4 for 64-byte rows)
template <class C>
__device__ __forceinline__ int swz(int row) {
  if constexpr (C::BK == 64)
    return (row >> 1) & 7;
  else
    return (row >> 2) & 3;
}


template <class C, int MODE, bool PARTIAL>
__global__ __launch_bounds__(256) void gemm_pipe_kernel(KParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[C::STAGES * C::SLAB];
  const GemmArgs& a = p.a;
  const int total = p.m_tiles * p.n_tiles * p.z_count;
  if ((int)blockIdx.x >= total) {               // extra blocks: the step's metadata copy
    const u32x4* src = (const u32x4*)a.meta.src;
    u32x4* dst = (u32x4*)a.meta.dst;
    const int64_t nb = gridDim.x - total;
    for (int64_t i = (int64_t)(blockIdx.x - total) * 256 + threadIdx.x; i < a.meta.n16; i += nb * 256)
      dst[i] = src[i];
    return;
  }
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
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;

  // DMA sources: instruction i of this wave fills slab rows (4i + wave) RPI ..
  // + RPI - 1; lane l takes row + l / CPR and physical chunk l % CPR (logical
  // chunk = physical ^ swz).  Byte offsets from the operand's base (32-bit:
  // the shape check keeps every operand under 4 GiB); the slab's K offset is
  // the scalar offset of each load.
  const __amdgpu_buffer_rsrc_t rA = buf_rsrc(a.A);
  const __amdgpu_buffer_rsrc_t rB = buf_rsrc(Bbase);
  const __amdgpu_buffer_rsrc_t rB2 = buf_rsrc(MODE == GEMM_SWIGLU ? B2base : Bbase);
  const __amdgpu_buffer_rsrc_t rNone = buf_rsrc_empty(a.A);
  uint32_t offA[C::A_IN], offB[C::B_IN];
  const int lrow = lane / C::CPR, pch = lane % C::CPR;
#pragma unroll
  for (int i = 0; i < C::A_IN; ++i) {
    const int row = (4 * i + wave) * C::RPI + lrow;
    const int local = min(m0 + row, rows - 1);            // clamp: rows past M are never stored
    int src = m_begin + local;
    if (a.a_rows) src = a.a_rows[src] / a.a_row_div;
    offA[i] = (uint32_t)(((int64_t)src * a.lda + k_lo + 8 * (pch ^ swz<C>(row))) * 2);
  }
#pragma unroll
  for (int i = 0; i < C::B_IN; ++i) {
    const int row = (4 * i + wave) * C::RPI + lrow;
    int n;
    if (MODE == GEMM_SWIGLU) {
      // an instruction's RPI rows lie in one half (gate rows, then up rows)
      constexpr int half = C::BN / 2;
      n = n_tile * half + (row < half ? row : row - half);
    } else {
      n = n_tile * C::BN + row;
    }
    n = min(n, a.N - 1);
    offB[i] = (uint32_t)(((int64_t)n * a.ldb + k_lo + 8 * (pch ^ swz<C>(row))) * 2);
  }
  // Load d (of X) of slab t into stage buffer buf.  Slabs past the end
  // (real == false) go through the empty resource: no memory moves, but every
  // wave issues the same X loads per slab, so the slab waits are constant
  // vmcnt counts.
  auto dma1 = [&](int t, int buf, bool real, int d) {
    const uint32_t koff = (uint32_t)(t * C::BK * 2);
    char* sA = smem + buf * C::SLAB;
    if (d < C::A_IN) {
      dma16_buf(real ? rA : rNone, offA[d], koff, sA + (4 * d + wave) * 1024);
    } else {
      const int i = d - C::A_IN;
      const bool up = MODE == GEMM_SWIGLU && (4 * i + wave) * C::RPI >= C::BN / 2;   // wave-uniform
      dma16_buf(real ? (up ? rB2 : rB) : rNone, offB[i], koff, sA + C::BM * C::ROWB + (4 * i + wave) * 1024);
    }
  };

  typedef typename Acc<C::MS>::T AccT;
  AccT acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int e = 0; e < C::NACC; ++e) acc[i][j][e] = 0.f;

  auto b_row = [&](int j) {
    if (MODE == GEMM_SWIGLU) {
      constexpr int HF = C::FN / 2;
      return j < HF ? wn * (C::WTN / 2) + j * C::MS : C::BN / 2 + wn * (C::WTN / 2) + (j - HF) * C::MS;
    }
    return wn * C::WTN + j * C::MS;
  };

  const int nk = (k_hi - k_lo) / C::BK;
  // row fragments of this wave that hold at least one live row (wave-uniform);
  // the rest skip their fragment loads and MFMAs (ragged groups, M % BM)
  const int live = __builtin_amdgcn_readfirstlane(min(C::FM, max(0, (rows - m0 - wm * C::WTM + C::MS - 1) / C::MS)));
  // prologue: every stage's buffer receives a slab (with SPREAD, slabs past
  // the end as empty loads)
#pragma unroll
  for (int t = 0; t < C::STAGES; ++t)
    if (C::SPREAD || t < nk)
#pragma unroll
      for (int d = 0; d < C::X; ++d) dma1(t, t, t < nk, d);
  const int fr = lane % C::MS, fq = lane / C::MS;
  // Fragment reads run L k-steps ahead of the MFMAs.  A slab's barrier sits
  // where its last reads have been issued: after it the slab's buffer takes
  // slab kt + STAGES, and the next slab's first L k-steps are read while the
  // MFMAs of this slab's last L k-steps run, so no LDS round trip is exposed
  // at a slab boundary.  With SPREAD the refill loads are spread evenly over
  // those MFMAs: the CU's path from L2 takes about as long to accept a slab
  // as the MFMAs of half a slab take, and a wave waiting to issue a load
  // issues no MFMA, so a burst of loads would leave the matrix unit idle.
  // The instruction order is fixed by scheduling barriers (the compiler's own
  // interleaving bunched the loads).  The k loop is instantiated twice:
  // without the live-row checks when every row fragment of the wave is live
  // (straight-line code), and with them for the ragged tiles.
  constexpr int KS = C::KS;
  constexpr int L = KS > 2 ? 2 : 1;
  auto k_loop_spread = [&](auto checked) {
    constexpr bool CHECK = decltype(checked)::value;
    bf16x8 af[KS][C::FM], bfr[KS][C::FN];
    // fragment read r of k-step s: A row fragments first, then B
    auto read1 = [&](const char* sA, int s, int r) {
      const int c = s * (C::KSTEP / 8) + fq;
      if (r < C::FM) {
        if (CHECK && r >= live) return;
        const int row = wm * C::WTM + r * C::MS + fr;
        af[s][r] = *(const bf16x8*)(sA + row * C::ROWB + ((c ^ swz<C>(row)) << 4));
      } else {
        const int row = b_row(r - C::FM) + fr;
        bfr[s][r - C::FM] = *(const bf16x8*)(sA + C::BM * C::ROWB + row * C::ROWB + ((c ^ swz<C>(row)) << 4));
      }
    };
    auto mma1 = [&](int s, int q) {
      const int i = q / C::FN, j = q % C::FN;
      if (CHECK && i >= live) return;
      acc[i][j] = mfma<C::MS>(af[s][i], bfr[s][j], acc[i][j]);
    };
    // One k-step: after MFMA q come the fragment reads of step `rs` from
    // `src` assigned to it (RPM each for the first MFMAs, so the last read has
    // half the step's MFMAs to land) and the refill loads d0 .. d0 + D - 1
    // whose even spacing over the NM MFMAs falls on q.
    constexpr int NR = C::FM + C::FN, NM = C::FM * C::FN;
    constexpr int HALF = NM / 2 > 0 ? NM / 2 : 1;
    constexpr int RPM = (NR + HALF - 1) / HALF;
    auto step = [&](int s, const char* src, int rs, int D, int d0, int t, int buf, bool real) {
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        mma1(s, q);
#pragma unroll
        for (int r = min(q * RPM, NR); r < min((q + 1) * RPM, NR); ++r) read1(src, rs, r);
#pragma unroll
        for (int d = (q * D + NM - 1) / NM; d < ((q + 1) * D + NM - 1) / NM; ++d) dma1(t, buf, real, d0 + d);
        if constexpr (!CHECK) __builtin_amdgcn_sched_barrier(0);
      }
    };
    constexpr int D_FIRST = (C::X + L - 1) / L, D_REST = (C::X - D_FIRST) / (L > 1 ? L - 1 : 1);
    static_assert(D_FIRST + (L - 1) * D_REST == C::X, "refill loads per k-step");
    wait_vmcnt<(C::STAGES - 1) * C::X>();
    barrier_lds();
#pragma unroll
    for (int s = 0; s < L; ++s)
#pragma unroll
      for (int r = 0; r < NR; ++r) read1(smem, s, r);
    // Slab kt lives in stage buffer U = kt % STAGES.  The loop is unrolled by
    // STAGES so that U is a constant in each copy: every fragment address is
    // then a per-lane register plus an immediate offset, where a run-time
    // buffer index cost vector adds for every read of every slab.
    auto slab = [&](int kt, auto u_c) {
      constexpr int U = decltype(u_c)::value;
      const char* cur = smem + U * C::SLAB;
      const char* nxt = smem + ((U + 1) % C::STAGES) * C::SLAB;
#pragma unroll
      for (int s = 0; s < KS - L; ++s) step(s, cur, s + L, 0, 0, 0, 0, false);
      // every wave holds this slab's last fragments and slab kt + 1 has landed
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<(C::STAGES - 2) * C::X>();
      barrier_lds();
      const int t = kt + C::STAGES;
      const bool real = t < nk;
#pragma unroll
      for (int s = KS - L; s < KS; ++s) {
        // the next slab's first k-steps (after the last slab these reads go unused)
        const int first = s == KS - L;
        step(s, nxt, s + L - KS, first ? D_FIRST : D_REST, first ? 0 : D_FIRST + (s - KS + L - 1) * D_REST, t, U, real);
      }
    };
    for (int kt = 0; kt < nk; kt += C::STAGES)
      unroll_n<0, C::STAGES>([&](auto u) {
        if (kt + decltype(u)::value < nk) slab(kt + decltype(u)::value, u);
      });
    wait_vmcnt<0>();                     // the empty loads too: none may land during the epilogue
  };
  // Burst refills: the slab's loads are issued together right after the
  // barrier, only for slabs that exist, and the compiler interleaves the
  // fragment reads with the MFMAs.
  auto k_loop_burst = [&](auto checked) {
    constexpr bool CHECK = decltype(checked)::value;
    bf16x8 af[KS][C::FM], bfr[KS][C::FN];
    auto load_frags = [&](const char* sA, int s) {
      const char* sB = sA + C::BM * C::ROWB;
      const int c = s * (C::KSTEP / 8) + fq;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        if (CHECK && i >= live) break;
        const int r = wm * C::WTM + i * C::MS + fr;
        af[s][i] = *(const bf16x8*)(sA + r * C::ROWB + ((c ^ swz<C>(r)) << 4));
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int r = b_row(j) + fr;
        bfr[s][j] = *(const bf16x8*)(sB + r * C::ROWB + ((c ^ swz<C>(r)) << 4));
      }
    };
    auto mma_step = [&](int s) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        if (CHECK && i >= live) break;
#pragma unroll
        for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma<C::MS>(af[s][i], bfr[s][j], acc[i][j]);
      }
    };
    // issue order of a k-step: the NR fragment reads of step s + L go out
    // RPM at a time after each of its first MFMAs, all within the first half
    // of them, so the last read has half the step's MFMAs to land
    constexpr int NR = C::FM + C::FN, NM = C::FM * C::FN;
    constexpr int HALF = NM / 2 > 0 ? NM / 2 : 1;
    constexpr int RPM = (NR + HALF - 1) / HALF;
    auto order = [&]() {
      if constexpr (!CHECK) {
        constexpr int NI = (NR + RPM - 1) / RPM;       // MFMAs with reads after them
        constexpr int LAST = NR - (NI - 1) * RPM;
#pragma unroll
        for (int q = 0; q < NI - 1; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, LAST, 0);
        if constexpr (NM > NI) __builtin_amdgcn_sched_group_barrier(0x008, NM - NI, 0);
      }
    };
    wait_slab<C, C::STAGES - 1>(min(C::STAGES, nk) - 1);
    barrier_lds();
#pragma unroll
    for (int s = 0; s < L; ++s) load_frags(smem, s);
    for (int kt = 0; kt < nk; ++kt) {
      const char* cur = smem + (kt % C::STAGES) * C::SLAB;
      const char* nxt = smem + ((kt + 1) % C::STAGES) * C::SLAB;
#pragma unroll
      for (int s = 0; s < KS - L; ++s) {
        mma_step(s);
        load_frags(cur, s + L);
        order();
      }
      // every wave holds this slab's last fragments and slab kt + 1 has landed
      // (nothing of the k-steps above moves below the wait)
      __builtin_amdgcn_sched_barrier(0);
      wait_slab<C>(max(0, min(C::STAGES - 2, nk - kt - 2)));
      barrier_lds();
      if (kt + C::STAGES < nk)
#pragma unroll
        for (int d = 0; d < C::X; ++d) dma1(kt + C::STAGES, kt % C::STAGES, true, d);
#pragma unroll
      for (int s = KS - L; s < KS; ++s) {
        mma_step(s);
        load_frags(nxt, s + L - KS);     // after the last slab these reads go unused
        order();
      }
    }
  };
  auto k_loop = [&](auto checked) {
    if constexpr (C::SPREAD)
      k_loop_spread(checked);
    else
      k_loop_burst(checked);
  };
  // grouped GEMMs stream weights: their MFMAs on clamped rows past a
  // group's end cost nothing, the checked loop's waits would
  if (live == C::FM || a.group_off)
    k_loop(std::false_type{});
  else
    k_loop(std::true_type{});

  const int ec = lane % C::MS;
  constexpr int NJ = (MODE == GEMM_SWIGLU) ? C::FN / 2 : C::FN;
  constexpr int BNO = (MODE == GEMM_SWIGLU) ? C::BN / 2 : C::BN;    // output columns per tile
  const int n0 = n_tile * BNO;

  if constexpr (!PARTIAL && MODE != GEMM_F32OUT) {
    if (p.vec_epi) {
      // The tile leaves through LDS: waves write their accumulators (after
      // SwiGLU, rounded to bf16; fp32 for the residual add so it rounds
      // once), then every thread moves 16-byte row chunks to C, adding 16
      // bytes of R for the residual.  Rows are padded so the rows 4 apart
      // that one accumulator write covers fall on different banks.
      constexpr bool F32S = MODE == GEMM_RESIDUAL;
      constexpr int ES = F32S ? 4 : 2;
      constexpr int ROWB_O = BNO * ES + (F32S ? 32 : 16);
      constexpr int FIT = (C::STAGES * C::SLAB) / ROWB_O;
      constexpr int RP = stage_rows(C::BM, FIT);          // rows per pass
      static_assert(RP >= 32 && C::BM % RP == 0, "staging");
      constexpr int CH = BNO / 8;                          // 16-byte output chunks per row
      // Residual chunks are loaded two passes ahead (the first two passes'
      // right after the k loop, into registers the operand fragments held),
      // so a pass's loads have two passes to land.
      constexpr int NPASS = C::BM / RP, PER = RP * CH / 256;
      static_assert(RP * CH % 256 == 0, "chunks per thread");
      bf16x8 res[F32S ? NPASS : 1][F32S ? PER : 1];
      auto load_res = [&](int pass) {
        if constexpr (F32S) {
#pragma unroll
          for (int e = 0; e < PER; ++e) {
            const int idx = threadIdx.x + e * 256;
            const int local = m0 + pass * RP + idx / CH, col = n0 + (idx % CH) * 8;
            if (local < rows && col < a.N)
              res[pass][e] = *(const bf16x8*)((const bf16*)a.R + (m_begin + local) * a.ldr + col);
          }
        }
      };
      constexpr int AHEAD = NPASS < 2 ? NPASS : 2;
#pragma unroll
      for (int pass = 0; pass < AHEAD; ++pass) load_res(pass);
#pragma unroll
      for (int pass = 0; pass < NPASS; ++pass) {
        __syncthreads();                                   // LDS free (slabs, or the previous pass)
        const int r_lo = pass * RP;
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
          // wave-uniform: this fragment row block lies in the pass or not
          const int blk = wm * C::WTM + i * C::MS;
          if (blk + C::MS <= r_lo || blk >= r_lo + RP) continue;
#pragma unroll
          for (int r = 0; r < C::NACC; ++r) {
            const int rt = blk + acc_row<C::MS>(lane, r) - r_lo;
            char* row = smem + rt * ROWB_O;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              if (MODE == GEMM_SWIGLU) {
                const int ct = wn * (C::WTN / 2) + j * C::MS + ec;
                const float g = acc[i][j][r], u = acc[i][j + C::FN / 2][r];
                *(bf16*)(row + ct * 2) = (bf16)(silu_f(g) * u);
              } else if (F32S) {
                *(float*)(row + (wn * C::WTN + j * C::MS + ec) * 4) = acc[i][j][r];
              } else {
                *(bf16*)(row + (wn * C::WTN + j * C::MS + ec) * 2) = (bf16)acc[i][j][r];
              }
            }
          }
        }
        __syncthreads();
        if (pass + AHEAD < NPASS) load_res(pass + AHEAD);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int idx = threadIdx.x + e * 256;
          const int rr = idx / CH, ch = idx % CH;
          const int local = m0 + r_lo + rr;
          const int col = n0 + ch * 8;
          if (local >= rows || col >= a.N) continue;
          const int64_t orow = m_begin + local;
          bf16x8 out;
          if constexpr (F32S) {
            const f32x4 v0 = *(const f32x4*)(smem + rr * ROWB_O + ch * 32);
            const f32x4 v1 = *(const f32x4*)(smem + rr * ROWB_O + ch * 32 + 16);
            const bf16x8 rv = res[pass][e];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              out[q] = (bf16)(v0[q] + (float)rv[q]);
              out[q + 4] = (bf16)(v1[q] + (float)rv[q + 4]);
            }
          } else {
            out = *(const bf16x8*)(smem + rr * ROWB_O + ch * 16);
          }
          *(bf16x8*)((bf16*)a.C + orow * a.ldc + col) = out;
        }
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int r = 0; r < C::NACC; ++r) {
      const int local = m0 + wm * C::WTM + i * C::MS + acc_row<C::MS>(lane, r);
      if (local >= rows) continue;
      const int64_t orow = m_begin + local;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        if (MODE == GEMM_SWIGLU) {
          const int col = n0 + wn * (C::WTN / 2) + j * C::MS + ec;
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
          const int col = n0 + wn * C::WTN + j * C::MS + ec;
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

template <class C>
hipError_t launch_pipe(const GemmArgs& a, const GemmPlan& pl, void* ws, hipStream_t s,
                       const LaunchHook* hook) {
  KParams p;
  p.a = a;
  const int rows = a.group_off ? a.max_group_rows : a.M;
  p.m_tiles = (rows + C::BM - 1) / C::BM;
  p.n_tiles = (a.N + (a.mode == GEMM_SWIGLU ? C::BN / 2 : C::BN) - 1) / (a.mode == GEMM_SWIGLU ? C::BN / 2 : C::BN);
  p.part_ld = a.mode == GEMM_SWIGLU ? 2 * (int64_t)a.N : a.N;
  const bool split = pl.k_splits > 1 && !a.group_off;
  if (split) {
    const int kb = a.K / 64;
    p.k_per = ((kb + pl.k_splits - 1) / pl.k_splits) * 64;
    p.z_count = (a.K + p.k_per - 1) / p.k_per;
      p.part = (float*)ws;
    if (!ws && p.z_count > 1) return hipErrorInvalidValue;  // split-K needs the workspace
  } else {
    p.k_per = a.K;
    p.z_count = a.group_off ? a.n_groups : 1;
      p.part = nullptr;
  }
  const int total = p.m_tiles * p.n_tiles * p.z_count;
  if (total == 0) return hipSuccess;
  // blocks after the tiles copy the step's metadata (a.meta), then exit
  const int grid = total + (a.meta.n16 > 0 ? (int)std::min<int64_t>((a.meta.n16 + 255) / 256, 64) : 0);
  auto al16 = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
  p.vec_epi = a.N % 8 == 0 && a.ldc % 8 == 0 && al16(a.C) &&
              (a.mode != GEMM_RESIDUAL || (a.ldr % 8 == 0 && al16(a.R)));
  if (split && p.z_count > 1) {
    if (a.mode == GEMM_SWIGLU)
      launch(gemm_pipe_kernel<C, GEMM_SWIGLU, true>, grid, 256, 0, s, p);
    else
      launch(gemm_pipe_kernel<C, GEMM_STORE, true>, grid, 256, 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.defer_reduce) return e;
    if (hook && hook->fn) hook->fn(hook->ctx, 1);
    return splitk_reduce(a, p.part, p.part_ld, p.z_count, s);
  }
  switch (a.mode) {
    case GEMM_STORE: launch(gemm_pipe_kernel<C, GEMM_STORE, false>, grid, 256, 0, s, p); break;
    case GEMM_RESIDUAL: launch(gemm_pipe_kernel<C, GEMM_RESIDUAL, false>, grid, 256, 0, s, p); break;
    case GEMM_SWIGLU: launch(gemm_pipe_kernel<C, GEMM_SWIGLU, false>, grid, 256, 0, s, p); break;
    default: launch(gemm_pipe_kernel<C, GEMM_F32OUT, false>, grid, 256, 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

namespace {
// (BM, BN of the B slab) of each tile configuration id
void tile_dims(int cfg, int& bm, int& bn) {
  switch (cfg) {
    case 1: bm = 64; bn = 128; return;
    case 2: bm = 256; bn = 128; return;
    case 3: bm = 32; bn = 128; return;
    case 4: bm = 128; bn = 256; return;
    case 5: bm = 256; bn = 256; return;
    case 6: bm = 64; bn = 128; return;
    case 10: bm = 256; bn = 256; return;
    case 11: bm = 256; bn = 128; return;
    case 12: bm = 128; bn = 256; return;
    case 13: case 14: bm = 128; bn = 128; return;
    case 15: bm = 64; bn = 128; return;
    case 16: bm = 32; bn = 128; return;
    case 17: bm = 64; bn = 256; return;
    case 18: bm = 64; bn = 128; return;
    case 19: case 20: bm = 32; bn = 128; return;
    case 21: bm = 256; bn = 256; return;
    case 22: case 23: bm = 128; bn = 128; return;
    case 24: bm = 256; bn = 128; return;
    case 25: bm = 128; bn = 256; return;
    case 26: case 27: bm = 256; bn = 256; return;
    case 28: bm = 256; bn = 128; return;
    case 29: bm = 128; bn = 128; return;
    case 30: bm = 160; bn = 256; return;
    default: bm = 128; bn = 128; return;
  }
}
int n_tiles_of(const GemmArgs& a, int bn) {
  const int c = a.mode == GEMM_SWIGLU ? bn / 2 : bn;
  return (a.N + c - 1) / c;
}
}  // namespace

// Tile choice (from sweeps on MI355X, timed inside the layer step: a GEMM
// timed back to back on its own runs up to 20% faster than between the
// step's other kernels, and ranks the tiles differently).  K % 64 == 0
// problems use the pipelined kernel: decode-sized M streams weights with 32-
// or 64-row tiles; larger M uses 128 x 128 tiles, two workgroups per CU, or
// 256 x 256 tiles (one per CU) when there are enough of them.  When the tiles
// cannot give every CU about two workgroups, K is split (up to 8 ways for
// weight streaming, 4 otherwise, keeping >= 512 of K per piece) and a reduce
// kernel applies the epilogue.
namespace {
// Split count of a weight-streaming launch from a time model fitted on
// MI355X: a workgroup streams at most kWgGBps, at most two workgroups share a
// CU, and the chip at most kHbmGBps; split-K adds its fp32 partial slices
// (written, then read again by the reduce).
// (the double-buffered configurations 46..51 keep a second chunk in
// flight: about 24 GB/s per workgroup)
constexpr double kWgGBps = 20.0, kWgGBpsDB = 24.0, kHbmGBps = 6000.0;
int stream_splits(const GemmArgs& a, int cfg, int cus) {
  const double wg_gbps = (cfg >= 46 && cfg <= 51) ? kWgGBpsDB : kWgGBps;
  const bool sw = a.mode == GEMM_SWIGLU;
  const int nbw = stream_nbw(cfg);
  const int nbt = (sw ? 2 : 1) * (a.N / 32);
  const int n_wg = (nbt + 4 * nbw - 1) / (4 * nbw);
  const int nch = a.K / 16 / stream_kc(cfg);
  const double wbytes = (double)nbt * 32 * a.K * 2 * a.n_groups;
  const double pld = sw ? 2.0 * a.N : a.N;
  int best = 1;
  double best_t = 1e30;
  for (int want = 1; want <= std::min(nch, 16); ++want) {
    const int ch_per = (nch + want - 1) / want;
    const int z = (nch + ch_per - 1) / ch_per;
    const double wgs = (double)n_wg * z * a.n_groups;
    const double bw = std::min(kHbmGBps, std::min(wgs, 2.0 * cus) * wg_gbps) * 1e9;
    const double t = (wbytes + (z > 1 ? 2.0 * z * a.M * pld * 4 : 0.0)) / bw;
    if (t < best_t * 0.98) {
      best_t = t;
      best = z;
    }
  }
  return best;
}
}  // namespace

// Tuning knob for timing tile configurations inside the step:
// NF_GEMM_OVERRIDE="M,N,K,mode=cfg:splits;..." makes every dense GEMM of that
// shape and mode run LDS-pipelined configuration cfg (10..30) with the given
// K split.  Read once per process; shapes the configuration cannot take
// (K not a multiple of 64, grouped GEMMs) keep the regular choice.
struct GemmOverride {
  int M, N, K, mode, cfg, splits;
};

const std::vector<GemmOverride>& gemm_overrides() {
  static const std::vector<GemmOverride> table = [] {
    std::vector<GemmOverride> t;
    const char* v = std::getenv("NF_GEMM_OVERRIDE");
    while (v && *v) {
      GemmOverride o{};
      if (std::sscanf(v, "%d,%d,%d,%d=%d:%d", &o.M, &o.N, &o.K, &o.mode, &o.cfg, &o.splits) == 6 && o.cfg >= 10 &&
          o.cfg <= 30 && o.splits >= 1)
        t.push_back(o);
      v = std::strchr(v, ';');
      if (v) ++v;
    }
    return t;
  }();
  return table;
}

GemmPlan gemm_choose(const GemmArgs& a, int cus, bool coresident) {
  GemmPlan p;
  if (cus <= 0) cus = 256;
  if (!a.group_off && !a.Bp && a.K % 64 == 0)
    for (const GemmOverride& o : gemm_overrides())
      if (o.M == a.M && o.N == a.N && o.K == a.K && o.mode == a.mode) {
        p.cfg = o.cfg;
        p.k_splits = std::min(o.splits, a.K / 64);
        return p;
      }
  if (a.Bp) {                   // packed weights: stream them for expert groups
    // (measured: for dense decode-sized M the pipelined LDS kernel below is
    // faster, so configurations 40..43 are chosen only on request; on the
    // 8-expert workload the double-buffered 46 / 47 beat 44 / 45, and for
    // the down projection (112 chunks per workgroup) 48, which loads A two
    // chunks ahead, beats 46 by a fifth; for gate/up (32 chunks per
    // workgroup, 3.5 rounds) 49 did not beat 47; a 160 x 256 LDS-pipelined
    // tile (configuration 30) ties with 46 / 47; 50 / 51, which issue the
    // next chunk's loads spread among this chunk's MFMAs, beat 48 / 47 by
    // an eighth and a tenth)
    const bool sw = a.mode == GEMM_SWIGLU;
    int cfg = 0;
    if (a.group_off && a.max_group_rows / std::max(1, a.n_groups) <= 160) cfg = sw ? 51 : 50;
    if (cfg && a.N % 32 == 0 && a.K % (16 * stream_kc(cfg)) == 0) {
      p.cfg = cfg;
      p.k_splits = stream_splits(a, cfg, cus);
      return p;
    }
  }
  const bool pipe = a.K % 64 == 0;
  if (a.group_off) {            // grouped (experts): rows per group ~ tokens*k/E
    // 128 x 128 tiles (measured best of the pipelined configurations on the
    // 8-expert workload); fragments past a group's rows do no work
    p.cfg = pipe ? 14 : 0;
    return p;
  }
  const int M = a.M;
  const bool stream_w = M <= 64;
  if (stream_w)
    p.cfg = pipe ? (M <= 32 ? 16 : 15) : (M <= 32 ? 3 : 1);
  else
    p.cfg = pipe ? 14 : 0;
  // 256 x 256 tiles halve the operand traffic per FLOP of 128 x 128 ones
  // but run one workgroup per CU.  Timed inside the layer step (1024- and
  // 2048-token batches of the Llama-3-8B and Llama-2-70B-shard layers) they
  // win once there are about 0.75 of them per CU with K >= 2048, and, for
  // K >= 8192, when split-K brings them there with >= 2048 of K per piece
  // (shorter K, or fewer tiles: 128 x 128 tiles, whose split partials the
  // consumers reduce more cheaply)
  // Short K (1024..2047) takes them only when they fill exactly one round:
  // the Llama-2-70B-shard O projection (2048 x 8192 x 1024) 53.3 -> 50.2 us
  // inside the step against 128 x 128 tiles (three alternating runs).
  if (p.cfg == 14 && a.K >= 1024 && a.K < 2048 && !coresident) {
    const int64_t t256 = (int64_t)((M + 255) / 256) * n_tiles_of(a, 256);
    if (4 * t256 >= 3 * (int64_t)cus && t256 <= cus) {
      p.cfg = 10;
      p.k_splits = 1;
      return p;
    }
  }
  if (p.cfg == 14 && a.K >= 2048 && !coresident) {
    const int64_t t256 = (int64_t)((M + 255) / 256) * n_tiles_of(a, 256);
    const int64_t enough = (3 * (int64_t)cus + 3) / 4;
    int ks = 0;
    if (t256 >= enough) {
      ks = 1;
    } else if (const int64_t t12 = (int64_t)((M + 127) / 128) * n_tiles_of(a, 256), t13 = (int64_t)((M + 127) / 128) * n_tiles_of(a, 128);
               (a.K < 8192 || a.mode == GEMM_SWIGLU) &&
               ((t12 >= enough && t12 <= cus) || (t13 >= enough && t13 <= cus))) {
      // a grid of 128-row tiles that fills one round runs unsplit, with no
      // partials to write and reduce: 128 x 256 (configuration 12) before
      // 128 x 128 (13).  Inside the step: the Llama-3-8B QKV of 1024 tokens
      // 74 -> 55 us; the Llama-2-70B-shard gate/up of 1024 and 512 tokens
      // (whose split partials are twice as wide) alone 109 us against 118
      // plus a reduce, and 64 against 70 plus a reduce.  Long-K projections
      // keep the split 256 x 256 tiles (the 1024-token Llama-3-8B down
      // projection: 117 us split, 134 as 128 x 128 tiles).
      p.cfg = (t12 >= enough && t12 <= cus) ? 12 : 13;
      p.k_splits = 1;
      // plain stores (the QKV projection) as 256 x 128 tiles when those fill
      // the round as well: the 1024-token Llama-3-8B QKV 56.3 -> 53.1 us
      // inside the step (two alternating runs)
      const int64_t t11 = (int64_t)((M + 255) / 256) * n_tiles_of(a, 128);
      if (a.mode == GEMM_STORE && t11 >= enough && t11 <= cus) p.cfg = 11;
      return p;
    } else if (a.K >= 8192) {
      for (int k = 2; k <= 8 && a.K / k >= 2048; k *= 2)
        if (t256 * k >= enough) {
          ks = k;
          break;
        }
    }
    if (ks) {
      p.cfg = 10;
      p.k_splits = ks;
      return p;
    }
  }
  // A long-K projection to a narrow output (the Llama-2-70B-shard QKV:
  // 1280 x 8192) has too few 256 x 256 tiles even split four ways; 128 x 256
  // tiles split until they fill one round (at least 1024 of K per piece) run
  // it inside the step in 61 us at 2048 tokens (3 pieces) against 73-75 for
  // split 128 x 128 tiles, and in 2 x 32 us at 1024 tokens (5 pieces) against
  // 2 x 45 (the partials go to the RoPE kernel, which reduces them)
  // The same tiles as 256 x 128 (configuration 11) ran it in 53.0 us against
  // 54.7 (three pieces; two alternating runs inside the step), so the split
  // is sized on those.
  if (p.cfg == 14 && a.K >= 8192 && !coresident && a.mode == GEMM_STORE) {
    const int64_t t11 = (int64_t)((M + 255) / 256) * n_tiles_of(a, 128);
    const int64_t enough = (3 * (int64_t)cus + 3) / 4;
    for (int k = 2; k <= 8 && a.K / k >= 1024; ++k)
      if (t11 * k >= enough && t11 * k <= cus) {
        p.cfg = 11;
        p.k_splits = k;
        return p;
      }
  }
  // 128 x 128 tiles that fill one round on the CUs (at least three quarters
  // of them) run unsplit, one workgroup per CU with three stages and the
  // refill spread over the MFMAs (configuration 13).  Inside the step: the
  // 1024 x 4096 x 4096 O projection and its FFN norm 56 -> 45 us (no split-K
  // partials to reduce), the 512 x 6144 x 4096 QKV with RoPE 45 -> 41 us; with
  // fewer tiles (160 or 128 for 256 CUs) the split 128 x 128 tiles were faster
  if (p.cfg == 14 && a.K >= 1024 && !coresident) {
    const int64_t t128 = (int64_t)((M + 127) / 128) * n_tiles_of(a, 128);
    if (4 * t128 >= 3 * (int64_t)cus && t128 <= cus) {
      p.cfg = 13;
      p.k_splits = 1;
      return p;
    }
  }
  int bm, bn;
  tile_dims(p.cfg, bm, bn);
  const int tiles = ((M + bm - 1) / bm) * n_tiles_of(a, bn);
  const int want = stream_w ? cus : 2 * cus;      // workgroups that keep every CU busy
  int ks = 1;
  while (ks * 2 * tiles <= want && ks < (stream_w ? 8 : 4) && a.K / (ks * 2) >= 512) ks *= 2;
  p.k_splits = ks;
  return p;
}

hipError_t splitk_reduce(const GemmArgs& a, const float* part, int64_t part_ld, int splits, hipStream_t s) {
  return splitk_reduce_impl(a, part, part_ld, splits, s);
}

int gemm_partials(const GemmArgs& a, const GemmPlan& p) {
  if (p.cfg >= 40) {            // streaming kernels split K in whole chunks
    const int kc = stream_kc(p.cfg);
    const int nch = a.K / 16 / kc;
    if (p.k_splits <= 1 || nch <= 1) return 1;
    const int ch_per = (nch + std::min(p.k_splits, nch) - 1) / std::min(p.k_splits, nch);
    return (nch + ch_per - 1) / ch_per;
  }
  if (p.k_splits <= 1 || a.group_off || a.M == 0 || a.N == 0) return 1;
  // both kernels split K in whole 64-wide blocks, as launch_cfg / launch_pipe do
  const int kb = (a.K + 63) / 64;
  const int k_per = ((kb + p.k_splits - 1) / p.k_splits) * 64;
  return (a.K + k_per - 1) / k_per;
}

size_t gemm_workspace_bytes(const GemmArgs& a, const GemmPlan& p) {
  if (p.cfg >= 40) {
    const int z = gemm_partials(a, p);
    return z > 1 ? (size_t)z * a.M * (a.mode == GEMM_SWIGLU ? 2 * (int64_t)a.N : a.N) * sizeof(float) : 0;
  }
  if (p.k_splits <= 1 || a.group_off) return 0;
  const int64_t ld = a.mode == GEMM_SWIGLU ? 2 * (int64_t)a.N : a.N;
  int bm, bn;
  tile_dims(p.cfg, bm, bn);
  const int tiles = ((a.M + bm - 1) / bm) * n_tiles_of(a, bn);
  (void)tiles;
  return (size_t)p.k_splits * a.M * ld * sizeof(float);
}

hipError_t gemm_bf16(const GemmArgs& a, const GemmPlan& p, void* ws, hipStream_t s, const LaunchHook* hook) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (p.cfg >= 40) return a.Bp ? gemm_stream(a, p, ws, s, hook) : hipErrorInvalidValue;
  if (p.cfg >= 10 && a.K % 64 != 0) return hipErrorInvalidValue;
  switch (p.cfg) {
    case 1: return launch_cfg<Cfg1>(a, p, ws, s, hook);
    case 2: return launch_cfg<Cfg2>(a, p, ws, s, hook);
    case 3: return launch_cfg<Cfg3>(a, p, ws, s, hook);
    case 4: return launch_cfg<Cfg4>(a, p, ws, s, hook);
    case 5: return launch_cfg<Cfg5>(a, p, ws, s, hook);
    case 6: return launch_cfg<Cfg6>(a, p, ws, s, hook);
    case 10: return launch_pipe<P10>(a, p, ws, s, hook);
    case 11: return launch_pipe<P11>(a, p, ws, s, hook);
    case 12: return launch_pipe<P12>(a, p, ws, s, hook);
    case 13: return launch_pipe<P13>(a, p, ws, s, hook);
    case 14: return launch_pipe<P14>(a, p, ws, s, hook);
    case 15: return launch_pipe<P15>(a, p, ws, s, hook);
    case 16: return launch_pipe<P16>(a, p, ws, s, hook);
    case 17: return launch_pipe<P17>(a, p, ws, s, hook);
    case 18: return launch_pipe<P18>(a, p, ws, s, hook);
    case 19: return launch_pipe<P19>(a, p, ws, s, hook);
    case 20: return launch_pipe<P20>(a, p, ws, s, hook);
    case 21: return launch_pipe<P21>(a, p, ws, s, hook);
    case 22: return launch_pipe<P22>(a, p, ws, s, hook);
    case 23: return launch_pipe<P23>(a, p, ws, s, hook);
    case 24: return launch_pipe<P24>(a, p, ws, s, hook);
    case 25: return launch_pipe<P25>(a, p, ws, s, hook);
    case 26: return launch_pipe<P26>(a, p, ws, s, hook);
    case 27: return launch_pipe<P27>(a, p, ws, s, hook);
    case 28: return launch_pipe<P28>(a, p, ws, s, hook);
    case 29: return launch_pipe<P29>(a, p, ws, s, hook);
    case 30: return launch_pipe<P30>(a, p, ws, s, hook);
    default: return launch_cfg<Cfg0>(a, p, ws, s, hook);
  }
}

hipError_t gemm_f32(const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
  switch (a.mode) {
    case GEMM_RESIDUAL: launch(gemm_f32_kernel<GEMM_RESIDUAL>, grid, 256, 0, s, a); break;
    case GEMM_SWIGLU: launch(gemm_f32_kernel<GEMM_SWIGLU>, grid, 256, 0, s, a); break;
    default: launch(gemm_f32_kernel<GEMM_STORE>, grid, 256, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace nf
