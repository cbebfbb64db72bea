// Weight-streaming bf16 GEMM for the decode-sized GEMMs of a step (M up to
// 64 rows) and for the per-expert GEMMs of a mixture-of-experts layer (about
// 128 rows per expert).  At these M the GEMM reads every weight byte once
// and does little arithmetic per byte, so its time is the HBM stream of the
// weights, and what matters is how many weight bytes each CU keeps in flight.
//
// The weights are copied once, at layer creation, into the operand order of
// v_mfma_f32_32x32x16_bf16: block (n-block b of 32 output features, k-step
// s of 16) is 1 KB holding, for lane l, the 8 K-consecutive values
// W[32 b + l % 32][16 s + 8 (l / 32) ..].  A wavefront then fetches its B
// operand for one k-step with one linear 16-byte-per-lane load straight into
// registers (no LDS), and it issues a whole chunk of k-steps ahead.  The
// activations (A) are small and shared by the four waves of a workgroup:
// they are staged in LDS through registers, one K-chunk at a time, and the
// chunk's B loads stay in flight while the A part is written and the
// workgroup synchronises.
//
// Split-K writes fp32 partial slices in the same layout as the pipelined
// GEMM's, so the same reduce kernel (or a fused consumer) finishes them.
#include <type_traits>

#include "nf_device.h"
#include "nf_internal.h"

namespace nf {
namespace {

constexpr int SB = 32;   // rows / columns of one MFMA block
constexpr int SK = 16;   // K of one MFMA

struct SParams {
  GemmArgs a;
  int nbt;          // packed n-blocks per group (SWIGLU: gate and up blocks interleaved)
  int kbt;          // K / 16
  int n_wg;         // workgroups along N
  int splits;       // K pieces
  int ks_per;       // k-steps per piece (a multiple of the chunk)
  float* part;      // partial slices [splits][M][part_ld] (split-K only)
  int64_t part_ld;
};

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (within a 32 x 32 block) of accumulator element r held by `lane`; the
// column is lane % 32.
__device__ __forceinline__ int acc_row32(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// MB m-blocks of 32 rows per pass, NBW packed n-blocks per wave, KC k-steps
// per A chunk.  MODE as in GemmMode; PARTIAL writes fp32 partial slices.
// PIPE 1 double-buffers the chunks (two LDS A buffers, two register sets of
// B): chunk c + 1's loads are in flight while chunk c's MFMAs run.  Only
// register loads are used: a buffer-to-LDS fill in flight beside register
// loads made in-order vmcnt counting unsafe (the two kinds completed out of
// order on MI355X; wrong sums, found by the streaming-configuration tests).
template <int MB, int NBW, int KC, int MODE, bool PARTIAL, int PIPE>
__global__ __launch_bounds__(256, MB <= 2 ? 2 : 1) void gemm_stream_kernel(SParams p) {
  constexpr int ROWS = MB * SB;
  constexpr int PR = KC * 2;                 // 16-byte pieces of one A row in a chunk
  constexpr int CH = ROWS * PR * 16;         // bytes of one A chunk
  constexpr int NA = CH / 4096;              // 16-byte A loads per lane per chunk
  constexpr int NB = KC * NBW;               // B loads per wave per chunk
  static_assert(CH % 4096 == 0 && NA >= 1, "chunk");
  static_assert((PIPE >= 1 ? 2 : 1) * (NA + NB) + (PIPE == 3 ? NA : 0) <= 63, "vmcnt range");
  static_assert(PIPE != 5 || NA + NB <= KC * MB * 4, "loads per MFMA slot");
  static_assert((MODE == GEMM_SWIGLU) == (NBW == 2), "SWIGLU pairs a gate and an up block per wave");
  __shared__ __attribute__((aligned(1024))) char smem[(PIPE >= 1 ? 2 : 1) * CH];

  const GemmArgs& a = p.a;
  const int total = p.n_wg * p.splits * a.n_groups;
  const int logical = xcd_logical(blockIdx.x, total);
  const int wg_n = logical % p.n_wg;
  const int rest = logical / p.n_wg;
  const int z = rest % p.splits;
  const int grp = rest / p.splits;
  int m_begin = 0, rows = a.M;
  if (a.group_off) {
    m_begin = a.group_off[grp];
    rows = a.group_off[grp + 1] - m_begin;
  }
  if (rows <= 0) return;                                   // whole workgroup exits together
  const int ks0 = z * p.ks_per;
  const int nch = min(p.ks_per, p.kbt - ks0) / KC;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // B sources: this wave's packed n-blocks, clamped into range so that every
  // wave issues the same number of loads (the vmcnt arithmetic relies on it)
  const bf16x8* bsrc[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const int nb = min((wg_n * 4 + wave) * NBW + j, p.nbt - 1);
    bsrc[j] = (const bf16x8*)((const bf16*)a.Bp + (int64_t)grp * a.bp_group_stride +
                              ((int64_t)nb * p.kbt + ks0) * 512) + lane;
  }

  for (int m0 = 0; m0 < rows; m0 += ROWS) {
    const int live_mb = min(MB, (rows - m0 + SB - 1) / SB);
    // A sources: load i of this wave fills chunk bytes [(wave NA + i) KB, +1 KB):
    // piece (row r, physical slot sl) holds logical piece sl ^ (r % PR), so
    // fragment reads (32 rows, one piece) spread over the LDS banks
    const bf16* asrc[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int piece = (wave * NA + i) * 64 + lane;
      const int r = piece / PR, q = (piece % PR) ^ (r % PR);
      int src = m_begin + min(m0 + r, rows - 1);          // rows past the group repeat its last row
      if (a.a_rows) src = a.a_rows[src] / a.a_row_div;
      asrc[i] = (const bf16*)a.A + (int64_t)src * a.lda + (int64_t)ks0 * SK + q * 8;
    }

    f32x16 acc[MB][NBW];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[m][j][e] = 0.f;

    // Per chunk: the chunk's A is loaded to registers and all KC * NBW of its
    // weight loads are issued at once; A goes to LDS as soon as it lands and
    // the MFMAs consume the weights in issue order (the compiler waits per
    // register).  Only register loads are used, and a chunk's loads are
    // consumed in the same iteration, so the compiler's in-order counting
    // stays exact; the other waves of the CU keep HBM busy while one wave
    // computes.
    bf16x8 ar[NA];
    if constexpr (PIPE == 5) {
      // PIPE 5: as PIPE 1 (chunk c + 1's loads in flight while chunk c's
      // MFMAs run), but the NA + NB loads of chunk c + 1 are issued spread
      // over chunk c's MFMAs in a fixed order, not in a block before them:
      // the CU's path from L2 accepts about one 1 KB load per 16 cycles, and
      // a wave waiting to issue a load issues no MFMA (per-wave timing: the
      // block of 26 loads took ~2500 cycles per chunk beside ~3200 of MFMAs).
      const __amdgpu_buffer_rsrc_t rA = buf_rsrc(a.A);
      uint32_t aoff[NA];
#pragma unroll
      for (int i = 0; i < NA; ++i) aoff[i] = (uint32_t)((asrc[i] - (const bf16*)a.A) * 2);
      __amdgpu_buffer_rsrc_t rB[NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) rB[j] = buf_rsrc(bsrc[j] - lane);
      bf16x8 bq[2][KC][NBW];
      bf16x8 aq[NA];
      // load d of chunk c: A pieces first (they go to LDS right after the
      // MFMAs), then the weights (the chunk after the last reloads the last,
      // so every wave issues the same loads and the in-order waits stay exact)
      auto load1 = [&](int c, int d, bf16x8 (&bdst)[KC][NBW]) {
        c = min(c, nch - 1);
        if (d < NA) {
          aq[d] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rA, aoff[d], c * KC * SK * 2, 0));
        } else {
          const int q = d - NA, st = q / NBW, j = q % NBW;
          bdst[st][j] = __builtin_bit_cast(
              bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rB[j], lane * 16, (c * KC + st) * 1024, 2));
        }
      };
      auto put_a = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NA; ++i) *(bf16x8*)(smem + buf * CH + ((wave * NA + i) * 64 + lane) * 16) = aq[i];
      };
      auto frag = [&](int buf, int idx) {
        const int st = idx / MB, m = idx % MB;
        const int r = m * SB + (lane & 31);
        const int sl = (2 * st + (lane >> 5)) ^ (r % PR);
        return *(const bf16x8*)(smem + buf * CH + r * PR * 16 + sl * 16);
      };
      constexpr int NI = KC * MB, NL = NA + NB;
      // chunk c's MFMAs from LDS buffer buf and registers src, with chunk
      // c + 1's loads (into aq and bnext) spread over them
      auto mma_load = [&](int buf, const bf16x8 (&src)[KC][NBW], int cnext, bf16x8 (&bnext)[KC][NBW]) {
        bf16x8 af[3];
        af[0] = frag(buf, 0);
        if (NI > 1) af[1] = frag(buf, 1);
#pragma unroll
        for (int idx = 0; idx < NI; ++idx) {
          if (idx + 2 < NI) af[(idx + 2) % 3] = frag(buf, idx + 2);
          const int st = idx / MB, m = idx % MB;
#pragma unroll
          for (int j = 0; j < NBW; ++j) acc[m][j] = mfma32(af[idx % 3], src[st][j], acc[m][j]);
#pragma unroll
          for (int d = (idx * NL + NI - 1) / NI; d < ((idx + 1) * NL + NI - 1) / NI; ++d) load1(cnext, d, bnext);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // prologue: chunk 0 to LDS and registers
#pragma unroll
      for (int d = 0; d < NL; ++d) load1(0, d, bq[0]);
      put_a(0);
      int c = 0;
      for (; c + 1 < nch; c += 2) {
        barrier_lds();                // chunk c's A is in buffer 0; chunk c - 1 is done with buffer 1
        mma_load(0, bq[0], c + 1, bq[1]);
        put_a(1);
        barrier_lds();
        mma_load(1, bq[1], c + 2, bq[0]);
        put_a(0);
      }
      if (c < nch) {
        barrier_lds();
        mma_load(0, bq[0], c + 1, bq[1]);
      }
      barrier_lds();                  // LDS may take the next pass
    } else if constexpr (PIPE == 1 || PIPE == 3) {
      // PIPE 3 loads A two chunks ahead (a second register set), so the A
      // written to LDS after chunk c's MFMAs has been in flight for a chunk
      // and a half instead of for the MFMAs alone.
      constexpr bool A2 = PIPE == 3;
      // Every load is unconditional (the chunk after the last one reloads
      // the last), so the compiler's in-order wait counts stay exact across
      // the loop; one barrier per chunk separates the A writes of chunk c + 1
      // from the fragment reads of chunk c - 1 in the same buffer.
      // buffer loads: a scalar base per operand (per packed n-block for B)
      // and 32-bit lane offsets, with the chunk's offset in the scalar
      // offset, keep the address registers few
      const __amdgpu_buffer_rsrc_t rA = buf_rsrc(a.A);
      uint32_t aoff[NA];
#pragma unroll
      for (int i = 0; i < NA; ++i) aoff[i] = (uint32_t)((asrc[i] - (const bf16*)a.A) * 2);
      __amdgpu_buffer_rsrc_t rB[NBW];
#pragma unroll
      for (int j = 0; j < NBW; ++j) rB[j] = buf_rsrc(bsrc[j] - lane);      // wave-uniform: the wave's n-block
      bf16x8 bq[2][KC][NBW];
      bf16x8 aq[A2 ? 2 : 1][NA];
      auto load_a = [&](int c, bf16x8 (&dst)[NA]) {
        c = min(c, nch - 1);
#pragma unroll
        for (int i = 0; i < NA; ++i)
          dst[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rA, aoff[i], c * KC * SK * 2, 0));
      };
      auto load_b = [&](int c, bf16x8 (&dst)[KC][NBW]) {
        c = min(c, nch - 1);
#pragma unroll
        for (int s = 0; s < KC; ++s)
#pragma unroll
          for (int j = 0; j < NBW; ++j)      // nontemporal: each weight byte is read once
            dst[s][j] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rB[j], lane * 16, (c * KC + s) * 1024, 2));
      };
      auto put_a = [&](int buf, const bf16x8 (&src)[NA]) {
#pragma unroll
        for (int i = 0; i < NA; ++i) *(bf16x8*)(smem + buf * CH + ((wave * NA + i) * 64 + lane) * 16) = src[i];
      };
      auto mma = [&](int buf, const bf16x8 (&src)[KC][NBW]) {
#pragma unroll
        for (int s = 0; s < KC; ++s) {
#pragma unroll
          for (int m = 0; m < MB; ++m) {
            const int r = m * SB + (lane & 31);
            const int sl = (2 * s + (lane >> 5)) ^ (r % PR);
            const bf16x8 af = *(const bf16x8*)(smem + buf * CH + r * PR * 16 + sl * 16);
#pragma unroll
            for (int j = 0; j < NBW; ++j) acc[m][j] = mfma32(af, src[s][j], acc[m][j]);
          }
        }
        // fragment reads run two ahead of their MFMAs (hoisting all of them
        // would take 4 registers each)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < KC * MB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, NBW, 0);
          if (i + 2 < KC * MB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      };
      // chunks in pairs (no exit between the halves, so the accumulators
      // keep their registers), an odd last chunk after the loop
      int c = 0;
      if constexpr (!A2) {
        load_a(0, aq[0]);
        load_b(0, bq[0]);
        put_a(0, aq[0]);
        for (; c + 1 < nch; c += 2) {
          load_a(c + 1, aq[0]);
          load_b(c + 1, bq[1]);
          barrier_lds();              // chunk c's A is in buffer 0; chunk c - 1 is done with buffer 1
          mma(0, bq[0]);
          put_a(1, aq[0]);
          load_a(c + 2, aq[0]);
          load_b(c + 2, bq[0]);
          barrier_lds();
          mma(1, bq[1]);
          put_a(0, aq[0]);
        }
      } else {
        load_a(0, aq[0]);
        load_b(0, bq[0]);
        load_a(1, aq[1]);
        put_a(0, aq[0]);
        for (; c + 1 < nch; c += 2) {
          load_a(c + 2, aq[0]);       // aq[0] went to LDS as chunk c's A
          load_b(c + 1, bq[1]);
          barrier_lds();              // chunk c's A is in buffer 0; chunk c - 1 is done with buffer 1
          mma(0, bq[0]);
          put_a(1, aq[1]);            // chunk c + 1's A, loaded a chunk earlier
          load_a(c + 3, aq[1]);
          load_b(c + 2, bq[0]);
          barrier_lds();
          mma(1, bq[1]);
          put_a(0, aq[0]);
        }
      }
      if (c < nch) {
        barrier_lds();
        mma(0, bq[0]);
      }
      barrier_lds();                  // LDS may take the next pass
    } else {
    bf16x8 br[KC][NBW];
    for (int c = 0; c < nch; ++c) {
#pragma unroll
      for (int i = 0; i < NA; ++i) ar[i] = *(const bf16x8*)(asrc[i] + (int64_t)c * KC * SK);
#pragma unroll
      for (int s = 0; s < KC; ++s)
#pragma unroll
        for (int j = 0; j < NBW; ++j) br[s][j] = __builtin_nontemporal_load(bsrc[j] + (int64_t)(c * KC + s) * 64);
#pragma unroll
      for (int i = 0; i < NA; ++i) *(bf16x8*)(smem + ((wave * NA + i) * 64 + lane) * 16) = ar[i];
      barrier_lds();                  // every wave's part of the chunk's A is in LDS
#pragma unroll
      for (int s = 0; s < KC; ++s) {
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const int r = m * SB + (lane & 31);
          const int sl = (2 * s + (lane >> 5)) ^ (r % PR);
          const bf16x8 af = *(const bf16x8*)(smem + r * PR * 16 + sl * 16);
#pragma unroll
          for (int j = 0; j < NBW; ++j) acc[m][j] = mfma32(af, br[s][j], acc[m][j]);
        }
      }
      barrier_lds();                  // LDS may take the next chunk
    }
    }

    // epilogue: lane holds D[acc_row32(lane, r)][lane % 32] of each block
    constexpr int NOUT = MODE == GEMM_SWIGLU ? 1 : NBW;     // output blocks per wave
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (m >= live_mb) break;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int local = m0 + m * SB + acc_row32(lane, r);
        if (local >= rows) continue;
        const int64_t orow = m_begin + local;
#pragma unroll
        for (int j = 0; j < NOUT; ++j) {
          const int ob = MODE == GEMM_SWIGLU ? wg_n * 4 + wave : (wg_n * 4 + wave) * NBW + j;
          const int col = ob * SB + (lane & 31);
          if (col >= a.N) continue;
          if (MODE == GEMM_SWIGLU) {
            const float g = acc[m][0][r], u = acc[m][1][r];
            if (PARTIAL) {
              float* P = p.part + (int64_t)z * a.M * p.part_ld + orow * p.part_ld;
              P[col] = g;
              P[a.N + col] = u;
            } else {
              ((bf16*)a.C)[orow * a.ldc + col] = (bf16)(silu_f(g) * u);
            }
          } else {
            const float v = acc[m][j][r];
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
}

// Packs W [groups][N][K] (row stride ldw, group stride gs) into operand
// order: block (n-block b, k-step s) of group g goes to packed n-block
// b * nb_stride + nb_offset.  One thread per 16-byte piece.
__global__ __launch_bounds__(256) void pack_b_kernel(const bf16* __restrict__ W, int64_t ldw, int64_t gs, int N,
                                                     int K, int groups, bf16* __restrict__ P, int nb_stride,
                                                     int nb_offset, int nbt_packed, int64_t pgs) {
  const int kbt = K / SK, nbt = N / SB;
  const int64_t pieces = (int64_t)groups * nbt * kbt * 64;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < pieces; i += (int64_t)gridDim.x * 256) {
    const int lane = (int)(i % 64);
    const int64_t blk = i / 64;
    const int s = (int)(blk % kbt);
    const int64_t gb = blk / kbt;
    const int b = (int)(gb % nbt);
    const int g = (int)(gb / nbt);
    const bf16x8 v = *(const bf16x8*)(W + g * gs + (int64_t)(b * SB + (lane & 31)) * ldw + s * SK + 8 * (lane >> 5));
    const int64_t pb = (int64_t)b * nb_stride + nb_offset;
    *(bf16x8*)(P + g * pgs + ((pb * kbt + s) * 64 + lane) * 8) = v;
    (void)nbt_packed;
  }
}

template <int MB, int NBW, int KC, int PIPE = 0>
hipError_t launch_stream(const GemmArgs& a, const GemmPlan& pl, void* ws, hipStream_t s, const LaunchHook* hook) {
  if (a.N % SB || a.K % (KC * SK)) return hipErrorInvalidValue;
  SParams p;
  p.a = a;
  const bool sw = a.mode == GEMM_SWIGLU;
  p.kbt = a.K / SK;
  p.nbt = (sw ? 2 : 1) * (a.N / SB);
  p.n_wg = (p.nbt + 4 * NBW - 1) / (4 * NBW);
  const int nch = p.kbt / KC;
  const int want = std::max(1, std::min(pl.k_splits, nch));
  const int ch_per = (nch + want - 1) / want;
  p.ks_per = ch_per * KC;
  p.splits = (nch + ch_per - 1) / ch_per;
  p.part_ld = sw ? 2 * (int64_t)a.N : a.N;
  p.part = p.splits > 1 ? (float*)ws : nullptr;
  if (p.splits > 1 && !ws) return hipErrorInvalidValue;     // split-K needs the workspace
  const int total = p.n_wg * p.splits * a.n_groups;
  if (total == 0) return hipSuccess;
  if (sw != (NBW == 2)) return hipErrorInvalidValue;    // SWIGLU configurations pair gate and up blocks
  if (p.splits > 1) {
    if constexpr (NBW == 2)
      launch(gemm_stream_kernel<MB, NBW, KC, GEMM_SWIGLU, true, PIPE>, total, 256, 0, s, p);
    else
      launch(gemm_stream_kernel<MB, NBW, KC, GEMM_STORE, true, PIPE>, total, 256, 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.defer_reduce) return e;
    if (hook && hook->fn) hook->fn(hook->ctx, 1);
    return splitk_reduce(a, p.part, p.part_ld, p.splits, s);
  }
  if constexpr (NBW == 2) {
    launch(gemm_stream_kernel<MB, NBW, KC, GEMM_SWIGLU, false, PIPE>, total, 256, 0, s, p);
  } else {
    switch (a.mode) {
      case GEMM_STORE: launch(gemm_stream_kernel<MB, NBW, KC, GEMM_STORE, false, PIPE>, total, 256, 0, s, p); break;
      case GEMM_RESIDUAL: launch(gemm_stream_kernel<MB, NBW, KC, GEMM_RESIDUAL, false, PIPE>, total, 256, 0, s, p); break;
      default: launch(gemm_stream_kernel<MB, NBW, KC, GEMM_F32OUT, false, PIPE>, total, 256, 0, s, p); break;
    }
  }
  return hipGetLastError();
}

}  // namespace

// Configurations: (rows per pass, packed n-blocks per wave, k-steps per chunk)
//   40: 32 rows,  1 block, 16    41: 64 rows, 1 block, 16
//   42: 32 rows,  2 blocks, 16   43: 64 rows, 2 blocks, 16  (SWIGLU)
//   44: 160 rows, 1 block, 16    45: 160 rows, 2 blocks, 16 (expert groups; one
//   workgroup per CU, so that an expert of up to 160 rows streams its weights once)
//   46, 47: as 44, 45 with 8 k-steps per chunk, double-buffered
//   48, 49: as 46, 47 with A loaded two chunks ahead
//   50, 51: as 46, 47 with the next chunk's loads spread over the MFMAs
hipError_t gemm_stream(const GemmArgs& a, const GemmPlan& p, void* ws, hipStream_t s, const LaunchHook* hook) {
  switch (p.cfg) {
    case 40: return launch_stream<1, 1, 16>(a, p, ws, s, hook);
    case 41: return launch_stream<2, 1, 16>(a, p, ws, s, hook);
    case 42: return launch_stream<1, 2, 16>(a, p, ws, s, hook);
    case 43: return launch_stream<2, 2, 16>(a, p, ws, s, hook);
    case 44: return launch_stream<5, 1, 16>(a, p, ws, s, hook);
    case 45: return launch_stream<5, 2, 16>(a, p, ws, s, hook);
    case 46: return launch_stream<5, 1, 8, 1>(a, p, ws, s, hook);
    case 47: return launch_stream<5, 2, 8, 1>(a, p, ws, s, hook);
    case 48: return launch_stream<5, 1, 8, 3>(a, p, ws, s, hook);
    case 49: return launch_stream<5, 2, 8, 3>(a, p, ws, s, hook);
    case 50: return launch_stream<5, 1, 8, 5>(a, p, ws, s, hook);
    case 51: return launch_stream<5, 2, 8, 5>(a, p, ws, s, hook);
    default: return hipErrorInvalidValue;
  }
}

int stream_nbw(int cfg) {
  switch (cfg) {
    case 42: case 43: case 45: case 47: case 49: case 51: return 2;
    case 40: case 41: case 44: case 46: case 48: case 50: return 1;
    default: return 0;
  }
}

int stream_kc(int cfg) {
  switch (cfg) {
    case 40: case 41: case 42: case 43: case 44: case 45: return 16;
    case 46: case 47: case 48: case 49: case 50: case 51: return 8;
    default: return 0;
  }
}

hipError_t pack_b(const void* W, int64_t ldw, int64_t group_stride, int N, int K, int groups, void* P,
                  int nb_stride, int nb_offset, int64_t packed_group_stride, hipStream_t s) {
  if (N % SB || K % SK) return hipErrorInvalidValue;
  const int64_t pieces = (int64_t)groups * (N / SB) * (K / SK) * 64;
  const int blocks = (int)std::min<int64_t>((pieces + 255) / 256, 4096);
  launch(pack_b_kernel, blocks, 256, 0, s, (const bf16*)W, ldw, group_stride, N, K, groups, (bf16*)P, nb_stride,
         nb_offset, 0, packed_group_stride);
  return hipGetLastError();
}

}  // namespace nf
