// Device probes: dense bf16 matrix-core peak, HBM read bandwidth, and the
// hardware identity (XCC / CU) a workgroup lands on.
#include <algorithm>

#include "nf_device.h"
#include "nf_internal.h"

namespace nf {
namespace {

// Eight independent accumulator chains of one bf16 MFMA shape per wave,
// operands in registers only.  SHAPE 0: 16x16x32, SHAPE 1: 32x32x16.
template <int SHAPE>
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* sink) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (bf16)(float)((threadIdx.x + e) & 3);
    b[e] = (bf16)(float)((threadIdx.x * 3 + e) & 3);
  }
  float s = 0.f;
  if (SHAPE == 0) {
    f32x4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  } else {
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) s += acc[c][0] + acc[c][5] + acc[c][10] + acc[c][15];
  }
  if (s == 12345.678f) sink[threadIdx.x] = s;     // keeps the chains live
}

// Deterministic pseudo-random bf16 fill: element i gets scale * u, with u
// uniform in [-1, 1) taken from the MurmurHash3 32-bit finaliser of i ^ seed.
// Constant operands would understate the matrix cores' switching power and so
// overstate the clock a GEMM holds on real data.
__global__ __launch_bounds__(256) void probe_fill_bf16_kernel(bf16* p, int64_t n, uint32_t seed, float scale) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    uint32_t h = (uint32_t)i ^ (uint32_t)(i >> 32) * 0x9e3779b9u ^ seed;
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    p[i] = (bf16)(scale * ((float)(h >> 8) * (1.0f / 8388608.0f) - 1.0f));
  }
}

// Streams the buffer once, 16 bytes per lane per load, grid-strided.
template <int U>
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ buf, size_t n16, float* sink) {
  uint32_t x = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u][0] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = buf[i];
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (x == 0x9e3779b9u) sink[threadIdx.x] = (float)x;
}

// HW_ID (hwreg 4) and XCC_ID (hwreg 20) of the first wave of each workgroup.
__global__ void probe_hwid_kernel(uint32_t* out) {
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = __builtin_amdgcn_s_getreg((4) | (0 << 6) | ((32 - 1) << 11));
    out[2 * blockIdx.x + 1] = __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((16 - 1) << 11));
  }
}

}  // namespace

hipError_t probe_mfma(int shape, int n_blocks, int iters, float* sink, hipStream_t s) {
  if (shape == 0)
    probe_mfma_kernel<0><<<n_blocks, 256, 0, s>>>(iters, sink);
  else
    probe_mfma_kernel<1><<<n_blocks, 256, 0, s>>>(iters, sink);
  return hipGetLastError();
}

hipError_t probe_read(const void* buf, size_t bytes, float* sink, int n_blocks, hipStream_t s) {
  probe_read_kernel<8><<<n_blocks, 256, 0, s>>>((const u32x4*)buf, bytes / 16, sink);
  return hipGetLastError();
}

hipError_t probe_hwid(uint32_t* out, int n_blocks, hipStream_t s) {
  probe_hwid_kernel<<<n_blocks, 64, 0, s>>>(out);
  return hipGetLastError();
}

hipError_t probe_fill_bf16(void* p, int64_t n, uint32_t seed, float scale, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
  launch(probe_fill_bf16_kernel, blocks, 256, 0, s, (bf16*)p, n, seed, scale);
  return hipGetLastError();
}

}  // namespace nf
