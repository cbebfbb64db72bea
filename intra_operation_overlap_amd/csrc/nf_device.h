// Device-side types and helpers shared by the HIP kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Storage conversions.  float -> bf16 rounds to nearest even (the compiler
// emits gfx950's v_cvt_pk_bf16_f32 for this cast).
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// SiLU z * sigmoid(z), the reciprocal by v_rcp_f32 (1 ulp; the result is
// rounded to bf16).  Large negative z gives -0, as the quotient does.
__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Element offsets inside one (page, KV head) block of 16 key slots x D dims
// (D % 32 == 0): the KV pool stores each block in the operand order of the
// attention MFMAs, so a wavefront fetches a 512-element run with one linear
// 16-byte-per-lane load.
//   K: chunk c = d / 32 holds, for lane l = 16 * ((d % 32) / 8) + s, the 8
//      dims 32c + 8 (l / 16) .. of key s (the A operand of S^T = K Q^T).
//   V: chunk c = d / 32 holds, for lane l = (d % 16) + 16 * (s / 4), keys
//      4 (l / 16) .. +3 of dim 32c + l % 16 and then of dim 32c + 16 + l % 16
//      (A operands of O^T = V^T P^T for two 16-dim blocks).
__device__ __forceinline__ int kv_k_off(int s, int d) {
  return (d >> 5) * 512 + ((((d & 31) >> 3) << 4) + s) * 8 + (d & 7);
}
__device__ __forceinline__ int kv_v_off(int s, int d) {
  return (d >> 5) * 512 + ((d & 15) + ((s >> 2) << 4)) * 8 + ((d >> 4) & 1) * 4 + (s & 3);
}

// Sum of `splits` fp32 partial slices p[0], p[zstride], p[2 zstride], ...
// (V: float or an fp32 vector) added in slice order from zero, so the result
// is bit-identical to a sequential loop; the loads of up to 8 slices are
// issued together instead of one memory latency per slice.
template <typename V>
__device__ __forceinline__ V sum_slices(const float* p, int64_t zstride, int splits) {
  V acc = V{};
  for (int z0 = 0; z0 < splits; z0 += 8) {
    V buf[8];
#pragma unroll
    for (int z = 0; z < 8; ++z)
      if (z0 + z < splits) buf[z] = *(const V*)(p + (int64_t)(z0 + z) * zstride);
#pragma unroll
    for (int z = 0; z < 8; ++z)
      if (z0 + z < splits) acc += buf[z];
  }
  return acc;
}

// ---------------------------------------------------------------- launch and memory helpers

// The dispatcher deals workgroups round-robin over the 8 XCDs; this maps the
// hardware order to a logical tile index such that each XCD is handed one
// contiguous range of tiles (so neighbouring tiles share that XCD's L2).
constexpr int NXCD = 8;
__device__ __forceinline__ int xcd_logical(int hw, int total) {
  const int xcd = hw % NXCD, slot = hw / NXCD;
  const int q = total / NXCD, r = total % NXCD;
  return xcd * q + min(xcd, r) + slot;
}

// Raw buffer resource over `base`: byte offsets up to 4 GiB, no range check
// (word 3 is the gfx9-family data format for untyped dword access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)0xffffffff, 0x00020000);
}

// Buffer resource with no records: every load through it is out of range, so
// it moves no memory (a load with it stands in for a load that must not run,
// keeping loop bodies branch-free and per-wave load counts constant).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc_empty(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0, 0x00020000);
}

// 16 bytes per lane from base + soff + voff straight into LDS through the
// buffer unit (buffer_load_dwordx4 ... lds): lane l writes lds + 16 l, so one
// instruction fills 1 KB.  The global form (global_load_lds) would do the
// same, but as a FLAT-family instruction it makes the compiler wait for all
// LDS reads (lgkmcnt(0)) wherever fragment reads are in flight.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff,
                                           (int)soff, 0, 0);
}

// Wait until at most N of this wave's vector-memory loads are outstanding
// (loads retire in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that waits only for this wave's LDS operations, not for
// its global loads still in flight.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
