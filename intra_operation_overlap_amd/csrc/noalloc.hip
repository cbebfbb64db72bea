// nf_gemm_bf16_noalloc: the layer's bf16 GEMM for callers that cannot
// allocate device memory (code under stream capture, tight serving loops).
// Its only scratch memory -- the fp32 split-K partial slices -- lives in a
// file-scope device array of fixed size instead of a hipMalloc'd workspace.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "nf_internal.h"

using namespace nf;

static constexpr size_t kScratchBytes = NF_NOALLOC_SCRATCH_BYTES;   // per device

// Split-K partials of nf_gemm_bf16_noalloc.  Host code never passes this name
// to a kernel (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

nf_status fail(nf_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
nf_status fail(nf_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return nf::set_error(st, buf);
}

// This device's address of `scratch`, looked up on the first call made with
// the device current.
nf_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(NF_ERR_HIP, "nf_gemm_bf16_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(NF_ERR_UNSUPPORTED, "nf_gemm_bf16_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(NF_ERR_HIP, "nf_gemm_bf16_noalloc: hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return NF_OK;
}

}  // namespace

extern "C" nf_status nf_gemm_bf16_noalloc(int32_t M, int32_t N, int32_t K, int32_t mode, const void* A, int64_t lda,
                                          const void* Bw, const void* B2, int64_t ldb, const void* R, int64_t ldr,
                                          void* C, int64_t ldc, int32_t tile_cfg, int32_t k_splits, int32_t cus,
                                          void* stream, int32_t* out_cfg, int32_t* out_splits) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 8 || N % 8 || mode < 0 || mode > 2 || !A || !Bw || !C ||
      (mode == GEMM_RESIDUAL && !R) || (mode == GEMM_SWIGLU && !B2) || lda < K || ldb < K || ldc < N ||
      (mode == GEMM_RESIDUAL && ldr < N))
    return fail(NF_ERR_INVALID_ARG, "nf_gemm_bf16_noalloc: bad argument");
  if (tile_cfg >= 40)
    return fail(NF_ERR_UNSUPPORTED, "nf_gemm_bf16_noalloc: tile_cfg %d: the weight-streaming configurations need "
                "an operand-order copy of B; use nf_gemm_bf16", tile_cfg);
  if (tile_cfg >= 0 && !((tile_cfg <= 6) || (tile_cfg >= 10 && tile_cfg <= 30 && K % 64 == 0)))
    return fail(NF_ERR_INVALID_ARG, "nf_gemm_bf16_noalloc: tile_cfg %d not available for N %d K %d mode %d", tile_cfg,
                N, K, mode);
  if ((int64_t)M * lda * 2 >= (int64_t(1) << 32) || (int64_t)N * ldb * 2 >= (int64_t(1) << 32))
    return fail(NF_ERR_OUT_OF_RANGE, "nf_gemm_bf16_noalloc: an operand would exceed 4 GiB");
  GemmArgs g;
  g.A = A; g.lda = lda;
  g.B = Bw; g.B2 = B2; g.ldb = ldb;
  g.C = C; g.ldc = ldc; g.R = R; g.ldr = ldr;
  g.M = M; g.N = N; g.K = K; g.mode = mode;
  GemmPlan p = gemm_choose(g, cus > 0 ? cus : 256);
  if (tile_cfg >= 0) p.cfg = tile_cfg;
  if (k_splits > 0) p.k_splits = k_splits;
  if (p.cfg >= 40)
    return fail(NF_ERR_UNSUPPORTED, "nf_gemm_bf16_noalloc: configuration %d streams an operand-order copy of B",
                p.cfg);
  const size_t wsb = gemm_workspace_bytes(g, p);
  if (wsb > kScratchBytes)
    return fail(NF_ERR_OUT_OF_RANGE, "nf_gemm_bf16_noalloc: split-K partials need %zu bytes, the scratch array "
                "holds %zu (M x N x splits x 4 bytes; N doubled for SwiGLU): fewer splits or a smaller problem",
                wsb, kScratchBytes);
  void* ws = nullptr;
  if (wsb) {
    nf_status st = scratch_ptr(&ws);
    if (st != NF_OK) return st;
  }
  hipError_t e = gemm_bf16(g, p, ws, (hipStream_t)stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(NF_ERR_HIP, "nf_gemm_bf16_noalloc: %s", hipGetErrorString(e));
  }
  if (out_cfg) *out_cfg = p.cfg;
  if (out_splits) *out_splits = p.k_splits;
  return NF_OK;
}
