// gpt_gemm_noalloc: the single-product entry point for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The split-K partial sums that gpt_gemm
// keeps in a caller workspace live here in a file-scope device array.
//
// The array is a symbol of this library's code object: each GPU the library
// runs on holds its own copy, at its own address, until the process ends.  In
// host code its name is only a stand-in, so its device address is looked up
// once per device with hipGetSymbolAddress (on the first call with that
// device current) and only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "model.h"

using namespace gk;
using namespace gm;

// The split-K partial sums of gpt_gemm_noalloc (one copy per GPU).
static __device__ __align__(256) float scratch[(size_t)GPT_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr size_t SCRATCH_BYTES = (size_t)GPT_NOALLOC_SCRATCH_BYTES;
constexpr size_t SCRATCH_FLOATS = SCRATCH_BYTES / sizeof(float);
constexpr int MAX_DEVICES = 64;

std::mutex g_mu;
float* g_ptr[MAX_DEVICES] = {};

// Device address of the current device's copy of `scratch` (looked up on
// the first call per device).
int scratch_ptr(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GPT_EHIP, std::string("gpt_gemm_noalloc: hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(GPT_EINVAL, "gpt_gemm_noalloc: device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(GPT_EHIP, std::string("gpt_gemm_noalloc: hipGetSymbolAddress: ") + hipGetErrorString(e));
    g_ptr[dev] = (float*)p;
  }
  *out = g_ptr[dev];
  return GPT_OK;
}

}  // namespace

extern "C" int gpt_gemm_noalloc(int dtype, int layout, int M, int N, int K, const void* A, const void* B, float* C,
                                int splits, int tile, void* stream) {
  int rc = gemm_check(dtype, layout, M, N, K, A, B, C, splits, tile, "gpt_gemm_noalloc");
  if (rc) return rc;
  if (splits > 1) {
    const size_t need = (size_t)gemm_real_splits(dtype, K, splits, nullptr) * (size_t)M * (size_t)N;
    if (need > SCRATCH_FLOATS)
      return fail(GPT_EINVAL, "gpt_gemm_noalloc: splits * M * N = " + std::to_string(need) +
                                  " partial sums exceed the scratch limit of " + std::to_string(SCRATCH_FLOATS) +
                                  " floats");
  }
  float* part = nullptr;
  if (splits > 1 && (rc = scratch_ptr(&part))) return rc;
  // every partial is written before it is read (each split stores its whole
  // M x N block), so nothing needs clearing between calls
  return gemm_entry(dtype, layout, M, N, K, A, B, C, part, splits, tile, stream, "gpt_gemm_noalloc");
}
