// Per-tensor FP8 quantisation for the FP8 linear layers.
//
// Current scaling: s = fmax / amax(|x|) over the whole tensor (s = 1 when the
// tensor is all zeros, and s is capped at 2^64 so that it stays finite for
// tensors of vanishing magnitude), all in fp32; code = round-to-nearest-even(clamp(x * s, +-fmax)) in
// the OCP E4M3 (fmax 448) or E5M2 (fmax 57344) format.  A product of two
// quantised operands is rescaled by 1 / (s_a * s_b) in the GEMM epilogue.
//
// The quantiser writes the codes row-major and, optionally, transposed
// ([C][R]), so that every FP8 product can take both operands K-contiguous:
// the forward uses X and W, the input gradient dY and W^T, the weight
// gradient dY^T and X^T.
#include "common.h"
#include "kernels.h"

namespace gk {

static_assert(AMAX_SLOT == AMAX_WAYS, "amax slot size must match the device-side spreading");

__device__ __forceinline__ float fp8_max(int fmt) { return fmt == FP8_E4M3 ? 448.f : 57344.f; }

// Two fp32 values -> two codes in the low 16 bits (round to nearest even).
__device__ __forceinline__ uint32_t cvt2(int fmt, float a, float b) {
  return fmt == FP8_E4M3 ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)
                         : __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
}

// Folds max |x| into the AMAX_WAYS words at amax (zeroed beforehand).  Each
// work-group reduces its share through LDS and issues one atomic.
__global__ __launch_bounds__(256) void amax_kernel(const bf16* __restrict__ x, long n, unsigned* amax) {
  __shared__ float red[4];
  float m = 0.f;
  const long n8 = n / 8;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n8; i += (long)gridDim.x * 256) {
    const bf16x8 v = *(const bf16x8*)(x + i * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)v[e]));
  }
  for (long i = n8 * 8 + (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256)
    m = fmaxf(m, fabsf((float)x[i]));
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(amax + (blockIdx.x & (AMAX_WAYS - 1)), __float_as_uint(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

// Sixteen consecutive values of row r as fp32: bf16 (widened exactly) or
// fp32, times rowscale[r] when given, or max(x, 0)^2 with RELU2.
template <bool RELU2>
__device__ __forceinline__ void load16(const bf16* src, const float*, int, float* f) {
  const bf16x8 v0 = *(const bf16x8*)src;
  const bf16x8 v1 = *(const bf16x8*)(src + 8);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    f[e] = (float)v0[e];
    f[8 + e] = (float)v1[e];
  }
}
template <bool RELU2>
__device__ __forceinline__ void load16(const float* src, const float* rowscale, int r, float* f) {
  const float rs = rowscale ? rowscale[r] : 1.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const floatx4 v = *(const floatx4*)(src + 4 * k);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (RELU2) {
        const float x = fmaxf(v[e], 0.f);
        f[4 * k + e] = x * x;
      } else {
        f[4 * k + e] = rowscale ? v[e] * rs : v[e];
      }
    }
  }
}

// Grid (C/64, ceil(R/64)), 256 threads: a 64x64 tile; thread t converts 16
// consecutive elements of row t/4.  Codes go to q[r][c] and (if qT) to
// qT[c][r] through an LDS transpose.  scale_out (if set) receives s.
template <int FMT, typename TI, bool RELU2>
__global__ __launch_bounds__(256) void quant_kernel(const TI* __restrict__ x, const float* __restrict__ rowscale,
                                                    int R, int C, const unsigned* __restrict__ amax,
                                                    float* scale_out, uint8_t* __restrict__ q,
                                                    uint8_t* __restrict__ qT) {
  __shared__ uint8_t tile[64][64 + 4];
  __shared__ float amax_s;
  const float fmax = fp8_max(FMT);
  if (threadIdx.x < 64) {
    const float w = wave_max(__uint_as_float(amax[threadIdx.x & (AMAX_WAYS - 1)]));
    if (threadIdx.x == 0) amax_s = w;
  }
  __syncthreads();
  const float a = amax_s;
  const float s = a > 0.f ? fminf(fmax / a, 0x1p64f) : 1.f;
  if (scale_out && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) scale_out[0] = s;
  const int t = threadIdx.x;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int rl = t >> 2, cl = (t & 3) * 16;
  const int r = r0 + rl;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (r < R) {
    float f[16];
    load16<RELU2>(x + (long)r * C + c0 + cl, rowscale, r, f);
#pragma unroll
    for (int e = 0; e < 16; ++e) f[e] = fminf(fmaxf(f[e] * s, -fmax), fmax);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (cvt2(FMT, f[4 * k], f[4 * k + 1]) & 0xFFFFu) | (cvt2(FMT, f[4 * k + 2], f[4 * k + 3]) << 16);
    *(u32x4*)(q + (long)r * C + c0 + cl) = u32x4{w[0], w[1], w[2], w[3]};
  }
  if (!qT) return;
#pragma unroll
  for (int k = 0; k < 16; ++k) tile[rl][cl + k] = (uint8_t)(w[k >> 2] >> (8 * (k & 3)));
  __syncthreads();
  // transposed: row c0 + t/4 of qT, 16 codes from rows r0 + (t%4)*16 ..
  const int cr = t >> 2, rc = (t & 3) * 16;
  if (r0 + rc >= R) return;
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = (uint32_t)tile[rc + 4 * k][cr] | ((uint32_t)tile[rc + 4 * k + 1][cr] << 8) |
           ((uint32_t)tile[rc + 4 * k + 2][cr] << 16) | ((uint32_t)tile[rc + 4 * k + 3][cr] << 24);
  uint8_t* dst = qT + (long)(c0 + cr) * R + r0 + rc;
  if ((R & 15) == 0 && r0 + rc + 16 <= R) {
    *(u32x4*)dst = u32x4{o[0], o[1], o[2], o[3]};
  } else {
    for (int k = 0; k < 16 && r0 + rc + k < R; ++k) dst[k] = (uint8_t)(o[k >> 2] >> (8 * (k & 3)));
  }
}

__global__ void zero_u32_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

void zero_u32(unsigned* p, int n, hipStream_t st) {
  hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
}

void fp8_amax(const void* x, long n, unsigned* amax, hipStream_t st) {
  long blocks = (n / 8 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const bf16*)x, n, amax);
}

template <typename TI, bool RELU2>
static void quantize_t(int fmt, const TI* x, const float* rowscale, int R, int C, const unsigned* amax,
                       float* scale_out, void* q, void* qT, hipStream_t st) {
  dim3 g(C / 64, (R + 63) / 64);
  if (fmt == FP8_E4M3)
    hipLaunchKernelGGL((quant_kernel<FP8_E4M3, TI, RELU2>), g, dim3(256), 0, st, x, rowscale, R, C, amax,
                       scale_out, (uint8_t*)q, (uint8_t*)qT);
  else
    hipLaunchKernelGGL((quant_kernel<FP8_E5M2, TI, RELU2>), g, dim3(256), 0, st, x, rowscale, R, C, amax,
                       scale_out, (uint8_t*)q, (uint8_t*)qT);
}

void fp8_quantize(int fmt, const void* x, int R, int C, const unsigned* amax, float* scale_out, void* q, void* qT,
                  hipStream_t st, int x_f32, const float* rowscale, int relu2) {
  if (x_f32 && relu2) quantize_t<float, true>(fmt, (const float*)x, nullptr, R, C, amax, scale_out, q, qT, st);
  else if (x_f32) quantize_t<float, false>(fmt, (const float*)x, rowscale, R, C, amax, scale_out, q, qT, st);
  else quantize_t<bf16, false>(fmt, (const bf16*)x, nullptr, R, C, amax, scale_out, q, qT, st);
}

}  // namespace gk
