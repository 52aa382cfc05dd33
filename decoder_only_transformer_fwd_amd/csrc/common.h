// Shared device-side definitions for the gfx950 kernels of the GPT step.
//
// Element types: float (fp32 configuration), bf16 (stored as __bf16), and the
// OCP fp8 formats (stored as uint8).  MFMA traits describe, per operand type,
// how many elements one lane feeds into a 32x32 MFMA (EPL) and the K depth
// of one instruction (KM).  For every 32x32 MFMA used here the A operand of
// lane l is row (l % 32) and the B operand is column (l % 32); lane group
// g = l / 32 supplies a fixed K subset, the same for A and B.  The 16 fp32
// accumulators of lane l hold D[8*(r/4) + 4*g + r%4][l % 32], r = 0..15.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gk {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct fp8e4 { uint8_t v; };   // OCP E4M3FN code
struct fp8e5 { uint8_t v; };   // OCP E5M2 code

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Store 4 consecutive fp32 values as T (8 or 16 bytes, naturally aligned).
__device__ __forceinline__ void store4(float* p, floatx4 v) { *(floatx4*)p = v; }
__device__ __forceinline__ void store4(bf16* p, floatx4 v) {
  bf16x4 r = __builtin_convertvector(v, bf16x4);
  *(bf16x4*)p = r;
}
__device__ __forceinline__ floatx4 load4(const float* p) { return *(const floatx4*)p; }
__device__ __forceinline__ floatx4 load4(const bf16* p) {
  bf16x4 r = *(const bf16x4*)p;
  return __builtin_convertvector(r, floatx4);
}

// ---------------------------------------------------------------- MFMA traits
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KM = 16;   // K per instruction
  static constexpr int EPL = 8;   // elements per lane per operand
  typedef bf16x8 frag;
  __device__ __forceinline__ static floatx16 mma(frag a, frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KM = 2;
  static constexpr int EPL = 1;
  typedef float frag;
  __device__ __forceinline__ static floatx16 mma(frag a, frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// fp8 x fp8 with neutral (2^0) block scales: format codes 0 = E4M3, 1 = E5M2
// (FA for the first operand, FB for the second).  Each lane supplies 32
// codes of one row (first operand) / column (second operand).
template <int FA, int FB> struct MfmaF8 {
  static constexpr int KM = 64;
  static constexpr int EPL = 32;
  typedef intx8 frag;
  __device__ __forceinline__ static floatx16 mma(frag a, frag b, floatx16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 127, 0, 127);
  }
};

// ---------------------------------------------------------------- LDS layout
// Tiles are stored row by row; each row is cut into 16-byte chunks and chunk c
// of row r lives at chunk slot c ^ swz(r) so that 16 consecutive rows read at
// the same chunk hit distinct bank groups (64 banks x 4 bytes).
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int row) {
  constexpr int NCH = ROW_BYTES / 16;
  constexpr int RP = (256 / ROW_BYTES) > 0 ? (256 / ROW_BYTES) : 1;
  return (row / RP) & (NCH - 1);
}
template <int ROW_BYTES>
__device__ __forceinline__ int lds_off(int row, int byte_in_row) {
  const int c = byte_in_row >> 4;
  return row * ROW_BYTES + (((c ^ swz<ROW_BYTES>(row))) << 4) + (byte_in_row & 15);
}

// Read `bytes` (4, 8, 16 or 32) at (row, byte) of a swizzled LDS tile.
template <int ROW_BYTES, int BYTES>
__device__ __forceinline__ void lds_read(const char* base, int row, int byte, void* out) {
  if constexpr (BYTES == 32) {
    *(u32x4*)out = *(const u32x4*)(base + lds_off<ROW_BYTES>(row, byte));
    *((u32x4*)out + 1) = *(const u32x4*)(base + lds_off<ROW_BYTES>(row, byte + 16));
  } else if constexpr (BYTES == 16) {
    *(u32x4*)out = *(const u32x4*)(base + lds_off<ROW_BYTES>(row, byte));
  } else if constexpr (BYTES == 8) {
    *(u32x2*)out = *(const u32x2*)(base + lds_off<ROW_BYTES>(row, byte));
  } else {
    *(uint32_t*)out = *(const uint32_t*)(base + lds_off<ROW_BYTES>(row, byte));
  }
}

// Raw buffer resource for `nbytes` bytes at `base`.  Both are uniform across
// the wave by construction; taking them through readfirstlane lets the
// compiler prove it and keep the descriptor in scalar registers (a
// descriptor it cannot prove uniform is wrapped in a per-load loop over
// lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int nbytes) {
  const unsigned long long bp = (unsigned long long)base;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)bp);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(bp >> 32));
  const int nb = __builtin_amdgcn_readfirstlane(nbytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((unsigned long long)hi << 32) | lo), 0, nb, 0x00020000);
}

// Rows of a global matrix copied straight into a swizzled LDS tile by buffer
// loads with the LDS bit (no registers).  One wave instruction writes 64
// lanes x 16 bytes = RPI consecutive LDS rows of RB bytes; the lane owning
// LDS slot p of row r fetches source chunk p ^ swz(r).  Source row r of the
// tile starts at base + row_off + r * stride; bytes at or past `nbytes` from
// base read as zero.
// One wave instruction: 64 lanes x 16 bytes from the buffer into LDS at
// lds + 16 * lane.  Bytes at or past the buffer's size read as zero.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds, int off, int soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, soff, 0, 0);
}

template <int ROWS, int RB, int NW>
struct RowDma {
  static constexpr int CPR = RB / 16;
  static constexpr int RPI = 64 / CPR;
  static constexpr int PER_WAVE = ROWS / (RPI * NW);
  static_assert(ROWS % (RPI * NW) == 0, "tile rows must split evenly over the waves");
  __amdgpu_buffer_rsrc_t rsrc;
  int voff[PER_WAVE];
  __device__ __forceinline__ void init(const void* base, int stride, long nbytes, int wave, int lane) {
    if (nbytes > 0x7FFFFFF0L) nbytes = 0x7FFFFFF0L;
    if (nbytes < 0) nbytes = 0;
    rsrc = uniform_rsrc(base, (int)nbytes);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int r = (wave * PER_WAVE + i) * RPI + lane / CPR;
      const int c = (lane % CPR) ^ swz<RB>(r);
      voff[i] = r * stride + c * 16;
    }
  }
  // row_off is uniform and goes in the scalar offset, so the per-lane offset
  // registers are never rewritten: no later register write has to wait for a
  // copy still reading them.
  __device__ __forceinline__ void issue(char* lds, int row_off, int wave) const {
    const int so = __builtin_amdgcn_readfirstlane(row_off);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) dma16(rsrc, lds + (wave * PER_WAVE + i) * RPI * RB, voff[i], so);
  }
};

// Transposing LDS read (16-bit elements).  Within each group of 16 lanes,
// lane 4a+b receives as its element e the b-th 16-bit value of the 8 bytes
// addressed by lane 4e+a of the same group (measured on gfx950).
typedef short shortx4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ shortx4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)p);
}

// Work-group barrier without the release/acquire fences of __syncthreads.
// Those fences make every wave wait for all of its outstanding global->LDS
// copies (vmcnt 0) at each barrier, which would drain a multi-stage pipeline;
// callers wait for exactly the copies and LDS reads they depend on.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// ---------------------------------------------------------------- reductions
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
// Sum over aligned groups of W lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// A tensor's running max |x| is kept in AMAX_WAYS words (bit patterns of
// non-negative floats, all starting at 0); writers spread their atomics over
// the words so that thousands of waves do not queue on one address, and the
// reader takes the max of all of them.  Max is order-independent, so the
// result is deterministic.
constexpr int AMAX_WAYS = 64;
__device__ __forceinline__ int amax_way() {
  return (blockIdx.x + blockIdx.y * 17 + blockIdx.z * 31) & (AMAX_WAYS - 1);
}
// Fold the work-group's largest |value| in: one atomic per work-group of NW
// waves, reduced through `red` (NW floats of LDS).  Every thread of the
// work-group must call it.
template <int NW>
__device__ __forceinline__ void block_amax(unsigned* amax, float m, float* red) {
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = fmaxf(r, red[w]);
    atomicMax(amax + amax_way(), __float_as_uint(r));
  }
}
// Largest |x_e| of 4 values after rounding to T (the values actually stored).
template <typename T>
__device__ __forceinline__ float abs_max4(floatx4 v) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(to_f32(from_f32<T>(v[e]))));
  return m;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace gk
