// Bandwidth-bound kernels of the GPT step: embedding, RMSNorm, rotary + QK
// norm, attention-backward preparation, cross-entropy row reduction and the
// embedding-gradient segmented sum.  Each kernel reads and writes every byte
// once with 8- or 16-byte accesses; per-row statistics are wave reductions.
#include "common.h"
#include "kernels.h"

namespace gk {

// ------------------------------------------------------------------ embedding
// h[r, :] = E[tokens[r], :] (fp32).  An id outside [0, vocab) sets *flag and
// writes a zero row.
template <typename T>
__global__ __launch_bounds__(256) void embed_fwd_kernel(const int32_t* __restrict__ tok,
                                                        const int32_t* __restrict__ tgt,
                                                        const T* __restrict__ E, float* __restrict__ h,
                                                        int rows, int d, int vocab, int* flag) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int id = tok[row];
  const int y = tgt[row];
  const bool ok = id >= 0 && id < vocab;
  if ((!ok || y < 0 || y >= vocab) && lane == 0) atomicOr(flag, 1);
  for (int c = lane * 4; c < d; c += 256) {
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (ok) v = load4(E + (long)id * d + c);
    store4(h + (long)row * d + c, v);
  }
}

// ------------------------------------------------------------------ rmsnorm
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const float* __restrict__ x, T* __restrict__ y,
                                                          float* __restrict__ rstd, int rows, int d,
                                                          float eps, unsigned* __restrict__ amax) {
  __shared__ float red[4];
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float m = 0.f;
  if (row < rows) {
    const float* xr = x + (long)row * d;
    float ss = 0.f;
    for (int c = lane * 4; c < d; c += 256) {
      const floatx4 v = load4(xr + c);
      ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    for (int c = lane * 4; c < d; c += 256) {
      const floatx4 v = load4(xr + c) * r;
      store4(y + (long)row * d + c, v);
      if (amax) m = fmaxf(m, abs_max4<float>(v));
    }
    if (lane == 0) rstd[row] = r;
  }
  if (amax) block_amax<4>(amax, m, red);
}

// Register-resident variants for d <= 512 * NCH, d % 8 == 0: one wave per
// row, each lane holding NCH chunks of 8 consecutive elements (32-byte fp32
// and 16-byte bf16 accesses), so every input byte is read exactly once.
__device__ __forceinline__ void load8(const float* p, floatx4& lo, floatx4& hi) {
  lo = *(const floatx4*)p;
  hi = *(const floatx4*)(p + 4);
}
__device__ __forceinline__ void load8(const bf16* p, floatx4& lo, floatx4& hi) {
  const bf16x8 v = *(const bf16x8*)p;
  lo = __builtin_convertvector(__builtin_shufflevector(v, v, 0, 1, 2, 3), floatx4);
  hi = __builtin_convertvector(__builtin_shufflevector(v, v, 4, 5, 6, 7), floatx4);
}
__device__ __forceinline__ void store8(float* p, floatx4 lo, floatx4 hi) {
  *(floatx4*)p = lo;
  *(floatx4*)(p + 4) = hi;
}
__device__ __forceinline__ void store8(bf16* p, floatx4 lo, floatx4 hi) {
  const bf16x4 a = __builtin_convertvector(lo, bf16x4), b = __builtin_convertvector(hi, bf16x4);
  *(bf16x8*)p = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <typename T, int NCH>
__global__ __launch_bounds__(256) void rmsnorm_fwd_reg_kernel(const float* __restrict__ x, T* __restrict__ y,
                                                              float* __restrict__ rstd, int rows, int d, float eps,
                                                              unsigned* __restrict__ amax) {
  __shared__ float red[4];
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float m = 0.f;
  if (row < rows) {
    const float* xr = x + (long)row * d;
    floatx4 v[NCH][2];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c = (k * 64 + lane) * 8;
      if (c < d) {
        load8(xr + c, v[k][0], v[k][1]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) ss = __builtin_fmaf(v[k][h][e], v[k][h][e], ss);
      }
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c = (k * 64 + lane) * 8;
      if (c < d) {
        const floatx4 lo = v[k][0] * r, hi = v[k][1] * r;
        store8(y + (long)row * d + c, lo, hi);
        if (amax) m = fmaxf(m, fmaxf(abs_max4<float>(lo), abs_max4<float>(hi)));
      }
    }
    if (lane == 0) rstd[row] = r;
  }
  if (amax) block_amax<4>(amax, m, red);
}

template <typename T, int NCH>
__global__ __launch_bounds__(256) void rmsnorm_bwd_reg_kernel(const void* __restrict__ dy, int dy_act,
                                                              const T* __restrict__ y,
                                                              const float* __restrict__ rstd, float* __restrict__ dx,
                                                              T* __restrict__ dxa, int rows, int d, int accumulate,
                                                              unsigned* __restrict__ amax) {
  __shared__ float red[4];
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float m = 0.f;
  if (row < rows) {
    const long base = (long)row * d;
    floatx4 a[NCH][2], b[NCH][2], acc[NCH][2];
    float dot = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c = (k * 64 + lane) * 8;
      if (c < d) {
        if (dy_act) load8((const T*)dy + base + c, a[k][0], a[k][1]);   // dy in the activation type
        else load8((const float*)dy + base + c, a[k][0], a[k][1]);
        load8(y + base + c, b[k][0], b[k][1]);
        if (accumulate) load8(dx + base + c, acc[k][0], acc[k][1]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) dot = __builtin_fmaf(a[k][h][e], b[k][h][e], dot);
      }
    }
    dot = wave_sum(dot) / (float)d;
    const float r = rstd[row];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c = (k * 64 + lane) * 8;
      if (c < d) {
        floatx4 g[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          g[h] = (a[k][h] - b[k][h] * dot) * r;
          if (accumulate) g[h] += acc[k][h];
        }
        store8(dx + base + c, g[0], g[1]);
        store8(dxa + base + c, g[0], g[1]);
        if (amax) m = fmaxf(m, fmaxf(abs_max4<float>(g[0]), abs_max4<float>(g[1])));
      }
    }
  }
  if (amax) block_amax<4>(amax, m, red);
}

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const float* __restrict__ dy, const T* __restrict__ y,
                                                          const float* __restrict__ rstd, float* __restrict__ dx,
                                                          T* __restrict__ dxa, int rows, int d, int accumulate,
                                                          unsigned* __restrict__ amax) {
  __shared__ float red[4];
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float m = 0.f;
  if (row < rows) {
    const long base = (long)row * d;
    float dot = 0.f;
    for (int c = lane * 4; c < d; c += 256) {
      const floatx4 a = load4(dy + base + c);
      const floatx4 b = load4(y + base + c);
      dot += a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
    }
    dot = wave_sum(dot) / (float)d;
    const float r = rstd[row];
    for (int c = lane * 4; c < d; c += 256) {
      floatx4 g = (load4(dy + base + c) - load4(y + base + c) * dot) * r;
      if (accumulate) g += load4(dx + base + c);
      store4(dx + base + c, g);
      store4(dxa + base + c, g);
      if (amax) m = fmaxf(m, abs_max4<float>(g));
    }
  }
  if (amax) block_amax<4>(amax, m, red);
}

// ------------------------------------------------------------------ rotary + QK norm
// Column of head h's part (0 q, 1 k, 2 v) in a qkv row: q heads, then the Hkv
// key heads, then the Hkv value heads.
__device__ __forceinline__ int qkv_col(int part, int h, int H, int Hkv, int DH) {
  return part == 0 ? h * DH : part == 1 ? (H + h) * DH : (H + Hkv + h) * DH;
}

// Grid (ceil(T/64), H, B); 256 threads.  For q of head h, and k of head h
// when h < Hkv: rotate the half-split pairs (x[i], x[i+Dh/2]) by t*theta_i,
// RMS-normalise the head vector, write it back in place and into the
// transposed copy [B][heads][Dh][Tp]; v (h < Hkv) is only transposed.  Tokens
// t >= T are written as zeros in the copies.
template <typename T, int DH>
__global__ __launch_bounds__(256) void rope_qknorm_fwd_kernel(T* __restrict__ qkv, float* __restrict__ rstd_qk,
                                                              T* __restrict__ qT, T* __restrict__ kT,
                                                              T* __restrict__ vT, const float* __restrict__ cosb,
                                                              const float* __restrict__ sinb, int Tn, int Tp,
                                                              int H, int Hkv, float eps) {
  constexpr int HALF = DH / 2;
  constexpr int TPP = 64 / HALF;      // tokens per wave pass
  constexpr int LDW = 64 + 16 / sizeof(T) * 2;  // padded tile row (elements), 16-byte multiple
  __shared__ __attribute__((aligned(16))) T tile[DH * LDW];
  const int t0 = blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / HALF, i = lane % HALF;
  const long row3 = (long)(H + 2 * Hkv) * DH;
  const int nparts = h < Hkv ? 3 : 1;   // block-uniform
  for (int part = 0; part < nparts; ++part) {
    const int col = qkv_col(part, h, H, Hkv, DH);
    for (int tt = wave * 16; tt < wave * 16 + 16; tt += TPP) {
      const int tl = tt + sub;
      const int t = t0 + tl;
      const bool ok = t < Tn;
      float y1 = 0.f, y2 = 0.f;
      T* px = qkv + ((long)b * Tn + t) * row3 + col;
      if (ok) {
        y1 = to_f32(px[i]);
        y2 = to_f32(px[i + HALF]);
      }
      if (part < 2) {
        float c = 0.f, s = 0.f;
        if (ok) {
          c = cosb[t * HALF + i];
          s = sinb[t * HALF + i];
        }
        const float r1 = y1 * c - y2 * s;
        const float r2 = y1 * s + y2 * c;
        const float ss = group_sum<HALF>(r1 * r1 + r2 * r2);
        const float r = 1.0f / sqrtf(ss / (float)DH + eps);
        y1 = r1 * r;
        y2 = r2 * r;
        if (ok) {
          px[i] = from_f32<T>(y1);
          px[i + HALF] = from_f32<T>(y2);
          if (i == 0) rstd_qk[((long)b * Tn + t) * (H + Hkv) + part * H + h] = r;
        }
      }
      tile[i * LDW + tl] = from_f32<T>(ok ? y1 : 0.f);
      tile[(i + HALF) * LDW + tl] = from_f32<T>(ok ? y2 : 0.f);
    }
    __syncthreads();
    T* dst = part == 0 ? qT : (part == 1 ? kT : vT);
    const int nh = part == 0 ? H : Hkv;
    constexpr int EPC = 16 / sizeof(T);
    constexpr int CPR = 64 / EPC;    // chunks per row
    for (int c = threadIdx.x; c < DH * CPR; c += 256) {
      const int r = c / CPR, cc = c % CPR;
      if (t0 + cc * EPC < Tp)
        *(u32x4*)(dst + (((long)b * nh + h) * DH + r) * Tp + t0 + cc * EPC) =
            *(const u32x4*)(tile + r * LDW + cc * EPC);
    }
    __syncthreads();
  }
}

// The same for bf16 heads of 128: grid (ceil(T/128), H, B), 512 threads.
// Thread (p, c) = (tid / 8, tid % 8) owns tokens 2p and 2p+1 of the 128-token
// tile and the 16-byte chunks c and c+8 of each head vector (elements 8c..
// and 64+8c.., the rotation pairs).  The head's sum of squares is a reduction
// over the 8 lanes sharing p.  All twelve 16-byte loads of q, k and v (and
// the rotation table) are issued before any arithmetic, so a thread has them
// in flight together.  The transposed copies go through LDS as 4-byte words
// holding one dimension of two consecutive tokens; the word stride per
// dimension is odd (65), so the word writes are free of bank conflicts.  Each
// dimension then leaves as one 256-byte run of the transposed row (chunks at
// or past Tp, a multiple of 64, are not stored).
__global__ __launch_bounds__(512) void rope_qknorm_fwd128_kernel(bf16* __restrict__ qkv, float* __restrict__ rstd_qk,
                                                                 bf16* __restrict__ qT, bf16* __restrict__ kT,
                                                                 bf16* __restrict__ vT, const float* __restrict__ cosb,
                                                                 const float* __restrict__ sinb, int Tn, int Tp,
                                                                 int H, int Hkv, float eps) {
  constexpr int DH = 128, HALF = 64, TT = 128, S = TT / 2 + 1;
  __shared__ uint32_t tile[DH * S];
  const int t0 = blockIdx.x * TT, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, p = tid >> 3, c = tid & 7;
  const long row3 = (long)(H + 2 * Hkv) * DH;
  const bool kv = h < Hkv;   // this block also owns key/value head h (block-uniform)
  bf16x8 raw[3][2][2];
  floatx4 cs[2][2], sn[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = t0 + 2 * p + u;
    const bool ok = t < Tn;
#pragma unroll
    for (int part = 0; part < 3; ++part) {
      const bool okp = ok && (part == 0 || kv);
      const bf16* px = qkv + ((long)b * Tn + t) * row3 + qkv_col(part, h, H, Hkv, DH);
      raw[part][u][0] = okp ? *(const bf16x8*)(px + 8 * c) : bf16x8{};
      raw[part][u][1] = okp ? *(const bf16x8*)(px + HALF + 8 * c) : bf16x8{};
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      cs[u][q] = ok ? *(const floatx4*)(cosb + (long)t * HALF + 8 * c + 4 * q) : floatx4{};
      sn[u][q] = ok ? *(const floatx4*)(sinb + (long)t * HALF + 8 * c + 4 * q) : floatx4{};
    }
  }
#pragma unroll
  for (int part = 0; part < 3; ++part) {
    if (part > 0 && !kv) break;   // block-uniform: every thread leaves together
    float x[2][16];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = t0 + 2 * p + u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[u][e] = (float)raw[part][u][0][e];
        x[u][8 + e] = (float)raw[part][u][1][e];
      }
      if (part < 2) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ce = cs[u][e >> 2][e & 3], se = sn[u][e >> 2][e & 3];
          const float r1 = x[u][e] * ce - x[u][8 + e] * se;
          const float r2 = x[u][e] * se + x[u][8 + e] * ce;
          x[u][e] = r1;
          x[u][8 + e] = r2;
          ss += r1 * r1 + r2 * r2;
        }
        ss = group_sum<8>(ss);
        const float r = 1.0f / sqrtf(ss / (float)DH + eps);
#pragma unroll
        for (int e = 0; e < 16; ++e) x[u][e] *= r;
        if (t < Tn) {
          bf16* px = qkv + ((long)b * Tn + t) * row3 + qkv_col(part, h, H, Hkv, DH);
          bf16x8 ylo, yhi;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            ylo[e] = (bf16)x[u][e];
            yhi[e] = (bf16)x[u][8 + e];
          }
          *(bf16x8*)(px + 8 * c) = ylo;
          *(bf16x8*)(px + HALF + 8 * c) = yhi;
          if (c == 0) rstd_qk[((long)b * Tn + t) * (H + Hkv) + part * H + h] = r;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int dim = (e < 8 ? 8 * c : HALF + 8 * c) + (e & 7);
      const uint32_t w = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)x[0][e]) |
                         ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)x[1][e]) << 16);
      tile[dim * S + p] = w;
    }
    __syncthreads();
    // 16-byte stores: thread (dim, q) writes tokens 8q .. 8q+7 of one dimension
    bf16* dst = (part == 0 ? qT : (part == 1 ? kT : vT)) + ((long)b * (part == 0 ? H : Hkv) + h) * DH * Tp + t0;
#pragma unroll
    for (int k = 0; k < DH * (TT / 8) / 512; ++k) {
      const int idx = tid + 512 * k, dim = idx / (TT / 8), q = idx % (TT / 8);
      const uint32_t* w = tile + dim * S + 4 * q;
      if (t0 + 8 * q < Tp) *(u32x4*)(dst + (long)dim * Tp + 8 * q) = u32x4{w[0], w[1], w[2], w[3]};
    }
    __syncthreads();
  }
}

// Backward of the rotation + QK norm for bf16 heads of 128, in place on the q
// and k columns of dqkv.  A group of 8 lanes takes one head vector (q or k of
// one head of one token, numbered row * (H + Hkv) + v, which is also its rstd
// index; v < H is q head v, v >= H k head v - H, and either sits at column
// v * Dh of the row); lane c holds elements 8c.. and 64+8c.. (the rotation
// pairs) of the gradient and of the normalised output, each as one 16-byte
// load.
__global__ __launch_bounds__(256) void rope_qknorm_bwd128_kernel(bf16* __restrict__ dqkv, const bf16* __restrict__ qkv,
                                                                 const float* __restrict__ rstd_qk,
                                                                 const float* __restrict__ cosb,
                                                                 const float* __restrict__ sinb, long nvec, int Tn,
                                                                 int H, int Hkv, unsigned* __restrict__ amax) {
  constexpr int DH = 128, HALF = 64;
  __shared__ float red[4];
  const long vec = (long)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int c = threadIdx.x & 7;
  const bool ok = vec < nvec;
  const int nv = H + Hkv;
  const long row = ok ? vec / nv : 0;
  const int v = (int)(vec - row * nv);
  const int t = (int)(row % Tn);
  const long off = row * (long)(H + 2 * Hkv) * DH + (long)v * DH;
  bf16x8 g[2], y[2];
  floatx4 cs[2], sn[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    g[hf] = ok ? *(const bf16x8*)(dqkv + off + hf * HALF + 8 * c) : bf16x8{};
    y[hf] = ok ? *(const bf16x8*)(qkv + off + hf * HALF + 8 * c) : bf16x8{};
    cs[hf] = ok ? *(const floatx4*)(cosb + (long)t * HALF + 8 * c + 4 * hf) : floatx4{};
    sn[hf] = ok ? *(const floatx4*)(sinb + (long)t * HALF + 8 * c + 4 * hf) : floatx4{};
  }
  const float r = ok ? rstd_qk[vec] : 0.f;
  float dot = 0.f;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = __builtin_fmaf((float)g[hf][e], (float)y[hf][e], dot);
  dot = group_sum<8>(dot) / (float)DH;
  bf16x8 o[2];
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float ce = cs[e >> 2][e & 3], se = sn[e >> 2][e & 3];
    const float d1 = r * ((float)g[0][e] - (float)y[0][e] * dot);
    const float d2 = r * ((float)g[1][e] - (float)y[1][e] * dot);
    o[0][e] = (bf16)(d1 * ce + d2 * se);
    o[1][e] = (bf16)(-d1 * se + d2 * ce);
    m = fmaxf(m, fmaxf(fabsf((float)o[0][e]), fabsf((float)o[1][e])));
  }
  if (ok) {
    *(bf16x8*)(dqkv + off + 8 * c) = o[0];
    *(bf16x8*)(dqkv + off + HALF + 8 * c) = o[1];
  }
  if (amax) block_amax<4>(amax, m, red);
}

// dq' = r * (g - y * mean(g*y)), then the inverse rotation; in place on the
// q and k columns of dqkv.  One wave per token row.
template <typename T, int DH>
__global__ __launch_bounds__(256) void rope_qknorm_bwd_kernel(T* __restrict__ dqkv, const T* __restrict__ qkv,
                                                              const float* __restrict__ rstd_qk,
                                                              const float* __restrict__ cosb,
                                                              const float* __restrict__ sinb, int rows, int Tn,
                                                              int H, int Hkv, unsigned* __restrict__ amax) {
  constexpr int HALF = DH / 2;
  constexpr int VPP = 64 / HALF;   // head vectors per pass
  __shared__ float red[4];
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int t = row % Tn;
  const int sub = lane / HALF, i = lane % HALF;
  const int nv = H + Hkv;
  const bool ok = row < rows;
  const float c = ok ? cosb[t * HALF + i] : 0.f, s = ok ? sinb[t * HALF + i] : 0.f;
  float m = 0.f;
  for (int v0 = 0; ok && v0 < nv; v0 += VPP) {
    const int v = v0 + sub;       // q heads then k heads, head v at column v * DH
    if (v >= nv) continue;
    const long off = (long)row * (H + 2 * Hkv) * DH + (long)v * DH;
    const float g1 = to_f32(dqkv[off + i]), g2 = to_f32(dqkv[off + i + HALF]);
    const float y1 = to_f32(qkv[off + i]), y2 = to_f32(qkv[off + i + HALF]);
    const float dot = group_sum<HALF>(g1 * y1 + g2 * y2) / (float)DH;
    const float r = rstd_qk[(long)row * nv + v];
    const float d1 = r * (g1 - y1 * dot), d2 = r * (g2 - y2 * dot);
    const T o1 = from_f32<T>(d1 * c + d2 * s), o2 = from_f32<T>(-d1 * s + d2 * c);
    dqkv[off + i] = o1;
    dqkv[off + i + HALF] = o2;
    m = fmaxf(m, fmaxf(fabsf(to_f32(o1)), fabsf(to_f32(o2))));
  }
  if (amax) block_amax<4>(amax, m, red);
}

// D[b,h,t] = sum_c dO[t, h*Dh + c] * O[t, h*Dh + c]; dO^T copy [B][H][Dh][Tp].
template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(const T* __restrict__ dO, const T* __restrict__ O,
                                                           float* __restrict__ Dv, T* __restrict__ dOT, int Tn,
                                                           int Tp, int H) {
  constexpr int HALF = DH / 2;
  constexpr int TPP = 64 / HALF;
  constexpr int LDW = 64 + 16 / sizeof(T) * 2;
  __shared__ __attribute__((aligned(16))) T tile[DH * LDW];
  const int t0 = blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / HALF, i = lane % HALF;
  const int d = H * DH;
  for (int tt = wave * 16; tt < wave * 16 + 16; tt += TPP) {
    const int tl = tt + sub;
    const int t = t0 + tl;
    const bool ok = t < Tn;
    float g1 = 0.f, g2 = 0.f, o1 = 0.f, o2 = 0.f;
    if (ok) {
      const long off = ((long)b * Tn + t) * d + h * DH;
      g1 = to_f32(dO[off + i]);
      g2 = to_f32(dO[off + i + HALF]);
      o1 = to_f32(O[off + i]);
      o2 = to_f32(O[off + i + HALF]);
    }
    const float s = group_sum<HALF>(g1 * o1 + g2 * o2);
    if (i == 0 && t < Tp) Dv[((long)b * H + h) * Tp + t] = ok ? s : 0.f;
    tile[i * LDW + tl] = from_f32<T>(g1);
    tile[(i + HALF) * LDW + tl] = from_f32<T>(g2);
  }
  __syncthreads();
  constexpr int EPC = 16 / sizeof(T);
  constexpr int CPR = 64 / EPC;
  for (int c = threadIdx.x; c < DH * CPR; c += 256) {
    const int r = c / CPR, cc = c % CPR;
    if (t0 + cc * EPC < Tp)
      *(u32x4*)(dOT + (((long)b * H + h) * DH + r) * Tp + t0 + cc * EPC) =
          *(const u32x4*)(tile + r * LDW + cc * EPC);
  }
}

// The same for bf16 heads of 128: grid (ceil(T/128), H, B), 512 threads.
// Thread (p, j) = (tid / 16, tid % 16) owns the 16-byte chunk j (dimensions
// 8j .. 8j+7) of tokens 2p, 2p+1 and 64+2p, 65+2p of the 128-token tile; all
// eight 16-byte loads go out together.  D is a sum over the 16 lanes sharing
// a token.  dO^T goes through LDS as 4-byte words holding one dimension of two
// consecutive tokens (odd word stride 65), then out in 16-byte stores, one
// 256-byte run per dimension (chunks at or past Tp are not stored).
__global__ __launch_bounds__(512) void attn_bwd_pre128_kernel(const bf16* __restrict__ dO, const bf16* __restrict__ O,
                                                              float* __restrict__ Dv, bf16* __restrict__ dOT, int Tn,
                                                              int Tp, int H) {
  constexpr int DH = 128, TT = 128, S = TT / 2 + 1;
  __shared__ uint32_t tile[DH * S];
  const int t0 = blockIdx.x * TT, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, p = tid >> 4, j = tid & 15;
  const int d = H * DH;
  bf16x8 g[2][2], o[2][2];   // [half of the tile][token of the pair]
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = t0 + 64 * hf + 2 * p + u;
      const long off = ((long)b * Tn + t) * d + h * DH + 8 * j;
      g[hf][u] = t < Tn ? *(const bf16x8*)(dO + off) : bf16x8{};
      o[hf][u] = t < Tn ? *(const bf16x8*)(O + off) : bf16x8{};
    }
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = __builtin_fmaf((float)g[hf][u][e], (float)o[hf][u][e], s);
      s = group_sum<16>(s);
      const int t = t0 + 64 * hf + 2 * p + u;
      if (j == 0 && t < Tp) Dv[((long)b * H + h) * Tp + t] = s;   // zero past Tn: the loads were zero
    }
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // (a vector element is copied out before the bit cast: taking the cast
      // of the element expression itself read element 0)
      const bf16 lo = g[hf][0][e], hi = g[hf][1][e];
      tile[(8 * j + e) * S + 32 * hf + p] =
          (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
  __syncthreads();
  bf16* dst = dOT + ((long)b * H + h) * DH * Tp + t0;
#pragma unroll
  for (int k = 0; k < DH * (TT / 8) / 512; ++k) {
    const int idx = tid + 512 * k, dim = idx / (TT / 8), q = idx % (TT / 8);
    const uint32_t* w = tile + dim * S + 4 * q;
    if (t0 + 8 * q < Tp) *(u32x4*)(dst + (long)dim * Tp + 8 * q) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// ------------------------------------------------------------------ cross-entropy rows
// lse[m] = log sum_b se_b * exp(mx_b - M), row_loss[m] = lse[m] - z[m, y_m].
__global__ __launch_bounds__(256) void xent_reduce_kernel(const float* __restrict__ part,
                                                          const float* __restrict__ tgt, int rows, int nblk,
                                                          float* __restrict__ lse, float* __restrict__ row_loss) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* p = part + (long)row * nblk * 2;
  float mx = -INFINITY;
  for (int b = lane; b < nblk; b += 64) mx = fmaxf(mx, p[2 * b]);
  mx = wave_max(mx);
  float s = 0.f;
  for (int b = lane; b < nblk; b += 64) {
    const float m = p[2 * b];
    if (m > -INFINITY) s += p[2 * b + 1] * expf(m - mx);
  }
  s = wave_sum(s);
  if (lane == 0) {
    const float l = mx + logf(s);
    lse[row] = l;
    row_loss[row] = l - tgt[row];
  }
}

// out[0] = (sum x) / n, summed in a fixed order by one work-group.
__global__ __launch_bounds__(1024) void mean_reduce_kernel(const float* __restrict__ x, int n, float* out) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 1024) s += (double)x[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = (float)(red[0] / (double)n);
}

// ------------------------------------------------------------------ embedding gradient
// dE[id] = sum of the dh rows whose token is id, each id's rows added in
// position order (deterministic, no atomics on values).  A stable counting
// sort by id, over chunks of EMB_CHUNK positions, gives each id's positions
// in order:
//   1. per chunk: the chunk's keys (id, position) sorted in LDS; a position's
//      rank among the chunk's earlier positions with the same id is its
//      distance from the start of its id's run there, and the run's last
//      entry records the id's count in the chunk, cnt[c][id] (zeroed
//      beforehand);
//   2. per id: cnt[c][id] becomes the id's count in the chunks before c, and
//      tot[id] its count in all of them; per block of 256 ids, the exclusive
//      prefix sum of tot (lstart) and the block's total (bsum);
//   3. one work-group scans the block totals (boff; boff[nb] = all valid
//      positions), so that an id's first sorted index is
//      start(id) = boff[id / 256] + lstart[id];
//   4. position p goes to sorted[start(id) + cnt[c][id] + rank[p]]; the
//      position that lands at start(id) appends id to the list of ids with
//      few rows or to the list of ids with many (the lists' order varies, the
//      sums do not).
// Then each id's rows are added in sorted order: by one wave over the whole
// row for ids with few rows, by eight waves per 256-column slice (partial sums
// added in wave order) for ids with many.  Ids outside [0, vocab) take no part
// (the step reports them through its token check).
constexpr int EMB_CHUNK = 1024;

__device__ __forceinline__ int emb_start(const int* lstart, const int* boff, int id) {
  return boff[id >> 8] + lstart[id];
}

__global__ __launch_bounds__(1024) void emb_rank_kernel(const int32_t* __restrict__ tok, int rows, int vocab,
                                                        int* __restrict__ rank, int* __restrict__ cnt) {
  __shared__ uint32_t sk[EMB_CHUNK];
  const int c = blockIdx.x, t = threadIdx.x, p = c * EMB_CHUNK + t;
  const int id = p < rows ? tok[p] : -1;
  // key: id above the position in the chunk (ids < 65536, 10 position bits)
  sk[t] = (id >= 0 && id < vocab) ? ((uint32_t)id << 10) | (uint32_t)t : 0xFFFFFFFFu;
  __syncthreads();
  // bitonic sort, ascending: each thread keeps the smaller or the larger
  // key of its pair (t, t ^ jj), as the pair's direction asks
  for (int k = 2; k <= EMB_CHUNK; k <<= 1)
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      const uint32_t a = sk[t], b = sk[t ^ jj];
      const bool lower = (t & jj) == 0, up = (t & k) == 0;
      const uint32_t keep = (lower == up) ? min(a, b) : max(a, b);
      __syncthreads();
      sk[t] = keep;
      __syncthreads();
    }
  const uint32_t key = sk[t];
  if (key == 0xFFFFFFFFu) return;
  const uint32_t kid = key >> 10;
  // first entry of this id's run: lower bound of (kid << 10)
  int lo = 0, hi = t;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((sk[mid] >> 10) < kid) lo = mid + 1;
    else hi = mid;
  }
  rank[c * EMB_CHUNK + (int)(key & 1023u)] = t - lo;
  if (t + 1 == EMB_CHUNK || sk[t + 1] == 0xFFFFFFFFu || (sk[t + 1] >> 10) != kid)
    cnt[(long)c * vocab + kid] = t - lo + 1;
}

__global__ __launch_bounds__(256) void emb_prefix_kernel(int* __restrict__ cnt, int chunks, int vocab,
                                                         int* __restrict__ tot, int* __restrict__ lstart,
                                                         int* __restrict__ bsum) {
  __shared__ int ws[4];
  const int id = blockIdx.x * 256 + threadIdx.x;
  int run = 0;
  if (id < vocab)
    for (int c = 0; c < chunks; ++c) {
      const int v = cnt[(long)c * vocab + id];
      cnt[(long)c * vocab + id] = run;
      run += v;
    }
  // exclusive scan of the block's totals: wave scans, then the wave offsets
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) ws[w] = incl;
  __syncthreads();
  int off = 0;
  for (int u = 0; u < w; ++u) off += ws[u];
  if (id < vocab) {
    tot[id] = run;
    lstart[id] = off + incl - run;
  }
  if (threadIdx.x == 255) bsum[blockIdx.x] = off + incl;
}

// boff[b] = sum of bsum[0 .. b), for b = 0 .. nb (nb <= 256), one work-group
__global__ __launch_bounds__(256) void emb_scan_kernel(const int* __restrict__ bsum, int nb, int* __restrict__ boff) {
  __shared__ int ws[4];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int v0 = t < nb ? bsum[t] : 0;
  int incl = v0;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) ws[w] = incl;
  __syncthreads();
  int off = 0;
  for (int u = 0; u < w; ++u) off += ws[u];
  if (t < nb) boff[t] = off + incl - v0;
  if (t == nb - 1) boff[nb] = off + incl;
}

// Ids with at most EMB_LONG rows go to the short list, the others to the
// long list: heads[0] and heads[1] count them; the short list fills heads
// from index 2 upwards and the long list from the top (index 1 + vocab)
// downwards.
constexpr int EMB_LONG = 256;

__global__ __launch_bounds__(256) void emb_scatter_kernel(const int32_t* __restrict__ tok, int rows, int vocab,
                                                          const int* __restrict__ rank, const int* __restrict__ cnt,
                                                          const int* __restrict__ lstart, const int* __restrict__ boff,
                                                          const int* __restrict__ tot, int* __restrict__ sorted,
                                                          int* __restrict__ heads) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= rows) return;
  const int id = tok[p];
  if (id < 0 || id >= vocab) return;
  const int within = cnt[(long)(p / EMB_CHUNK) * vocab + id] + rank[p];
  sorted[emb_start(lstart, boff, id) + within] = p;
  if (within == 0) {
    if (tot[id] <= EMB_LONG) heads[2 + atomicAdd(heads, 1)] = id;
    else heads[1 + vocab - atomicAdd(heads + 1, 1)] = id;
  }
}

// Short runs: one wave per id, over the whole row in blocks of 2048 columns
// (lane l holds columns 256 g + 4 l .. +3 of group g); the id's rows are
// added one after another in sorted order, two rows' loads in flight.  Loads
// past the row's end read a clamped in-row address and are not added, so no
// load sits behind a branch.
__global__ __launch_bounds__(256) void emb_short_kernel(const int* __restrict__ sorted, const int* __restrict__ heads,
                                                        const int* __restrict__ lstart, const int* __restrict__ boff,
                                                        const int* __restrict__ tot, const float* __restrict__ dh,
                                                        float* __restrict__ dE, int d, int accumulate) {
  const int nh = heads[0];
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), nw = gridDim.x * 4;
  for (int h = gw; h < nh; h += nw) {
    const int id = heads[2 + h];
    const int i0 = emb_start(lstart, boff, id), n = tot[id];
    for (int cb = 0; cb < d; cb += 2048) {
      int col[8];
      bool ok[8];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        ok[g] = cb + g * 256 + lane * 4 < d;
        col[g] = ok[g] ? cb + g * 256 + lane * 4 : d - 4;
      }
      floatx4 s[8];
#pragma unroll
      for (int g = 0; g < 8; ++g) s[g] = floatx4{0.f, 0.f, 0.f, 0.f};
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
      int r = 0;
      for (; r + 1 < n; r += 2) {
        const float* x0 = dh + (long)sorted[i0 + r] * d;
        const float* x1 = dh + (long)sorted[i0 + r + 1] * d;
        floatx4 a[8], b[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          a[g] = load4(x0 + col[g]);
          b[g] = load4(x1 + col[g]);
        }
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          s[g] += ok[g] ? a[g] : z;
          s[g] += ok[g] ? b[g] : z;
        }
      }
      if (r < n) {
        const float* x0 = dh + (long)sorted[i0 + r] * d;
        floatx4 a[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) a[g] = load4(x0 + col[g]);
#pragma unroll
        for (int g = 0; g < 8; ++g) s[g] += ok[g] ? a[g] : z;
      }
      floatx4 o[8];
      if (accumulate) {
#pragma unroll
        for (int g = 0; g < 8; ++g) o[g] = load4(dE + (long)id * d + col[g]);
      }
#pragma unroll
      for (int g = 0; g < 8; ++g)
        if (ok[g]) store4(dE + (long)id * d + col[g], accumulate ? o[g] + s[g] : s[g]);
    }
  }
}

// Long runs are cut into segments of EMB_SEG rows.  Segment work: work-group
// b takes the segments b, b + gridDim.x, ... of the flattened (long id,
// segment) sequence, for its 256-column slice; wave w adds rows w, w+8, ... of
// the segment (sixteen loads in flight per lane) and the eight wave sums are
// added in wave order into part[segment] (the long ids' segments are numbered
// in the order of the long list).  Then emb_long_sum_kernel adds each long
// id's segment sums in segment order.  Both orders are fixed, so the result
// does not depend on timing.
constexpr int EMB_SEG = 128;
constexpr int EMB_MAXLONG = 256;   // long ids hold > EMB_LONG rows each: at most rows / EMB_LONG of them

__device__ __forceinline__ void emb_long_table(const int* heads, const int* tot, int vocab, int nl, int* lid,
                                               int* lseg) {
  // lid[k]: k-th long id; lseg[k]: its first segment (lseg[nl]: all)
  for (int k = threadIdx.x; k < nl; k += blockDim.x) {
    const int id = heads[1 + vocab - k];
    lid[k] = id;
    lseg[k + 1] = (tot[id] + EMB_SEG - 1) / EMB_SEG;   // segment counts, summed below
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    lseg[0] = 0;
    for (int k = 0; k < nl; ++k) lseg[k + 1] += lseg[k];
  }
  __syncthreads();
}

__global__ __launch_bounds__(512) void emb_long_kernel(const int* __restrict__ sorted, const int* __restrict__ heads,
                                                       const int* __restrict__ lstart, const int* __restrict__ boff,
                                                       const int* __restrict__ tot, const float* __restrict__ dh,
                                                       float* __restrict__ part, int vocab, int d) {
  __shared__ floatx4 wsum[7][64];
  __shared__ int lid[EMB_MAXLONG], lseg[EMB_MAXLONG + 1];
  const int nl = min(heads[1], EMB_MAXLONG);
  emb_long_table(heads, tot, vocab, nl, lid, lseg);
  const int nseg = lseg[nl];
  const int c = blockIdx.y * 256 + (threadIdx.x & 63) * 4;
  const int w = threadIdx.x >> 6;
  for (int sg = blockIdx.x; sg < nseg; sg += gridDim.x) {
    int k = 0;
    while (lseg[k + 1] <= sg) ++k;                 // the long id owning segment sg
    const int id = lid[k];
    const int i0 = emb_start(lstart, boff, id) + (sg - lseg[k]) * EMB_SEG;
    const int m = min(EMB_SEG, tot[id] - (sg - lseg[k]) * EMB_SEG);
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
    if (c < d) {
      int j = w;
      for (; j + 120 < m; j += 128) {
        floatx4 a[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) a[u] = load4(dh + (long)sorted[i0 + j + 8 * u] * d + c);
#pragma unroll
        for (int u = 0; u < 16; ++u) s += a[u];
      }
      for (; j < m; j += 8) s += load4(dh + (long)sorted[i0 + j] * d + c);
    }
    if (w > 0) wsum[w - 1][threadIdx.x & 63] = s;
    __syncthreads();
    if (w == 0 && c < d) {
#pragma unroll
      for (int u = 0; u < 7; ++u) s += wsum[u][threadIdx.x];
      store4(part + (long)sg * d + c, s);
    }
    __syncthreads();   // wsum is rewritten by the next segment
  }
}

__global__ __launch_bounds__(256) void emb_long_sum_kernel(const int* __restrict__ heads, const int* __restrict__ tot,
                                                           const float* __restrict__ part, float* __restrict__ dE,
                                                           int vocab, int d, int accumulate) {
  __shared__ int lid[EMB_MAXLONG], lseg[EMB_MAXLONG + 1];
  const int nl = min(heads[1], EMB_MAXLONG);
  emb_long_table(heads, tot, vocab, nl, lid, lseg);
  const int c = blockIdx.y * 1024 + threadIdx.x * 4;
  if (c >= d) return;
  for (int k = blockIdx.x; k < nl; k += gridDim.x) {
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
    for (int sg = lseg[k]; sg < lseg[k + 1]; ++sg) s += load4(part + (long)sg * d + c);
    const long o = (long)lid[k] * d + c;
    if (accumulate) s += load4(dE + o);
    store4(dE + o, s);
  }
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* p, long n, float v) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// ------------------------------------------------------------------ launchers
void embed_fwd(int dtype, const int32_t* tokens, const int32_t* targets, const void* E, float* h, int rows, int d,
               int vocab, int* flag, hipStream_t st) {
  dim3 g((rows + 3) / 4);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(embed_fwd_kernel<bf16>, g, dim3(256), 0, st, tokens, targets, (const bf16*)E, h, rows, d,
                       vocab, flag);
  else
    hipLaunchKernelGGL(embed_fwd_kernel<float>, g, dim3(256), 0, st, tokens, targets, (const float*)E, h, rows, d,
                       vocab, flag);
}

template <typename T>
static void rmsnorm_fwd_reg(const float* x, T* y, float* rstd, int rows, int d, float eps, hipStream_t st,
                            unsigned* amax) {
  dim3 g((rows + 3) / 4);
  switch (norm_chunks(d)) {
    case 1: hipLaunchKernelGGL((rmsnorm_fwd_reg_kernel<T, 1>), g, dim3(256), 0, st, x, y, rstd, rows, d, eps, amax); break;
    case 2: hipLaunchKernelGGL((rmsnorm_fwd_reg_kernel<T, 2>), g, dim3(256), 0, st, x, y, rstd, rows, d, eps, amax); break;
    case 3: hipLaunchKernelGGL((rmsnorm_fwd_reg_kernel<T, 3>), g, dim3(256), 0, st, x, y, rstd, rows, d, eps, amax); break;
    default: hipLaunchKernelGGL((rmsnorm_fwd_reg_kernel<T, 4>), g, dim3(256), 0, st, x, y, rstd, rows, d, eps, amax);
  }
}

template <typename T>
static void rmsnorm_bwd_reg(const void* dy, int dy_act, const T* y, const float* rstd, float* dx, T* dxa, int rows,
                            int d, int accumulate, hipStream_t st, unsigned* amax) {
  dim3 g((rows + 3) / 4);
#define RBR(N)                                                                                                 \
  case N:                                                                                                      \
    hipLaunchKernelGGL((rmsnorm_bwd_reg_kernel<T, N>), g, dim3(256), 0, st, dy, dy_act, y, rstd, dx, dxa, rows, d, \
                       accumulate, amax);                                                                      \
    break;
  switch (norm_chunks(d)) { RBR(1) RBR(2) RBR(3) default: RBR(4) }
#undef RBR
}

void rmsnorm_fwd(int dtype, const float* x, void* y, float* rstd, int rows, int d, float eps, hipStream_t st,
                 unsigned* amax) {
  dim3 g((rows + 3) / 4);
  if (norm_chunks(d)) {
    if (dtype == DT_BF16) rmsnorm_fwd_reg(x, (bf16*)y, rstd, rows, d, eps, st, amax);
    else rmsnorm_fwd_reg(x, (float*)y, rstd, rows, d, eps, st, amax);
    return;
  }
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<bf16>, g, dim3(256), 0, st, x, (bf16*)y, rstd, rows, d, eps, amax);
  else
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<float>, g, dim3(256), 0, st, x, (float*)y, rstd, rows, d, eps, amax);
}

int rmsnorm_bwd(int dtype, const void* dy, int dy_act, const void* y, const float* rstd, float* dx, void* dxa,
                int rows, int d, int accumulate, hipStream_t st, unsigned* amax) {
  dim3 g((rows + 3) / 4);
  if (norm_chunks(d)) {
    if (dtype == DT_BF16) rmsnorm_bwd_reg(dy, dy_act, (const bf16*)y, rstd, dx, (bf16*)dxa, rows, d, accumulate, st, amax);
    else rmsnorm_bwd_reg(dy, dy_act, (const float*)y, rstd, dx, (float*)dxa, rows, d, accumulate, st, amax);
    return 0;
  }
  if (dy_act && dtype != DT_F32) return -1;   // the row-loop form reads fp32 dy only
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<bf16>, g, dim3(256), 0, st, (const float*)dy, (const bf16*)y, rstd, dx,
                       (bf16*)dxa, rows, d, accumulate, amax);
  else
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<float>, g, dim3(256), 0, st, (const float*)dy, (const float*)y, rstd, dx,
                       (float*)dxa, rows, d, accumulate, amax);
  return 0;
}

template <typename T, int DH>
static void rope_fwd_t(void* qkv, float* rq, void* qT, void* kT, void* vT, const float* c, const float* s, int B,
                       int T_, int Tp, int H, int Hkv, float eps, hipStream_t st) {
  dim3 g((T_ + 63) / 64, H, B);
  if constexpr (sizeof(T) == 2 && DH == 128) {
    hipLaunchKernelGGL(rope_qknorm_fwd128_kernel, dim3((T_ + 127) / 128, H, B), dim3(512), 0, st, (bf16*)qkv, rq,
                       (bf16*)qT, (bf16*)kT, (bf16*)vT, c, s, T_, Tp, H, Hkv, eps);
    return;
  }
  hipLaunchKernelGGL((rope_qknorm_fwd_kernel<T, DH>), g, dim3(256), 0, st, (T*)qkv, rq, (T*)qT, (T*)kT, (T*)vT, c,
                     s, T_, Tp, H, Hkv, eps);
}

void rope_qknorm_fwd(int dtype, void* qkv, float* rq, void* qT, void* kT, void* vT, const float* c,
                     const float* s, int B, int T_, int Tp, int H, int Hkv, int Dh, float eps, hipStream_t st) {
#define RF(TT, D) \
  if (Dh == D) return rope_fwd_t<TT, D>(qkv, rq, qT, kT, vT, c, s, B, T_, Tp, H, Hkv, eps, st);
  if (dtype == DT_BF16) { RF(bf16, 32) RF(bf16, 64) RF(bf16, 128) }
  else { RF(float, 32) RF(float, 64) RF(float, 128) }
#undef RF
}

template <typename T, int DH>
static void rope_bwd_t(void* dqkv, const void* qkv, const float* rq, const float* c, const float* s, int B, int T_,
                       int H, int Hkv, hipStream_t st, unsigned* amax) {
  const int rows = B * T_;
  if constexpr (sizeof(T) == 2 && DH == 128) {
    const long nvec = (long)rows * (H + Hkv);
    hipLaunchKernelGGL(rope_qknorm_bwd128_kernel, dim3((unsigned)((nvec + 31) / 32)), dim3(256), 0, st, (bf16*)dqkv,
                       (const bf16*)qkv, rq, c, s, nvec, T_, H, Hkv, amax);
    return;
  }
  hipLaunchKernelGGL((rope_qknorm_bwd_kernel<T, DH>), dim3((rows + 3) / 4), dim3(256), 0, st, (T*)dqkv,
                     (const T*)qkv, rq, c, s, rows, T_, H, Hkv, amax);
}

void rope_qknorm_bwd(int dtype, void* dqkv, const void* qkv, const float* rq, const float* c, const float* s,
                     int B, int T_, int H, int Hkv, int Dh, hipStream_t st, unsigned* amax) {
#define RB(TT, D) \
  if (Dh == D) return rope_bwd_t<TT, D>(dqkv, qkv, rq, c, s, B, T_, H, Hkv, st, amax);
  if (dtype == DT_BF16) { RB(bf16, 32) RB(bf16, 64) RB(bf16, 128) }
  else { RB(float, 32) RB(float, 64) RB(float, 128) }
#undef RB
}

template <typename T, int DH>
static void pre_t(const void* dO, const void* O, float* Dv, void* dOT, int B, int T_, int Tp, int H, hipStream_t st) {
  dim3 g((T_ + 63) / 64, H, B);
  if constexpr (sizeof(T) == 2 && DH == 128) {
    hipLaunchKernelGGL(attn_bwd_pre128_kernel, dim3((T_ + 127) / 128, H, B), dim3(512), 0, st, (const bf16*)dO, (const bf16*)O, Dv, (bf16*)dOT,
                       T_, Tp, H);
    return;
  }
  hipLaunchKernelGGL((attn_bwd_pre_kernel<T, DH>), g, dim3(256), 0, st, (const T*)dO, (const T*)O, Dv, (T*)dOT, T_,
                     Tp, H);
}

void attn_bwd_pre(int dtype, const void* dO, const void* O, float* Dv, void* dOT, int B, int T_, int Tp, int H,
                  int Dh, hipStream_t st) {
#define PB(TT, D) \
  if (Dh == D) return pre_t<TT, D>(dO, O, Dv, dOT, B, T_, Tp, H, st);
  if (dtype == DT_BF16) { PB(bf16, 32) PB(bf16, 64) PB(bf16, 128) }
  else { PB(float, 32) PB(float, 64) PB(float, 128) }
#undef PB
}

void xent_reduce(const float* part, const float* tgt, int rows, int nblk, float* lse, float* row_loss,
                 hipStream_t st) {
  hipLaunchKernelGGL(xent_reduce_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, part, tgt, rows, nblk, lse,
                     row_loss);
}

void mean_reduce(const float* x, int n, float* out, hipStream_t st) {
  hipLaunchKernelGGL(mean_reduce_kernel, dim3(1), dim3(1024), 0, st, x, n, out);
}

void embed_bwd(const int32_t* tokens, const float* dh, float* dE, int rows, int d, int vocab, int* sorted, int* rank,
               int* cnt, int* tot, int* lstart, int* bsum, int* heads, float* part, int accumulate, hipStream_t st) {
  const int chunks = (rows + EMB_CHUNK - 1) / EMB_CHUNK;
  const int nb = (vocab + 255) / 256;   // <= 256 (vocab <= 65536)
  int* boff = bsum + nb;
  if (!accumulate) fill_f32(dE, (long)vocab * d, 0.f, st);
  fill_f32((float*)cnt, (long)chunks * vocab, 0.f, st);   // all-zero bits: integer zeros
  fill_f32((float*)heads, 2, 0.f, st);
  hipLaunchKernelGGL(emb_rank_kernel, dim3(chunks), dim3(EMB_CHUNK), 0, st, tokens, rows, vocab, rank, cnt);
  hipLaunchKernelGGL(emb_prefix_kernel, dim3(nb), dim3(256), 0, st, cnt, chunks, vocab, tot, lstart, bsum);
  hipLaunchKernelGGL(emb_scan_kernel, dim3(1), dim3(256), 0, st, bsum, nb, boff);
  hipLaunchKernelGGL(emb_scatter_kernel, dim3((rows + 255) / 256), dim3(256), 0, st, tokens, rows, vocab, rank, cnt,
                     lstart, boff, tot, sorted, heads);
  hipLaunchKernelGGL(emb_short_kernel, dim3(1024), dim3(256), 0, st, sorted, heads, lstart, boff, tot, dh, dE, d,
                     accumulate);
  hipLaunchKernelGGL(emb_long_kernel, dim3(256, (d + 255) / 256), dim3(512), 0, st, sorted, heads, lstart, boff, tot,
                     dh, part, vocab, d);
  hipLaunchKernelGGL(emb_long_sum_kernel, dim3(64, (d + 1023) / 1024), dim3(256), 0, st, heads, tot, part, dE, vocab,
                     d, accumulate);
}

void fill_f32(float* p, long n, float v, hipStream_t st) {
  hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, v);
}

}  // namespace gk
