// Kernels of incremental decoding with a KV cache: one new token per
// sequence per step.  At this size every product is a matrix-vector-like
// pass over the weights and attention is a pass over the cached keys and
// values, so both are HBM-bound; they are written for bandwidth (many
// loads in flight, every byte read once) rather than for MFMA throughput.
//
// KV cache layout (bf16): layer l, K then V, each [B][H][Tmax][Dh]; the key
// and value rows of one head are contiguous in position.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gk {

// ------------------------------------------------------------------ skinny GEMM
// out[b][n] = sum_k x[b][k] W[n][k] for b < B <= 32: work-group (i, y) takes
// weight rows 32i..32i+31 and the y-th of gridDim.y equal runs of K, its
// waves splitting the run in interleaved 16-wide steps (neighbouring waves
// read neighbouring 32-byte pieces of the same cache lines; measured faster
// than a contiguous run per wave).  The 32x32x16 MFMA takes 32 weight rows
// as its A operand and the (zero-padded) batch as its B operand, so a wave
// streams 1 KB of weights per MFMA, with eight steps' loads issued before
// their MFMAs.  The wave partials are summed in a fixed order through LDS.
// Products with few weight rows split K over gridDim.y work-groups
// (EPI_PARTIAL: part[y][b][n]); the consumer adds the partials in order.
constexpr int SK_UNROLL = 8;

template <int EPI, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void skinny_gemm_kernel(const bf16* __restrict__ x, long ldx, int B, int K,
                                                                  const bf16* __restrict__ W, int N,
                                                                  void* __restrict__ C, int ldc,
                                                                  void* __restrict__ C2) {
  __shared__ floatx16 red[WAVES][64];
  const int n0 = blockIdx.x * 32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 5, l32 = lane & 31;
  const int nrow = min(n0 + l32, N - 1);   // rows past N load a valid row and are never stored
  const bool bok = l32 < B;
  const u32x4 bmask = bok ? u32x4{~0u, ~0u, ~0u, ~0u} : u32x4{0u, 0u, 0u, 0u};
  const bf16* wr = W + (long)nrow * K + g * 8;
  const bf16* xr = x + (long)(bok ? l32 : 0) * ldx + g * 8;   // batch lanes past B read row 0, masked to zero
  const int nsteps = K / 16;
  const int per = (nsteps + gridDim.y - 1) / gridDim.y;
  const int s_end = min(nsteps, (int)(blockIdx.y + 1) * per);
  floatx16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  auto xload = [&](int st) {
    const u32x4 v = *(const u32x4*)(xr + (long)st * 16) & bmask;
    return __builtin_bit_cast(bf16x8, v);
  };
  int s = blockIdx.y * per + wave;
  for (; s + WAVES * (SK_UNROLL - 1) < s_end; s += WAVES * SK_UNROLL) {
    bf16x8 a[SK_UNROLL], b[SK_UNROLL];
#pragma unroll
    for (int u = 0; u < SK_UNROLL; ++u) {
      a[u] = *(const bf16x8*)(wr + (long)(s + WAVES * u) * 16);
      b[u] = xload(s + WAVES * u);
    }
#pragma unroll
    for (int u = 0; u < SK_UNROLL; ++u) acc = Mfma<bf16>::mma(a[u], b[u], acc);
  }
  for (; s < s_end; s += WAVES) {
    const bf16x8 a = *(const bf16x8*)(wr + (long)s * 16);
    acc = Mfma<bf16>::mma(a, xload(s), acc);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  floatx16 t = red[0][lane];
#pragma unroll
  for (int w = 1; w < WAVES; ++w) t += red[w][lane];
  if (!bok) return;
  // lane (g, l32) holds D[8*(r/4) + 4*g + r%4][l32]: weight row, batch column
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int n = n0 + 8 * (r / 4) + 4 * g + (r % 4);
    if (n >= N) continue;
    const long o = (long)l32 * ldc + n;
    const float v = t[r];
    if constexpr (EPI == EPI_STORE) {
      ((bf16*)C)[o] = (bf16)v;
    } else if constexpr (EPI == EPI_STORE_F32) {
      ((float*)C)[o] = v;
    } else if constexpr (EPI == EPI_PARTIAL) {
      ((float*)C)[(long)blockIdx.y * B * ldc + o] = v;
    } else if constexpr (EPI == EPI_RELU2) {
      ((bf16*)C)[o] = (bf16)v;
      const float y = fmaxf(v, 0.f);
      ((bf16*)C2)[o] = (bf16)(y * y);
    }
  }
}

int skinny_gemm(int epi, const void* x, long ldx, int B, int K, const void* W, int N, void* C, int ldc, void* C2,
                int ksplit, hipStream_t st) {
  if (B < 1 || B > 32 || K % 16 || ksplit < 1 || (ksplit > 1) != (epi == EPI_PARTIAL)) return -1;
  const bf16* xb = (const bf16*)x;
  const bf16* wb = (const bf16*)W;
  const dim3 grid((N + 31) / 32, ksplit);
#define SK(E, WV) hipLaunchKernelGGL((skinny_gemm_kernel<E, WV>), grid, dim3(64 * WV), 0, st, xb, ldx, B, K, wb, N, C, ldc, C2)
  switch (epi) {
    case EPI_STORE: SK(EPI_STORE, 16); break;
    case EPI_STORE_F32: SK(EPI_STORE_F32, 16); break;
    case EPI_RELU2: SK(EPI_RELU2, 16); break;
    case EPI_PARTIAL: SK(EPI_PARTIAL, 4); break;
    default: return -1;
  }
#undef SK
  return 0;
}

// ------------------------------------------------------------------ residual add + RMSNorm
// h[b] += sum_{s < nsplit} part[s][b] (in split order), then
// y[b] = bf16(h[b] / sqrt(mean(h[b]^2) + eps)).  One work-group of 512
// threads per row: a row of up to 2048 values takes one pass, with the
// partials' loads of a thread issued together.
constexpr int AN_THREADS = 512, AN_MAXSPLIT = 8;

__global__ __launch_bounds__(AN_THREADS) void decode_add_rmsnorm_kernel(float* __restrict__ h,
                                                                        const float* __restrict__ part, int nsplit,
                                                                        int B, int d, bf16* __restrict__ y,
                                                                        float eps) {
  __shared__ float red[AN_THREADS / 64];
  const int b = blockIdx.x;
  float* hr = h + (long)b * d;
  float ss = 0.f;
  for (int c = threadIdx.x * 4; c < d; c += AN_THREADS * 4) {
    floatx4 p[AN_MAXSPLIT];
#pragma unroll
    for (int sp = 0; sp < AN_MAXSPLIT; ++sp)
      if (sp < nsplit) p[sp] = load4(part + ((long)sp * B + b) * d + c);
    floatx4 v = load4(hr + c);
#pragma unroll
    for (int sp = 0; sp < AN_MAXSPLIT; ++sp)
      if (sp < nsplit) v += p[sp];
    if (nsplit) store4(hr + c, v);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < AN_THREADS / 64; ++w) tot += red[w];
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
  for (int c = threadIdx.x * 4; c < d; c += AN_THREADS * 4) store4(y + (long)b * d + c, load4(hr + c) * r);
}

void decode_add_rmsnorm(float* h, const float* part, int nsplit, int B, int d, void* y, float eps, hipStream_t st) {
  hipLaunchKernelGGL(decode_add_rmsnorm_kernel, dim3(B), dim3(AN_THREADS), 0, st, h, part, nsplit, B, d, (bf16*)y,
                     eps);
}

// ------------------------------------------------------------------ prefill: cache fill
// kc/vc[b][g][t][:] = k^ / v of key/value head g of row (b, t) of qkv
// [B*T][d + 2*Hkv*Dh], t < T.
__global__ __launch_bounds__(256) void kv_fill_kernel(const bf16* __restrict__ qkv, bf16* __restrict__ kc,
                                                      bf16* __restrict__ vc, int T, int H, int Hkv, int Dh,
                                                      int Tmax) {
  const int t = blockIdx.x, b = blockIdx.y;
  const int d = H * Dh, dkv = Hkv * Dh;
  const bf16* row = qkv + ((long)b * T + t) * (d + 2 * dkv);
  for (int i = threadIdx.x * 8; i < 2 * dkv; i += 256 * 8) {
    const int part = i / dkv, c = i % dkv, g = c / Dh, e = c % Dh;
    const bf16x8 v = *(const bf16x8*)(row + d + i);
    bf16* dst = (part == 0 ? kc : vc) + (((long)b * Hkv + g) * Tmax + t) * Dh + e;
    *(bf16x8*)dst = v;
  }
}

void kv_fill(const void* qkv, void* kc, void* vc, int B, int T, int H, int Hkv, int Dh, int Tmax, hipStream_t st) {
  hipLaunchKernelGGL(kv_fill_kernel, dim3(T, B), dim3(256), 0, st, (const bf16*)qkv, (bf16*)kc, (bf16*)vc, T, H, Hkv,
                     Dh, Tmax);
}

// ------------------------------------------------------------------ attention over the cache
// Split pass: work-group (split, h, b) takes keys [lo + split*128, +128)
// of the visible range [lo, pos], lo = max(0, pos - window + 1); 16 (Dh 128)
// or 8 (Dh 64) lanes share one key row, so a wave covers 4 or 8 keys per
// load.  The new token's rotary embedding and QK norm are done here: every
// work-group forms q^ from the raw q of qkv [B][3d]; the one whose split
// holds pos also forms k^ of the new token, writes k^ and v into the cache
// at pos for later steps, and uses them from registers for key pos.
// QK-normalised queries and keys bound every score by sqrt(Dh), so the
// softmax uses a fixed exponent offset M = 1.01 sqrt(Dh) log2(e) and the
// splits only add their (sum p, sum p v) partials: part[b][h][split] =
// {o[Dh], l}.  The grid covers the most splits the window can need, so it
// does not depend on pos (read from device memory); splits past pos write
// zero partials.
// keys per split (a wave takes a quarter: one load of each of its rows in
// flight at once)
constexpr int ATT_SPLIT = 128;

// Rotary embedding by +pos*theta_i over half-split pairs, then unit RMS over
// the head, for the 8 values this lane holds (lane li of an LPK-lane group
// holds elements 8li..8li+7; its pair partner is lane li ^ LPK/2); the
// result is rounded to bf16, as a stored q^ / k^ is.
template <int LPK>
__device__ __forceinline__ void rope_norm8(const bf16x8 xv, const float* cs, const float* sn, bool first, float eps,
                                           float* out) {
  constexpr int DH = LPK * 8;
  float y[8];
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = (float)xv[e];
    const float pr = __shfl_xor(x, LPK / 2, 64);
    y[e] = first ? x * cs[e] - pr * sn[e] : pr * sn[e] + x * cs[e];
    ss += y[e] * y[e];
  }
#pragma unroll
  for (int o = LPK / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  const float r = 1.0f / sqrtf(ss / (float)DH + eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (float)(bf16)(y[e] * r);
}

template <int DH>
__global__ __launch_bounds__(256) void attn_decode_split_kernel(const bf16* __restrict__ qkv, bf16* __restrict__ kc,
                                                                bf16* __restrict__ vc, float* __restrict__ part,
                                                                const float* __restrict__ cosb,
                                                                const float* __restrict__ sinb, int H, int Hkv,
                                                                int Tmax, const int* __restrict__ posp, int window,
                                                                float scale_log2, float eps) {
  constexpr int LPK = DH / 8, KPI = 64 / LPK, HALF = DH / 2;
  __shared__ float red[4][DH + 1];
  const int sp = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nsplit = gridDim.x;
  const int pos = *posp;
  const int lo = max(0, pos - window + 1);
  if (lo + sp * ATT_SPLIT > pos) {   // nothing visible in this split
    float* out = part + (((long)b * H + h) * nsplit + sp) * (DH + 1);
    for (int i = threadIdx.x; i <= DH; i += 256) out[i] = 0.f;
    return;
  }
  const bool has_pos = pos < lo + (sp + 1) * ATT_SPLIT;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kg = lane / LPK, li = lane % LPK;
  const bool first = li < LPK / 2;
  const int d = H * DH, dkv = Hkv * DH;
  const int G = H / Hkv, hk = h / G;   // key/value head of query head h
  const bf16* row = qkv + (long)b * (d + 2 * dkv) + h * DH + li * 8;
  const bf16* kvrow = qkv + (long)b * (d + 2 * dkv) + d + hk * DH + li * 8;
  float cs[8], sn[8];
  {
    const float* c = cosb + (long)pos * HALF + (li % (LPK / 2)) * 8;
    const float* s = sinb + (long)pos * HALF + (li % (LPK / 2)) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      cs[e] = c[e];
      sn[e] = s[e];
    }
  }
  float q[8];
  rope_norm8<LPK>(*(const bf16x8*)row, cs, sn, first, eps, q);
  const long base = ((long)b * Hkv + hk) * Tmax * DH;
  bf16x8 knew = bf16x8{}, vnew = bf16x8{};
  if (has_pos) {   // uniform over the work-group
    float k[8];
    rope_norm8<LPK>(*(const bf16x8*)kvrow, cs, sn, first, eps, k);
#pragma unroll
    for (int e = 0; e < 8; ++e) knew[e] = (bf16)k[e];
    vnew = *(const bf16x8*)(kvrow + dkv);
    // the first query head of the group writes the shared key and value
    if (wave == 0 && kg == 0 && h % G == 0) {
      *(bf16x8*)(kc + base + (long)pos * DH + li * 8) = knew;
      *(bf16x8*)(vc + base + (long)pos * DH + li * 8) = vnew;
    }
  }
  const float M = 1.01f * scale_log2 * (float)DH;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  const int k0 = lo + sp * ATT_SPLIT + wave * (ATT_SPLIT / 4);
#pragma unroll 8
  for (int it = 0; it < ATT_SPLIT / 4 / KPI; ++it) {
    const int j = k0 + it * KPI + kg;
    const bool ok = j <= pos;
    const int jj = ok ? j : pos;   // a valid row; its weight is zero
    bf16x8 kv = *(const bf16x8*)(kc + base + (long)jj * DH + li * 8);
    bf16x8 vv = *(const bf16x8*)(vc + base + (long)jj * DH + li * 8);
    if (jj == pos) {   // the new token: its key and value come from registers
      kv = knew;
      vv = vnew;
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += q[e] * (float)kv[e];
#pragma unroll
    for (int o = LPK / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    const float p = ok ? exp2f(s * scale_log2 - M) : 0.f;
    l += p;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += p * (float)vv[e];
  }
  // add the key groups of the wave (lanes li, li + LPK, ...)
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1) {
    l += __shfl_xor(l, o, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
  }
  if (kg == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wave][li * 8 + e] = acc[e];
    if (li == 0) red[wave][DH] = l;
  }
  __syncthreads();
  float* out = part + (((long)b * H + h) * nsplit + sp) * (DH + 1);
  for (int i = threadIdx.x; i <= DH; i += 256) out[i] = (red[0][i] + red[1][i]) + (red[2][i] + red[3][i]);
}

// o[b][h*Dh + i] = sum_split o_i / sum_split l, added in split order.
template <int DH>
__global__ __launch_bounds__(DH) void attn_decode_combine_kernel(const float* __restrict__ part, bf16* __restrict__ o,
                                                                 int H, int nsplit) {
  const int h = blockIdx.x, b = blockIdx.y, i = threadIdx.x;
  const float* p = part + ((long)b * H + h) * nsplit * (DH + 1);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    num += p[s * (DH + 1) + i];
    den += p[s * (DH + 1) + DH];
  }
  o[(long)b * H * DH + h * DH + i] = (bf16)(num / den);
}

int attn_decode(const void* qkv, void* kc, void* vc, const float* cosb, const float* sinb, float* part, void* o,
                int B, int H, int Hkv, int Dh, int Tmax, const int* posp, int window, float eps, hipStream_t st) {
  const int nsplit = (std::min(window, Tmax) + ATT_SPLIT - 1) / ATT_SPLIT;
  const float sl2 = (float)(1.4426950408889634 / sqrt((double)Dh));
  const dim3 g1(nsplit, H, B), g2(H, B);
  if (Dh == 128) {
    hipLaunchKernelGGL(attn_decode_split_kernel<128>, g1, dim3(256), 0, st, (const bf16*)qkv, (bf16*)kc, (bf16*)vc,
                       part, cosb, sinb, H, Hkv, Tmax, posp, window, sl2, eps);
    hipLaunchKernelGGL(attn_decode_combine_kernel<128>, g2, dim3(128), 0, st, part, (bf16*)o, H, nsplit);
  } else if (Dh == 64) {
    hipLaunchKernelGGL(attn_decode_split_kernel<64>, g1, dim3(256), 0, st, (const bf16*)qkv, (bf16*)kc, (bf16*)vc,
                       part, cosb, sinb, H, Hkv, Tmax, posp, window, sl2, eps);
    hipLaunchKernelGGL(attn_decode_combine_kernel<64>, g2, dim3(64), 0, st, part, (bf16*)o, H, nsplit);
  } else {
    return -1;
  }
  return 0;
}

// ------------------------------------------------------------------ step inputs
// Copies the step's token ids and position into the decoder's own device
// buffers (the kernels of a step, and a captured graph of them, read them
// there) and clears the token-range flag.
__global__ __launch_bounds__(64) void decode_stage_kernel(const int32_t* __restrict__ tokens, int B, int pos,
                                                          int32_t* __restrict__ tok, int* __restrict__ posp,
                                                          int* __restrict__ flag) {
  for (int i = threadIdx.x; i < B; i += 64) tok[i] = tokens[i];
  if (threadIdx.x == 0) {
    *posp = pos;
    *flag = 0;
  }
}

void decode_stage(const int32_t* tokens, int B, int pos, int32_t* tok, int* posp, int* flag, hipStream_t st) {
  hipLaunchKernelGGL(decode_stage_kernel, dim3(1), dim3(64), 0, st, tokens, B, pos, tok, posp, flag);
}

}  // namespace gk
