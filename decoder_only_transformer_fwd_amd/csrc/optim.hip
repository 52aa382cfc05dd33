// Bandwidth-bound kernels of the optimizer step: the global gradient norm,
// AdamW on the embedding and lm_head, and Muon's momentum, normalisation and
// weight update (its Newton-Schulz products run on the GEMM kernel).
//
// Every pass walks a list of tensors in chunks of OPT_CHUNK elements, one
// work-group per chunk; a chunk finds its tensor by binary search over the
// list's first-chunk indices.  Reductions are two-level and in a fixed
// order (per-chunk partial sums, then one ordered sum), so every pass is
// deterministic.
#include "common.h"
#include "kernels.h"

namespace gk {

namespace {

// the list entry that owns chunk b: the last i with seg[i].blk0 <= b
__device__ __forceinline__ int find_seg(const OptSeg* __restrict__ seg, int nseg, int b) {
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seg[mid].blk0 <= b) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// sum over the 256 threads of a work-group, in a fixed order
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float s = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return s;
}

constexpr int VPT = OPT_CHUNK / (256 * 4);   // float4 groups per thread

}  // namespace

// part[b] = sum of squares of chunk b of the list (scaled by nothing).
__global__ __launch_bounds__(256) void opt_sumsq_kernel(const float* __restrict__ x, const OptSeg* __restrict__ seg,
                                                        int nseg, float* __restrict__ part) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const OptSeg s = seg[find_seg(seg, nseg, b)];
  const long c0 = (long)(b - s.blk0) * OPT_CHUNK;
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const long i = c0 + (long)(j * 256 + threadIdx.x) * 4;
    if (i < s.n) {
      const floatx4 v = load4(x + s.off + i);
      acc += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    }
  }
  acc = block_sum256(acc, red);
  if (threadIdx.x == 0) part[b] = acc;
}

// hdr[0] = sqrt(sum part), hdr[1] = clip coefficient min(1, clip / (norm +
// 1e-6)) (1 when clip <= 0).  One work-group; the partials are added in a
// fixed order in double.
__global__ __launch_bounds__(1024) void opt_norm_kernel(const float* __restrict__ part, int nb, float clip,
                                                        float* __restrict__ hdr) {
  __shared__ double red[1024];
  // four independent running sums per thread keep four loads in flight
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  int i = threadIdx.x;
  for (; i + 3 * 1024 < nb; i += 4 * 1024) {
    a0 += (double)part[i];
    a1 += (double)part[i + 1024];
    a2 += (double)part[i + 2 * 1024];
    a3 += (double)part[i + 3 * 1024];
  }
  for (; i < nb; i += 1024) a0 += (double)part[i];
  red[threadIdx.x] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float norm = (float)sqrt(red[0]);
    hdr[0] = norm;
    hdr[1] = clip > 0.f ? fminf(1.f, clip / (norm + 1e-6f)) : 1.f;
  }
}

// AdamW over the list (E and U): m, v at state + soff, state + soff + n.
// w16: the bf16 weight copy to refresh (null when the weights are the fp32
// master itself).
__global__ __launch_bounds__(256) void opt_adamw_kernel(float* __restrict__ master, float* __restrict__ state,
                                                        const float* __restrict__ g, bf16* __restrict__ w16,
                                                        const OptSeg* __restrict__ seg, int nseg,
                                                        const float* __restrict__ hdr, AdamArgs a) {
  const int b = blockIdx.x;
  const OptSeg s = seg[find_seg(seg, nseg, b)];
  const long c0 = (long)(b - s.blk0) * OPT_CHUNK;
  const float cf = hdr[1];
  const float lr = s.which ? a.lr1 : a.lr0;
  const float decay = 1.f - lr * a.wd;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const long i = c0 + (long)(j * 256 + threadIdx.x) * 4;
    if (i < s.n) {
      const floatx4 gv = load4(g + s.off + i) * cf;
      floatx4 m = load4(state + s.soff + i);
      floatx4 v = load4(state + s.soff + s.n + i);
      floatx4 p = load4(master + s.off + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m[e] = a.b1 * m[e] + (1.f - a.b1) * gv[e];
        v[e] = a.b2 * v[e] + (1.f - a.b2) * gv[e] * gv[e];
        const float mh = m[e] * a.ibc1;
        const float den = sqrtf(v[e] * a.ibc2) + a.eps;
        p[e] = p[e] * decay - lr * (mh / den);
      }
      store4(state + s.soff + i, m);
      store4(state + s.soff + s.n + i, v);
      store4(master + s.off + i, p);
      if (w16) store4(w16 + s.off + i, p);
    }
  }
}

// Muon momentum: buf <- mu buf + (1 - mu) g (g clipped), u = Nesterov ?
// (1 - mu) g + mu buf : buf; part[b] = sum of u^2 over the chunk.
__global__ __launch_bounds__(256) void opt_muon_momentum_kernel(const float* __restrict__ g,
                                                                float* __restrict__ state,
                                                                const OptSeg* __restrict__ seg, int nseg,
                                                                const float* __restrict__ hdr, float mu,
                                                                int nesterov, float* __restrict__ part) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const OptSeg s = seg[find_seg(seg, nseg, b)];
  const long c0 = (long)(b - s.blk0) * OPT_CHUNK;
  const float cf = hdr[1];
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const long i = c0 + (long)(j * 256 + threadIdx.x) * 4;
    if (i < s.n) {
      const floatx4 gv = load4(g + s.off + i) * cf;
      floatx4 buf = load4(state + s.soff + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        buf[e] = mu * buf[e] + (1.f - mu) * gv[e];
        const float u = nesterov ? (1.f - mu) * gv[e] + mu * buf[e] : buf[e];
        acc += u * u;
      }
      store4(state + s.soff + i, buf);
    }
  }
  acc = block_sum256(acc, red);
  if (threadIdx.x == 0) part[b] = acc;
}

// X[xoff + i] = bf16(u / (||u||_F + 1e-7)), u recomputed from the gradient
// and the updated momentum exactly as the momentum pass formed it; the norm
// is the ordered sum of the matrix's chunk partials (every chunk of a matrix
// adds them in the same order, so all see the same value).
__global__ __launch_bounds__(256) void opt_muon_normalise_kernel(const float* __restrict__ g,
                                                                 const float* __restrict__ state,
                                                                 const OptSeg* __restrict__ seg, int nseg,
                                                                 const float* __restrict__ hdr, float mu,
                                                                 int nesterov, const float* __restrict__ part,
                                                                 bf16* __restrict__ X) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const int k = find_seg(seg, nseg, b);
  const OptSeg s = seg[k];
  const int nb = seg[k + 1].blk0 - s.blk0;   // the list ends with a sentinel entry
  float ss = 0.f;
  for (int i = threadIdx.x; i < nb; i += 256) ss += part[s.blk0 + i];
  ss = block_sum256(ss, red);
  const float inv = 1.f / (sqrtf(ss) + 1e-7f);
  const long c0 = (long)(b - s.blk0) * OPT_CHUNK;
  const float cf = hdr[1];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const long i = c0 + (long)(j * 256 + threadIdx.x) * 4;
    if (i < s.n) {
      const floatx4 gv = load4(g + s.off + i) * cf;
      const floatx4 buf = load4(state + s.soff + i);
      floatx4 u;
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = (nesterov ? (1.f - mu) * gv[e] + mu * buf[e] : buf[e]) * inv;
      store4(X + s.xoff + i, u);
    }
  }
}

// Muon update: p <- p (1 - lr wd) - lr * scale * O, scale = sqrt(max(1, rows/cols)).
__global__ __launch_bounds__(256) void opt_muon_update_kernel(float* __restrict__ master, const bf16* __restrict__ X,
                                                              bf16* __restrict__ w16, const OptSeg* __restrict__ seg,
                                                              int nseg, float lr, float scale, float wd) {
  const int b = blockIdx.x;
  const OptSeg s = seg[find_seg(seg, nseg, b)];
  const long c0 = (long)(b - s.blk0) * OPT_CHUNK;
  const float decay = 1.f - lr * wd;
  const float step = lr * scale;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const long i = c0 + (long)(j * 256 + threadIdx.x) * 4;
    if (i < s.n) {
      const floatx4 o = load4(X + s.xoff + i);
      floatx4 p = load4(master + s.off + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = p[e] * decay - step * o[e];
      store4(master + s.off + i, p);
      if (w16) store4(w16 + s.off + i, p);
    }
  }
}

// fp32 master weights from the bf16 parameters, over the list.
__global__ __launch_bounds__(256) void opt_widen_kernel(const bf16* __restrict__ w16, float* __restrict__ master,
                                                        const OptSeg* __restrict__ seg, int nseg) {
  const int b = blockIdx.x;
  const OptSeg s = seg[find_seg(seg, nseg, b)];
  const long c0 = (long)(b - s.blk0) * OPT_CHUNK;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const long i = c0 + (long)(j * 256 + threadIdx.x) * 4;
    if (i < s.n) store4(master + s.off + i, load4(w16 + s.off + i));
  }
}

// ------------------------------------------------------------------ launchers
void opt_sumsq(const float* x, const OptSeg* seg, int nseg, int nblk, float* part, hipStream_t st) {
  hipLaunchKernelGGL(opt_sumsq_kernel, dim3(nblk), dim3(256), 0, st, x, seg, nseg, part);
}
void opt_norm(const float* part, int nblk, float clip, float* hdr, hipStream_t st) {
  hipLaunchKernelGGL(opt_norm_kernel, dim3(1), dim3(1024), 0, st, part, nblk, clip, hdr);
}
void opt_adamw(float* master, float* state, const float* g, void* w16, const OptSeg* seg, int nseg, int nblk,
               const float* hdr, const AdamArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(opt_adamw_kernel, dim3(nblk), dim3(256), 0, st, master, state, g, (bf16*)w16, seg, nseg, hdr,
                     a);
}
void opt_muon_momentum(const float* g, float* state, const OptSeg* seg, int nseg, int nblk, const float* hdr,
                       float mu, int nesterov, float* part, hipStream_t st) {
  hipLaunchKernelGGL(opt_muon_momentum_kernel, dim3(nblk), dim3(256), 0, st, g, state, seg, nseg, hdr, mu, nesterov,
                     part);
}
void opt_muon_normalise(const float* g, const float* state, const OptSeg* seg, int nseg, int nblk,
                        const float* hdr, float mu, int nesterov, const float* part, void* X, hipStream_t st) {
  hipLaunchKernelGGL(opt_muon_normalise_kernel, dim3(nblk), dim3(256), 0, st, g, state, seg, nseg, hdr, mu,
                     nesterov, part, (bf16*)X);
}
void opt_muon_update(float* master, const void* X, void* w16, const OptSeg* seg, int nseg, int nblk, float lr,
                     float scale, float wd, hipStream_t st) {
  hipLaunchKernelGGL(opt_muon_update_kernel, dim3(nblk), dim3(256), 0, st, master, (const bf16*)X, (bf16*)w16, seg,
                     nseg, lr, scale, wd);
}
void opt_widen(const void* w16, float* master, const OptSeg* seg, int nseg, int nblk, hipStream_t st) {
  hipLaunchKernelGGL(opt_widen_kernel, dim3(nblk), dim3(256), 0, st, (const bf16*)w16, master, seg, nseg);
}

}  // namespace gk
