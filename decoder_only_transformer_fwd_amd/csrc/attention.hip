// Causal / sliding-window softmax attention, forward and backward, for gfx950.
//
// Visible pairs: key j is visible to query i when 0 <= i - j <= W - 1 (W = T
// for full causal layers).  Scores are q^.k^ / sqrt(Dh) on the QK-normalised
// heads; probabilities use exp2 with the scale folded into log2(e)/sqrt(Dh),
// and the forward stores the per-query log-sum-exp in that base-2 domain.
//
// MFMA formulation.  The forward computes S^T = K Q^T so that each lane owns
// one query (its column) and reduces over keys in-lane plus one swap with the
// other half-wave; the output is accumulated transposed, O^T = V^T P^T, so the
// online-softmax rescale is a per-lane scalar.  The accumulator registers of S
// are fed directly as the B operand of the next MFMA: the K index of that
// operand runs over the keys in the accumulator's register order, and the
// matching A operand (V^T) is read from LDS in the same order.  Operands that
// would need a strided read (V for the forward, Q and dO for dK/dV, K for dQ)
// come from transposed copies [B][H][Dh][Tp] written by the producing kernels,
// so every LDS read is one contiguous 8- or 16-byte access.
//
// Backward: D_i = rowsum(dO*O) comes from a separate pass; dK/dV are produced
// by one kernel per 128-key tile iterating over query tiles, dQ by one kernel
// per 128-query tile iterating over key tiles.  No atomics: the result is
// bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace gk {

template <int ROWS, int ROW_BYTES>
struct RowTile {
  static constexpr int NCH = ROW_BYTES / 16;
  static constexpr int TOTAL = ROWS * NCH;
  static constexpr int PER = (TOTAL + 255) / 256;
  u32x4 reg[PER];
  __device__ __forceinline__ void load(const char* __restrict__ base, long stride, int nvalid, int t) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = t + p * 256;
      const int row = c / NCH, ch = c % NCH;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (c < TOTAL && row < nvalid) v = *(const u32x4*)(base + (long)row * stride + ch * 16);
      reg[p] = v;
    }
  }
  __device__ __forceinline__ void store(char* __restrict__ lds, int t) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = t + p * 256;
      if (c < TOTAL) *(u32x4*)(lds + lds_off<ROW_BYTES>(c / NCH, (c % NCH) * 16)) = reg[p];
    }
  }
};

// Fragment of a row-major operand: EPL contiguous elements at K offset
// s*KM + g*EPL of `row`.
template <typename T, int ROW_BYTES>
__device__ __forceinline__ typename Mfma<T>::frag row_frag(const char* lds, int row, int s, int g) {
  typedef Mfma<T> MF;
  typename MF::frag f;
  lds_read<ROW_BYTES, MF::EPL * (int)sizeof(T)>(lds, row, (s * MF::KM + g * MF::EPL) * (int)sizeof(T), &f);
  return f;
}

// Fragment whose K index follows accumulator register order: register f of a
// 32-wide block jb = f/16 holds column 32*jb + 8*(r/4) + 4*g + r%4, r = f%16.
template <typename T, int ROW_BYTES>
__device__ __forceinline__ typename Mfma<T>::frag perm_frag(const char* lds, int row, int s, int g) {
  typedef Mfma<T> MF;
  typename MF::frag out;
  if constexpr (MF::EPL == 8) {
#pragma unroll
    for (int run = 0; run < 2; ++run) {
      const int f = s * 8 + run * 4;
      const int col = (f >> 4) * 32 + 8 * ((f & 15) >> 2) + 4 * g;
      lds_read<ROW_BYTES, 8>(lds, row, col * 2, ((u32x2*)&out) + run);
    }
  } else {
    const int f = s;
    const int col = (f >> 4) * 32 + 8 * ((f & 15) >> 2) + 4 * g + (f & 3);
    lds_read<ROW_BYTES, 4>(lds, row, col * 4, &out);
  }
  return out;
}

// The matching B operand built from accumulator registers p[jb][r].
template <typename T, int NBLK>
__device__ __forceinline__ typename Mfma<T>::frag acc_frag(const floatx16 (&p)[NBLK], int s) {
  typedef Mfma<T> MF;
  typename MF::frag out;
  if constexpr (MF::EPL == 8) {
    const int jb = s >> 1, r0 = (s & 1) * 8;
    floatx4 a = {p[jb][r0], p[jb][r0 + 1], p[jb][r0 + 2], p[jb][r0 + 3]};
    floatx4 b = {p[jb][r0 + 4], p[jb][r0 + 5], p[jb][r0 + 6], p[jb][r0 + 7]};
    bf16x4 ca = __builtin_convertvector(a, bf16x4);
    bf16x4 cb = __builtin_convertvector(b, bf16x4);
    out = __builtin_shufflevector(ca, cb, 0, 1, 2, 3, 4, 5, 6, 7);
  } else {
    out = p[s >> 4][s & 15];
  }
  return out;
}

__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

__device__ __forceinline__ bool visible(int i, int j, int W, int Tn) {
  return j <= i && i - j < W && i < Tn;
}

// ------------------------------------------------------------------ forward
template <typename T, int DH>
__global__ __launch_bounds__(256, 1) void attn_fwd_kernel(AttnArgs a) {
  typedef Mfma<T> MF;
  constexpr int ES = sizeof(T);
  constexpr int BQ = 128, BKV = 64;
  constexpr int KROW = DH * ES, VROW = BKV * ES;
  constexpr int KS = DH / MF::KM;          // k-steps over the head dim
  constexpr int PS = BKV / MF::KM;         // k-steps over the keys of a tile
  constexpr int DB = DH / 32;              // 32-row blocks of the head dim
  constexpr int STAGE = BKV * KROW + DH * VROW;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, g = lane >> 5, l32 = lane & 31;
  const int qb = gridDim.x - 1 - blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Tn = a.T, W = a.window, d = a.d;
  const long row3 = 3L * d;
  const int i0 = qb * BQ, iw0 = i0 + wave * 32, i = iw0 + l32;

  const char* qkv = (const char*)a.qkv;
  typename MF::frag qf[KS];
  {
    const char* qrow = qkv + (((long)b * Tn + i) * row3 + h * DH) * ES;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (i < Tn)
        qf[s] = *(const typename MF::frag*)(qrow + (s * MF::KM + g * MF::EPL) * ES);
      else
        __builtin_memset(&qf[s], 0, sizeof(qf[s]));
    }
  }

  const int jb0 = max(0, i0 - W + 1) / BKV * BKV;
  const int jend = min(Tn, i0 + BQ);
  const int nt = jend > jb0 ? (jend - jb0 + BKV - 1) / BKV : 0;

  const char* kbase = qkv + (((long)b * Tn) * row3 + d + h * DH) * ES;
  const char* vtbase = (const char*)a.vT + (((long)b * a.H + h) * DH) * (long)a.Tp * ES;
  RowTile<BKV, KROW> lk;
  RowTile<DH, VROW> lv;

  floatx16 acc[DB];
#pragma unroll
  for (int x = 0; x < DB; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[x][r] = 0.f;
  float m = -1e30f, l = 0.f;

  if (nt > 0) {
    lk.load(kbase + (long)jb0 * row3 * ES, row3 * ES, Tn - jb0, t);
    lv.load(vtbase + (long)jb0 * ES, (long)a.Tp * ES, DH, t);
    lk.store(smem, t);
    lv.store(smem + BKV * KROW, t);
  }
  __syncthreads();

  for (int it = 0; it < nt; ++it) {
    const int j0 = jb0 + it * BKV;
    const int s = it & 1;
    const bool more = it + 1 < nt;
    if (more) {
      lk.load(kbase + (long)(j0 + BKV) * row3 * ES, row3 * ES, Tn - j0 - BKV, t);
      lv.load(vtbase + (long)(j0 + BKV) * ES, (long)a.Tp * ES, DH, t);
    }
    const char* ks = smem + s * STAGE;
    const char* vs = ks + BKV * KROW;
    const bool skip = j0 > iw0 + 31 || iw0 - (j0 + BKV - 1) >= W || iw0 >= Tn;
    if (!skip) {
      floatx16 sc[2];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[jb][r] = 0.f;
#pragma unroll
        for (int k = 0; k < KS; ++k) sc[jb] = MF::mma(row_frag<T, KROW>(ks, jb * 32 + l32, k, g), qf[k], sc[jb]);
      }
      const bool need_mask = (j0 + BKV - 1 > iw0) || (iw0 + 31 - j0 >= W) || (j0 + BKV > Tn);
      float mloc = -1e30f;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = sc[jb][r] * a.scale_log2;
          if (need_mask && !visible(i, j0 + jb * 32 + acc_row(r, g), W, Tn)) x = -INFINITY;
          sc[jb][r] = x;
          mloc = fmaxf(mloc, x);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float mnew = fmaxf(m, mloc);
      const float alpha = fast_exp2(m - mnew);
      m = mnew;
      float ps = 0.f;
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(sc[jb][r] - mnew);
          sc[jb][r] = p;
          ps += p;
        }
      l = l * alpha + ps;
#pragma unroll
      for (int x = 0; x < DB; ++x)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[x][r] *= alpha;
#pragma unroll
      for (int k = 0; k < PS; ++k) {
        const typename MF::frag pf = acc_frag<T, 2>(sc, k);
#pragma unroll
        for (int x = 0; x < DB; ++x) acc[x] = MF::mma(perm_frag<T, VROW>(vs, x * 32 + l32, k, g), pf, acc[x]);
      }
    }
    if (more) {
      lk.store(smem + (s ^ 1) * STAGE, t);
      lv.store(smem + (s ^ 1) * STAGE + BKV * KROW, t);
    }
    __syncthreads();
  }

  const float lt = l + __shfl_xor(l, 32, 64);
  if (i < Tn) {
    const float inv = 1.0f / lt;
    T* orow = (T*)a.o + ((long)b * Tn + i) * d + h * DH;
#pragma unroll
    for (int x = 0; x < DB; ++x)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        floatx4 v = {acc[x][4 * q] * inv, acc[x][4 * q + 1] * inv, acc[x][4 * q + 2] * inv, acc[x][4 * q + 3] * inv};
        store4(orow + x * 32 + 8 * q + 4 * g, v);
      }
  }
  if (g == 0 && i < a.Tp) a.lse2[((long)b * a.H + h) * a.Tp + i] = i < Tn ? m + fast_log2(lt) : 0.f;
}

// ------------------------------------------------------------------ backward: dK, dV
template <typename T, int DH>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_kernel(AttnArgs a) {
  typedef Mfma<T> MF;
  constexpr int ES = sizeof(T);
  constexpr int BKV = 128, BQ = 32;
  constexpr int RROW = DH * ES, TROW = BQ * ES;
  constexpr int KS = DH / MF::KM;
  constexpr int PS = BQ / MF::KM;
  constexpr int DB = DH / 32;
  constexpr int STAGE = 2 * BQ * RROW + 2 * DH * TROW + 2 * BQ * 4;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, g = lane >> 5, l32 = lane & 31;
  const int kb = gridDim.x - 1 - blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Tn = a.T, W = a.window, d = a.d, Tp = a.Tp;
  const long row3 = 3L * d;
  const int j0 = kb * BKV, jw0 = j0 + wave * 32, j = jw0 + l32;

  const char* qkv = (const char*)a.qkv;
  typename MF::frag kf[KS], vf[KS];
  {
    const char* krow = qkv + (((long)b * Tn + j) * row3 + d + h * DH) * ES;
    const char* vrow = krow + (long)d * ES;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (j < Tn) {
        kf[s] = *(const typename MF::frag*)(krow + (s * MF::KM + g * MF::EPL) * ES);
        vf[s] = *(const typename MF::frag*)(vrow + (s * MF::KM + g * MF::EPL) * ES);
      } else {
        __builtin_memset(&kf[s], 0, sizeof(kf[s]));
        __builtin_memset(&vf[s], 0, sizeof(vf[s]));
      }
    }
  }

  const int ib = j0;
  const int iend = min(Tn, j0 + BKV - 1 + W);
  const int nq = iend > ib ? (iend - ib + BQ - 1) / BQ : 0;

  const char* qbase = qkv + (((long)b * Tn) * row3 + h * DH) * ES;
  const char* dobase = (const char*)a.dO + (((long)b * Tn) * d + h * DH) * ES;
  const long hoff = ((long)b * a.H + h);
  const char* qtbase = (const char*)a.qT + hoff * DH * Tp * ES;
  const char* dotbase = (const char*)a.dOT + hoff * DH * Tp * ES;
  const float* lseb = a.lse2 + hoff * Tp;
  const float* Db = a.Dv + hoff * Tp;

  RowTile<BQ, RROW> lq, ldo;
  RowTile<DH, TROW> lqt, ldot;
  float lse_r = 0.f, d_r = 0.f;   // thread t < BQ stages lse/D of query i0 + t

  floatx16 dk[DB], dv[DB];
#pragma unroll
  for (int x = 0; x < DB; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[x][r] = dv[x][r] = 0.f;

  auto load = [&](int i0) {
    lq.load(qbase + (long)i0 * row3 * ES, row3 * ES, Tn - i0, t);
    ldo.load(dobase + (long)i0 * d * ES, (long)d * ES, Tn - i0, t);
    lqt.load(qtbase + (long)i0 * ES, (long)Tp * ES, DH, t);
    ldot.load(dotbase + (long)i0 * ES, (long)Tp * ES, DH, t);
    if (t < BQ) {
      lse_r = i0 + t < Tp ? lseb[i0 + t] : 0.f;
      d_r = i0 + t < Tp ? Db[i0 + t] : 0.f;
    }
  };
  auto store = [&](char* st) {
    lq.store(st, t);
    ldo.store(st + BQ * RROW, t);
    lqt.store(st + 2 * BQ * RROW, t);
    ldot.store(st + 2 * BQ * RROW + DH * TROW, t);
    float* f = (float*)(st + 2 * BQ * RROW + 2 * DH * TROW);
    if (t < BQ) {
      f[t] = lse_r;
      f[BQ + t] = d_r;
    }
  };

  if (nq > 0) {
    load(ib);
    store(smem);
  }
  __syncthreads();

  for (int it = 0; it < nq; ++it) {
    const int i0 = ib + it * BQ;
    const int s = it & 1;
    const bool more = it + 1 < nq;
    if (more) load(i0 + BQ);
    const char* qs = smem + s * STAGE;
    const char* dos = qs + BQ * RROW;
    const char* qts = qs + 2 * BQ * RROW;
    const char* dots = qts + DH * TROW;
    const float* lses = (const float*)(dots + DH * TROW);
    const float* Ds = lses + BQ;
    const bool skip = i0 + BQ - 1 < jw0 || i0 - (jw0 + 31) >= W || jw0 >= Tn || i0 >= Tn;
    if (!skip) {
      floatx16 sc[1], dp[1];
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[0][r] = dp[0][r] = 0.f;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        sc[0] = MF::mma(row_frag<T, RROW>(qs, l32, k, g), kf[k], sc[0]);
        dp[0] = MF::mma(row_frag<T, RROW>(dos, l32, k, g), vf[k], dp[0]);
      }
      const bool need_mask = (i0 < jw0 + 31) || (i0 + BQ - 1 - jw0 >= W) || (i0 + BQ > Tn) || (jw0 + 31 >= Tn);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int il = acc_row(r, g);
        const float p0 = fast_exp2(sc[0][r] * a.scale_log2 - lses[il]);
        const float p = (!need_mask || visible(i0 + il, j, W, Tn)) ? p0 : 0.f;
        sc[0][r] = p;
        dp[0][r] = p * (dp[0][r] - Ds[il]);
      }
#pragma unroll
      for (int k = 0; k < PS; ++k) {
        const typename MF::frag pf = acc_frag<T, 1>(sc, k);
        const typename MF::frag sf = acc_frag<T, 1>(dp, k);
#pragma unroll
        for (int x = 0; x < DB; ++x) {
          dv[x] = MF::mma(perm_frag<T, TROW>(dots, x * 32 + l32, k, g), pf, dv[x]);
          dk[x] = MF::mma(perm_frag<T, TROW>(qts, x * 32 + l32, k, g), sf, dk[x]);
        }
      }
    }
    if (more) store(smem + (s ^ 1) * STAGE);
    __syncthreads();
  }

  if (j < Tn) {
    T* base = (T*)a.dqkv + ((long)b * Tn + j) * row3 + h * DH;
#pragma unroll
    for (int x = 0; x < DB; ++x)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = x * 32 + 8 * q + 4 * g;
        floatx4 vk = {dk[x][4 * q], dk[x][4 * q + 1], dk[x][4 * q + 2], dk[x][4 * q + 3]};
        floatx4 vv = {dv[x][4 * q], dv[x][4 * q + 1], dv[x][4 * q + 2], dv[x][4 * q + 3]};
        store4(base + d + c, vk * a.scale);
        store4(base + 2 * d + c, vv);
      }
  }
}

// ------------------------------------------------------------------ backward: dQ
template <typename T, int DH>
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_kernel(AttnArgs a) {
  typedef Mfma<T> MF;
  constexpr int ES = sizeof(T);
  constexpr int BQ = 128, BKV = 64;
  constexpr int RROW = DH * ES, TROW = BKV * ES;
  constexpr int KS = DH / MF::KM;
  constexpr int PS = BKV / MF::KM;
  constexpr int DB = DH / 32;
  constexpr int STAGE = 2 * BKV * RROW + DH * TROW;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, g = lane >> 5, l32 = lane & 31;
  const int qb = gridDim.x - 1 - blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Tn = a.T, W = a.window, d = a.d, Tp = a.Tp;
  const long row3 = 3L * d;
  const int i0 = qb * BQ, iw0 = i0 + wave * 32, i = iw0 + l32;
  const long hoff = ((long)b * a.H + h);

  const char* qkv = (const char*)a.qkv;
  typename MF::frag qf[KS], df[KS];
  {
    const char* qrow = qkv + (((long)b * Tn + i) * row3 + h * DH) * ES;
    const char* drow = (const char*)a.dO + (((long)b * Tn + i) * d + h * DH) * ES;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (i < Tn) {
        qf[s] = *(const typename MF::frag*)(qrow + (s * MF::KM + g * MF::EPL) * ES);
        df[s] = *(const typename MF::frag*)(drow + (s * MF::KM + g * MF::EPL) * ES);
      } else {
        __builtin_memset(&qf[s], 0, sizeof(qf[s]));
        __builtin_memset(&df[s], 0, sizeof(df[s]));
      }
    }
  }
  const float lse_i = i < Tn ? a.lse2[hoff * Tp + i] : 0.f;
  const float D_i = i < Tn ? a.Dv[hoff * Tp + i] : 0.f;

  const int jb0 = max(0, i0 - W + 1) / BKV * BKV;
  const int jend = min(Tn, i0 + BQ);
  const int nt = jend > jb0 ? (jend - jb0 + BKV - 1) / BKV : 0;

  const char* kbase = qkv + (((long)b * Tn) * row3 + d + h * DH) * ES;
  const char* vbase = kbase + (long)d * ES;
  const char* ktbase = (const char*)a.kT + hoff * DH * Tp * ES;
  RowTile<BKV, RROW> lk, lv;
  RowTile<DH, TROW> lkt;

  floatx16 dq[DB];
#pragma unroll
  for (int x = 0; x < DB; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[x][r] = 0.f;

  auto load = [&](int j0) {
    lk.load(kbase + (long)j0 * row3 * ES, row3 * ES, Tn - j0, t);
    lv.load(vbase + (long)j0 * row3 * ES, row3 * ES, Tn - j0, t);
    lkt.load(ktbase + (long)j0 * ES, (long)Tp * ES, DH, t);
  };
  auto store = [&](char* st) {
    lk.store(st, t);
    lv.store(st + BKV * RROW, t);
    lkt.store(st + 2 * BKV * RROW, t);
  };
  if (nt > 0) {
    load(jb0);
    store(smem);
  }
  __syncthreads();

  for (int it = 0; it < nt; ++it) {
    const int j0 = jb0 + it * BKV;
    const int s = it & 1;
    const bool more = it + 1 < nt;
    if (more) load(j0 + BKV);
    const char* ks = smem + s * STAGE;
    const char* vs = ks + BKV * RROW;
    const char* kts = vs + BKV * RROW;
    const bool skip = j0 > iw0 + 31 || iw0 - (j0 + BKV - 1) >= W || iw0 >= Tn;
    if (!skip) {
      floatx16 sc[2], dp[2];
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[jb][r] = dp[jb][r] = 0.f;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          sc[jb] = MF::mma(row_frag<T, RROW>(ks, jb * 32 + l32, k, g), qf[k], sc[jb]);
          dp[jb] = MF::mma(row_frag<T, RROW>(vs, jb * 32 + l32, k, g), df[k], dp[jb]);
        }
      }
      const bool need_mask = (j0 + BKV - 1 > iw0) || (iw0 + 31 - j0 >= W) || (j0 + BKV > Tn) || (iw0 + 31 >= Tn);
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p0 = fast_exp2(sc[jb][r] * a.scale_log2 - lse_i);
          const float p = (!need_mask || visible(i, j0 + jb * 32 + acc_row(r, g), W, Tn)) ? p0 : 0.f;
          dp[jb][r] = p * (dp[jb][r] - D_i);
        }
#pragma unroll
      for (int k = 0; k < PS; ++k) {
        const typename MF::frag sf = acc_frag<T, 2>(dp, k);
#pragma unroll
        for (int x = 0; x < DB; ++x) dq[x] = MF::mma(perm_frag<T, TROW>(kts, x * 32 + l32, k, g), sf, dq[x]);
      }
    }
    if (more) store(smem + (s ^ 1) * STAGE);
    __syncthreads();
  }

  if (i < Tn) {
    T* base = (T*)a.dqkv + ((long)b * Tn + i) * row3 + h * DH;
#pragma unroll
    for (int x = 0; x < DB; ++x)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        floatx4 v = {dq[x][4 * q], dq[x][4 * q + 1], dq[x][4 * q + 2], dq[x][4 * q + 3]};
        store4(base + x * 32 + 8 * q + 4 * g, v * a.scale);
      }
  }
}

// ------------------------------------------------------------------ launchers
template <typename T, int DH>
static void fwd_t(const AttnArgs& a, hipStream_t st) {
  dim3 g((a.T + 127) / 128, a.H, a.B);
  hipLaunchKernelGGL((attn_fwd_kernel<T, DH>), g, dim3(256), 0, st, a);
}
template <typename T, int DH>
static void bwd_t(const AttnArgs& a, int part, hipStream_t st) {
  dim3 g((a.T + 127) / 128, a.H, a.B);
  if (part == 0)
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, DH>), g, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_bwd_dq_kernel<T, DH>), g, dim3(256), 0, st, a);
}

int attn_fwd(int dtype, int Dh, const AttnArgs& a, hipStream_t st) {
#define AF(TT, D) if (Dh == D) { fwd_t<TT, D>(a, st); return 0; }
  if (dtype == DT_BF16) { AF(bf16, 64) AF(bf16, 128) }
  else { AF(float, 32) AF(float, 64) }
#undef AF
  return -1;
}

int attn_bwd(int dtype, int Dh, const AttnArgs& a, int part, hipStream_t st) {
#define AB(TT, D) if (Dh == D) { bwd_t<TT, D>(a, part, st); return 0; }
  if (dtype == DT_BF16) { AB(bf16, 64) AB(bf16, 128) }
  else { AB(float, 32) AB(float, 64) }
#undef AB
  return -1;
}

}  // namespace gk
