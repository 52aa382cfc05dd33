// Causal / sliding-window softmax attention, forward and backward, for gfx950.
//
// Visible pairs: key j is visible to query i when 0 <= i - j <= W - 1 (W = T
// for full causal layers).  Scores are q^.k^ / sqrt(Dh) on the QK-normalised
// heads; probabilities use exp2 with the scale folded into log2(e)/sqrt(Dh),
// and the forward stores the per-query log-sum-exp in that base-2 domain.
//
// MFMA formulation.  The forward computes S^T = K Q^T so that each lane owns
// one query (its column) and reduces over keys in-lane plus one swap with the
// other half-wave; the output is accumulated transposed, O^T = V^T P^T, and
// normalised per lane at the end.  The softmax needs no running maximum: the
// heads are QK-normalised, so the scores are bounded and a fixed exponent
// offset keeps every exponential in range.  The accumulator registers of S
// are fed directly as the B operand of the next MFMA: the K index of that
// operand runs over the keys in the accumulator's register order, and the
// matching A operand (V^T) is read from LDS in the same order.  Operands that
// would need a strided read (V for the forward, Q and dO for dK/dV, K for dQ)
// come from transposed copies [B][H][Dh][Tp] written by the producing kernels,
// so every LDS read is one contiguous 8- or 16-byte access.
//
// Backward: D_i = rowsum(dO*O) comes from a separate pass; dV and dK are
// produced by two passes over 128-key tiles iterating over query tiles (of
// every query head that shares the key/value head, with grouped-query
// attention), dQ by one pass over 128-query tiles iterating over key tiles.
// No atomics: the result is bitwise reproducible.
#include "common.h"
#include "kernels.h"

namespace gk {

// Work-group -> (tile, head, batch).  Work-groups are dealt round-robin to
// the 8 XCDs (each with its own L2); the linear id is remapped so that all
// tiles of one (batch, head) run on the same XCD and share its K/V (or Q/dO)
// reads from L2.  Tiles are taken in reverse so the longest causal rows
// start first.
__device__ __forceinline__ void attn_coords(int& tile, int& h, int& b) {
  const int nt = gridDim.x, H = gridDim.y;
  const int L = blockIdx.x + nt * (blockIdx.y + H * blockIdx.z);
  const int per = nt * H * gridDim.z / 8;
  const int Lp = (per > 0 && L < per * 8) ? (L & 7) * per + (L >> 3) : L;
  tile = nt - 1 - Lp % nt;
  h = (Lp / nt) % H;
  b = Lp / nt / H;
}

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

// Visibility from the offset i - j alone: 0 <= i - j < W, one unsigned
// compare.  Positions past T need no test: their query, key, value, dO and
// D entries are zero (padded copies, zero-filled tile loads), so they add
// nothing to any stored result, and a valid query never sees a padded key
// (j <= i < T).
__device__ __forceinline__ bool visible_off(int i_minus_j, int W) { return (unsigned)i_minus_j < (unsigned)W; }

// ------------------------------------------------------------------ forward
// Work-group: 4 waves x 32 queries; key tiles of 64 (K rows and V^T columns)
// arrive by direct-to-LDS loads one tile ahead.  Two work-groups fit per CU
// (64 KB LDS, <= 256 registers per lane) so one work-group's softmax overlaps
// the other's MFMAs.
template <typename T, int DH>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs a) {
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
  int qb, h, b;
  attn_coords(qb, h, b);
  const int Tn = a.T, W = a.window, d = a.d;
  const long row3 = a.ldqkv;
  const int hk = h / (a.H / a.Hkv);   // key/value head of query head h
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

  RowDma<BKV, KROW, 4> lk;
  RowDma<DH, VROW, 4> lv;
  {
    const char* kbase = qkv + (((long)b * Tn) * row3 + d + hk * DH) * ES;
    lk.init(kbase, (int)(row3 * ES), (long)(Tn - 1) * row3 * ES + KROW, wave, lane);
    const char* vtbase = (const char*)a.vT + (((long)b * a.Hkv + hk) * DH) * (long)a.Tp * ES;
    lv.init(vtbase, a.Tp * ES, (long)DH * a.Tp * ES, wave, lane);
  }

  floatx16 acc[DB];
#pragma unroll
  for (int x = 0; x < DB; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[x][r] = 0.f;
  // Softmax with a fixed exponent offset instead of a running maximum.  The
  // heads are QK-normalised (|q^|, |k^| <= sqrt(Dh), up to bf16 rounding), so
  // every scaled score s * c lies within +-c * Dh; with the offset
  // M = 1.01 * c * Dh every exponent is <= 0 and >= -2M (2^-33 at Dh = 128),
  // well inside fp32 and bf16 range.  No running max, no rescaling of the
  // accumulators, and the same probabilities as the online form.
  const float c = a.scale_log2;
  const float M = 1.01f * c * DH;
  float l = 0.f;   // sum of this lane's exponentials

  if (nt > 0) {
    lk.issue(smem, jb0 * (int)(row3 * ES), wave);
    lv.issue(smem + BKV * KROW, jb0 * ES, wave);
  }
  for (int it = 0; it < nt; ++it) {
    const int j0 = jb0 + it * BKV;
    const int s = it & 1;
    __builtin_amdgcn_s_waitcnt(0x0070);   // this tile's loads have landed
    __syncthreads();                      // ... for every wave; stage s^1 is free
    if (it + 1 < nt) {
      char* nx = smem + (s ^ 1) * STAGE;
      lk.issue(nx, (j0 + BKV) * (int)(row3 * ES), wave);
      lv.issue(nx + BKV * KROW, (j0 + BKV) * ES, wave);
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
      const bool need_mask = (j0 + BKV - 1 > iw0) || (iw0 + 31 - j0 >= W);
      if (need_mask) {
        const int dij = i - j0;   // i - j of key row jb * 32 + acc_row(r, g)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float x = __builtin_fmaf(sc[jb][r], c, -M);
            sc[jb][r] = visible_off(dij - jb * 32 - acc_row(r, g), W) ? x : -INFINITY;
          }
      } else {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[jb][r] = __builtin_fmaf(sc[jb][r], c, -M);
      }
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(sc[jb][r]);
          sc[jb][r] = p;
          l += p;
        }
#pragma unroll
      for (int k = 0; k < PS; ++k) {
        const typename MF::frag pf = acc_frag<T, 2>(sc, k);
#pragma unroll
        for (int x = 0; x < DB; ++x) acc[x] = MF::mma(perm_frag<T, VROW>(vs, x * 32 + l32, k, g), pf, acc[x]);
      }
    }
  }

  const float lt = l + __shfl_xor(l, 32, 64);
  float om = 0.f;
  if (i < Tn) {
    const float inv = 1.0f / lt;
    T* orow = (T*)a.o + ((long)b * Tn + i) * d + h * DH;
#pragma unroll
    for (int x = 0; x < DB; ++x)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        floatx4 v = {acc[x][4 * q] * inv, acc[x][4 * q + 1] * inv, acc[x][4 * q + 2] * inv, acc[x][4 * q + 3] * inv};
        store4(orow + x * 32 + 8 * q + 4 * g, v);
        if (a.amax_o) om = fmaxf(om, abs_max4<T>(v));
      }
  }
  if (a.amax_o) {
    __syncthreads();   // every wave is done reading the K/V stages
    block_amax<4>(a.amax_o, om, (float*)smem);
  }
  // log-sum-exp of the scaled scores, base 2
  if (g == 0 && i < a.Tp) a.lse2[((long)b * a.H + h) * a.Tp + i] = i < Tn ? M + fast_log2(lt) : 0.f;
}

// ------------------------------------------------------------------ backward: dK, dV
// Work-group: 4 waves x 32 keys (K and V fragments held in registers), looping
// over query tiles of BQ that arrive by direct-to-LDS loads one tile ahead (Q
// and dO rows, and their transposed copies for the dV / dK products); the
// per-query lse and D values are 16-byte loads issued as a tile starts.
// MODE 1 produces dV and MODE 2 dK: each pass is small enough for two or
// three waves per SIMD, which on MI355X beats a single pass holding both
// accumulators at one wave per SIMD, even though the scores are computed in
// both passes.
template <typename T, int DH, int BQ, int MODE>
__global__ __launch_bounds__(256, MODE == 1 ? 3 : 2) void attn_bwd_dkdv_kernel(AttnArgs a) {
  typedef Mfma<T> MF;
  static_assert(MODE == 1 || MODE == 2, "MODE 1 = dV pass, MODE 2 = dK pass");
  constexpr bool DO_DV = MODE == 1, DO_DK = MODE == 2;
  constexpr int ES = sizeof(T);
  constexpr int BKV = 128;
  constexpr int QB = BQ / 32;                 // 32-query blocks per tile
  constexpr int RROW = DH * ES, TROW = BQ * ES;
  constexpr int KS = DH / MF::KM;
  constexpr int PS = BQ / MF::KM;
  constexpr int DB = DH / 32;
  // stage layout: Q rows | dO rows (dK) | Q^T (dK) | dO^T (dV) | lse | D (dK);
  // lse and D of the tile's BQ queries arrive with the tile (one 64-lane
  // copy each, 1 KB of LDS of which the first BQ * 4 bytes are used)
  constexpr int OFF_DO = BQ * RROW;
  constexpr int OFF_QT = OFF_DO + (DO_DK ? BQ * RROW : 0);
  constexpr int OFF_DOT = OFF_QT + (DO_DK ? DH * TROW : 0);
  constexpr int OFF_LSE = OFF_DOT + (DO_DV ? DH * TROW : 0);
  constexpr int OFF_D = OFF_LSE + 1024;
  constexpr int STAGE = OFF_D + (DO_DK ? 1024 : 0);
  static_assert(BQ / 4 <= 64, "one 64-lane copy holds the tile's lse / D");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, g = lane >> 5, l32 = lane & 31;
  int kb, hk, b;   // key tile, key/value head, batch row
  attn_coords(kb, hk, b);
  const int Tn = a.T, W = a.window, d = a.d, Tp = a.Tp;
  const long row3 = a.ldqkv;
  const int dkv = a.Hkv * DH;
  const int G = a.H / a.Hkv;   // query heads per key/value head
  const int j0 = kb * BKV, jw0 = j0 + wave * 32, j = jw0 + l32;
  const float c = a.scale_log2;

  const char* qkv = (const char*)a.qkv;
  typename MF::frag kf[KS], vf[DO_DK ? KS : 1];
  {
    const char* krow = qkv + (((long)b * Tn + j) * row3 + d + hk * DH) * ES;
    const char* vrow = krow + (long)dkv * ES;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (j < Tn) {
        kf[s] = *(const typename MF::frag*)(krow + (s * MF::KM + g * MF::EPL) * ES);
        if constexpr (DO_DK) vf[s] = *(const typename MF::frag*)(vrow + (s * MF::KM + g * MF::EPL) * ES);
      } else {
        __builtin_memset(&kf[s], 0, sizeof(kf[s]));
        if constexpr (DO_DK) __builtin_memset(&vf[s], 0, sizeof(vf[s]));
      }
    }
  }

  const int ib = j0;
  const int iend = min(Tn, j0 + BKV - 1 + W);
  const int nq = iend > ib ? (iend - ib + BQ - 1) / BQ : 0;

  // The G query heads that share this key/value head are walked one after
  // another, as one sequence of G * nq query tiles.  Each operand's buffer
  // covers the whole group (its first head's columns / rows onwards), and a
  // head's offset within it goes into the scalar offset of the copies.
  const int hq0 = hk * G;                  // first query head of the group
  const long hoff0 = (long)b * a.H + hq0;
  RowDma<BQ, RROW, 4> lq, ldo;
  RowDma<DH, TROW, 4> lqt, ldot;
  lq.init(qkv + (((long)b * Tn) * row3 + hq0 * DH) * ES, (int)(row3 * ES),
          (long)(Tn - 1) * row3 * ES + (long)G * RROW, wave, lane);
  if constexpr (DO_DK) {
    ldo.init((const char*)a.dO + (((long)b * Tn) * d + hq0 * DH) * ES, d * ES,
             (long)(Tn - 1) * d * ES + (long)G * RROW, wave, lane);
    lqt.init((const char*)a.qT + hoff0 * DH * Tp * ES, Tp * ES, (long)G * DH * Tp * ES, wave, lane);
  }
  if constexpr (DO_DV) ldot.init((const char*)a.dOT + hoff0 * DH * Tp * ES, Tp * ES, (long)G * DH * Tp * ES, wave, lane);
  const __amdgpu_buffer_rsrc_t rs_lse = uniform_rsrc(a.lse2 + hoff0 * Tp, G * Tp * 4);
  const __amdgpu_buffer_rsrc_t rs_D = uniform_rsrc(a.Dv + hoff0 * Tp, G * Tp * 4);

  floatx16 dk[DO_DK ? DB : 1], dv[DO_DV ? DB : 1];
#pragma unroll
  for (int x = 0; x < DB; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if constexpr (DO_DK) dk[x][r] = 0.f;
      if constexpr (DO_DV) dv[x][r] = 0.f;
    }

  // tile itx of the sequence: query head hq0 + gq, queries from i0
  auto issue = [&](int itx, int stage) {
    const int gq = itx / nq, i0 = ib + (itx - gq * nq) * BQ;
    char* st = smem + stage * STAGE;
    lq.issue(st, i0 * (int)(row3 * ES) + gq * RROW, wave);
    if constexpr (DO_DK) {
      ldo.issue(st + OFF_DO, i0 * d * ES + gq * RROW, wave);
      lqt.issue(st + OFF_QT, (gq * DH * Tp + i0) * ES, wave);
    }
    if constexpr (DO_DV) ldot.issue(st + OFF_DOT, (gq * DH * Tp + i0) * ES, wave);
    if (wave == 0) {
      const int off = lane < BQ / 4 ? (gq * Tp + i0 + 4 * lane) * 4 : (int)0x80000000;
      dma16(rs_lse, st + OFF_LSE, off);
      if constexpr (DO_DK) dma16(rs_D, st + OFF_D, off);
    }
  };

  const int ntot = G * nq;
  if (ntot > 0) issue(0, 0);
  for (int it = 0; it < ntot; ++it) {
    const int gq = it / nq;
    const int i0 = ib + (it - gq * nq) * BQ;
    const int s = it & 1;
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    if (it + 1 < ntot) issue(it + 1, s ^ 1);
    const char* qs = smem + s * STAGE;
    const bool skip = i0 + BQ - 1 < jw0 || i0 - (jw0 + 31) >= W || jw0 >= Tn || i0 >= Tn;
    if (!skip) {
      // lse / D of the queries this lane's accumulator rows cover: i0 + 32qb + 8q + 4g + e
      floatx4 lse_c[QB][4], D_c[DO_DK ? QB : 1][4];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          lse_c[qb][q] = *(const floatx4*)(qs + OFF_LSE + (32 * qb + 8 * q + 4 * g) * 4);
          if constexpr (DO_DK) D_c[qb][q] = *(const floatx4*)(qs + OFF_D + (32 * qb + 8 * q + 4 * g) * 4);
        }
      floatx16 sc[QB], dp[DO_DK ? QB : 1];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[qb][r] = 0.f;
          if constexpr (DO_DK) dp[qb][r] = 0.f;
        }
      }
#pragma unroll
      for (int k = 0; k < KS; ++k)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          sc[qb] = MF::mma(row_frag<T, RROW>(qs, qb * 32 + l32, k, g), kf[k], sc[qb]);
          if constexpr (DO_DK) dp[qb] = MF::mma(row_frag<T, RROW>(qs + OFF_DO, qb * 32 + l32, k, g), vf[k], dp[qb]);
        }
      const bool need_mask = (i0 < jw0 + 31) || (i0 + BQ - 1 - jw0 >= W);
      // invisible pairs get a -inf exponent (exp2 -> 0); the exponentials
      // themselves are unconditional so the loop stays branch-free
      if (need_mask) {
        const int dij = i0 - j;   // i - j of accumulator row il is dij + il
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int il = qb * 32 + acc_row(r, g);
            const float x = __builtin_fmaf(sc[qb][r], c, -lse_c[qb][r >> 2][r & 3]);
            sc[qb][r] = visible_off(dij + il, W) ? x : -INFINITY;
          }
      } else {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[qb][r] = __builtin_fmaf(sc[qb][r], c, -lse_c[qb][r >> 2][r & 3]);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(sc[qb][r]);
          sc[qb][r] = p;
          if constexpr (DO_DK) dp[qb][r] = p * (dp[qb][r] - D_c[qb][r >> 2][r & 3]);
        }
#pragma unroll
      for (int k = 0; k < PS; ++k) {
#pragma unroll
        for (int x = 0; x < DB; ++x) {
          if constexpr (DO_DV)
            dv[x] = MF::mma(perm_frag<T, TROW>(qs + OFF_DOT, x * 32 + l32, k, g), acc_frag<T, QB>(sc, k), dv[x]);
          if constexpr (DO_DK)
            dk[x] = MF::mma(perm_frag<T, TROW>(qs + OFF_QT, x * 32 + l32, k, g), acc_frag<T, QB>(dp, k), dk[x]);
        }
      }
    }
  }

  float vm = 0.f;
  if (j < Tn) {
    T* base = (T*)a.dqkv + ((long)b * Tn + j) * row3 + hk * DH;
#pragma unroll
    for (int x = 0; x < DB; ++x)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cc = x * 32 + 8 * q + 4 * g;
        if constexpr (DO_DK) {
          floatx4 vk = {dk[x][4 * q], dk[x][4 * q + 1], dk[x][4 * q + 2], dk[x][4 * q + 3]};
          store4(base + d + cc, vk * a.scale);
        }
        if constexpr (DO_DV) {
          floatx4 vv = {dv[x][4 * q], dv[x][4 * q + 1], dv[x][4 * q + 2], dv[x][4 * q + 3]};
          store4(base + d + dkv + cc, vv);
          if (a.amax_dv) vm = fmaxf(vm, abs_max4<T>(vv));
        }
      }
  }
  if constexpr (DO_DV) {
    if (a.amax_dv) {
      __syncthreads();   // every wave is done reading the stages
      block_amax<4>(a.amax_dv, vm, (float*)smem);
    }
  }
}

// ------------------------------------------------------------------ backward: dQ
// Work-group: 4 waves x 32 queries (Q and dO fragments in registers), looping
// over key tiles of 32 (K and V rows plus K^T columns) that arrive by
// direct-to-LDS loads one tile ahead.
template <typename T, int DH>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(AttnArgs a) {
  typedef Mfma<T> MF;
  constexpr int ES = sizeof(T);
  constexpr int BQ = 128, BKV = 32;
  constexpr int RROW = DH * ES, TROW = BKV * ES;
  constexpr int KS = DH / MF::KM;
  constexpr int PS = BKV / MF::KM;
  constexpr int DB = DH / 32;
  constexpr int STAGE = 2 * BKV * RROW + DH * TROW;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, g = lane >> 5, l32 = lane & 31;
  int qb, h, b;
  attn_coords(qb, h, b);
  const int Tn = a.T, W = a.window, d = a.d, Tp = a.Tp;
  const long row3 = a.ldqkv;
  const int hk = h / (a.H / a.Hkv);   // key/value head of query head h
  const int i0 = qb * BQ, iw0 = i0 + wave * 32, i = iw0 + l32;
  const long hoff = ((long)b * a.H + h);
  const float c = a.scale_log2;

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

  RowDma<BKV, RROW, 4> lk, lv;
  RowDma<DH, TROW, 4> lkt;
  {
    const char* kbase = qkv + (((long)b * Tn) * row3 + d + hk * DH) * ES;
    lk.init(kbase, (int)(row3 * ES), (long)(Tn - 1) * row3 * ES + RROW, wave, lane);
    lv.init(kbase + (long)a.Hkv * DH * ES, (int)(row3 * ES), (long)(Tn - 1) * row3 * ES + RROW, wave, lane);
    lkt.init((const char*)a.kT + ((long)b * a.Hkv + hk) * DH * Tp * ES, Tp * ES, (long)DH * Tp * ES, wave, lane);
  }

  floatx16 dq[DB];
#pragma unroll
  for (int x = 0; x < DB; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[x][r] = 0.f;

  auto issue = [&](int j0, int stage) {
    char* st = smem + stage * STAGE;
    lk.issue(st, j0 * (int)(row3 * ES), wave);
    lv.issue(st + BKV * RROW, j0 * (int)(row3 * ES), wave);
    lkt.issue(st + 2 * BKV * RROW, j0 * ES, wave);
  };
  if (nt > 0) issue(jb0, 0);
  for (int it = 0; it < nt; ++it) {
    const int j0 = jb0 + it * BKV;
    const int s = it & 1;
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    if (it + 1 < nt) issue(j0 + BKV, s ^ 1);
    const char* ks = smem + s * STAGE;
    const char* vs = ks + BKV * RROW;
    const char* kts = vs + BKV * RROW;
    const bool skip = j0 > iw0 + 31 || iw0 - (j0 + BKV - 1) >= W || iw0 >= Tn;
    if (!skip) {
      floatx16 sc[1], dp[1];
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[0][r] = dp[0][r] = 0.f;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        sc[0] = MF::mma(row_frag<T, RROW>(ks, l32, k, g), qf[k], sc[0]);
        dp[0] = MF::mma(row_frag<T, RROW>(vs, l32, k, g), df[k], dp[0]);
      }
      const bool need_mask = (j0 + BKV - 1 > iw0) || (iw0 + 31 - j0 >= W);
      // invisible pairs get a -inf exponent (exp2 -> 0), branch-free
      if (need_mask) {
        const int dij = i - j0;   // i - j of accumulator row r is dij - acc_row(r, g)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = __builtin_fmaf(sc[0][r], c, -lse_i);
          sc[0][r] = visible_off(dij - acc_row(r, g), W) ? x : -INFINITY;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[0][r] = __builtin_fmaf(sc[0][r], c, -lse_i);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[0][r] = fast_exp2(sc[0][r]) * (dp[0][r] - D_i);
#pragma unroll
      for (int k = 0; k < PS; ++k) {
        const typename MF::frag sf = acc_frag<T, 1>(dp, k);
#pragma unroll
        for (int x = 0; x < DB; ++x) dq[x] = MF::mma(perm_frag<T, TROW>(kts, x * 32 + l32, k, g), sf, dq[x]);
      }
    }
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
  dim3 gkv((a.T + 127) / 128, a.Hkv, a.B);   // dK / dV: one work-group per key/value head
  if (part == 0) hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, DH, 32, 1>), gkv, dim3(256), 0, st, a);
  else if (part == 1) hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, DH, 32, 2>), gkv, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((attn_bwd_dq_kernel<T, DH>), g, dim3(256), 0, st, a);
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
