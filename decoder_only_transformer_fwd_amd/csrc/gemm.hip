// Tiled MFMA GEMM for gfx950 with fused epilogues.
//
// C[M,N] = alpha * sum_k A(m,k) B(n,k), where A is stored either K-contiguous
// ([M][K], "row") or M-contiguous ([K][M]), and B either K-contiguous ([N][K],
// a linear layer's weight) or N-contiguous ([K][N]).  These three layouts
// cover the forward (activation x weight^T), the input-gradient
// (grad x weight) and the weight-gradient (grad^T x activation) products of
// every linear layer of the step.
//
// Structure: 256 threads = 4 waves in a 2x2 arrangement; each wave owns a
// (BM/2)x(BN/2) block of 32x32 MFMA tiles.  K advances in steps of 128 bytes
// per row (64 bf16, 32 fp32, 128 fp8).  Global tiles are fetched into
// registers one step ahead, written to a double-buffered, XOR-swizzled LDS
// tile, and consumed by MFMA with one barrier per step.  An M-contiguous or
// N-contiguous operand is transposed in registers (blocks of 16 bytes x 16
// bytes) on its way into LDS so that every MFMA fragment is a contiguous LDS
// read.  The MFMA is issued with the B tile as its first operand, so each
// lane's accumulators hold one output row and 4-wide runs of columns, which
// keeps every epilogue store vectorised and every row reduction in-lane.
//
// Work-group order is remapped so that the tiles one XCD (a group of 32 CUs
// with its own L2) runs are neighbours, and grouped along M so that a band of
// A rows is reused from L2 by several column tiles.
#include "common.h"
#include "kernels.h"

namespace gk {

template <int ES, int ROWS, bool KC>
struct TileLoader {
  static constexpr int EPC = 16 / ES;                      // elements per 16 bytes
  static constexpr int NBLK_TOTAL = 8 * ROWS / EPC;        // MN-contiguous blocks
  static constexpr int NREG = KC ? (ROWS * 8) / 256 : ((NBLK_TOTAL + 255) / 256) * EPC;
  u32x4 reg[NREG];

  // base: operand base pointer; ld: leading dimension in elements; r0/nrows:
  // first row of the tile and the operand's row count (M or N); k0/K: the
  // same along K.
  __device__ __forceinline__ void load(const char* __restrict__ base, long ld, int r0, int nrows,
                                       int k0, int K, int t) {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NREG; ++i) {
        const int row = i * 32 + (t >> 3);
        const int c = t & 7;
        const int gr = r0 + row;
        const int gk = k0 + c * EPC;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (gr < nrows && gk < K) v = *(const u32x4*)(base + ((long)gr * ld + gk) * ES);
        reg[i] = v;
      }
    } else {
#pragma unroll
      for (int bi = 0; bi < NREG / EPC; ++bi) {
        const int blk = t + bi * 256;
        const int kb = blk / (ROWS / EPC);
        const int rb = blk % (ROWS / EPC);
        const int gr = r0 + rb * EPC;
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const int gk = k0 + kb * EPC + e;
          u32x4 v = {0u, 0u, 0u, 0u};
          if (blk < NBLK_TOTAL && gk < K && gr < nrows)
            v = *(const u32x4*)(base + ((long)gk * ld + gr) * ES);
          reg[bi * EPC + e] = v;
        }
      }
    }
  }

  __device__ __forceinline__ void store(char* __restrict__ lds, int t) const {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NREG; ++i) {
        const int row = i * 32 + (t >> 3);
        *(u32x4*)(lds + lds_off<128>(row, (t & 7) * 16)) = reg[i];
      }
    } else {
#pragma unroll
      for (int bi = 0; bi < NREG / EPC; ++bi) {
        const int blk = t + bi * 256;
        if (blk >= NBLK_TOTAL) continue;
        const int kb = blk / (ROWS / EPC);
        const int rb = blk % (ROWS / EPC);
        const u32x4* in = &reg[bi * EPC];
#pragma unroll
        for (int e2 = 0; e2 < EPC; ++e2) {
          u32x4 o;
          if constexpr (ES == 4) {
#pragma unroll
            for (int w = 0; w < 4; ++w) o[w] = in[w][e2];
          } else if constexpr (ES == 2) {
            const uint32_t sel = (e2 & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
            for (int w = 0; w < 4; ++w)
              o[w] = __builtin_amdgcn_perm(in[2 * w + 1][e2 >> 1], in[2 * w][e2 >> 1], sel);
          } else {
            const int sh = (e2 & 3) * 8;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              uint32_t x = 0;
#pragma unroll
              for (int q = 0; q < 4; ++q) x |= ((in[4 * w + q][e2 >> 2] >> sh) & 0xFFu) << (8 * q);
              o[w] = x;
            }
          }
          *(u32x4*)(lds + lds_off<128>(rb * EPC + e2, kb * 16)) = o;
        }
      }
    }
  }
};

__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nwg = tiles_m * tiles_n;
  // XCD remap: hardware deals work-groups round-robin over 8 XCDs; give each
  // XCD a contiguous range of tile ids.
  int tile = wg;
  const int per = nwg / 8;
  if (per > 0 && wg < per * 8) tile = (wg & 7) * per + (wg >> 3);
  // Grouped order along M.
  constexpr int GROUP_M = 8;
  const int group = tile / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in_group = tile % (GROUP_M * tiles_n);
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

template <typename TA, typename MF, int BM, int BN, bool A_KC, bool B_KC, int EPI, typename TC>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmArgs p) {
  constexpr int ES = sizeof(TA);
  constexpr int BK = 128 / ES;
  constexpr int KM = MF::KM;
  constexpr int EPL = MF::EPL;
  constexpr int FB = EPL * ES;         // fragment bytes per lane
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MB = WM / 32, NB = WN / 32;

  constexpr int STAGE = (BM + BN) * 128;   // A tile, then B tile
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 5, l32 = lane & 31;

  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int kbeg = blockIdx.z * p.k_split;
  const int kend = min(p.K, kbeg + p.k_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  TileLoader<ES, BM, A_KC> la;
  TileLoader<ES, BN, B_KC> lb;
  const char* Ab = (const char*)p.A;
  const char* Bb = (const char*)p.B;

  floatx16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (nk > 0) {
    la.load(Ab, p.lda, m0, p.M, kbeg, kend, t);
    lb.load(Bb, p.ldb, n0, p.N, kbeg, kend, t);
    la.store(smem, t);
    lb.store(smem + BM * 128, t);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int s = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = kbeg + (kt + 1) * BK;
      la.load(Ab, p.lda, m0, p.M, k0, kend, t);
      lb.load(Bb, p.ldb, n0, p.N, k0, kend, t);
    }
    const char* a_s = smem + s * STAGE;
    const char* b_s = a_s + BM * 128;
#pragma unroll
    for (int kk = 0; kk < BK / KM; ++kk) {
      typename MF::frag af[MB], bfr[NB];
      const int kb = (kk * KM + g * EPL) * ES;
#pragma unroll
      for (int i = 0; i < MB; ++i) lds_read<128, FB>(a_s, wm * WM + i * 32 + l32, kb, &af[i]);
#pragma unroll
      for (int j = 0; j < NB; ++j) lds_read<128, FB>(b_s, wn * WN + j * 32 + l32, kb, &bfr[j]);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = MF::mma(bfr[j], af[i], acc[i][j]);
    }
    if (more) {
      la.store(smem + (s ^ 1) * STAGE, t);
      lb.store(smem + (s ^ 1) * STAGE + BM * 128, t);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ epilogue
  const float alpha = p.alpha;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = m0 + wm * WM + i * 32 + l32;
    const bool mok = m < p.M;
    if constexpr (EPI == EPI_XENT_FWD) {
      // per-row partial (max, sum of exp) over this wave's WN columns
      const int ncol0 = n0 + wn * WN;
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = ncol0 + j * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (n < p.N) mx = fmaxf(mx, acc[i][j][r] * alpha);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float se = 0.f;
      const float L2E = 1.4426950408889634f;
      const int y = mok ? ((const int*)p.aux)[m] : -1;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int n = ncol0 + j * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          const float v = acc[i][j][r] * alpha;
          if (n < p.N) se += fast_exp2((v - mx) * L2E);
          if (n == y) p.tgt[m] = v;
        }
      se += __shfl_xor(se, 32, 64);
      const int blk = ncol0 / WN;
      if (mok && g == 0 && ncol0 < p.N) {
        p.part[((long)m * p.nblk + blk) * 2 + 0] = mx;
        p.part[((long)m * p.nblk + blk) * 2 + 1] = se;
      }
      continue;
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * g;
        if (!mok || n >= p.N) continue;
        floatx4 v = {acc[i][j][4 * q] * alpha, acc[i][j][4 * q + 1] * alpha,
                     acc[i][j][4 * q + 2] * alpha, acc[i][j][4 * q + 3] * alpha};
        const long off = (long)m * p.ldc + n;
        if constexpr (EPI == EPI_STORE) {
          store4((TC*)p.C + off, v);
        } else if constexpr (EPI == EPI_STORE_F32) {
          store4((float*)p.C + off, v);
        } else if constexpr (EPI == EPI_ACCUM_F32) {
          float* c = (float*)p.C + off;
          store4(c, load4(c) + v);
        } else if constexpr (EPI == EPI_RELU2) {
          store4((TC*)p.C + off, v);
          floatx4 r;
#pragma unroll
          for (int e = 0; e < 4; ++e) { const float x = fmaxf(v[e], 0.f); r[e] = x * x; }
          store4((TC*)p.C2 + off, r);
        } else if constexpr (EPI == EPI_DRELU2) {
          const floatx4 u = load4((const TC*)p.aux + off);
          floatx4 r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = v[e] * 2.f * fmaxf(u[e], 0.f);
          store4((TC*)p.C + off, r);
        } else if constexpr (EPI == EPI_XENT_BWD) {
          const float L2E = 1.4426950408889634f;
          const float lse = p.auxf[m];
          const int y = ((const int*)p.aux)[m];
          floatx4 r;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            r[e] = (fast_exp2((v[e] - lse) * L2E) - (n + e == y ? 1.f : 0.f)) * p.beta;
          store4((TC*)p.C + off, r);
        } else if constexpr (EPI == EPI_PARTIAL) {
          store4(p.part + (long)blockIdx.z * p.M * p.N + (long)m * p.N + n, v);
        }
      }
    }
  }
}

// Sum split-K partials in split order: out[m, n] (+)= sum_z part[z, m, n].
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits,
                                                            long mn, float* __restrict__ out,
                                                            int accumulate) {
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  floatx4 s = accumulate ? *(const floatx4*)(out + i) : floatx4{0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < splits; ++z) s += *(const floatx4*)(part + (long)z * mn + i);
  *(floatx4*)(out + i) = s;
}

// ------------------------------------------------------------------ dispatch

template <typename TA, typename MF, int BM, int BN, bool AK, bool BK_, int EPI, typename TC>
static void launch_cfg(const GemmArgs& a, int splits, hipStream_t st) {
  dim3 grid(((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN), 1, splits);
  hipLaunchKernelGGL((gemm_kernel<TA, MF, BM, BN, AK, BK_, EPI, TC>), grid, dim3(256), 0, st, a);
}

template <typename TA, typename MF, bool AK, bool BK_, int EPI, typename TC>
static void launch_tiles(const GemmArgs& a, int tile, int splits, hipStream_t st) {
  if constexpr (sizeof(TA) == 4) {
    if (tile == TILE_128x128) launch_cfg<TA, MF, 128, 128, AK, BK_, EPI, TC>(a, splits, st);
    else launch_cfg<TA, MF, 64, 64, AK, BK_, EPI, TC>(a, splits, st);
  } else {
    if (tile == TILE_256x256) launch_cfg<TA, MF, 256, 256, AK, BK_, EPI, TC>(a, splits, st);
    else if (tile == TILE_256x128) launch_cfg<TA, MF, 256, 128, AK, BK_, EPI, TC>(a, splits, st);
    else launch_cfg<TA, MF, 128, 128, AK, BK_, EPI, TC>(a, splits, st);
  }
}

template <typename TA, typename MF, typename TC>
static int launch_epi(const GemmArgs& a, int layout, int epi, int tile, int splits, hipStream_t st) {
#define GK_CASE(L, AK, BK_, E)                                             \
  if (layout == L && epi == E) {                                           \
    launch_tiles<TA, MF, AK, BK_, E, TC>(a, tile, splits, st);             \
    return 0;                                                              \
  }
  // forward products: activation [M][K] x weight [N][K]
  GK_CASE(LAYOUT_KK, true, true, EPI_STORE)
  GK_CASE(LAYOUT_KK, true, true, EPI_ACCUM_F32)
  GK_CASE(LAYOUT_KK, true, true, EPI_RELU2)
  GK_CASE(LAYOUT_KK, true, true, EPI_XENT_FWD)
  GK_CASE(LAYOUT_KK, true, true, EPI_XENT_BWD)
  GK_CASE(LAYOUT_KK, true, true, EPI_STORE_F32)
  // input gradients: grad [M][K] x weight [K][N]
  GK_CASE(LAYOUT_KN, true, false, EPI_STORE)
  GK_CASE(LAYOUT_KN, true, false, EPI_STORE_F32)
  GK_CASE(LAYOUT_KN, true, false, EPI_DRELU2)
  GK_CASE(LAYOUT_KN, true, false, EPI_PARTIAL)
  // weight gradients: grad [K][M] x activation [K][N]
  GK_CASE(LAYOUT_MN, false, false, EPI_STORE_F32)
  GK_CASE(LAYOUT_MN, false, false, EPI_PARTIAL)
#undef GK_CASE
  return -1;
}

int gemm_launch(const GemmArgs& a, int dtype, int layout, int epi, int tile, int splits,
                hipStream_t st) {
  if (dtype == DT_BF16) return launch_epi<bf16, Mfma<bf16>, bf16>(a, layout, epi, tile, splits, st);
  if (dtype == DT_F32) return launch_epi<float, Mfma<float>, float>(a, layout, epi, tile, splits, st);
  return -1;
}

void splitk_reduce(const float* part, int splits, long mn, float* out, int accumulate,
                   hipStream_t st) {
  const long n4 = (mn + 3) / 4;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, part,
                     splits, mn, out, accumulate);
}

}  // namespace gk
