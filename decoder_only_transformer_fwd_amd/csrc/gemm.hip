// Tiled MFMA GEMM for gfx950 with fused epilogues.
//
// C[M,N] = alpha * sum_k A(m,k) B(n,k), where A is stored either K-contiguous
// ([M][K]) or M-contiguous ([K][M]), and B either K-contiguous ([N][K], a
// linear layer's weight) or N-contiguous ([K][N]).  These three layouts cover
// the forward (activation x weight^T), the input-gradient (grad x weight) and
// the weight-gradient (grad^T x activation) products of every linear layer.
//
// Structure: WGM x WGN waves (4 or 8) per work-group, each owning a
// (BM/WGM) x (BN/WGN) block of 32x32 MFMA tiles.  K advances in steps of 128
// bytes per row (64 bf16, 32 fp32).  A K-contiguous operand tile travels
// straight from global memory into LDS (buffer loads with the LDS bit, no
// registers); an M/N-contiguous one is loaded into registers, transposed in
// 16x16-byte blocks and written to LDS, so every MFMA fragment is one
// contiguous LDS read.  LDS is double-buffered with one barrier per K step;
// within a step the fragment reads for sub-step kk+1 are issued before the
// MFMAs of sub-step kk.  The MFMA takes the B tile as its first operand, so
// each lane's accumulators hold one output row and 4-wide runs of columns:
// epilogue stores are vectorised and row reductions stay in-lane.
//
// Work-group order is remapped so that the tiles one XCD (32 CUs sharing an
// L2) runs are neighbours, grouped along M so a band of A rows is reused from
// L2 by several column tiles.
#include "common.h"
#include "kernels.h"

#include <cstdio>

namespace gk {

constexpr uint32_t BUF_DWORD3 = 0x00020000u;   // raw buffer, 32-bit data format

// M/N-contiguous operand: blocks of 16 bytes (EPC elements) along the rows
// x EPC K-rows, transposed in registers, then stored K-contiguous in LDS.
template <int ES, int ROWS, int THREADS>
struct TransLoader {
  static constexpr int EPC = 16 / ES;
  static constexpr int NBLK_TOTAL = 8 * ROWS / EPC;
  static constexpr int NB = (NBLK_TOTAL + THREADS - 1) / THREADS;
  u32x4 reg[NB * EPC];

  // base: operand [K][ld]; rows r0.. of the tile are its contiguous index.
  __device__ __forceinline__ void load(const char* __restrict__ base, long ld, int r0, int nrows, int k0, int K,
                                       int t) {
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
      const int blk = t + bi * THREADS;
      const int kb = blk / (ROWS / EPC);
      const int rb = blk % (ROWS / EPC);
      const int gr = r0 + rb * EPC;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const int gk = k0 + kb * EPC + e;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (blk < NBLK_TOTAL && gk < K && gr < nrows) v = *(const u32x4*)(base + ((long)gk * ld + gr) * ES);
        reg[bi * EPC + e] = v;
      }
    }
  }

  __device__ __forceinline__ void store(char* __restrict__ lds, int t) const {
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
      const int blk = t + bi * THREADS;
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
          for (int w = 0; w < 4; ++w) o[w] = __builtin_amdgcn_perm(in[2 * w + 1][e2 >> 1], in[2 * w][e2 >> 1], sel);
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
};

// K-contiguous operand tile fetched straight from global memory into LDS.
// Each wave instruction fills 8 consecutive 128-byte LDS rows, lane l writing
// slot l%8 of row l/8; the swizzle is applied on the source side (the lane
// owning LDS slot p of row r fetches K-chunk p ^ swz(r)).  Rows past the
// operand and K-chunks past the end of the K range are outside the buffer's
// range and arrive as zeros.
template <int ES, int ROWS, int NWAVES, int RB>
struct DmaLoader {
  static constexpr int EPC = 16 / ES;
  static constexpr int CPR = RB / 16;             // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;            // rows per wave instruction
  static constexpr int RPW = ROWS / NWAVES;       // rows per wave
  static constexpr int PER_WAVE = RPW / RPI;
  static_assert(RPW % RPI == 0, "tile rows must be a multiple of the rows one wave instruction fills");
  __amdgpu_buffer_rsrc_t rsrc;
  int voff[PER_WAVE];
  int kel[PER_WAVE];

  __device__ __forceinline__ void init(const char* base, long ld, int r0, int nrows, int wave, int lane) {
    const long rows_left = nrows > r0 ? (long)(nrows - r0) : 0;
    long bytes = rows_left * ld * ES;
    if (bytes > 0x7FFFFFF0L) bytes = 0x7FFFFFF0L;
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(base + (long)r0 * ld * ES), 0, (int)bytes, BUF_DWORD3);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int r = wave * RPW + i * RPI + lane / CPR;
      const int c = (lane % CPR) ^ swz<RB>(r);
      voff[i] = (int)(r * ld * ES) + c * 16;
      kel[i] = c * EPC;
    }
  }
  __device__ __forceinline__ void issue(char* lds, int k0, int kend, int wave) const {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int off = (k0 + kel[i] < kend) ? voff[i] + k0 * ES : (int)0x80000000;
      dma16(rsrc, lds + (wave * RPW + i * RPI) * RB, off);
    }
  }
};

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nwg = tiles_m * tiles_n;
  // Hardware deals work-groups round-robin over 8 XCDs; give each XCD a
  // contiguous range of tile ids.
  int tile = wg;
  const int per = nwg / 8;
  if (per > 0 && wg < per * 8) tile = (wg & 7) * per + (wg >> 3);
  constexpr int GROUP_M = 8;
  const int group = tile / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in_group = tile % (GROUP_M * tiles_n);
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

template <typename TA, typename MF, int BM, int BN, int WGM, int WGN, int RB, int NS, bool A_KC, bool B_KC, int EPI,
          typename TC>
__global__ __launch_bounds__(64 * WGM * WGN, 1) void gemm_kernel(GemmArgs p) {
  constexpr int THREADS = 64 * WGM * WGN;
  constexpr int NW = WGM * WGN;
  constexpr int ES = sizeof(TA);
  constexpr int BK = RB / ES;         // K elements per step
  static_assert(NS == 2 || (A_KC && B_KC), "deeper pipelines need both operands on the direct-to-LDS path");
  static_assert(RB == 128 || (A_KC && B_KC), "register-transposed operands use 128-byte rows");
  constexpr int KM = MF::KM;
  constexpr int EPL = MF::EPL;
  constexpr int FB = EPL * ES;         // fragment bytes per lane
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int STAGE = (BM + BN) * RB;   // A tile, then B tile
  __shared__ __attribute__((aligned(16))) char smem[NS * STAGE];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int g = lane >> 5, l32 = lane & 31;

  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = (p.N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int kbeg = blockIdx.z * p.k_split;
  const int kend = min(p.K, kbeg + p.k_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  TransLoader<ES, BM, THREADS> la;
  TransLoader<ES, BN, THREADS> lb;
  DmaLoader<ES, BM, NW, RB> da;
  DmaLoader<ES, BN, NW, RB> db;
  const char* Ab = (const char*)p.A;
  const char* Bb = (const char*)p.B;
  if constexpr (A_KC) da.init(Ab, p.lda, m0, p.M, wave, lane);
  if constexpr (B_KC) db.init(Bb, p.ldb, n0, p.N, wave, lane);

  floatx16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto fetch = [&](int k0, int stage) {
    char* st = smem + stage * STAGE;
    if constexpr (A_KC) da.issue(st, k0, kend, wave);
    else la.load(Ab, p.lda, m0, p.M, k0, kend, t);
    if constexpr (B_KC) db.issue(st + BM * RB, k0, kend, wave);
    else lb.load(Bb, p.ldb, n0, p.N, k0, kend, t);
  };
  auto commit = [&](int stage) {   // register-staged operands into LDS
    char* st = smem + stage * STAGE;
    if constexpr (!A_KC) la.store(st, t);
    if constexpr (!B_KC) lb.store(st + BM * RB, t);
  };
  constexpr int KK = BK / KM;
  auto compute = [&](int stage) {
    const char* a_s = smem + stage * STAGE;
    const char* b_s = a_s + BM * RB;
    typename MF::frag af[2][MB], bfr[2][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i) lds_read<RB, FB>(a_s, wm * WM + i * 32 + l32, (g * EPL) * ES, &af[0][i]);
#pragma unroll
    for (int j = 0; j < NB; ++j) lds_read<RB, FB>(b_s, wn * WN + j * 32 + l32, (g * EPL) * ES, &bfr[0][j]);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cur = kk & 1;
      // fragment reads for the next sub-step go out before this sub-step's
      // MFMAs (the fences keep the scheduler from sinking them to their uses)
      if (kk + 1 < KK) {
        const int kb = ((kk + 1) * KM + g * EPL) * ES;
#pragma unroll
        for (int i = 0; i < MB; ++i) lds_read<RB, FB>(a_s, wm * WM + i * 32 + l32, kb, &af[cur ^ 1][i]);
#pragma unroll
        for (int j = 0; j < NB; ++j) lds_read<RB, FB>(b_s, wn * WN + j * 32 + l32, kb, &bfr[cur ^ 1][j]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = MF::mma(bfr[cur][j], af[cur][i], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if constexpr (NS == 2) {
    // Two stages: the next tile is requested at the top of a step and must
    // have landed (vmcnt 0) by the barrier that ends it.
    if (nk > 0) {
      fetch(kbeg, 0);
      commit(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int s = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) fetch(kbeg + (kt + 1) * BK, s ^ 1);
      compute(s);
      if (more) commit(s ^ 1);
      __builtin_amdgcn_s_waitcnt(0x0070);
      __syncthreads();
    }
  } else {
    // NS stages, all by direct-to-LDS loads: NS-1 steps are in flight.  Every
    // step issues its loads (past the K range they fetch zeros), so a fixed
    // vmcnt threshold waits for exactly the stage about to be consumed.
    constexpr int LPS = DmaLoader<ES, BM, NW, RB>::PER_WAVE + DmaLoader<ES, BN, NW, RB>::PER_WAVE;
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) fetch(kbeg + st * BK, st);
    for (int kt = 0; kt < nk; ++kt) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * LPS));
      __syncthreads();
      fetch(kbeg + (kt + NS - 1) * BK, (kt + NS - 1) % NS);
      compute(kt % NS);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);
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
        floatx4 v = {acc[i][j][4 * q] * alpha, acc[i][j][4 * q + 1] * alpha, acc[i][j][4 * q + 2] * alpha,
                     acc[i][j][4 * q + 3] * alpha};
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
          for (int e = 0; e < 4; ++e) {
            const float x = fmaxf(v[e], 0.f);
            r[e] = x * x;
          }
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
          for (int e = 0; e < 4; ++e) r[e] = (fast_exp2((v[e] - lse) * L2E) - (n + e == y ? 1.f : 0.f)) * p.beta;
          store4((TC*)p.C + off, r);
        } else if constexpr (EPI == EPI_PARTIAL) {
          store4(p.part + (long)blockIdx.z * p.M * p.N + (long)m * p.N + n, v);
        }
      }
    }
  }
}

// Sum split-K partials in split order: out[m, n] (+)= sum_z part[z, m, n].
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits, long mn,
                                                            float* __restrict__ out, int accumulate) {
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  floatx4 s = accumulate ? *(const floatx4*)(out + i) : floatx4{0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < splits; ++z) s += *(const floatx4*)(part + (long)z * mn + i);
  *(floatx4*)(out + i) = s;
}

// ------------------------------------------------------------------ dispatch

// Tile table: id -> (BM, BN, waves M x N, bytes per K step per row, stages).
struct TileCfg {
  int bm, bn, wgm, wgn, rb, ns;
};
static constexpr TileCfg TILES[] = {
    {256, 256, 2, 2, 128, 2},  // TILE_256x256
    {256, 128, 2, 2, 128, 2},  // TILE_256x128
    {128, 128, 2, 2, 128, 2},  // TILE_128x128
    {64, 64, 2, 2, 128, 2},    // TILE_64x64
    {256, 256, 2, 4, 128, 2},  // TILE_256x256_W8
    {256, 128, 2, 4, 128, 2},  // TILE_256x128_W8
    {256, 256, 2, 4, 64, 4},   // TILE_256x256_W8_S4
    {256, 256, 2, 2, 64, 4},   // TILE_256x256_S4
    {256, 128, 2, 4, 128, 3},  // TILE_256x128_W8_S3
    {128, 128, 2, 2, 64, 4},   // TILE_128x128_S4
};
int tile_bm(int tile) { return TILES[tile].bm; }
int tile_bn(int tile) { return TILES[tile].bn; }
int tile_wn(int tile) { return TILES[tile].bn / TILES[tile].wgn; }
bool tile_needs_kc(int tile) { return TILES[tile].ns > 2 || TILES[tile].rb != 128; }

void gemm_kernel_label(int dtype, int layout, int epi, int tile, char* buf, int n) {
  const TileCfg& c = TILES[tile];
  snprintf(buf, n, "gemm_kernel<%s, %d, %d, %d, %d, %d, %d, %s, %s, %d>", dtype == DT_BF16 ? "bf16" : "float", c.bm,
           c.bn, c.wgm, c.wgn, c.rb, c.ns, layout == LAYOUT_MN ? "false" : "true", layout == LAYOUT_KK ? "true" : "false",
           epi);
}

template <typename TA, typename MF, int T, bool AK, bool BK_, int EPI, typename TC>
static void launch_cfg(const GemmArgs& a, int splits, hipStream_t st) {
  constexpr TileCfg c = TILES[T];
  dim3 grid(((a.M + c.bm - 1) / c.bm) * ((a.N + c.bn - 1) / c.bn), 1, splits);
  hipLaunchKernelGGL((gemm_kernel<TA, MF, c.bm, c.bn, c.wgm, c.wgn, c.rb, c.ns, AK, BK_, EPI, TC>), grid,
                     dim3(64 * c.wgm * c.wgn), 0, st, a);
}

template <typename TA, typename MF, bool AK, bool BK_, int EPI, typename TC>
static void launch_tiles(const GemmArgs& a, int tile, int splits, hipStream_t st) {
  if constexpr (sizeof(TA) == 4) {
    if (tile == TILE_128x128) launch_cfg<TA, MF, TILE_128x128, AK, BK_, EPI, TC>(a, splits, st);
    else launch_cfg<TA, MF, TILE_64x64, AK, BK_, EPI, TC>(a, splits, st);
  } else {
#define GK_T(T) case T: launch_cfg<TA, MF, T, AK, BK_, EPI, TC>(a, splits, st); return;
    switch (tile) {
      GK_T(TILE_256x256) GK_T(TILE_256x128) GK_T(TILE_256x256_W8) GK_T(TILE_256x128_W8)
      default: break;
    }
    if constexpr (AK && BK_) {
      switch (tile) {
        GK_T(TILE_256x256_W8_S4) GK_T(TILE_256x256_S4) GK_T(TILE_256x128_W8_S3) GK_T(TILE_128x128_S4)
        default: break;
      }
    }
#undef GK_T
    launch_cfg<TA, MF, TILE_128x128, AK, BK_, EPI, TC>(a, splits, st);
  }
}

template <typename TA, typename MF, typename TC>
static int launch_epi(const GemmArgs& a, int layout, int epi, int tile, int splits, hipStream_t st) {
#define GK_CASE(L, AK, BK_, E)                                 \
  if (layout == L && epi == E) {                               \
    launch_tiles<TA, MF, AK, BK_, E, TC>(a, tile, splits, st); \
    return 0;                                                  \
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

int gemm_launch(const GemmArgs& a, int dtype, int layout, int epi, int tile, int splits, hipStream_t st) {
  if (dtype == DT_BF16) return launch_epi<bf16, Mfma<bf16>, bf16>(a, layout, epi, tile, splits, st);
  if (dtype == DT_F32) return launch_epi<float, Mfma<float>, float>(a, layout, epi, tile, splits, st);
  return -1;
}

void splitk_reduce(const float* part, int splits, long mn, float* out, int accumulate, hipStream_t st) {
  const long n4 = (mn + 3) / 4;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, part, splits, mn,
                     out, accumulate);
}

}  // namespace gk
