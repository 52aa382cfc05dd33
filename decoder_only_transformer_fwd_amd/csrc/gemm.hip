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
// bytes per row (64 bf16, 32 fp32).  Operand tiles travel straight from global
// memory into LDS (buffer loads with the LDS bit, no registers): a
// K-contiguous tile is read back as one contiguous 16-byte fragment per lane,
// a 16-bit M/N-contiguous tile with two transposing LDS reads per fragment.
// 32-bit M/N-contiguous operands (fp32 workloads) are instead transposed in
// registers on their way into LDS.  LDS is double-buffered with one barrier per K step;
// within a step the fragment reads for sub-step kk+1 are issued before the
// MFMAs of sub-step kk.  The MFMA takes the B tile as its first operand, so
// each lane's accumulators hold one output row and 4-wide runs of columns:
// row reductions (the cross-entropy statistics) stay in-lane, and the other
// epilogues stage 32-row blocks through LDS to load and store whole rows.
//
// Work-group order is remapped so that the tiles one XCD (32 CUs sharing an
// L2) runs are neighbours, grouped along M so a band of A rows is reused from
// L2 by several column tiles.
#include "common.h"
#include "kernels.h"

#include <cstdio>

namespace gk {


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
    rsrc = uniform_rsrc(base + (long)r0 * ld * ES, (int)bytes);
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

// M/N-contiguous 16-bit operand ([K][rows]) copied row-for-row into LDS by
// direct-to-LDS loads: the tile holds BK K-rows of ROWS*2 bytes, 16-byte
// chunk c of K-row k at slot c ^ swz_tr(k).  Each stage re-bases the buffer
// at K-row k0 so offsets stay small, and K-rows at or past the end of the K
// range fall outside the buffer and arrive as zeros.  MFMA fragments are then
// assembled with transposing LDS reads (tr_frag).
template <int RBT>
__device__ __forceinline__ int swz_tr(int k) {
  return (4 * (k & 3)) & (RBT / 16 - 1);
}

template <int ES, int ROWS, int NWAVES, int BK>
struct DmaTrLoader {
  static constexpr int RBT = ROWS * ES;            // bytes per K-row in LDS
  static constexpr int TOTAL = BK * RBT / 1024;    // wave instructions per stage
  static constexpr int PER_WAVE = TOTAL / NWAVES;
  static_assert(TOTAL % NWAVES == 0 && RBT <= 1024 && 1024 % RBT == 0, "tile shape");
  const char* base;     // operand + r0 columns
  long ldb;             // leading dimension in bytes
  long col_bytes_left;  // bytes of a K-row from column r0 to the end of the row
  int voff[PER_WAVE];   // offset of this lane's chunk relative to K-row k0
  int krow[PER_WAVE];

  __device__ __forceinline__ void init(const char* op, long ld, int r0, int wave, int lane) {
    base = op + (long)r0 * ES;
    ldb = ld * ES;
    col_bytes_left = ldb - (long)r0 * ES;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int pos = (wave * PER_WAVE + i) * 1024 + lane * 16;
      const int k = pos / RBT, p = (pos % RBT) / 16;
      krow[i] = k;
      voff[i] = (int)(k * ldb) + ((p ^ swz_tr<RBT>(k)) << 4);
    }
  }
  __device__ __forceinline__ void issue(char* lds, int k0, int kend, int wave) const {
    long bytes = (long)(kend - k0 - 1) * ldb + col_bytes_left;
    if (bytes < 0) bytes = 0;
    if (bytes > 0x7FFFFFF0L) bytes = 0x7FFFFFF0L;
    const __amdgpu_buffer_rsrc_t r = uniform_rsrc(base + (long)k0 * ldb, (int)bytes);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i)
      dma16(r, lds + (wave * PER_WAVE + i) * 1024, k0 + krow[i] < kend ? voff[i] : (int)0x80000000);
  }
};

// Fragment of 32 rows (M or N indices rb..rb+31) x 16 K values from a
// [K][rows] tile: lane (row rb + l%32, group g) gets K-rows kbase + 8g + e,
// e = 0..7 -- the same K order as a K-contiguous fragment.
template <int RBT>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int rb, int kbase, int lane) {
  const int s = lane & 15, q = (lane >> 4) & 1, g = lane >> 5;
  const int byte = (rb + 16 * q + 4 * (s & 3)) * 2;
  shortx4 v[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = kbase + 8 * g + 4 * h + (s >> 2);
    v[h] = lds_read_tr16(tile + k * RBT + (((byte >> 4) ^ swz_tr<RBT>(k)) << 4) + (byte & 15));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Tiles are taken in groups of GROUP_M rows of tiles (about 1024 rows of A,
// measured best at the step's shapes) across all tile columns.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int wg, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int nwg = tiles_m * tiles_n;
  // Hardware deals work-groups round-robin over 8 XCDs; give each XCD a
  // contiguous range of tile ids.
  int tile = wg;
  const int per = nwg / 8;
  if (per > 0 && wg < per * 8) tile = (wg & 7) * per + (wg >> 3);
  const int group = tile / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in_group = tile % (GROUP_M * tiles_n);
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Rotary embedding + QK RMS norm of one 32-row block of the fused QKV
// product (EPI_ROPE_QKN), in the accumulators of a wave that owns one whole
// head of 128 columns: lane (l32, g) holds row l32 of the block and columns
// j*32 + 8q + 4g + e (j < 4), so the rotation pair (x[i], x[i+64]) of each of
// its values is in the same lane (j and j+2), and the other half of the
// head's squares sits in lane l32 ^ 32.  q and k heads: rotate each pair by
// the token's angle, scale by rstd = 1/sqrt(mean square + eps) (written by
// the g = 0 lanes); v heads pass through.  Then the wave writes its 32
// tokens x 128 dimensions transposed into its own LDS region `wr` and from
// there 16-byte runs of 8 tokens into the transposed copy.  The accumulators
// leave holding the results (alpha applied); the caller stores them
// row-major through the same region.  No work-group barrier.
__device__ __forceinline__ void rope_qkn_block(const GemmArgs& p, floatx16 (&acc)[4], char* wr, int lane,
                                               int mrow0, int hcol, float alpha) {
  const int g = lane >> 5, l32 = lane & 31;
  if (hcol >= p.N) return;                    // wave-uniform
  const int H = p.nH, Hkv = p.nHkv;
  const int slot = hcol >> 7;                 // head slot in the row
  const int part = slot < H ? 0 : slot < H + Hkv ? 1 : 2;
  const int m = mrow0 + l32;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] *= alpha;
  if (part < 2) {
    const int tok = m % p.seqT;
    floatx4 c[2][4], sn[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[j][q] = *(const floatx4*)(p.rope_cos + (long)tok * 64 + j * 32 + 8 * q + 4 * g);
        sn[j][q] = *(const floatx4*)(p.rope_sin + (long)tok * 64 + j * 32 + 8 * q + 4 * g);
      }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x1 = acc[j][4 * q + e], x2 = acc[j + 2][4 * q + e];
          const float r1 = x1 * c[j][q][e] - x2 * sn[j][q][e];
          const float r2 = x1 * sn[j][q][e] + x2 * c[j][q][e];
          ss += r1 * r1 + r2 * r2;
          acc[j][4 * q + e] = r1;
          acc[j + 2][4 * q + e] = r2;
        }
    ss += __shfl_xor(ss, 32, 64);
    const float r = 1.0f / sqrtf(ss / 128.f + p.eps);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] *= r;
    if (g == 0 && m < p.M) p.rqk[(long)m * (H + Hkv) + slot] = r;
  }
  constexpr int LDT = 40;   // bf16 per transposed row: 32 tokens + padding (80 bytes, 16-byte aligned)
  bf16* tb = (bf16*)wr;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) tb[(j * 32 + 8 * q + 4 * g + e) * LDT + l32] = (bf16)acc[j][4 * q + e];
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  const int hh = part == 0 ? slot : part == 1 ? slot - H : slot - H - Hkv;
  const int nh = part == 0 ? H : Hkv;
  bf16* dst = (bf16*)(part == 0 ? p.qT : part == 1 ? p.kT : p.vT);
#pragma unroll
  for (int ps = 0; ps < 8; ++ps) {
    const int dim = ps * 16 + (lane >> 2), tq = (lane & 3) * 8;
    const int mf = mrow0 + tq;               // 8 tokens of one sequence (seqT % 64 == 0)
    if (mf < p.M) {
      const int b = mf / p.seqT, t = mf % p.seqT;
      const u32x4 v = *(const u32x4*)(tb + dim * LDT + tq);
      *(u32x4*)(dst + (((long)b * nh + hh) * 128 + dim) * p.seqT + t) = v;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // transposed reads done before the region is rewritten
  __builtin_amdgcn_wave_barrier();
}

template <typename TA, typename MF, int BM, int BN, int WGM, int WGN, int RB, int NS, bool A_KC, bool B_KC, int EPI,
          typename TC, bool PP, bool BATCHED>
// Two waves per SIMD except for the 4-wave tiles whose accumulators need the
// whole register file.
__global__ __launch_bounds__(64 * WGM * WGN, (WGM * WGN == 4 && BM * BN >= 256 * 128) ? 1 : 2) void gemm_kernel(GemmArgs p) {
  // symmetric variants: the base epilogue E, upper-triangle tiles, mirrored stores
  constexpr bool SYM = EPI == EPI_STORE_SYM || EPI == EPI_AXPBY_SYM;
  constexpr int E = EPI == EPI_STORE_SYM ? EPI_STORE : EPI == EPI_AXPBY_SYM ? EPI_AXPBY : EPI;
  static_assert(!SYM || BATCHED, "symmetric products are batched launches");
  // batched products: this work-group's member of the batch
  if constexpr (BATCHED) {
    const long bz = blockIdx.y;
    p.A = (const char*)p.A + bz * p.bsA * (long)sizeof(TA);
    p.B = (const char*)p.B + bz * p.bsB * (long)sizeof(TA);
    p.C = (char*)p.C + bz * p.bsC * (long)sizeof(TC);
    p.aux = (const char*)p.aux + bz * p.bsC * (long)sizeof(TC);
  }
  constexpr int THREADS = 64 * WGM * WGN;
  constexpr int NW = WGM * WGN;
  constexpr int ES = sizeof(TA);
  constexpr int BK = RB / ES;         // K elements per step
  // 16-bit M/N-contiguous operands take the direct-to-LDS path with
  // transposing fragment reads; 32-bit ones are transposed in registers.
  constexpr bool A_TR = !A_KC && ES == 2, B_TR = !B_KC && ES == 2;
  constexpr bool A_REG = !A_KC && !A_TR, B_REG = !B_KC && !B_TR;
  static_assert(NS == 2 || (!A_REG && !B_REG), "deeper pipelines need both operands on the direct-to-LDS path");
  static_assert(RB == 128 || (A_KC && B_KC) || PP, "transposed operands use 128-byte K steps");
  static_assert(!PP || (WGM * WGN == 8 && WGM % 2 == 0 && !A_REG && !B_REG), "ping-pong: two groups of four waves");
  // every wave issues its share of the global->LDS copies (in the ping-pong
  // schedule, each group during its own memory phase: spreading the copies
  // over 8 waves and two issue points per step keeps more of them in flight
  // than one group issuing all of them)
  constexpr int LW = WGM * WGN;
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
  if constexpr (SYM) {
    // tiles on or above the diagonal, row by row
    int idx = blockIdx.x;
    tm = 0;
    while (idx >= tiles_n - tm) idx -= tiles_n - tm++;
    tn = tm + idx;
  } else {
    tile_coords<(BM >= 1024 ? 1 : 1024 / BM)>(blockIdx.x, tiles_m, tiles_n, tm, tn);
  }
  const int m0 = tm * BM, n0 = tn * BN;

  const int kbeg = blockIdx.z * p.k_split;
  const int kend = min(p.K, kbeg + p.k_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  TransLoader<ES, BM, THREADS> la;
  TransLoader<ES, BN, THREADS> lb;
  DmaLoader<ES, BM, LW, RB> da;
  DmaLoader<ES, BN, LW, RB> db;
  DmaTrLoader<ES, BM, LW, BK> ta;
  DmaTrLoader<ES, BN, LW, BK> tb;
  const char* Ab = (const char*)p.A;
  const char* Bb = (const char*)p.B;
  if (wave < LW) {
    if constexpr (A_KC) da.init(Ab, p.lda, m0, p.M, wave, lane);
    if constexpr (B_KC) db.init(Bb, p.ldb, n0, p.N, wave, lane);
    if constexpr (A_TR) ta.init(Ab, p.lda, m0, wave, lane);
    if constexpr (B_TR) tb.init(Bb, p.ldb, n0, wave, lane);
  }

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
    else if constexpr (A_TR) ta.issue(st, k0, kend, wave);
    else la.load(Ab, p.lda, m0, p.M, k0, kend, t);
    if constexpr (B_KC) db.issue(st + BM * RB, k0, kend, wave);
    else if constexpr (B_TR) tb.issue(st + BM * RB, k0, kend, wave);
    else lb.load(Bb, p.ldb, n0, p.N, k0, kend, t);
  };
  auto commit = [&](int stage) {   // register-staged operands into LDS
    char* st = smem + stage * STAGE;
    if constexpr (A_REG) la.store(st, t);
    if constexpr (B_REG) lb.store(st + BM * RB, t);
  };
  // fragment of 32 A rows / B columns at K sub-step kk
  auto frag_a = [&](const char* a_s, int i, int kk, typename MF::frag* out) {
    if constexpr (A_TR) *out = tr_frag<BM * ES>(a_s, wm * WM + i * 32, kk * KM, lane);
    else lds_read<RB, FB>(a_s, wm * WM + i * 32 + l32, (kk * KM + g * EPL) * ES, out);
  };
  auto frag_b = [&](const char* b_s, int j, int kk, typename MF::frag* out) {
    if constexpr (B_TR) *out = tr_frag<BN * ES>(b_s, wn * WN + j * 32, kk * KM, lane);
    else lds_read<RB, FB>(b_s, wn * WN + j * 32 + l32, (kk * KM + g * EPL) * ES, out);
  };
  constexpr int KK = BK / KM;
  static_assert(KK % 2 == 0, "fragment double-buffering assumes an even number of K sub-steps");
  // fragment buffers: two, double-buffering the sub-steps, or in the
  // ping-pong schedule one per sub-step of a phase (two sub-steps)
  constexpr int PSUB = 2;             // ping-pong: K sub-steps per phase
  constexpr int FBUF = PP ? PSUB : 2;
  typename MF::frag af[FBUF][MB], bfr[FBUF][NB];
  auto read_frags = [&](const char* a_s, int kk, int buf) {
#pragma unroll
    for (int i = 0; i < MB; ++i) frag_a(a_s, i, kk, &af[buf][i]);
#pragma unroll
    for (int j = 0; j < NB; ++j) frag_b(a_s + BM * RB, j, kk, &bfr[buf][j]);
  };
  auto mma_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = MF::mma(bfr[buf][j], af[buf][i], acc[i][j]);
  };
  // Sub-steps 0 .. KK-2 of a stage whose sub-step-0 fragments are already in
  // buffer 0; the fragment reads for the next sub-step go out before this
  // sub-step's MFMAs (the fences keep the scheduler from sinking them to
  // their uses).  Sub-step KK-1's fragments are left in buffer 1.
  auto compute_head = [&](int stage) {
    const char* a_s = smem + stage * STAGE;
#pragma unroll
    for (int kk = 0; kk + 1 < KK; ++kk) {
      read_frags(a_s, kk + 1, (kk + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      mma_step(kk & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto compute = [&](int stage) {
    read_frags(smem + stage * STAGE, 0, 0);
    compute_head(stage);
    mma_step(1);
  };

  if constexpr (PP) {
    // Ping-pong: waves 0-3 (group 0, output rows 0..BM/2-1) and 4-7 (group 1,
    // the other half) share the SIMDs pairwise and run one phase apart.  While
    // one group multiplies fragments already in its registers, the other
    // reads the next phase's fragments from LDS and, at the start of a step,
    // issues its half of the global->LDS copies for the stage NS-1 steps
    // ahead; each SIMD's matrix unit thus alternates between the two groups'
    // MFMA blocks.  Every phase ends with a barrier of all 8 waves; group 1
    // starts one barrier late and group 0 ends with one extra barrier.
    //
    // Copy completion: stage s is first read by group 0 in its memory phase
    // of step s, after the barrier that ends group 0's compute phase and
    // group 1's memory phase of step s-1.  Each group therefore waits for
    // its copies of stage s at the end of that phase, leaving the two
    // younger stages (NS-2 of them) in flight.
    constexpr int LPS = (A_KC ? DmaLoader<ES, BM, LW, RB>::PER_WAVE : DmaTrLoader<ES, BM, LW, BK>::PER_WAVE) +
                        (B_KC ? DmaLoader<ES, BN, LW, RB>::PER_WAVE : DmaTrLoader<ES, BN, LW, BK>::PER_WAVE);
    const bool g0 = wave < NW / 2;
    static_assert(KK % PSUB == 0, "whole phases per K step");
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) fetch(kbeg + st * BK, st);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * LPS));
    barrier_only();
    if (!g0) barrier_only();
    for (int kt = 0; kt < nk; ++kt) {
      const char* a_s = smem + (kt % NS) * STAGE;
#pragma unroll
      for (int ph = 0; ph < KK / PSUB; ++ph) {
        // memory phase: this phase's fragments into registers (and, at the
        // start of a step, the copies for the stage NS-1 steps ahead)
#pragma unroll
        for (int u = 0; u < PSUB; ++u) read_frags(a_s, ph * PSUB + u, u);
        if (ph == 0) fetch(kbeg + (kt + NS - 1) * BK, (kt + NS - 1) % NS);
        if (ph == KK / PSUB - 1 && !g0)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * LPS));   // group 1's copies of the next stage
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): fragments are in registers
        barrier_only();
        // compute phase
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < PSUB; ++u) mma_step(u);
        __builtin_amdgcn_sched_barrier(0);
        if (ph == KK / PSUB - 1 && g0)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * LPS));   // group 0's copies of the next stage
        barrier_only();
      }
    }
    if (g0) barrier_only();
    __builtin_amdgcn_s_waitcnt(0x0070);
  } else if constexpr (NS == 2) {
    // Two stages: the next tile is requested at the top of a step and must
    // have landed (vmcnt 0) by the barrier that ends it.  (Moving the last
    // sub-step's MFMAs behind that barrier, to overlap the next stage's first
    // fragment reads, measured slower for the fp8 tiles and no faster for
    // bf16.)
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
    constexpr int LPS = (A_KC ? DmaLoader<ES, BM, NW, RB>::PER_WAVE : DmaTrLoader<ES, BM, NW, BK>::PER_WAVE) +
                        (B_KC ? DmaLoader<ES, BN, NW, RB>::PER_WAVE : DmaTrLoader<ES, BN, NW, BK>::PER_WAVE);
#pragma unroll
    for (int st = 0; st < NS - 1; ++st) fetch(kbeg + st * BK, st);
    for (int kt = 0; kt < nk; ++kt) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * LPS));
      barrier_only();
      fetch(kbeg + (kt + NS - 1) * BK, (kt + NS - 1) % NS);
      compute(kt % NS);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);
  }

  // ------------------------------------------------------------ epilogue
  float alpha = p.alpha;
  if constexpr (ES == 1) alpha = alpha / p.scale_a[0] / p.scale_b[0];
  static_assert(E != EPI_ROPE_QKN || (WN == 128 && ES == 2), "rotary epilogue: one head of 128 per wave");
  if constexpr (EPI == EPI_XENT_FWD) {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int m = m0 + wm * WM + i * 32 + l32;
      const bool mok = m < p.M;
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
    }
  } else {
    // Each wave stages its 32-row blocks of fp32 results through its own LDS
    // region and reads them back as whole rows, so that every global load and
    // store of the epilogue covers contiguous row segments (64 consecutive
    // columns per 16 lanes).
    constexpr int RBY = WN * 4;              // bytes per staged row
    constexpr int LPR = WN / 4;              // lanes per staged row (16 bytes each)
    constexpr int RPS = 64 / LPR;            // rows per read step
    static_assert(NW * 32 * RBY <= NS * STAGE, "epilogue staging must fit in the operand stages");
    char* region = smem + wave * 32 * RBY;
    __syncthreads();   // every wave is done with the operand stages
    // Epilogues that read C (accumulate) or the saved pre-activation
    // (dReLU^2) load those values for a whole 32-row block up front: the
    // compiler cannot move a load above an earlier store that may alias it.
    constexpr bool PRELOAD = E == EPI_ACCUM_F32 || E == EPI_DRELU2 || E == EPI_AXPBY;
    float amax_acc = 0.f;   // RELU2 / DRELU2: largest |stored activation|
    const float alpha_in = alpha;
    if constexpr (E == EPI_ROPE_QKN) alpha = 1.f;   // applied by the rotary step
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      if constexpr (E == EPI_ROPE_QKN) rope_qkn_block(p, acc[i], region, lane, m0 + wm * WM + i * 32, n0 + wn * WN,
                                                      alpha_in);
      floatx4 pre[PRELOAD ? 32 / RPS : 1];
      if constexpr (PRELOAD) {
        asm volatile("" ::: "memory");   // keep the next block's loads from being hoisted here
#pragma unroll
        for (int st = 0; st < 32 / RPS; ++st) {
          // out-of-range positions load a clamped in-range address (no
          // branches, so the array stays in registers) and are never stored
          const int m = min(m0 + wm * WM + i * 32 + st * RPS + lane / LPR, p.M - 1);
          const int n = min(n0 + wn * WN + (lane % LPR) * 4, p.N - 4);
          const long off = (long)m * p.ldc + n;
          if constexpr (E == EPI_ACCUM_F32) pre[st] = load4((const float*)p.C + off);
          else pre[st] = load4((const TC*)p.aux + off);
        }
      }
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = j * 32 + 8 * q + 4 * g;
          floatx4 v = {acc[i][j][4 * q] * alpha, acc[i][j][4 * q + 1] * alpha, acc[i][j][4 * q + 2] * alpha,
                       acc[i][j][4 * q + 3] * alpha};
          *(floatx4*)(region + lds_off<RBY>(l32, col * 4)) = v;
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's staging writes are done
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int st = 0; st < 32 / RPS; ++st) {
        const int r = st * RPS + lane / LPR;
        const int c4 = lane % LPR;
        const floatx4 v = *(const floatx4*)(region + lds_off<RBY>(r, c4 * 16));
        const int m = m0 + wm * WM + i * 32 + r;
        const int n = n0 + wn * WN + c4 * 4;
        if (m < p.M && n < p.N) {
          const long off = (long)m * p.ldc + n;
          if constexpr (E == EPI_STORE || E == EPI_ROPE_QKN) {
            store4((TC*)p.C + off, v);
            if constexpr (SYM)
              if (tm != tn)
#pragma unroll
                for (int e = 0; e < 4; ++e) ((TC*)p.C)[(long)(n + e) * p.ldc + m] = from_f32<TC>(v[e]);
          } else if constexpr (E == EPI_STORE_F32) {
            store4((float*)p.C + off, v);
          } else if constexpr (E == EPI_ACCUM_F32) {
            store4((float*)p.C + off, pre[st] + v);
          } else if constexpr (E == EPI_RELU2) {
            store4((TC*)p.C + off, v);
            floatx4 rr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = fmaxf(v[e], 0.f);
              rr[e] = x * x;
            }
            if (p.C2) store4((TC*)p.C2 + off, rr);   // without C2 only the amax of relu(u)^2 is taken
            if (p.amax) amax_acc = fmaxf(amax_acc, abs_max4<TC>(rr));
          } else if constexpr (E == EPI_DRELU2) {
            const floatx4 u = pre[st];
            floatx4 rr;
#pragma unroll
            for (int e = 0; e < 4; ++e) rr[e] = v[e] * 2.f * fmaxf(u[e], 0.f);
            store4((TC*)p.C + off, rr);
            if (p.amax) amax_acc = fmaxf(amax_acc, abs_max4<TC>(rr));
          } else if constexpr (E == EPI_XENT_BWD) {
            const float L2E = 1.4426950408889634f;
            const float lse = p.auxf[m];
            const int y = ((const int*)p.aux)[m];
            floatx4 rr;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              rr[e] = (fast_exp2((v[e] - lse) * L2E) - (p.col0 + n + e == y ? 1.f : 0.f)) * p.beta;
            store4((TC*)p.C + off, rr);
          } else if constexpr (E == EPI_PARTIAL) {
            store4(p.part + (long)blockIdx.z * p.M * p.N + (long)m * p.N + n, v);
          } else if constexpr (E == EPI_AXPBY) {
            floatx4 rr;
#pragma unroll
            for (int e = 0; e < 4; ++e) rr[e] = fmaf(p.beta, pre[st][e], v[e]);
            store4((TC*)p.C + off, rr);
            if constexpr (SYM)
              if (tm != tn)
#pragma unroll
                for (int e = 0; e < 4; ++e) ((TC*)p.C)[(long)(n + e) * p.ldc + m] = from_f32<TC>(rr[e]);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // staging reads done before the region is rewritten
      __builtin_amdgcn_wave_barrier();
    }
    if constexpr (E == EPI_RELU2 || E == EPI_DRELU2) {
      if (p.amax) {
        __syncthreads();   // every wave is done with its staging region
        block_amax<NW>(p.amax, amax_acc, (float*)smem);
      }
    }
  }
}

// Sum split-K partials in split order: out[m, n] (+)= sum_z part[z, m, n].
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits, long mn,
                                                            float* __restrict__ out, int accumulate) {
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  floatx4 s = {0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < splits; ++z) s += *(const floatx4*)(part + (long)z * mn + i);
  // accumulate: the product's value (as a storing call would write it) is
  // added to out with one rounding
  if (accumulate) s = *(const floatx4*)(out + i) + s;
  *(floatx4*)(out + i) = s;
}

// The same reduction into an M x N block of a matrix with row stride ldc.
// out_bf16: C holds bf16 (no accumulation), else fp32.
__global__ __launch_bounds__(256) void splitk_reduce_strided_kernel(const float* __restrict__ part, int splits, int M,
                                                                    int N, void* __restrict__ out, long ldc,
                                                                    int accumulate, int out_bf16) {
  const long i = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  const long mn = (long)M * N;
  if (i >= mn) return;
  const long m = i / N, n = i % N;
  floatx4 s = {0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < splits; ++z) s += *(const floatx4*)(part + (long)z * mn + i);
  if (out_bf16) {
    *(bf16x4*)((bf16*)out + m * ldc + n) = __builtin_convertvector(s, bf16x4);
    return;
  }
  float* o = (float*)out + m * ldc + n;
  if (accumulate) s = *(const floatx4*)o + s;
  *(floatx4*)o = s;
}

// ------------------------------------------------------------------ dispatch

// Tile table: id -> (BM, BN, waves M x N, bytes per K step per row, stages).
struct TileCfg {
  int bm, bn, wgm, wgn, rb, ns;
  bool pp;   // ping-pong schedule of two 4-wave groups
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
    {256, 256, 2, 4, 64, 4, true},   // TILE_256x256_PP4
    {256, 256, 2, 4, 64, 5, true},   // TILE_256x256_PP5
    {256, 128, 4, 2, 128, 3, true},  // TILE_256x128_PP3
    {256, 256, 4, 2, 64, 4, true},   // TILE_256x256_PP4_H
    {128, 128, 4, 1, 128, 2},        // TILE_128x128_H
};
int tile_bm(int tile) { return TILES[tile].bm; }
int tile_bn(int tile) { return TILES[tile].bn; }
int tile_wn(int tile) { return TILES[tile].bn / TILES[tile].wgn; }
bool tile_needs_kc(int tile) { return !TILES[tile].pp && (TILES[tile].ns > 2 || TILES[tile].rb != 128); }

void gemm_kernel_label(int dtype, int layout, int epi, int tile, char* buf, int n) {
  const TileCfg& c = TILES[tile];
  const char* ty = dtype == DT_BF16 ? "bf16" : dtype == DT_F32 ? "float" : dtype == DT_FP8_A4B4 ? "fp8 e4m3 x e4m3" : "fp8 e5m2 x e4m3";
  snprintf(buf, n, "gemm_kernel<%s, %d, %d, %d, %d, %d, %d, %s, %s, %d%s>", ty, c.bm,
           c.bn, c.wgm, c.wgn, c.rb, c.ns, layout == LAYOUT_MN ? "false" : "true", layout == LAYOUT_KK ? "true" : "false",
           epi, c.pp ? ", ping-pong" : "");
}

template <typename TA, typename MF, int T, bool AK, bool BK_, int EPI, typename TC>
static void launch_cfg(const GemmArgs& a, int splits, hipStream_t st) {
  constexpr TileCfg c = TILES[T];
  dim3 grid(((a.M + c.bm - 1) / c.bm) * ((a.N + c.bn - 1) / c.bn), 1, splits);
  hipLaunchKernelGGL((gemm_kernel<TA, MF, c.bm, c.bn, c.wgm, c.wgn, c.rb, c.ns, AK, BK_, EPI, TC, c.pp, false>), grid,
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
      GK_T(TILE_256x256_PP4) GK_T(TILE_256x256_PP5) GK_T(TILE_256x128_PP3)
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
  GK_CASE(LAYOUT_KK, true, true, EPI_PARTIAL)
  // input gradients: grad [M][K] x weight [K][N]
  GK_CASE(LAYOUT_KN, true, false, EPI_STORE)
  GK_CASE(LAYOUT_KN, true, false, EPI_STORE_F32)
  GK_CASE(LAYOUT_KN, true, false, EPI_ACCUM_F32)   // the lm_head's input gradient over vocabulary chunks
  GK_CASE(LAYOUT_KN, true, false, EPI_DRELU2)
  GK_CASE(LAYOUT_KN, true, false, EPI_PARTIAL)
  // the fused QKV product with its rotary epilogue: the two tiles whose
  // waves own 128 columns
  if constexpr (sizeof(TA) == 2) {
    if (layout == LAYOUT_KK && epi == EPI_ROPE_QKN) {
      if (tile == TILE_256x256_PP4_H) launch_cfg<TA, MF, TILE_256x256_PP4_H, true, true, EPI_ROPE_QKN, TC>(a, splits, st);
      else if (tile == TILE_128x128_H) launch_cfg<TA, MF, TILE_128x128_H, true, true, EPI_ROPE_QKN, TC>(a, splits, st);
      else return -1;
      return 0;
    }
  }
  // weight gradients: grad [K][M] x activation [K][N]
  GK_CASE(LAYOUT_MN, false, false, EPI_STORE_F32)
  GK_CASE(LAYOUT_MN, false, false, EPI_ACCUM_F32)
  GK_CASE(LAYOUT_MN, false, false, EPI_PARTIAL)
#undef GK_CASE
  return -1;
}

// FP8 products: both operands K-contiguous (the quantiser provides
// transposed copies), bf16 / fp32 outputs.  The MFMA is issued with the B
// tile first, so its first format code is B's.
template <typename MF>
static int launch_fp8(const GemmArgs& a, int layout, int epi, int tile, int splits, hipStream_t st) {
  if (layout != LAYOUT_KK) return -1;
  // ReLU^2 / dReLU^2 with fp32 outputs (and fp32 aux): the values the next
  // quantiser encodes
  if (epi == EPI_RELU2_F32) {
    launch_cfg<uint8_t, MF, TILE_128x128, true, true, EPI_RELU2, float>(a, splits, st);
    return 0;
  }
  if (epi == EPI_DRELU2_F32) {
    launch_cfg<uint8_t, MF, TILE_128x128, true, true, EPI_DRELU2, float>(a, splits, st);
    return 0;
  }
#define GK_F8(E)                                                                    \
  if (epi == E) {                                                                   \
    launch_cfg<uint8_t, MF, TILE_128x128, true, true, E, bf16>(a, splits, st);      \
    return 0;                                                                       \
  }
  GK_F8(EPI_STORE)
  GK_F8(EPI_STORE_F32)
  GK_F8(EPI_ACCUM_F32)
  GK_F8(EPI_RELU2)
  GK_F8(EPI_DRELU2)
  GK_F8(EPI_PARTIAL)
#undef GK_F8
  return -1;
}

template <typename TA, typename MF, typename TC, int T, bool AK, bool BK_, int EPI>
static void launch_batched_cfg(const GemmArgs& a, int batch, hipStream_t st) {
  constexpr TileCfg c = TILES[T];
  const int tm = (a.M + c.bm - 1) / c.bm, tn = (a.N + c.bn - 1) / c.bn;
  constexpr bool sym = EPI == EPI_STORE_SYM || EPI == EPI_AXPBY_SYM;
  dim3 grid(sym ? tn * (tn + 1) / 2 : tm * tn, batch, 1);
  hipLaunchKernelGGL((gemm_kernel<TA, MF, c.bm, c.bn, c.wgm, c.wgn, c.rb, c.ns, AK, BK_, EPI, TC, c.pp, true>), grid,
                     dim3(64 * c.wgm * c.wgn), 0, st, a);
}

template <bool AK, bool BK_, int EPI>
static int launch_batched_tile(const GemmArgs& a, int tile, int batch, hipStream_t st) {
  if (tile == TILE_256x256_PP4)
    launch_batched_cfg<bf16, Mfma<bf16>, bf16, TILE_256x256_PP4, AK, BK_, EPI>(a, batch, st);
  else if (tile == TILE_128x128)
    launch_batched_cfg<bf16, Mfma<bf16>, bf16, TILE_128x128, AK, BK_, EPI>(a, batch, st);
  else
    return -1;
  return 0;
}

int gemm_launch_batched(const GemmArgs& a, int layout, int epi, int tile, int batch, hipStream_t st) {
  if (batch < 1 || batch > 65535) return -1;
  if (epi == EPI_STORE_SYM || epi == EPI_AXPBY_SYM) {
    // square output, square tiles
    if (a.M != a.N || tile_bm(tile) != tile_bn(tile)) return -1;
    if (layout == LAYOUT_KK && epi == EPI_STORE_SYM)
      return launch_batched_tile<true, true, EPI_STORE_SYM>(a, tile, batch, st);
    if (layout == LAYOUT_MN && epi == EPI_STORE_SYM)
      return launch_batched_tile<false, false, EPI_STORE_SYM>(a, tile, batch, st);
    if (layout == LAYOUT_KK && epi == EPI_AXPBY_SYM)
      return launch_batched_tile<true, true, EPI_AXPBY_SYM>(a, tile, batch, st);
    return -1;
  }
  if (layout == LAYOUT_KK && epi == EPI_STORE) return launch_batched_tile<true, true, EPI_STORE>(a, tile, batch, st);
  if (layout == LAYOUT_KK && epi == EPI_AXPBY) return launch_batched_tile<true, true, EPI_AXPBY>(a, tile, batch, st);
  if (layout == LAYOUT_KN && epi == EPI_AXPBY) return launch_batched_tile<true, false, EPI_AXPBY>(a, tile, batch, st);
  if (layout == LAYOUT_MN && epi == EPI_STORE) return launch_batched_tile<false, false, EPI_STORE>(a, tile, batch, st);
  return -1;
}

int gemm_launch(const GemmArgs& a, int dtype, int layout, int epi, int tile, int splits, hipStream_t st) {
  if (dtype == DT_BF16) return launch_epi<bf16, Mfma<bf16>, bf16>(a, layout, epi, tile, splits, st);
  if (dtype == DT_F32) return launch_epi<float, Mfma<float>, float>(a, layout, epi, tile, splits, st);
  if (dtype == DT_FP8_A4B4) return launch_fp8<MfmaF8<FP8_E4M3, FP8_E4M3>>(a, layout, epi, tile, splits, st);
  if (dtype == DT_FP8_A5B4) return launch_fp8<MfmaF8<FP8_E4M3, FP8_E5M2>>(a, layout, epi, tile, splits, st);
  return -1;
}

void splitk_reduce(const float* part, int splits, long mn, float* out, int accumulate, hipStream_t st) {
  const long n4 = (mn + 3) / 4;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, part, splits, mn,
                     out, accumulate);
}

void splitk_reduce_strided(const float* part, int splits, int M, int N, void* out, long ldc, int accumulate,
                           int out_bf16, hipStream_t st) {
  const long n4 = ((long)M * N + 3) / 4;
  hipLaunchKernelGGL(splitk_reduce_strided_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, part, splits,
                     M, N, out, ldc, accumulate, out_bf16);
}

}  // namespace gk
