// Launcher interface between the host runtime (api.cpp) and the gfx950
// kernels.  Plain structs and functions; every launcher enqueues on the given
// stream and returns without synchronising.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gk {

enum DType {
  DT_F32 = 0,
  DT_BF16 = 1,
  DT_FP8_A4B4 = 2,   // fp8 GEMM: A E4M3, B E4M3 (forward)
  DT_FP8_A5B4 = 3,   // fp8 GEMM: A E5M2 (a gradient), B E4M3
};
enum Fp8Fmt { FP8_E4M3 = 0, FP8_E5M2 = 1 };   // also the MFMA operand format codes

enum Layout {
  LAYOUT_KK = 0,  // A [M][K], B [N][K]
  LAYOUT_KN = 1,  // A [M][K], B [K][N]
  LAYOUT_MN = 2,  // A [K][M], B [K][N]
};

enum Epi {
  EPI_STORE = 0,      // C (activation type) = acc
  EPI_STORE_F32 = 1,  // C (fp32) = acc
  EPI_ACCUM_F32 = 2,  // C (fp32) += acc
  EPI_RELU2 = 3,      // C = acc (u), C2 = relu(acc)^2 (g)
  EPI_DRELU2 = 4,     // C = acc * 2 * relu(aux)
  EPI_XENT_FWD = 5,   // per-row partial (max, sum exp) + target logit
  EPI_XENT_BWD = 6,   // C = (exp(acc - lse) - onehot(target)) * beta
  EPI_PARTIAL = 7,    // part[split][M][N] = acc (split-K)
  EPI_AXPBY = 8,      // C (activation type) = alpha * acc + beta * aux (aux laid out as C)
  // EPI_STORE / EPI_AXPBY for a product known to be symmetric (M == N, and a
  // symmetric aux): only the tiles on or above the diagonal are computed,
  // each stored also transposed (batched launches only)
  EPI_STORE_SYM = 9,
  EPI_AXPBY_SYM = 10,
  // fp8 products only: EPI_RELU2 / EPI_DRELU2 with fp32 outputs (and, for
  // EPI_DRELU2, an fp32 aux), so that the next quantiser encodes the fp32
  // values the epilogue computed
  EPI_RELU2_F32 = 11,
  EPI_DRELU2_F32 = 12,
  // the fused QKV product (bf16, heads of 128, one wave per head): rotate the
  // q and k heads, RMS-normalise them, store q^, k^, v row-major (C), their
  // rstd, and the transposed copies q^T, k^T, v^T
  EPI_ROPE_QKN = 13,
};

// Work-group tiles (M x N); _W8 variants use 8 waves (2 x 4) instead of 4 (2 x 2).
enum Tile {
  TILE_256x256 = 0, TILE_256x128 = 1, TILE_128x128 = 2, TILE_64x64 = 3,
  TILE_256x256_W8 = 4, TILE_256x128_W8 = 5,
  // deeper pipelines (K-contiguous operands only): 4 stages of 64-byte rows
  // or 3 stages of 128-byte rows
  TILE_256x256_W8_S4 = 6, TILE_256x256_S4 = 7, TILE_256x128_W8_S3 = 8, TILE_128x128_S4 = 9,
  // 8 waves in two ping-pong groups: 4 / 5 stages of 64-byte rows, 3 of 128
  TILE_256x256_PP4 = 10, TILE_256x256_PP5 = 11, TILE_256x128_PP3 = 12,
  TILE_COUNT = 13,
  // the rotary epilogue's tiles (EPI_ROPE_QKN only): PP4 and 128x128 with the
  // waves laid out so that each owns 128 whole columns, one head
  TILE_256x256_PP4_H = 13, TILE_128x128_H = 14,
};
bool tile_needs_kc(int tile);   // usable only when both operands are K-contiguous
// Readable template signature of the kernel a product launches (as profilers
// print it, without the MFMA-traits and output-type arguments).
void gemm_kernel_label(int dtype, int layout, int epi, int tile, char* buf, int n);
int tile_bm(int tile);
int tile_bn(int tile);
int tile_wn(int tile);   // output columns owned by one wave

struct GemmArgs {
  const void* A;
  const void* B;
  int M, N, K;
  long lda, ldb;   // leading dimensions, in elements
  void* C;
  long ldc;
  void* C2;        // EPI_RELU2: g (may be NULL: only u is stored, and the amax of g taken)
  const void* aux; // EPI_DRELU2: u; EPI_XENT_*: int32 targets
  const float* auxf; // EPI_XENT_BWD: per-row logsumexp
  float* part;     // EPI_XENT_FWD: [M][nblk][2]; EPI_PARTIAL: [splits][M][N]
  float* tgt;      // EPI_XENT_FWD: target logit per row
  float alpha;     // scales the accumulator before the epilogue
  const float* scale_a;  // fp8 products: quantisation scales of A and B (device);
  const float* scale_b;  // the accumulator is multiplied by alpha / (scale_a * scale_b)
  float beta;      // EPI_XENT_BWD: 1 / rows
  int k_split;     // K elements handled per blockIdx.z
  int nblk;        // EPI_XENT_FWD: number of column blocks of width BN/2
  int col0;        // EPI_XENT_BWD: vocabulary index of column 0 (a chunk of the vocabulary)
  unsigned* amax;  // EPI_RELU2 / EPI_DRELU2: if set, max |stored g / du| is folded in (float bits)
  // Batched products (grid y = batch index): element strides between the
  // batch's A, B and C (aux shares C's); zero for a single product.
  long bsA, bsB, bsC;
  // EPI_ROPE_QKN: the rotary table [seqT][64] (cos, sin); rstd out
  // [M][nH + nHkv]; the transposed copies [B][heads][128][seqT] (seqT a
  // multiple of 64, so that no padding columns exist); the C row holds nH q
  // heads, then nHkv k heads, then nHkv v heads.
  const float* rope_cos;
  const float* rope_sin;
  float* rqk;
  void* qT;
  void* kT;
  void* vT;
  int seqT, nH, nHkv;
  float eps;
};

int gemm_launch(const GemmArgs& a, int dtype, int layout, int epi, int tile, int splits,
                hipStream_t st);
// `batch` independent bf16 products of one shape (strides in a.bsA/bsB/bsC),
// one grid; no split-K.
int gemm_launch_batched(const GemmArgs& a, int layout, int epi, int tile, int batch, hipStream_t st);
void splitk_reduce(const float* part, int splits, long mn, float* out, int accumulate,
                   hipStream_t st);
// out[m * ldc + n] (+)= sum over z of part[z][m][n] for an M x N block of a
// wider fp32 matrix (N a multiple of 4, out and ldc 16-byte aligned), or, when
// out_bf16, out = the sum rounded to a bf16 matrix (8-byte aligned).
void splitk_reduce_strided(const float* part, int splits, int M, int N, void* out, long ldc, int accumulate,
                           int out_bf16, hipStream_t st);

// ---------------------------------------------------------------- elementwise
// Also checks that every token and target id is in [0, vocab) (sets *flag).
void embed_fwd(int dtype, const int32_t* tokens, const int32_t* targets, const void* E, float* h, int rows, int d,
               int vocab, int* flag, hipStream_t st);
// amax (optional): max |value| of the output, taken from the fp32 value before
// it is rounded to the stored type, folded in as float bits (fp8 scaling: the
// quantiser encodes the same fp32 values)
// Chunks of 8 elements per lane for the register-resident norm kernels (0:
// the row does not fit, the looping kernels run instead).
inline int norm_chunks(int d) {
  if (d % 8) return 0;
  return d <= 512 ? 1 : d <= 1024 ? 2 : d <= 1536 ? 3 : d <= 2048 ? 4 : 0;
}
void rmsnorm_fwd(int dtype, const float* x, void* y, float* rstd, int rows, int d, float eps,
                 hipStream_t st, unsigned* amax = nullptr);
// dx (+)= r * (dy - y * mean(dy*y)); also writes dx in the activation type.
// dy is fp32, or in the activation type when dy_act (register-chunk widths
// only: norm_chunks(d) != 0); returns -1 for a combination not built.
int rmsnorm_bwd(int dtype, const void* dy, int dy_act, const void* y, const float* rstd, float* dx,
                void* dx_act, int rows, int d, int accumulate, hipStream_t st, unsigned* amax = nullptr);
// qkv [B*T][H*Dh + 2*Hkv*Dh]: q heads, then k heads, then v heads; rstd_qk
// [B*T][H + Hkv] (q heads, then k heads); qT [B][H][Dh][Tp], kT, vT
// [B][Hkv][Dh][Tp].
void rope_qknorm_fwd(int dtype, void* qkv, float* rstd_qk, void* qT, void* kT, void* vT,
                     const float* cosb, const float* sinb, int B, int T, int Tp, int H, int Hkv, int Dh,
                     float eps, hipStream_t st);
void rope_qknorm_bwd(int dtype, void* dqkv, const void* qkv, const float* rstd_qk, const float* cosb,
                     const float* sinb, int B, int T, int H, int Hkv, int Dh, hipStream_t st,
                     unsigned* amax = nullptr);
void attn_bwd_pre(int dtype, const void* dO, const void* O, float* Dv, void* dOT, int B, int T, int Tp,
                  int H, int Dh, hipStream_t st);
void xent_reduce(const float* part, const float* tgt, int rows, int nblk, float* lse, float* row_loss,
                 hipStream_t st);
void mean_reduce(const float* x, int n, float* out, hipStream_t st);
// dE[id] = (accumulate ? dE[id] : 0) + sum of dh rows whose token is id, in
// position order (vocab <= 65536).  Scratch (int32): sorted and rank [rows],
// cnt [ceil(rows / 1024)][vocab], tot and lstart [vocab], bsum
// [2 * ceil(vocab / 256) + 1], heads [2 + vocab]; fp32 part [emb_part_rows(rows)][d].
void embed_bwd(const int32_t* tokens, const float* dh, float* dE, int rows, int d, int vocab, int* sorted, int* rank,
               int* cnt, int* tot, int* lstart, int* bsum, int* heads, float* part, int accumulate, hipStream_t st);
// segment sums of the ids with many rows (> 256 each, 128-row segments)
inline long emb_part_rows(long rows) { return rows / 128 + rows / 256 + 1; }
void fill_f32(float* p, long n, float v, hipStream_t st);

// ---------------------------------------------------------------- optimizer
// One tensor of a pass list.  Passes walk their list in chunks of OPT_CHUNK
// elements; blk0 is the tensor's first chunk index within the list, and every
// list ends with a sentinel entry whose blk0 is the list's chunk count.
constexpr int OPT_CHUNK = 4096;
struct OptSeg {
  long off;    // element offset in the parameter / gradient / master buffers
  long soff;   // element offset of its state (Muon: momentum; AdamW: m, then v at soff + n)
  long n;      // elements (a multiple of 4)
  long xoff;   // Muon: element offset of its matrix in the Newton-Schulz buffer
  int blk0;
  int which;   // AdamW: 0 takes AdamArgs::lr0, 1 takes lr1
};
struct AdamArgs {
  float b1, b2, eps, wd;
  float ibc1, ibc2;   // 1 / (1 - b1^t), 1 / (1 - b2^t)
  float lr0, lr1;
};
void opt_sumsq(const float* x, const OptSeg* seg, int nseg, int nblk, float* part, hipStream_t st);
void opt_norm(const float* part, int nblk, float clip, float* hdr, hipStream_t st);
void opt_adamw(float* master, float* state, const float* g, void* w16, const OptSeg* seg, int nseg, int nblk,
               const float* hdr, const AdamArgs& a, hipStream_t st);
void opt_muon_momentum(const float* g, float* state, const OptSeg* seg, int nseg, int nblk, const float* hdr,
                       float mu, int nesterov, float* part, hipStream_t st);
void opt_muon_normalise(const float* g, const float* state, const OptSeg* seg, int nseg, int nblk,
                        const float* hdr, float mu, int nesterov, const float* part, void* X, hipStream_t st);
// p <- p (1 - lr wd) - lr * scale * O
void opt_muon_update(float* master, const void* X, void* w16, const OptSeg* seg, int nseg, int nblk, float lr,
                     float scale, float wd, hipStream_t st);
void opt_widen(const void* w16, float* master, const OptSeg* seg, int nseg, int nblk, hipStream_t st);

// ---------------------------------------------------------------- decoding
// out[b][n] = sum_k x[b][k] W[n][k] (bf16 x with row stride ldx, W [N][K];
// B <= 32, K % 16 == 0) with epilogue EPI_STORE (bf16), EPI_STORE_F32 or
// EPI_RELU2 (C = u, C2 = relu(u)^2), C and C2 with row stride ldc; or, with
// ksplit > 1, EPI_PARTIAL: K in ksplit runs, C[y][b][n] (row stride ldc)
// the y-th run's sum.
int skinny_gemm(int epi, const void* x, long ldx, int B, int K, const void* W, int N, void* C, int ldc, void* C2,
                int ksplit, hipStream_t st);
// h [B][d] fp32 += sum of nsplit (<= 8) partials part[s][B][d] (in order),
// then y = bf16 RMSNorm(h)
void decode_add_rmsnorm(float* h, const float* part, int nsplit, int B, int d, void* y, float eps, hipStream_t st);
// caches[b][g][t] = k^ / v of key/value head g of qkv row (b, t) for t < T
// (qkv [B*T][d + 2*Hkv*Dh])
void kv_fill(const void* qkv, void* kc, void* vc, int B, int T, int H, int Hkv, int Dh, int Tmax, hipStream_t st);
// o [B][d] = attention of the new token over cached keys max(0, pos -
// window + 1) .. pos, pos = *posp (device).  qkv [B][d + 2*Hkv*Dh] holds the
// new token's raw q, k, v: its rotary embedding and QK norm are applied here,
// and k^ and v are written into the caches [B][Hkv][Tmax][Dh] at pos; query
// head h reads key/value head h / (H / Hkv).
// part: B * H * ceil(min(window, Tmax) / 128) * (Dh + 1) floats
int attn_decode(const void* qkv, void* kc, void* vc, const float* cosb, const float* sinb, float* part, void* o,
                int B, int H, int Hkv, int Dh, int Tmax, const int* posp, int window, float eps, hipStream_t st);
// tok[0..B) = tokens[0..B), *posp = pos, *flag = 0 (one small kernel)
void decode_stage(const int32_t* tokens, int B, int pos, int32_t* tok, int* posp, int* flag, hipStream_t st);

// ---------------------------------------------------------------- fp8
void zero_u32(unsigned* p, int n, hipStream_t st);
// Per-tensor amax: AMAX_SLOT words per tensor (see wave_amax), zeroed before
// the tensor is produced; fp8_amax folds in max |x| over n bf16 values.
constexpr int AMAX_SLOT = 64;
void fp8_amax(const void* x, long n, unsigned* amax, hipStream_t st);
// x [R][C] bf16, or fp32 when x_f32 (C a multiple of 64) -> codes q [R][C]
// and, if qT, [C][R].  fp32 x only: with rowscale the encoded value of
// x[r][c] is x[r][c] * rowscale[r] (a norm's output recomputed from its fp32
// input and rstd, exactly as the norm computes it); with relu2 it is
// max(x[r][c], 0)^2 (the MLP activation recomputed from u, as the W1
// epilogue computes it).
void fp8_quantize(int fmt, const void* x, int R, int C, const unsigned* amax, float* scale_out, void* q, void* qT,
                  hipStream_t st, int x_f32 = 0, const float* rowscale = nullptr, int relu2 = 0);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  // [B*T][ldqkv], ldqkv = d + 2*Hkv*Dh: q^ of head h at col h*Dh, k^ of
  // key/value head g at d + g*Dh, v at d + Hkv*Dh + g*Dh; query head h uses
  // key/value head h / (H / Hkv)
  const void* qkv;
  const void* qT;    // [B][H][Dh][Tp]
  const void* kT;    // [B][Hkv][Dh][Tp]
  const void* vT;
  void* o;           // [B*T][d]
  float* lse2;       // [B][H][Tp], log2 domain
  const void* dO;    // [B*T][d]
  const void* dOT;   // [B][H][Dh][Tp]
  const float* Dv;   // [B][H][Tp] rowsum(dO * O)
  void* dqkv;        // [B*T][ldqkv]
  int B, T, Tp, H, Hkv, d, ldqkv, window;
  float scale_log2;  // log2(e) / sqrt(Dh)
  unsigned* amax_o;   // forward: if set, max |stored o| (float bits)
  unsigned* amax_dv;  // dV pass: if set, max |stored dv| (float bits)
  float scale;       // 1 / sqrt(Dh)
};
int attn_fwd(int dtype, int Dh, const AttnArgs& a, hipStream_t st);
// part 0: dV, part 1: dK (one work-group per 128-key tile of a key/value
// head, summing over its query heads); part 2: dQ (per 128-query tile).
int attn_bwd(int dtype, int Dh, const AttnArgs& a, int part, hipStream_t st);

}  // namespace gk
