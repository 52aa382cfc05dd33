// Host runtime of the GPT step: configuration checks, parameter layout,
// workspace carve-up, and the launch sequence of one forward+backward pass on
// one HIP stream.  No device memory is allocated here: the caller passes the
// weights, gradients, tokens and one workspace buffer.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "model.h"

using namespace gk;
using namespace gm;

namespace gm __attribute__((visibility("hidden"))) {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}


int check_config(const gpt_config* c, Shape& s) {
  if (!c) return fail(GPT_ENULL, "cfg is NULL");
  if (c->precision != GPT_FP32 && c->precision != GPT_BF16 && c->precision != GPT_FP8)
    return fail(GPT_EINVAL, "unknown precision");
  s.fp8 = c->precision == GPT_FP8;
  s.dtype = c->precision == GPT_FP32 ? DT_F32 : DT_BF16;
  s.es = s.dtype == DT_F32 ? 4 : 2;
  s.L = c->depth; s.d = c->d_model; s.H = c->n_head; s.Dh = c->head_dim; s.F = c->mlp_hidden;
  s.V = c->vocab; s.T = c->seq_len; s.B = c->batch;
  s.eps = c->norm_eps; s.base = c->rope_base;
  if (s.L < 1 || s.d < 1 || s.H < 1 || s.F < 1 || s.V < 1 || s.T < 1 || s.B < 1)
    return fail(GPT_EINVAL, "all sizes must be positive");
  if ((long)s.H * s.Dh != s.d) return fail(GPT_EINVAL, "d_model must equal n_head * head_dim");
  s.Hkv = c->n_kv_head ? c->n_kv_head : s.H;
  if (s.Hkv < 1 || s.Hkv > s.H || s.H % s.Hkv) return fail(GPT_EINVAL, "n_kv_head must divide n_head");
  s.dkv = s.Hkv * s.Dh;
  s.Nqkv = s.d + 2 * s.dkv;
  const bool dh_ok = s.dtype == DT_F32 ? (s.Dh == 32 || s.Dh == 64) : (s.Dh == 64 || s.Dh == 128);
  if (!dh_ok) return fail(GPT_EINVAL, "unsupported head_dim for this precision");
  if (s.d % 64 || s.F % 64) return fail(GPT_EINVAL, "d_model and mlp_hidden must be multiples of 64");
  if (s.V % 8 || s.V > 65536) return fail(GPT_EINVAL, "vocab must be a multiple of 8 and <= 65536");
  if ((long)s.B * s.T > 32768) return fail(GPT_EINVAL, "batch * seq_len must be <= 32768");
  // eps > 0: the norms divide by sqrt(mean(x^2) + eps), and the attention
  // kernels' padded query/key positions are all-zero vectors
  if (!(c->norm_eps > 0.f) || !std::isfinite(c->norm_eps) || !(c->rope_base > 0.f) || !std::isfinite(c->rope_base))
    return fail(GPT_EINVAL, "norm_eps and rope_base must be positive and finite");
  s.BT = s.B * s.T;
  s.Tp = (s.T + 63) / 64 * 64;
  if (s.fp8 && s.BT % 64) return fail(GPT_EINVAL, "GPT_FP8 needs batch * seq_len to be a multiple of 64");
  const char* pat = c->window_pattern;
  size_t plen = strnlen(pat, sizeof(c->window_pattern));
  if (plen == 0 || plen == sizeof(c->window_pattern)) return fail(GPT_EINVAL, "window_pattern must be 1..7 chars");
  for (size_t k = 0; k < plen; ++k)
    if (pat[k] != 'S' && pat[k] != 'L') return fail(GPT_EINVAL, "window_pattern chars must be 'S' or 'L'");
  s.win.assign(s.L, s.T);
  for (int l = 0; l < s.L; ++l) {
    char ch = pat[l % plen];
    if (l == s.L - 1) ch = 'L';
    if (ch == 'S') {
      if (c->window < 1) return fail(GPT_EINVAL, "window must be >= 1 when the pattern has 'S'");
      s.win[l] = c->window < s.T ? c->window : s.T;
    } else if (ch != 'L') {
      return fail(GPT_EINVAL, "window_pattern chars must be 'S' or 'L'");
    }
  }
  return GPT_OK;
}

void param_offsets(const Shape& s, ParamOffsets& p) {
  long off = 0;
  auto add = [&](const char* name, int rows, int cols) {
    gpt_tensor_desc t;
    memset(&t, 0, sizeof(t));
    snprintf(t.name, sizeof(t.name), "%s", name);
    t.offset = off;
    t.rows = rows;
    t.cols = cols;
    p.descs.push_back(t);
    long o = off;
    off += (long)rows * cols;
    off = (off + 127) / 128 * 128;
    return o;
  };
  p.descs.clear();
  p.Wqkv.resize(s.L); p.Wo.resize(s.L); p.W1.resize(s.L); p.W2.resize(s.L);
  p.E = add("E", s.V, s.d);
  char nm[24];
  for (int l = 0; l < s.L; ++l) {
    snprintf(nm, sizeof nm, "L%d.Wq", l); p.Wqkv[l] = add(nm, s.d, s.d);
    snprintf(nm, sizeof nm, "L%d.Wk", l); add(nm, s.dkv, s.d);
    snprintf(nm, sizeof nm, "L%d.Wv", l); add(nm, s.dkv, s.d);
    snprintf(nm, sizeof nm, "L%d.Wo", l); p.Wo[l] = add(nm, s.d, s.d);
    snprintf(nm, sizeof nm, "L%d.W1", l); p.W1[l] = add(nm, s.F, s.d);
    snprintf(nm, sizeof nm, "L%d.W2", l); p.W2[l] = add(nm, s.d, s.F);
  }
  p.U = add("U", s.V, s.d);
  p.total = off;
}

// ------------------------------------------------------------------ GEMM planning
struct GemmPlan {
  int tile, splits, k_split;
};


// Tile and split-K choice, set from measurements of this kernel on MI355X at
// the step's shapes: the 256x256 ping-pong tile for every bf16 product
// (forward, input and weight gradients), 128x128 for fp8 and for fp32 (64x64
// for small fp32 outputs).  Weight gradients (K = B*T, few output tiles) are
// split along K by a cost model, over the ping-pong tile and, for bf16
// outputs small enough to need many splits, 128x128 (two work-groups per
// CU): waves of work-groups (512 resident at two per CU, 256 at one) times K
// steps per split, plus the fp32 partial-sum reduction at ~5 TB/s.
GemmPlan plan_gemm(int dtype, int layout, int M, int N, int K) {
  GemmPlan g{TILE_64x64, 1, K};
  const bool f8 = dtype == DT_FP8_A4B4 || dtype == DT_FP8_A5B4;
  const int bk = dtype == DT_F32 ? 32 : f8 ? 128 : 64;
  if (f8) {
    g.tile = TILE_128x128;
  } else if (dtype == DT_F32) {
    g.tile = (long)M * N >= 256L * 128 * 128 ? TILE_128x128 : TILE_64x64;
  } else if (layout == LAYOUT_KK) {
    // forward products: the ping-pong 256x256 tile at every step shape
    // (measured against 128x128, 256x128 and 8-wave tiles at 16384 x
    // {768 .. 4608} x {768 .. 6144}; in the d20 step the QKV product went
    // 8.96 -> 7.58 ms and d12's W2 1.39 -> 1.25 ms per step)
    g.tile = TILE_256x256_PP4;
  } else if (layout == LAYOUT_KN) {
    // input gradients: the ping-pong 256x256 tile measured best at every
    // step shape, narrow and wide
    g.tile = TILE_256x256_PP4;
  } else if (layout == LAYOUT_MN) {
    g.tile = TILE_256x256_PP4;
  } else {
    g.tile = TILE_128x128;
  }
  // Weight gradients (and fp8 weight gradients, K-contiguous with K = B*T):
  // split K by the cost model, over the candidate tiles (bf16: the ping-pong
  // 256x256 tile, or 128x128 for small outputs that need many splits).
  if (layout == LAYOUT_MN || (f8 && K >= 4096)) {
    double best = 1e300;
    const int tile_cand[2] = {g.tile, TILE_128x128};
    const int ntile = (layout == LAYOUT_MN && dtype == DT_BF16) ? 2 : 1;
    for (int ti = 0; ti < ntile; ++ti) {
      const int tile = tile_cand[ti];
      const bool pp = tile == TILE_256x256_PP4;
      const long tiles = (long)((M + tile_bm(tile) - 1) / tile_bm(tile)) * ((N + tile_bn(tile) - 1) / tile_bn(tile));
      const long slots = dtype == DT_F32 || pp ? 256 : 512;
      // one K step of one tile, seconds (the ping-pong tile steps 32 deep)
      const double t_step = dtype == DT_F32 ? 4e-6 : f8 ? 1.5e-6 : pp ? 0.95e-6 : 1.34e-6;
      const int step = pp ? 32 : bk;
      // split counts: up to 24 for 128x128; for the 256x256 tile up to 4, or
      // up to 8 for small outputs (a few tiles must fill the CUs, and the
      // fp32 partials stay small).  Measured: more splits of the 10-40 MB
      // outputs cost more in the reduction than they gain.
      const int cand_pp[8] = {1, 2, 3, 4, 5, 6, 7, 8};
      const int cand_128[9] = {1, 2, 3, 4, 6, 8, 12, 16, 24};
      const int ncand = pp ? ((double)M * N <= 2.5e6 ? 8 : 4) : 9;
      for (int c = 0; c < ncand; ++c) {
        const int sp = pp ? cand_pp[c] : cand_128[c];
        int ks = (K + sp - 1) / sp;
        ks = (ks + bk - 1) / bk * bk;
        const int real = (K + ks - 1) / ks;
        if (real != sp && sp > 1) continue;
        const long waves = (tiles * sp + slots - 1) / slots;
        double t = (double)waves * ((ks + step - 1) / step) * t_step;
        if (sp > 1) t += (sp + 1.0) * M * (double)N * 4.0 / 5e12;
        if (t < best) {
          best = t;
          g.tile = tile;
          g.splits = sp;
          g.k_split = ks;
        }
      }
    }
  }
  if (g.splits == 1) g.k_split = K;
  return g;
}

// Wave quantisation of long-K bf16 products whose 256x256 tiles fill a whole
// number of rounds of the 256 CUs only partly (e.g. 16384 x 1536: 384 tiles,
// 1.5 rounds run as 2).  The first n1 tile columns form whole rounds and run
// as usual; the remaining columns are split along K into `splits` parts that
// together fill one round, and their fp32 partials are summed (in split
// order) into C.  Plain stores (fp32 or bf16) and fp32 accumulation qualify.
struct TailPlan {
  int n1;       // tile columns of the whole-round part (0: no tail split)
  int splits;
};
TailPlan plan_tail(int dtype, int layout, int epi, int M, int N, int K) {
  TailPlan t{0, 1};
  if (dtype != DT_BF16 || layout == LAYOUT_MN || K < 4096) return t;
  if (epi != EPI_STORE_F32 && epi != EPI_ACCUM_F32 && epi != EPI_STORE) return t;
  if (plan_gemm(dtype, layout, M, N, K).tile != TILE_256x256_PP4) return t;
  const long tm = (M + 255) / 256, tn = (N + 255) / 256;
  if ((tm * tn) % 256 == 0) return t;
  for (long n1 = tn - 1; n1 >= 1; --n1) {
    if ((tm * n1) % 256) continue;
    const long r = tm * (tn - n1);
    const long sp = std::min<long>(4, 256 / r);
    if (sp < 2 || (N - n1 * 256) % 4) return t;
    t.n1 = (int)n1;
    t.splits = (int)sp;
    return t;
  }
  return t;
}

// Argument checks shared by gpt_gemm and gpt_gemm_noalloc (no device calls).
int gemm_check(int dtype, int layout, int M, int N, int K, const void* A, const void* B, const float* C, int splits,
               int tile, const char* who) {
  const std::string w(who);
  if (!A || !B || !C) return fail(GPT_ENULL, w + ": NULL operand");
  if (dtype != DT_F32 && dtype != DT_BF16) return fail(GPT_EINVAL, w + ": dtype");
  if (layout < 0 || layout > 2) return fail(GPT_EINVAL, w + ": layout");
  if (M < 1 || N < 1 || K < 1 || M % 8 || N % 8 || K % 8) return fail(GPT_EINVAL, w + ": sizes");
  if (splits < 1 || (splits > 1 && layout == LAYOUT_KK)) return fail(GPT_EINVAL, w + ": splits");
  if (tile < 0) tile = plan_gemm(dtype, layout, M, N, K).tile;
  if (dtype == DT_F32 && tile != TILE_128x128 && tile != TILE_64x64) return fail(GPT_EINVAL, w + ": tile");
  if (dtype == DT_BF16 && (tile == TILE_64x64 || tile >= TILE_COUNT || (tile_needs_kc(tile) && layout != LAYOUT_KK)))
    return fail(GPT_EINVAL, w + ": tile");
  return GPT_OK;
}

// K per split after rounding to whole K steps, and the number of splits
// that leaves (the partial buffer holds that many M x N blocks).
int gemm_real_splits(int dtype, int K, int splits, int* k_split) {
  const int bk = dtype == DT_F32 ? 32 : 64;
  int ks = (K + splits - 1) / splits;
  ks = (ks + bk - 1) / bk * bk;
  if (k_split) *k_split = ks;
  return (K + ks - 1) / ks;
}

// One product C = A B^T (layouts as in gpt_gemm); splits > 1 sums K splits
// through `workspace` (>= real splits * M * N floats) in split order.
// Arguments were checked by gemm_check.
int gemm_entry(int dtype, int layout, int M, int N, int K, const void* A, const void* B, float* C, float* workspace,
               int splits, int tile, void* stream, const char* who) {
  const std::string w(who);
  if (tile < 0) tile = plan_gemm(dtype, layout, M, N, K).tile;
  GemmArgs a{};
  a.A = A; a.B = B; a.M = M; a.N = N; a.K = K;
  a.lda = layout == LAYOUT_MN ? M : K;
  a.ldb = layout == LAYOUT_KK ? K : N;
  a.C = C; a.ldc = N; a.alpha = 1.f;
  hipStream_t st = (hipStream_t)stream;
  if (splits > 1) {
    int ks = 0;
    splits = gemm_real_splits(dtype, K, splits, &ks);
    a.k_split = ks;
    a.part = workspace;
    if (gemm_launch(a, dtype, layout, EPI_PARTIAL, tile, splits, st)) return fail(GPT_EINVAL, w + ": variant");
    splitk_reduce(workspace, splits, (long)M * N, C, 0, st);
  } else {
    a.k_split = K;
    if (gemm_launch(a, dtype, layout, EPI_STORE_F32, tile, 1, st)) return fail(GPT_EINVAL, w + ": variant");
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GPT_EHIP, w + ": launch: " + hipGetErrorString(e));
  return GPT_OK;
}

// RoPE table (nanochat User Guide, section 10, rotary embeddings): the pair
// (x[i], x[i + Dh/2]) of position t rotates by t * theta_i with
// theta_i = base^(-2i/Dh), i < Dh/2.  Evaluated in double, stored as fp32,
// [T][Dh/2] each for cos and sin.
void rope_table(const Shape& s, float* cosv, float* sinv) {
  const int half = s.Dh / 2;
  for (int t = 0; t < s.T; ++t)
    for (int i = 0; i < half; ++i) {
      const double th = std::pow((double)s.base, -2.0 * i / s.Dh);
      cosv[(size_t)t * half + i] = (float)std::cos(t * th);
      sinv[(size_t)t * half + i] = (float)std::sin(t * th);
    }
}

}  // namespace gm

namespace gm __attribute__((visibility("hidden"))) {

int build_layout(gpt_model& m) {
  const Shape& s = m.s;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t A = s.es;  // activation element size
  const size_t BT = s.BT;
  m.lay.resize(s.L);
  for (int l = 0; l < s.L; ++l) {
    auto& L = m.lay[l];
    L.n1 = take(BT * s.d * A);
    L.rstd1 = take(BT * 4);
    L.qkv = take(BT * s.Nqkv * A);
    L.rqk = take(BT * (s.H + s.Hkv) * 4);
    L.qT = take((size_t)s.B * s.H * s.Dh * s.Tp * A);
    L.kT = take((size_t)s.B * s.Hkv * s.Dh * s.Tp * A);
    L.vT = take((size_t)s.B * s.Hkv * s.Dh * s.Tp * A);
    L.o = take(BT * s.d * A);
    L.lse2 = take((size_t)s.B * s.H * s.Tp * 4);
    L.n2 = take(BT * s.d * A);
    L.rstd2 = take(BT * 4);
    // fp8: u is kept in fp32, so that du = dg * 2 relu(u) is computed from the
    // value the forward encoded
    L.u = take(BT * s.F * (s.fp8 ? 4 : A));
    L.g = take(BT * s.F * A);
  }
  m.h = take(BT * s.d * 4);
  m.nL = take(BT * s.d * A);
  m.rstdL = take(BT * 4);
  m.xent_tile = s.dtype == DT_F32 ? TILE_64x64 : TILE_256x256_W8;
  const int wn = tile_wn(m.xent_tile);
  m.xent_nblk = (s.V + wn - 1) / wn;
  m.part = take(BT * m.xent_nblk * 2 * 4);
  m.tgt = take(BT * 4);
  m.lse = take(BT * 4);
  m.rowloss = take(BT * 4);
  m.lossdev = take(64);
  m.flag = take(64);
  m.mloss = take((size_t)MAX_MICRO * 4);   // per-micro-batch losses of gpt_step_micro
  // decoding: attention split partials (128 keys per split), the step's
  // token ids and position
  m.dpart = take((size_t)s.B * s.H * ((s.T + 127) / 128) * (s.Dh + 1) * 4);
  m.dtok = take((size_t)s.B * 4);
  m.dsplit = take((size_t)DEC_KSPLIT * s.B * std::max(s.d, s.F) * 4);
  m.dpos = take(64);
  m.dz = take(BT * std::min(s.V, VOCAB_CHUNK) * A);   // one vocabulary chunk of the logit gradient
  m.dm = take(BT * s.d * 4);
  m.dh = take(BT * s.d * 4);
  m.dhA = take(BT * s.d * A);
  m.du = take(BT * s.F * A);
  m.dO = take(BT * s.d * A);
  m.dOT = take((size_t)s.B * s.H * s.Dh * s.Tp * A);
  m.Dv = take((size_t)s.B * s.H * s.Tp * 4);
  m.dqkv = take(BT * s.Nqkv * A);
  // split-K partials: the largest need among the planned products; the
  // weight-gradient products (which may run on the handle's second stream)
  // have a region of their own
  size_t need = 0, need2 = 0;
  auto consider = [&](int layout, int M, int N, int K) {
    size_t& nd = layout == LAYOUT_MN ? need2 : need;
    GemmPlan g = plan_gemm(s.dtype, layout, M, N, K);
    if (g.splits > 1) nd = std::max(nd, (size_t)g.splits * M * N);
    const TailPlan tp = plan_tail(s.dtype, layout, EPI_STORE_F32, M, N, K);
    if (tp.n1 > 0) nd = std::max(nd, (size_t)tp.splits * M * (N - tp.n1 * 256));
  };
  // the lm_head's products run one vocabulary chunk at a time
  const int vc = std::min(s.V, VOCAB_CHUNK);
  consider(LAYOUT_KN, s.BT, s.d, vc);
  consider(LAYOUT_MN, vc, s.d, s.BT);
  consider(LAYOUT_KN, s.BT, s.F, s.d);
  consider(LAYOUT_MN, s.d, s.F, s.BT);
  consider(LAYOUT_KN, s.BT, s.d, s.F);
  consider(LAYOUT_MN, s.F, s.d, s.BT);
  consider(LAYOUT_KN, s.BT, s.d, s.d);
  consider(LAYOUT_MN, s.d, s.d, s.BT);
  consider(LAYOUT_KN, s.BT, s.d, s.Nqkv);
  consider(LAYOUT_MN, s.Nqkv, s.d, s.BT);
  consider(LAYOUT_KK, s.BT, s.d, s.F);
  consider(LAYOUT_KK, s.BT, s.d, s.d);
  if (s.fp8) {
    for (int dty : {DT_FP8_A4B4, DT_FP8_A5B4}) {
      for (int K : {s.d, s.F, s.Nqkv}) {
        GemmPlan g = plan_gemm(dty, LAYOUT_KK, s.BT, s.d, K);
        if (g.splits > 1) need = std::max(need, (size_t)g.splits * s.BT * s.d);
      }
      const int MN[4][2] = {{s.Nqkv, s.d}, {s.d, s.d}, {s.F, s.d}, {s.d, s.F}};
      for (auto& mn : MN) {   // weight gradients
        GemmPlan g = plan_gemm(dty, LAYOUT_KK, mn[0], mn[1], s.BT);
        if (g.splits > 1) need2 = std::max(need2, (size_t)g.splits * mn[0] * mn[1]);
      }
    }
    const size_t wide = (size_t)std::max(s.F, s.Nqkv);
    for (int l = 0; l < s.L; ++l) {
      auto& L = m.lay[l];
      L.n1T = take(BT * s.d);
      L.oT = take(BT * s.d);
      L.n2T = take(BT * s.d);
      L.gT = take(BT * s.F);
      const size_t wsz[4] = {(size_t)s.Nqkv * s.d, (size_t)s.d * s.d, (size_t)s.F * s.d, (size_t)s.d * s.F};
      for (int k = 0; k < 4; ++k) {
        L.wq[k] = take(wsz[k]);
        L.wqT[k] = take(wsz[k]);
      }
    }
    m.q8row = take(BT * wide);
    m.f32w = take(BT * s.F * 4);
    m.q8T = take(BT * wide);
    m.q8T2 = take(BT * wide);   // the overlapped weight gradients alternate the transposed gradient codes
    m.n_slots = 12 * s.L;
    m.amax = take((size_t)m.n_slots * AMAX_SLOT * 4);
    m.scales = take((size_t)m.n_slots * 4);
  }
  m.splitk_floats = need;
  m.splitk = take(std::max<size_t>(need, 1) * 4);
  m.splitk2_floats = need2;
  m.splitk2 = take(std::max<size_t>(need2, 1) * 4);
  // second copies for the overlapped weight gradients: the residual
  // gradient's activation-type copy and the vocabulary chunk's logit gradient
  m.dhA2 = take(BT * s.d * A);
  m.dz2 = take(BT * std::min(s.V, VOCAB_CHUNK) * A);
  m.cosb = take((size_t)s.T * (s.Dh / 2) * 4);
  m.sinb = take((size_t)s.T * (s.Dh / 2) * 4);
  // the embedding gradient's counting sort: sorted positions, ranks, per-chunk
  // counts (chunks of 1024 positions), per-id totals and block-local starts,
  // block sums and offsets, the list of ids with rows
  m.keys = take(BT * 4);
  m.emb_rank = take(BT * 4);
  m.emb_cnt = take((BT + 1023) / 1024 * (size_t)s.V * 4);
  m.emb_tot = take((size_t)s.V * 4);
  m.emb_start = take((size_t)s.V * 4);
  m.emb_bsum = take((2 * (((size_t)s.V + 255) / 256) + 1) * 4);
  m.emb_heads = take(((size_t)s.V + 2) * 4);
  m.emb_part = take((size_t)emb_part_rows(s.BT) * s.d * 4);
  m.total = off;
  return GPT_OK;
}

// Site timing: prof_begin records an event before a launch, prof_end after
// it; gpt_step resolves the pairs once the stream has been synchronised.
hipEvent_t next_event(gpt_model& m) {
  if (m.ev_used == m.ev_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    m.ev_pool.push_back(e);
  }
  return m.ev_pool[m.ev_used++];
}

void prof_begin(gpt_model& m, const char* name, double work, int kind, const std::string& kernel) {
  if (!m.prof_on) return;
  int idx = -1;
  for (size_t i = 0; i < m.sites.size(); ++i)
    if (m.sites[i].name == name) { idx = (int)i; break; }
  if (idx < 0) {
    gpt_model::Site st;
    st.name = name;
    st.kernel = kernel;
    st.work_kind = kind;
    m.sites.push_back(st);
    idx = (int)m.sites.size() - 1;
  }
  hipEvent_t a = next_event(m), b = next_event(m);
  if (!a || !b) return;
  (void)hipEventRecord(a, m.st);
  m.pend.push_back(gpt_model::Pending{idx, work, a, b});
}

void prof_end(gpt_model& m) {
  if (!m.prof_on || m.pend.empty()) return;
  (void)hipEventRecord(m.pend.back().b, m.st);
}

void prof_collect(gpt_model& m) {
  for (auto& p : m.pend) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      m.sites[p.site].ms += ms;
      m.sites[p.site].launches += 1;
      m.sites[p.site].work += p.work;
    }
  }
  m.pend.clear();
  m.ev_used = 0;
}

// Causal / windowed visible (query, key) pairs of one sequence.
double visible_pairs(long T, long W) {
  if (W >= T) return 0.5 * (double)T * (double)(T + 1);
  return 0.5 * (double)W * (double)(W + 1) + (double)(T - W) * (double)W;
}

// One product with the planned tiling; splits go through the partial buffer
// and an ordered reduction into C (fp32).  Weight gradients (wgrad) keep the
// split plan of the storing form when they accumulate into C: the reduction
// then adds the partial sums to what C holds.
int gemm(gpt_model& m, const char* site, int layout, int epi, int M, int N, int K, const void* A, long lda,
         const void* B, long ldb, void* C, long ldc, GemmArgs extra = GemmArgs{}, int dtype = -1,
         bool wgrad = false) {
  const double flops = 2.0 * M * N * (double)K;
  const int dty = dtype < 0 ? m.s.dtype : dtype;
  GemmArgs a = extra;
  a.A = A; a.B = B; a.M = M; a.N = N; a.K = K; a.lda = lda; a.ldb = ldb; a.C = C; a.ldc = ldc;
  if (a.alpha == 0.f) a.alpha = 1.f;
  GemmPlan g = plan_gemm(dty, layout, M, N, K);
  if (epi == EPI_XENT_FWD) g = GemmPlan{m.xent_tile, 1, K};
  // the rotary epilogue runs the planned tile with one head of columns per wave
  if (epi == EPI_ROPE_QKN) g = GemmPlan{g.tile == TILE_256x256_PP4 ? TILE_256x256_PP4_H : TILE_128x128_H, 1, K};
  if (epi != EPI_STORE_F32 && !(wgrad && epi == EPI_ACCUM_F32)) g.splits = 1, g.k_split = K;
  if (g.splits > 1 && ldc != N) g.splits = 1, g.k_split = K;
  // A weight gradient on the second stream needs not fill the GPU alone,
  // since the input-gradient chain runs beside it: it takes the fewest K
  // splits (at most the planned ones) that give SIDE_WG_TARGET work-groups.
  // That saves most partial sums and their reduction while a product of a
  // few tiles does not run alone for its whole K.  Measured (ms per step):
  // unsplit d12 29.3 / d24 96.2 / d20 138.4; 64 work-groups 22.3 / 95.1 /
  // 136.6; the planned splits 22.0 / 98.9 / 140.7.  With the later plan
  // (input gradients keeping their last round), on one box: 64 work-groups
  // 22.1 / 96.5 / 137.2, 96 21.5 / 96.5 / 136.0, 128 21.4 / 97.3 / 136.8.
  if (wgrad && m.side && m.st == m.side) {
    const long tiles = (long)((M + tile_bm(g.tile) - 1) / tile_bm(g.tile)) * ((N + tile_bn(g.tile) - 1) / tile_bn(g.tile));
    int sp = 1;
    while (sp < g.splits && tiles * sp < SIDE_WG_TARGET) ++sp;
    if (sp == 1) g.splits = 1, g.k_split = K;
    else if (sp < g.splits) g.splits = gemm_real_splits(dty, K, sp, &g.k_split);
  }
  if (g.splits > 1) {
    // the partial sums must fit the workspace's split-K region (sized by
    // build_layout from the same plans); refuse rather than write past it
    if ((size_t)g.splits * M * N > (wgrad ? m.splitk2_floats : m.splitk_floats))
      return fail(GPT_EINVAL, std::string(site) + ": split-K partials exceed the planned workspace region");
    a.part = at<float>(m, wgrad ? m.splitk2 : m.splitk);
    a.k_split = g.k_split;
    char label[128];
    gemm_kernel_label(dty, layout, EPI_PARTIAL, g.tile, label, sizeof label);
    prof_begin(m, site, flops, 0, label);
    if (gemm_launch(a, dty, layout, EPI_PARTIAL, g.tile, g.splits, m.st))
      return fail(GPT_EINVAL, "gemm variant not instantiated (partial)");
    prof_end(m);
    const int acc = epi == EPI_ACCUM_F32;
    prof_begin(m, "splitk_reduce", (g.splits + 1.0 + acc) * M * N * 4.0, 1, "splitk_reduce_kernel");
    splitk_reduce(a.part, g.splits, (long)M * N, (float*)C, acc, m.st);
    prof_end(m);
    return GPT_OK;
  }
  a.k_split = K;
  char label[128];
  // An input gradient's partly filled last round of tiles is left as it is
  // when the weight gradients overlap the chain: their products fill the
  // idle CUs, and the K split of that round and its reduction are saved
  // (measured: d24 94.2 -> 93.7 ms, d20 133.6 -> 132.8 ms per step).
  const bool keep_tail = layout == LAYOUT_KN && m.overlap && m.side && !m.prof_on;
  const TailPlan tp = keep_tail ? TailPlan{0, 1} : plan_tail(dty, layout, epi, M, N, K);
  if (tp.n1 > 0) {
    // whole rounds: the first n1 tile columns
    const int N1 = tp.n1 * 256, N2 = N - N1;
    a.N = N1;
    gemm_kernel_label(dty, layout, epi, g.tile, label, sizeof label);
    prof_begin(m, site, flops * N1 / N, 0, label);
    if (gemm_launch(a, dty, layout, epi, g.tile, 1, m.st)) return fail(GPT_EINVAL, "gemm variant not instantiated");
    prof_end(m);
    // the remaining columns, split along K
    GemmArgs t = a;
    const size_t es = 2;   // bf16 operands (plan_tail admits no other type)
    t.B = (const char*)B + (layout == LAYOUT_KK ? (size_t)N1 * ldb : (size_t)N1) * es;
    t.N = N2;
    int ks = (K + tp.splits - 1) / tp.splits;
    ks = (ks + 63) / 64 * 64;
    const int sp = (K + ks - 1) / ks;
    if ((size_t)sp * M * N2 > (wgrad ? m.splitk2_floats : m.splitk_floats))
      return fail(GPT_EINVAL, std::string(site) + ": split-K partials exceed the planned workspace region");
    t.k_split = ks;
    t.part = at<float>(m, wgrad ? m.splitk2 : m.splitk);
    gemm_kernel_label(dty, layout, EPI_PARTIAL, g.tile, label, sizeof label);
    prof_begin(m, site, flops * N2 / N, 0, label);
    if (gemm_launch(t, dty, layout, EPI_PARTIAL, g.tile, sp, m.st))
      return fail(GPT_EINVAL, "gemm variant not instantiated (partial)");
    prof_end(m);
    const bool c16 = epi == EPI_STORE;   // bf16 C
    prof_begin(m, "splitk_reduce", (sp + (c16 ? 0.5 : 1.0 + (epi == EPI_ACCUM_F32))) * M * (double)N2 * 4.0, 1,
               "splitk_reduce_strided_kernel");
    splitk_reduce_strided(t.part, sp, M, N2, (char*)C + (size_t)N1 * (c16 ? 2 : 4), ldc, epi == EPI_ACCUM_F32, c16,
                          m.st);
    prof_end(m);
    return GPT_OK;
  }
  gemm_kernel_label(dty, layout, epi, g.tile, label, sizeof label);
  prof_begin(m, site, flops, 0, label);
  if (gemm_launch(a, dty, layout, epi, g.tile, 1, m.st))
    return fail(GPT_EINVAL, "gemm variant not instantiated");
  prof_end(m);
  return GPT_OK;
}

// One forward+backward pass.  Every gradient is linear in the logit gradient,
// so grad_scale is applied there (once); with accumulate set, the weight
// gradient products and the embedding scatter add to grads instead of
// overwriting it.  `shape` (default: the model's) may describe fewer tokens
// per row; forward_only stops after the final norm (prefill).
int run_step(gpt_model& m, const int32_t* tokens, const int32_t* targets, float* grads, float grad_scale,
             int accumulate, const Shape* shape, bool forward_only, float* loss_out, bool clear_flag,
             bool quant_weights) {
  const Shape& s = shape ? *shape : m.s;
  const ParamOffsets& P = m.po;
  const int dt = s.dtype;
  const size_t es = s.es;
  const char* W = m.W;
  auto wp = [&](long off) { return (const void*)(W + off * es); };
  hipStream_t st = m.st;
  const int BT = s.BT, d = s.d, F = s.F, V = s.V, H = s.H, Dh = s.Dh, Hkv = s.Hkv, Nqkv = s.Nqkv;
  float* h = at<float>(m, m.h);
  int* flag = at<int>(m, m.flag);
  const float* cosb = at<float>(m, m.cosb);
  const float* sinb = at<float>(m, m.sinb);
  int rc;

  const double es_d = (double)es;
  const std::string tname = dt == DT_BF16 ? "bf16" : "float";
  auto KL = [&](const char* k) { return std::string(k) + "<" + tname + ">"; };
  auto norm_label = [&](const char* k) {
    const int nch = norm_chunks(d);
    return nch ? std::string(k) + "_reg_kernel<" + tname + ", " + std::to_string(nch) + ">"
               : std::string(k) + "_kernel<" + tname + ">";
  };
  auto KLD = [&](const char* k, const char* extra = "") {
    return std::string(k) + "<" + tname + ", " + std::to_string(Dh) + extra + ">";
  };
  // kernels with a separate bf16, head-128 form
  auto KLV = [&](const char* k, const char* k128) { return dt == DT_BF16 && Dh == 128 ? std::string(k128) : KLD(k); };
  // fp8 linear layers: per-tensor scale slots (12 per layer), transient codes
  enum { SL_N1, SL_O, SL_N2, SL_G, SL_WQKV, SL_WO, SL_W1, SL_W2, SL_DH2, SL_DU, SL_DH1, SL_DQKV };
  const bool f8 = s.fp8;
  unsigned* amax8 = f8 ? at<unsigned>(m, m.amax) : nullptr;
  float* sc8 = f8 ? at<float>(m, m.scales) : nullptr;
  void* q8row = f8 ? m.ws + m.q8row : nullptr;
  void* q8T = f8 ? m.ws + m.q8T : nullptr;
  auto slot = [](int l, int k) { return 12 * l + k; };
  // Weights get their own amax pass; every activation and gradient operand's
  // amax is folded in by the kernel that produces it (the slot's pointer is
  // passed to that kernel), so its quantisation reads it once.
  // x32: the operand is fp32 (times rowscale[r], a norm's rstd, when given):
  // activations and gradients are encoded from the fp32 values their
  // producers computed, not from a bf16-rounded copy
  auto quant = [&](const char* site, int fmt, const void* x, int R, int C, int sl, void* q, void* qT,
                   bool amax_done = true, bool x32 = false, const float* rowscale = nullptr, bool relu2 = false) {
    prof_begin(m, site, (double)R * C * ((x32 ? 4.0 : 2.0) + (qT ? 2.0 : 1.0)), 1,
               std::string(amax_done ? "" : "amax_kernel + ") + "quant_kernel<" + (fmt == FP8_E4M3 ? "0" : "1") +
                   (x32 ? ", float" : ", bf16") + (relu2 ? ", relu2>" : ">"));
    unsigned* am = amax8 + (size_t)sl * AMAX_SLOT;
    if (!amax_done) fp8_amax(x, (long)R * C, am, st);
    fp8_quantize(fmt, x, R, C, am, sc8 + sl, q, qT, st, x32 ? 1 : 0, rowscale, relu2 ? 1 : 0);
    prof_end(m);
  };
  auto amx = [&](int l, int k) { return f8 && l >= 0 ? amax8 + (size_t)slot(l, k) * AMAX_SLOT : (unsigned*)nullptr; };
  auto gemm8 = [&](const char* site, int dty, int epi, int M, int N, int K, const void* A, const void* B, void* C,
                   long ldc, int sa, int sb, GemmArgs ex = GemmArgs{}) {
    ex.scale_a = sc8 + sa;
    ex.scale_b = sc8 + sb;
    return gemm(m, site, LAYOUT_KK, epi, M, N, K, A, K, B, K, C, ldc, ex, dty);
  };
  // weight-gradient products: store or accumulate into grads.  With overlap
  // they run on the handle's second stream: each forks from the main stream
  // once its inputs are written, and `done` receives an event after it, on
  // which the main stream waits before it overwrites a transient input of
  // that product (the activation gradient it reads).
  const int wepi = accumulate ? EPI_ACCUM_F32 : EPI_STORE_F32;
  const bool ov = m.overlap && m.side && !m.prof_on && !forward_only;
  hipEvent_t ev_last = nullptr;   // the side stream's last product
  auto ov_event = [&]() -> hipEvent_t {
    if (m.ov_next == m.ov_ev.size()) return nullptr;
    return m.ov_ev[m.ov_next++];
  };
  auto wait_for = [&](hipEvent_t& e) {
    if (!e) return GPT_OK;
    const hipError_t r = hipStreamWaitEvent(st, e, 0);
    e = nullptr;
    return r == hipSuccess ? GPT_OK : fail(GPT_EHIP, std::string("hipStreamWaitEvent: ") + hipGetErrorString(r));
  };
  auto wgrad = [&](const char* site, int M, int N, int K, const void* A, long lda, const void* B, long ldb,
                   float* C, long ldc, hipEvent_t* done = nullptr) {
    if (!ov) return gemm(m, site, LAYOUT_MN, wepi, M, N, K, A, lda, B, ldb, C, ldc, GemmArgs{}, -1, true);
    hipEvent_t fork = ov_event(), join = ov_event();
    if (!fork || !join) return fail(GPT_EINVAL, "overlap event ring exhausted");
    HIP_TRY(hipEventRecord(fork, st));
    HIP_TRY(hipStreamWaitEvent(m.side, fork, 0));
    m.st = m.side;
    const int r = gemm(m, site, LAYOUT_MN, wepi, M, N, K, A, lda, B, ldb, C, ldc, GemmArgs{}, -1, true);
    m.st = st;
    if (r) return r;
    HIP_TRY(hipEventRecord(join, m.side));
    ev_last = join;
    if (done) *done = join;
    return GPT_OK;
  };
  // fp8 weight gradients: the transposed gradient codes (A) are transient,
  // so with overlap the quantiser alternates two buffers (next_q8T), and
  // `done` receives the event after which the buffer this product read may
  // be rewritten
  auto wgrad8 = [&](const char* site, int M, int N, int K, const void* A, const void* B, float* C, long ldc, int sa,
                    int sb, hipEvent_t* done) {
    GemmArgs ex{};
    ex.scale_a = sc8 + sa;
    ex.scale_b = sc8 + sb;
    if (!ov) return gemm(m, site, LAYOUT_KK, wepi, M, N, K, A, K, B, K, C, ldc, ex, DT_FP8_A5B4, true);
    hipEvent_t fork = ov_event(), join = ov_event();
    if (!fork || !join) return fail(GPT_EINVAL, "overlap event ring exhausted");
    HIP_TRY(hipEventRecord(fork, st));
    HIP_TRY(hipStreamWaitEvent(m.side, fork, 0));
    m.st = m.side;
    const int r = gemm(m, site, LAYOUT_KK, wepi, M, N, K, A, K, B, K, C, ldc, ex, DT_FP8_A5B4, true);
    m.st = st;
    if (r) return r;
    HIP_TRY(hipEventRecord(join, m.side));
    ev_last = join;
    *done = join;
    return GPT_OK;
  };
  int kq = 0;
  hipEvent_t ev_q8T[2] = {nullptr, nullptr};
  auto next_q8T = [&](void*& qt) {
    if (ov) kq ^= 1;
    qt = kq ? m.ws + m.q8T2 : q8T;
    return wait_for(ev_q8T[kq]);   // the product that read this buffer last is done
  };

  m.ov_next = 0;
  if (clear_flag) fill_f32((float*)flag, 1, 0.f, st);
  // fp8: the weights' codes and scales are made here, unless the caller
  // knows they are those of the previous step (unchanged weights)
  if (f8) {
    zero_u32(amax8, m.n_slots * AMAX_SLOT, st);
    for (int l = 0; l < s.L && quant_weights; ++l) {
      auto& Ly = m.lay[l];
      quant("fp8_quant_weights", FP8_E4M3, wp(P.Wqkv[l]), Nqkv, d, slot(l, SL_WQKV), m.ws + Ly.wq[0], m.ws + Ly.wqT[0], false);
      quant("fp8_quant_weights", FP8_E4M3, wp(P.Wo[l]), d, d, slot(l, SL_WO), m.ws + Ly.wq[1], m.ws + Ly.wqT[1], false);
      quant("fp8_quant_weights", FP8_E4M3, wp(P.W1[l]), F, d, slot(l, SL_W1), m.ws + Ly.wq[2], m.ws + Ly.wqT[2], false);
      quant("fp8_quant_weights", FP8_E4M3, wp(P.W2[l]), d, F, slot(l, SL_W2), m.ws + Ly.wq[3], m.ws + Ly.wqT[3], false);
    }
  }
  prof_begin(m, "embed_fwd", (double)BT * d * (es_d + 4.0) + BT * 8.0, 1, KL("embed_fwd_kernel"));
  embed_fwd(dt, tokens, targets, wp(P.E), h, BT, d, V, flag, st);
  prof_end(m);
  // bf16 heads of 128 over whole 64-token blocks: the rotary step and QK norm
  // run in the QKV product's epilogue
  const bool rope_fused = dt == DT_BF16 && Dh == 128 && s.T % 64 == 0 && m.rope_epilogue;
  for (int l = 0; l < s.L; ++l) {
    auto& Ly = m.lay[l];
    const double pairs = (double)s.B * H * visible_pairs(s.T, s.win[l]);
    prof_begin(m, "rmsnorm_fwd", (double)BT * d * (4.0 + es_d) + BT * 4.0, 1, norm_label("rmsnorm_fwd"));
    rmsnorm_fwd(dt, h, m.ws + Ly.n1, at<float>(m, Ly.rstd1), BT, d, s.eps, st, amx(l, SL_N1));
    prof_end(m);
    if (f8) {
      quant("fp8_quant_act", FP8_E4M3, h, BT, d, slot(l, SL_N1), q8row, m.ws + Ly.n1T, true, true,
            at<float>(m, Ly.rstd1));
      rc = gemm8("gemm_qkv", DT_FP8_A4B4, EPI_STORE, BT, Nqkv, d, q8row, m.ws + Ly.wq[0], m.ws + Ly.qkv, Nqkv,
                 slot(l, SL_N1), slot(l, SL_WQKV));
    } else if (rope_fused) {
      // the product's epilogue rotates and normalises q and k and writes the
      // transposed copies
      GemmArgs ex{};
      ex.rope_cos = cosb; ex.rope_sin = sinb; ex.rqk = at<float>(m, Ly.rqk);
      ex.qT = m.ws + Ly.qT; ex.kT = m.ws + Ly.kT; ex.vT = m.ws + Ly.vT;
      ex.seqT = s.T; ex.nH = H; ex.nHkv = Hkv; ex.eps = s.eps;
      rc = gemm(m, "gemm_qkv_rope", LAYOUT_KK, EPI_ROPE_QKN, BT, Nqkv, d, m.ws + Ly.n1, d, wp(P.Wqkv[l]), d,
                m.ws + Ly.qkv, Nqkv, ex);
    } else {
      rc = gemm(m, "gemm_qkv", LAYOUT_KK, EPI_STORE, BT, Nqkv, d, m.ws + Ly.n1, d, wp(P.Wqkv[l]), d, m.ws + Ly.qkv,
                Nqkv);
    }
    if (rc) return rc;
    if (!rope_fused || f8) {
      // reads q, k, v; writes q^, k^ in place and the transposed q^, k^, v
      prof_begin(m, "rope_qknorm_fwd", (double)BT * (3.0 * d + 5.0 * s.dkv) * es_d + BT * (double)(H + Hkv) * 4.0, 1,
                 KLV("rope_qknorm_fwd_kernel", "rope_qknorm_fwd128_kernel"));
      rope_qknorm_fwd(dt, m.ws + Ly.qkv, at<float>(m, Ly.rqk), m.ws + Ly.qT, m.ws + Ly.kT, m.ws + Ly.vT, cosb, sinb,
                      s.B, s.T, s.Tp, H, Hkv, Dh, s.eps, st);
      prof_end(m);
    }
    AttnArgs aa{};
    aa.qkv = m.ws + Ly.qkv; aa.qT = m.ws + Ly.qT; aa.kT = m.ws + Ly.kT; aa.vT = m.ws + Ly.vT;
    aa.o = m.ws + Ly.o; aa.lse2 = at<float>(m, Ly.lse2);
    aa.B = s.B; aa.T = s.T; aa.Tp = s.Tp; aa.H = H; aa.Hkv = Hkv; aa.d = d; aa.ldqkv = Nqkv; aa.window = s.win[l];
    aa.scale = 1.0f / std::sqrt((float)Dh);
    aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)Dh));
    aa.amax_o = amx(l, SL_O);
    prof_begin(m, s.win[l] < s.T ? "attn_fwd_window" : "attn_fwd_causal", 4.0 * Dh * pairs, 0,
               KLD("attn_fwd_kernel"));
    if (attn_fwd(dt, Dh, aa, st)) return fail(GPT_EINVAL, "attention variant not instantiated");
    prof_end(m);
    if (f8) {
      quant("fp8_quant_act", FP8_E4M3, m.ws + Ly.o, BT, d, slot(l, SL_O), q8row, m.ws + Ly.oT);
      rc = gemm8("gemm_o", DT_FP8_A4B4, EPI_ACCUM_F32, BT, d, d, q8row, m.ws + Ly.wq[1], h, d, slot(l, SL_O),
                 slot(l, SL_WO));
    } else {
      rc = gemm(m, "gemm_o", LAYOUT_KK, EPI_ACCUM_F32, BT, d, d, m.ws + Ly.o, d, wp(P.Wo[l]), d, h, d);
    }
    if (rc) return rc;
    prof_begin(m, "rmsnorm_fwd", (double)BT * d * (4.0 + es_d) + BT * 4.0, 1, norm_label("rmsnorm_fwd"));
    rmsnorm_fwd(dt, h, m.ws + Ly.n2, at<float>(m, Ly.rstd2), BT, d, s.eps, st, amx(l, SL_N2));
    prof_end(m);
    GemmArgs ex{};
    ex.C2 = f8 ? nullptr : m.ws + Ly.g;   // fp8: relu(u)^2 is recomputed from u by its quantiser
    ex.amax = amx(l, SL_G);
    if (f8) {
      quant("fp8_quant_act", FP8_E4M3, h, BT, d, slot(l, SL_N2), q8row, m.ws + Ly.n2T, true, true,
            at<float>(m, Ly.rstd2));
      if ((rc = gemm8("gemm_w1_relu2", DT_FP8_A4B4, EPI_RELU2_F32, BT, F, d, q8row, m.ws + Ly.wq[2], m.ws + Ly.u, F,
                      slot(l, SL_N2), slot(l, SL_W1), ex)))
        return rc;
      quant("fp8_quant_act", FP8_E4M3, m.ws + Ly.u, BT, F, slot(l, SL_G), q8row, m.ws + Ly.gT, true, true, nullptr,
            true);
      rc = gemm8("gemm_w2", DT_FP8_A4B4, EPI_ACCUM_F32, BT, d, F, q8row, m.ws + Ly.wq[3], h, d, slot(l, SL_G),
                 slot(l, SL_W2));
    } else {
      if ((rc = gemm(m, "gemm_w1_relu2", LAYOUT_KK, EPI_RELU2, BT, F, d, m.ws + Ly.n2, d, wp(P.W1[l]), d, m.ws + Ly.u,
                     F, ex)))
        return rc;
      rc = gemm(m, "gemm_w2", LAYOUT_KK, EPI_ACCUM_F32, BT, d, F, m.ws + Ly.g, F, wp(P.W2[l]), F, h, d);
    }
    if (rc) return rc;
  }
  prof_begin(m, "rmsnorm_fwd", (double)BT * d * (4.0 + es_d) + BT * 4.0, 1, norm_label("rmsnorm_fwd"));
  rmsnorm_fwd(dt, h, m.ws + m.nL, at<float>(m, m.rstdL), BT, d, s.eps, st);
  prof_end(m);
  if (forward_only) {
    HIP_TRY(hipGetLastError());
    return GPT_OK;
  }
  {
    GemmArgs ex{};
    ex.aux = targets;
    ex.part = at<float>(m, m.part);
    ex.tgt = at<float>(m, m.tgt);
    ex.nblk = m.xent_nblk;
    if ((rc = gemm(m, "gemm_lm_head_xent_fwd", LAYOUT_KK, EPI_XENT_FWD, BT, V, d, m.ws + m.nL, d, wp(P.U), d, nullptr, V, ex))) return rc;
  }
  prof_begin(m, "xent_reduce", (double)BT * m.xent_nblk * 8.0 + BT * 12.0, 1, "xent_reduce_kernel + mean_reduce_kernel");
  xent_reduce(at<float>(m, m.part), at<float>(m, m.tgt), BT, m.xent_nblk, at<float>(m, m.lse),
              at<float>(m, m.rowloss), st);
  mean_reduce(at<float>(m, m.rowloss), BT, loss_out ? loss_out : at<float>(m, m.lossdev), st);
  prof_end(m);

  // ---------------------------------------------------------------- backward
  // The input gradients of the products that feed a norm backward (lm_head,
  // W1, Wqkv) are stored bf16 in the bf16 configuration, as the other
  // activation gradients are; the residual gradient dh stays fp32.
  void* dm = m.ws + m.dm;
  const bool dn_act = dt == DT_BF16 && !f8 && norm_chunks(d) != 0;
  const int epi_dn = dn_act ? EPI_STORE : EPI_STORE_F32;
  float* dh = at<float>(m, m.dh);
  // the norm backward writes the two copies of dhA in turn, so that a
  // weight gradient still reading one copy overlaps the next norm backward
  void* const dhAb[2] = {m.ws + m.dhA, m.ws + m.dhA2};
  hipEvent_t ev_dhA[2] = {nullptr, nullptr}, ev_du = nullptr, ev_dqkv = nullptr, ev_dz[2] = {nullptr, nullptr};
  int kA = 1;
  void* dhA = dhAb[0];
  auto norm_bwd = [&](const void* y, const float* rstd, int accumulate, unsigned* amax, bool dy_act) {
    kA ^= 1;
    int r = wait_for(ev_dhA[kA]);
    if (r) return r;
    dhA = dhAb[kA];
    const double dy_b = dy_act ? 2.0 : 4.0;   // bytes per dy element read
    prof_begin(m, "rmsnorm_bwd", (double)BT * d * (dy_b + 4.0 + 4.0 * accumulate + 2.0 * es_d), 1,
               norm_label("rmsnorm_bwd"));
    r = rmsnorm_bwd(dt, dm, dy_act, y, rstd, at<float>(m, m.dh), dhA, BT, d, accumulate, st, amax);
    prof_end(m);
    return r ? fail(GPT_EINVAL, "rmsnorm_bwd variant not built") : GPT_OK;
  };
  // Cross-entropy + lm_head backward, one vocabulary chunk of VOCAB_CHUNK
  // columns at a time: the chunk's logits are recomputed and its logit
  // gradient dz = (softmax - onehot) * grad_scale / BT formed in the
  // product's epilogue; the input gradient of the lm_head accumulates the
  // chunk's share (dn += dz U_c, fp32), and the chunk's rows of dU are
  // written.  Neither the logits nor their gradient exist for the whole
  // vocabulary at once.
  const bool vchunked = V > VOCAB_CHUNK;
  for (int v0 = 0; v0 < V; v0 += VOCAB_CHUNK) {
    const int vn = std::min(VOCAB_CHUNK, V - v0);
    GemmArgs ex{};
    ex.aux = targets;
    ex.auxf = at<float>(m, m.lse);
    ex.beta = grad_scale / (float)BT;
    ex.col0 = v0;
    const long uoff = P.U + (long)v0 * d;
    const int kz = (v0 / VOCAB_CHUNK) & 1;   // chunks alternate between two dz buffers
    void* dz = kz ? m.ws + m.dz2 : m.ws + m.dz;
    if ((rc = wait_for(ev_dz[kz]))) return rc;
    if ((rc = gemm(m, "gemm_lm_head_xent_bwd", LAYOUT_KK, EPI_XENT_BWD, BT, vn, d, m.ws + m.nL, d, wp(uoff), d, dz,
                   vn, ex)))
      return rc;
    const int epi = !vchunked ? epi_dn : v0 == 0 ? EPI_STORE_F32 : EPI_ACCUM_F32;
    if ((rc = gemm(m, "dgrad_lm_head", LAYOUT_KN, epi, BT, d, vn, dz, vn, wp(uoff), d, dm, d))) return rc;
    if ((rc = wgrad("wgrad_lm_head", vn, d, BT, dz, vn, m.ws + m.nL, d, grads + uoff, d, &ev_dz[kz]))) return rc;
  }
  if ((rc = norm_bwd(m.ws + m.nL, at<float>(m, m.rstdL), 0, amx(s.L - 1, SL_DH2), dn_act && !vchunked))) return rc;
  for (int l = s.L - 1; l >= 0; --l) {
    auto& Ly = m.lay[l];
    GemmArgs ex{};
    ex.aux = m.ws + Ly.u;
    ex.amax = amx(l, SL_DU);
    const double pairs = (double)s.B * H * visible_pairs(s.T, s.win[l]);
    if (f8) {
      void* qt = nullptr;
      if ((rc = next_q8T(qt))) return rc;
      quant("fp8_quant_grad", FP8_E5M2, dh, BT, d, slot(l, SL_DH2), q8row, qt, true, true);
      if ((rc = gemm8("dgrad_w2_drelu2", DT_FP8_A5B4, EPI_DRELU2_F32, BT, F, d, q8row, m.ws + Ly.wqT[3],
                      m.ws + m.f32w, F, slot(l, SL_DH2), slot(l, SL_W2), ex)))
        return rc;
      if ((rc = wgrad8("wgrad_w2", d, F, BT, qt, m.ws + Ly.gT, grads + P.W2[l], F, slot(l, SL_DH2),
                       slot(l, SL_G), &ev_q8T[kq])))
        return rc;
      if ((rc = next_q8T(qt))) return rc;
      quant("fp8_quant_grad", FP8_E5M2, m.ws + m.f32w, BT, F, slot(l, SL_DU), q8row, qt, true, true);
      if ((rc = gemm8("dgrad_w1", DT_FP8_A5B4, EPI_STORE_F32, BT, d, F, q8row, m.ws + Ly.wqT[2], dm, d,
                      slot(l, SL_DU), slot(l, SL_W1))))
        return rc;
      if ((rc = wgrad8("wgrad_w1", F, d, BT, qt, m.ws + Ly.n2T, grads + P.W1[l], d, slot(l, SL_DU),
                       slot(l, SL_N2), &ev_q8T[kq])))
        return rc;
    } else {
      if ((rc = wait_for(ev_du))) return rc;
      if ((rc = gemm(m, "dgrad_w2_drelu2", LAYOUT_KN, EPI_DRELU2, BT, F, d, dhA, d, wp(P.W2[l]), F, m.ws + m.du, F,
                     ex)))
        return rc;
      if ((rc = wgrad("wgrad_w2", d, F, BT, dhA, d, m.ws + Ly.g, F, grads + P.W2[l], F, &ev_dhA[kA])))
        return rc;
      if ((rc = gemm(m, "dgrad_w1", LAYOUT_KN, epi_dn, BT, d, F, m.ws + m.du, F, wp(P.W1[l]), d, dm, d)))
        return rc;
      if ((rc = wgrad("wgrad_w1", F, d, BT, m.ws + m.du, F, m.ws + Ly.n2, d, grads + P.W1[l], d, &ev_du)))
        return rc;
    }
    if ((rc = norm_bwd(m.ws + Ly.n2, at<float>(m, Ly.rstd2), 1, amx(l, SL_DH1), dn_act))) return rc;
    if (f8) {
      void* qt = nullptr;
      if ((rc = next_q8T(qt))) return rc;
      quant("fp8_quant_grad", FP8_E5M2, dh, BT, d, slot(l, SL_DH1), q8row, qt, true, true);
      if ((rc = gemm8("dgrad_o", DT_FP8_A5B4, EPI_STORE, BT, d, d, q8row, m.ws + Ly.wqT[1], m.ws + m.dO, d,
                      slot(l, SL_DH1), slot(l, SL_WO))))
        return rc;
      if ((rc = wgrad8("wgrad_o", d, d, BT, qt, m.ws + Ly.oT, grads + P.Wo[l], d, slot(l, SL_DH1),
                       slot(l, SL_O), &ev_q8T[kq])))
        return rc;
    } else {
      if ((rc = gemm(m, "dgrad_o", LAYOUT_KN, EPI_STORE, BT, d, d, dhA, d, wp(P.Wo[l]), d, m.ws + m.dO, d)))
        return rc;
      if ((rc = wgrad("wgrad_o", d, d, BT, dhA, d, m.ws + Ly.o, d, grads + P.Wo[l], d, &ev_dhA[kA])))
        return rc;
    }
    if ((rc = wait_for(ev_dqkv))) return rc;   // the attention backward rewrites dqkv
    prof_begin(m, "attn_bwd_pre", (double)BT * d * 3.0 * es_d + (double)s.B * H * s.Tp * 4.0, 1, KLV("attn_bwd_pre_kernel", "attn_bwd_pre128_kernel"));
    attn_bwd_pre(dt, m.ws + m.dO, m.ws + Ly.o, at<float>(m, m.Dv), m.ws + m.dOT, s.B, s.T, s.Tp, H, Dh, st);
    prof_end(m);
    AttnArgs aa{};
    aa.qkv = m.ws + Ly.qkv; aa.qT = m.ws + Ly.qT; aa.kT = m.ws + Ly.kT; aa.vT = m.ws + Ly.vT;
    aa.o = m.ws + Ly.o; aa.lse2 = at<float>(m, Ly.lse2);
    aa.dO = m.ws + m.dO; aa.dOT = m.ws + m.dOT; aa.Dv = at<float>(m, m.Dv); aa.dqkv = m.ws + m.dqkv;
    aa.amax_dv = amx(l, SL_DQKV);
    aa.B = s.B; aa.T = s.T; aa.Tp = s.Tp; aa.H = H; aa.Hkv = Hkv; aa.d = d; aa.ldqkv = Nqkv; aa.window = s.win[l];
    aa.scale = 1.0f / std::sqrt((float)Dh);
    aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)Dh));
    const bool win = s.win[l] < s.T;
    prof_begin(m, win ? "attn_bwd_dv_window" : "attn_bwd_dv_causal", 2.0 * Dh * pairs, 0,
               KLD("attn_bwd_dkdv_kernel", ", 32, 1"));
    if (attn_bwd(dt, Dh, aa, 0, st)) return fail(GPT_EINVAL, "attention variant not instantiated");
    prof_end(m);
    prof_begin(m, win ? "attn_bwd_dk_window" : "attn_bwd_dk_causal", 4.0 * Dh * pairs, 0,
               KLD("attn_bwd_dkdv_kernel", ", 32, 2"));
    if (attn_bwd(dt, Dh, aa, 1, st)) return fail(GPT_EINVAL, "attention variant not instantiated");
    prof_end(m);
    prof_begin(m, win ? "attn_bwd_dq_window" : "attn_bwd_dq_causal", 2.0 * Dh * pairs, 0,
               KLD("attn_bwd_dq_kernel"));
    if (attn_bwd(dt, Dh, aa, 2, st)) return fail(GPT_EINVAL, "attention variant not instantiated");
    prof_end(m);
    prof_begin(m, "rope_qknorm_bwd", (double)BT * (d + s.dkv) * 3.0 * es_d + BT * (double)(H + Hkv) * 4.0, 1,
               KLV("rope_qknorm_bwd_kernel", "rope_qknorm_bwd128_kernel"));
    rope_qknorm_bwd(dt, m.ws + m.dqkv, m.ws + Ly.qkv, at<float>(m, Ly.rqk), cosb, sinb, s.B, s.T, H, Hkv, Dh, st,
                    amx(l, SL_DQKV));
    prof_end(m);
    if (f8) {
      void* qt = nullptr;
      if ((rc = next_q8T(qt))) return rc;
      quant("fp8_quant_grad", FP8_E5M2, m.ws + m.dqkv, BT, Nqkv, slot(l, SL_DQKV), q8row, qt);
      if ((rc = gemm8("dgrad_qkv", DT_FP8_A5B4, EPI_STORE_F32, BT, d, Nqkv, q8row, m.ws + Ly.wqT[0], dm, d,
                      slot(l, SL_DQKV), slot(l, SL_WQKV))))
        return rc;
      if ((rc = wgrad8("wgrad_qkv", Nqkv, d, BT, qt, m.ws + Ly.n1T, grads + P.Wqkv[l], d, slot(l, SL_DQKV),
                       slot(l, SL_N1), &ev_q8T[kq])))
        return rc;
    } else {
      if ((rc = gemm(m, "dgrad_qkv", LAYOUT_KN, epi_dn, BT, d, Nqkv, m.ws + m.dqkv, Nqkv, wp(P.Wqkv[l]), d, dm,
                     d)))
        return rc;
      if ((rc = wgrad("wgrad_qkv", Nqkv, d, BT, m.ws + m.dqkv, Nqkv, m.ws + Ly.n1, d, grads + P.Wqkv[l], d,
                      &ev_dqkv)))
        return rc;
    }
    if ((rc = norm_bwd(m.ws + Ly.n1, at<float>(m, Ly.rstd1), 1, amx(l - 1, SL_DH2), dn_act))) return rc;
  }
  prof_begin(m, "embed_bwd", (double)BT * d * 4.0 + (double)V * d * (accumulate ? 8.0 : 4.0) + BT * 8.0, 1,
             "emb_rank_kernel + emb_prefix_kernel + emb_scan_kernel + emb_scatter_kernel + emb_short_kernel + emb_long_kernel + emb_long_sum_kernel");
  embed_bwd(tokens, dh, grads + P.E, BT, d, V, at<int>(m, m.keys), at<int>(m, m.emb_rank), at<int>(m, m.emb_cnt),
            at<int>(m, m.emb_tot), at<int>(m, m.emb_start), at<int>(m, m.emb_bsum), at<int>(m, m.emb_heads),
            at<float>(m, m.emb_part), accumulate, st);
  prof_end(m);
  if (ev_last) HIP_TRY(hipStreamWaitEvent(st, ev_last, 0));   // join: every weight gradient is written
  HIP_TRY(hipGetLastError());
  return GPT_OK;
}

// Graph-replay stream and events of the handle (created on first use).
int graph_stream(gpt_model& m) {
  auto& g = m.dg;
  if (!g.cs) {
    HIP_TRY(hipStreamCreateWithFlags(&g.cs, hipStreamNonBlocking));
    HIP_TRY(hipEventCreateWithFlags(&g.before, hipEventDisableTiming));
    HIP_TRY(hipEventCreateWithFlags(&g.after, hipEventDisableTiming));
  }
  return GPT_OK;
}

// The n micro-batch steps of gpt_step_micro, enqueued on m.st: the first
// stores or accumulates as asked, the rest accumulate; each writes its mean
// loss to mloss[i]; the token-range flag is cleared once and collects all.
// The weights cannot change within the call, so an fp8 model quantises them
// once, in the first step.
int run_micro(gpt_model& m, const int32_t* tokens, const int32_t* targets, int n, float* grads, float scale,
              int accumulate) {
  fill_f32(at<float>(m, m.flag), 1, 0.f, m.st);
  const long bt = m.s.BT;
  for (int i = 0; i < n; ++i) {
    const int rc = run_step(m, tokens + i * bt, targets + i * bt, grads, scale, i ? 1 : accumulate, nullptr, false,
                            at<float>(m, m.mloss) + i, false, i == 0);
    if (rc) return rc;
  }
  return GPT_OK;
}

// Replays the captured micro-batch sequence (capturing it first, or again
// when any argument differs from the captured one).
int micro_graph_launch(gpt_model& m, const int32_t* tokens, const int32_t* targets, int n, float* grads, float scale,
                       int accumulate) {
  int rc = graph_stream(m);
  if (rc) return rc;
  auto& g = m.mg;
  auto& d = m.dg;
  if (!g.exec || g.tokens != tokens || g.targets != targets || g.grads != grads || g.n != n ||
      g.accumulate != accumulate || g.scale != scale) {
    if (g.exec) (void)hipGraphExecDestroy(g.exec);
    if (g.graph) (void)hipGraphDestroy(g.graph);
    g.exec = nullptr;
    g.graph = nullptr;
    HIP_TRY(hipStreamBeginCapture(d.cs, hipStreamCaptureModeThreadLocal));
    hipStream_t saved = m.st;
    m.st = d.cs;
    rc = run_micro(m, tokens, targets, n, grads, scale, accumulate);
    m.st = saved;
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(d.cs, &graph);
    if (rc) {
      if (graph) (void)hipGraphDestroy(graph);
      return rc;
    }
    if (e != hipSuccess) return fail(GPT_EHIP, std::string("step graph capture: ") + hipGetErrorString(e));
    g.graph = graph;
    HIP_TRY(hipGraphInstantiate(&g.exec, g.graph, nullptr, nullptr, 0));
    g.tokens = tokens;
    g.targets = targets;
    g.grads = grads;
    g.n = n;
    g.accumulate = accumulate;
    g.scale = scale;
  }
  HIP_TRY(hipEventRecord(d.before, m.st));
  HIP_TRY(hipStreamWaitEvent(d.cs, d.before, 0));
  HIP_TRY(hipGraphLaunch(g.exec, d.cs));
  HIP_TRY(hipEventRecord(d.after, d.cs));
  HIP_TRY(hipStreamWaitEvent(m.st, d.after, 0));
  return GPT_OK;
}

}  // namespace gm

// ------------------------------------------------------------------ C ABI
extern "C" {

int gpt_param_layout(const gpt_config* cfg, gpt_tensor_desc* out, int capacity, int* n_tensors,
                     int64_t* total_elems) {
  Shape s;
  int rc = check_config(cfg, s);
  if (rc) return rc;
  ParamOffsets p;
  param_offsets(s, p);
  if (n_tensors) *n_tensors = (int)p.descs.size();
  if (total_elems) *total_elems = p.total;
  if (out) {
    if (capacity < (int)p.descs.size()) return fail(GPT_EINVAL, "capacity too small for the layout");
    for (size_t i = 0; i < p.descs.size(); ++i) out[i] = p.descs[i];
  }
  return GPT_OK;
}

int gpt_workspace_bytes(const gpt_config* cfg, size_t* bytes) {
  if (!bytes) return fail(GPT_ENULL, "bytes is NULL");
  gpt_model m{};
  int rc = check_config(cfg, m.s);
  if (rc) return rc;
  build_layout(m);
  *bytes = m.total;
  return GPT_OK;
}

int gpt_create(const gpt_config* cfg, gpt_model** out) {
  if (!out) return fail(GPT_ENULL, "out is NULL");
  *out = nullptr;
  gpt_model* m = new (std::nothrow) gpt_model();
  if (!m) return fail(GPT_EINVAL, "host allocation failed");
  int rc = check_config(cfg, m->s);
  if (rc) { delete m; return rc; }
  if (!cfg->weights || !cfg->workspace) { delete m; return fail(GPT_ENULL, "weights and workspace are required"); }
  if (((uintptr_t)cfg->weights | (uintptr_t)cfg->workspace) & (ALIGN - 1)) {
    delete m;
    return fail(GPT_EALIGN, "weights and workspace must be 256-byte aligned");
  }
  m->cfg = *cfg;
  param_offsets(m->s, m->po);
  build_layout(*m);
  if (cfg->workspace_bytes < m->total) {
    size_t need = m->total;
    delete m;
    return fail(GPT_ESPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  }
  m->st = (hipStream_t)cfg->stream;
  m->ws = (char*)cfg->workspace;
  m->W = (const char*)cfg->weights;
  // the second stream of the overlapped weight gradients (default priority)
  // and its fork / join events
  {
    hipError_t e = hipStreamCreateWithFlags(&m->side, hipStreamNonBlocking);
    for (int i = 0; e == hipSuccess && i < OV_EVENTS; ++i) {
      hipEvent_t ev;
      e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e == hipSuccess) m->ov_ev.push_back(ev);
    }
    if (e != hipSuccess) {
      delete m;
      return fail(GPT_EHIP, std::string("second stream / events: ") + hipGetErrorString(e));
    }
  }
  const int half = m->s.Dh / 2;
  std::vector<float> c((size_t)m->s.T * half), sn((size_t)m->s.T * half);
  rope_table(m->s, c.data(), sn.data());
  hipError_t e1 = hipMemcpyAsync(m->ws + m->cosb, c.data(), c.size() * 4, hipMemcpyHostToDevice, m->st);
  hipError_t e2 = hipMemcpyAsync(m->ws + m->sinb, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, m->st);
  hipError_t e3 = hipStreamSynchronize(m->st);
  if (e1 != hipSuccess || e2 != hipSuccess || e3 != hipSuccess) {
    delete m;
    return fail(GPT_EHIP, std::string("RoPE table upload failed: ") + hipGetErrorString(e1) + " / " +
                              hipGetErrorString(e2) + " / " + hipGetErrorString(e3));
  }
  *out = m;
  return GPT_OK;
}

int gpt_rope_table(const gpt_config* cfg, float* cos_out, float* sin_out) {
  if (!cos_out || !sin_out) return fail(GPT_ENULL, "gpt_rope_table: NULL output");
  Shape s;
  const int rc = check_config(cfg, s);
  if (rc) return rc;
  rope_table(s, cos_out, sin_out);
  return GPT_OK;
}

int gpt_step(gpt_model* m, const int32_t* tokens, const int32_t* targets, float* grads, float* loss) {
  return gpt_step_accum(m, tokens, targets, grads, 1.0f, 0, loss);
}

int gpt_step_accum(gpt_model* m, const int32_t* tokens, const int32_t* targets, float* grads, float grad_scale,
                   int accumulate, float* loss) {
  if (!m || !tokens || !targets || !grads || !loss) return fail(GPT_ENULL, "gpt_step: NULL argument");
  if ((uintptr_t)grads & (ALIGN - 1)) return fail(GPT_EALIGN, "grads must be 256-byte aligned");
  if (!std::isfinite(grad_scale)) return fail(GPT_EINVAL, "grad_scale must be finite");
  if (accumulate != 0 && accumulate != 1) return fail(GPT_EINVAL, "accumulate must be 0 or 1");
  int rc = run_step(*m, tokens, targets, grads, grad_scale, accumulate);
  if (rc) return rc;
  float lossv = 0.f;
  int flag = 0;
  HIP_TRY(hipMemcpyAsync(&lossv, m->ws + m->lossdev, 4, hipMemcpyDeviceToHost, m->st));
  HIP_TRY(hipMemcpyAsync(&flag, m->ws + m->flag, 4, hipMemcpyDeviceToHost, m->st));
  HIP_TRY(hipStreamSynchronize(m->st));
  if (m->prof_on) prof_collect(*m);
  *loss = lossv;
  if (flag) return fail(GPT_ETOKEN, "a token or target id is outside [0, vocab)");
  if (!std::isfinite(lossv)) return fail(GPT_ENONFINITE, "loss is not finite");
  return GPT_OK;
}

int gpt_step_micro(gpt_model* m, const int32_t* tokens, const int32_t* targets, int n_micro, float* grads,
                   float grad_scale, int accumulate, float* losses) {
  if (!m || !tokens || !targets || !grads || !losses) return fail(GPT_ENULL, "gpt_step_micro: NULL argument");
  if (n_micro < 1 || n_micro > MAX_MICRO) return fail(GPT_EINVAL, "n_micro must be in [1, 1024]");
  if ((uintptr_t)grads & (ALIGN - 1)) return fail(GPT_EALIGN, "grads must be 256-byte aligned");
  if (!std::isfinite(grad_scale)) return fail(GPT_EINVAL, "grad_scale must be finite");
  if (accumulate != 0 && accumulate != 1) return fail(GPT_EINVAL, "accumulate must be 0 or 1");
  int rc = m->prof_on ? run_micro(*m, tokens, targets, n_micro, grads, grad_scale, accumulate)
                      : micro_graph_launch(*m, tokens, targets, n_micro, grads, grad_scale, accumulate);
  if (rc) return rc;
  int flag = 0;
  HIP_TRY(hipMemcpyAsync(losses, m->ws + m->mloss, (size_t)n_micro * 4, hipMemcpyDeviceToHost, m->st));
  HIP_TRY(hipMemcpyAsync(&flag, m->ws + m->flag, 4, hipMemcpyDeviceToHost, m->st));
  HIP_TRY(hipStreamSynchronize(m->st));
  if (m->prof_on) prof_collect(*m);
  if (flag) return fail(GPT_ETOKEN, "a token or target id is outside [0, vocab)");
  for (int i = 0; i < n_micro; ++i)
    if (!std::isfinite(losses[i])) return fail(GPT_ENONFINITE, "a micro-batch loss is not finite");
  return GPT_OK;
}

void gpt_destroy(gpt_model* m) { delete m; }

int gpt_overlap_enable(gpt_model* m, int on) {
  if (!m) return fail(GPT_ENULL, "model is NULL");
  m->overlap = on != 0;
  return GPT_OK;
}

int gpt_rope_epilogue_enable(gpt_model* m, int on) {
  if (!m) return fail(GPT_ENULL, "model is NULL");
  m->rope_epilogue = on != 0;
  return GPT_OK;
}

int gpt_debug_tensor(gpt_model* m, int which, int layer, void** ptr, int64_t* rows, int64_t* cols,
                     int* elem_bytes) {
  if (!m || !ptr || !rows || !cols || !elem_bytes) return fail(GPT_ENULL, "NULL argument");
  const Shape& s = m->s;
  if ((which == 1 || which == 2 || which == 5) && (layer < 0 || layer >= s.L))
    return fail(GPT_EINVAL, "layer out of range");
  *rows = s.BT;
  *elem_bytes = s.es;
  switch (which) {
    case 0: *ptr = m->ws + m->h; *cols = s.d; *elem_bytes = 4; break;
    case 1: *ptr = m->ws + m->lay[layer].qkv; *cols = s.Nqkv; break;
    case 2: *ptr = m->ws + m->lay[layer].o; *cols = s.d; break;
    case 3: *ptr = m->ws + m->rowloss; *cols = 1; *elem_bytes = 4; break;
    case 4: *ptr = m->ws + m->lse; *cols = 1; *elem_bytes = 4; break;
    case 5: *ptr = m->ws + m->lay[layer].u; *cols = s.F; if (s.fp8) *elem_bytes = 4; break;
    default: return fail(GPT_EINVAL, "unknown tensor id");
  }
  return GPT_OK;
}

int gpt_gemm(int dtype, int layout, int M, int N, int K, const void* A, const void* B, float* C, float* workspace,
             int splits, int tile, void* stream) {
  int rc = gemm_check(dtype, layout, M, N, K, A, B, C, splits, tile, "gpt_gemm");
  if (rc) return rc;
  if (splits > 1 && !workspace) return fail(GPT_EINVAL, "gpt_gemm: splits > 1 needs a workspace");
  return gemm_entry(dtype, layout, M, N, K, A, B, C, workspace, splits, tile, stream, "gpt_gemm");
}

int gpt_fp8_quantize(int fmt, const void* x, int rows, int cols, uint32_t* amax, float* scale, void* q, void* qT,
                     void* stream) {
  if (!x || !amax || !scale || !q) return fail(GPT_ENULL, "gpt_fp8_quantize: NULL argument");
  if ((uintptr_t)x & 15) return fail(GPT_EALIGN, "gpt_fp8_quantize: x must be 16-byte aligned");
  if (fmt != FP8_E4M3 && fmt != FP8_E5M2) return fail(GPT_EINVAL, "gpt_fp8_quantize: fmt");
  if (rows < 1 || cols < 64 || cols % 64 || (long)rows * cols > (1L << 31))
    return fail(GPT_EINVAL, "gpt_fp8_quantize: sizes");
  hipStream_t st = (hipStream_t)stream;
  zero_u32(amax, AMAX_SLOT, st);
  fp8_amax(x, (long)rows * cols, amax, st);
  fp8_quantize(fmt, x, rows, cols, amax, scale, q, qT, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GPT_EHIP, std::string("launch: ") + hipGetErrorString(e));
  return GPT_OK;
}

int gpt_gemm_fp8(int fmt_a, int M, int N, int K, const void* A, const void* B, const float* scale_a,
                 const float* scale_b, float* C, float* workspace, int splits, void* stream) {
  if (!A || !B || !C || !scale_a || !scale_b) return fail(GPT_ENULL, "gpt_gemm_fp8: NULL argument");
  if (fmt_a != FP8_E4M3 && fmt_a != FP8_E5M2) return fail(GPT_EINVAL, "gpt_gemm_fp8: fmt_a");
  if (M < 1 || N < 1 || K < 16 || M % 8 || N % 8 || K % 16) return fail(GPT_EINVAL, "gpt_gemm_fp8: sizes");
  if (splits < 1 || (splits > 1 && !workspace)) return fail(GPT_EINVAL, "gpt_gemm_fp8: splits");
  const int dtype = fmt_a == FP8_E4M3 ? DT_FP8_A4B4 : DT_FP8_A5B4;
  GemmArgs a{};
  a.A = A; a.B = B; a.M = M; a.N = N; a.K = K; a.lda = K; a.ldb = K;
  a.C = C; a.ldc = N; a.alpha = 1.f; a.scale_a = scale_a; a.scale_b = scale_b;
  hipStream_t st = (hipStream_t)stream;
  if (splits > 1) {
    int ks = (K + splits - 1) / splits;
    ks = (ks + 127) / 128 * 128;
    splits = (K + ks - 1) / ks;
    a.k_split = ks;
    a.part = workspace;
    if (gemm_launch(a, dtype, LAYOUT_KK, EPI_PARTIAL, TILE_128x128, splits, st))
      return fail(GPT_EINVAL, "gpt_gemm_fp8: variant");
    splitk_reduce(workspace, splits, (long)M * N, C, 0, st);
  } else {
    a.k_split = K;
    if (gemm_launch(a, dtype, LAYOUT_KK, EPI_STORE_F32, TILE_128x128, 1, st))
      return fail(GPT_EINVAL, "gpt_gemm_fp8: variant");
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GPT_EHIP, std::string("launch: ") + hipGetErrorString(e));
  return GPT_OK;
}

int gpt_profile_enable(gpt_model* m, int on) {
  if (!m) return fail(GPT_ENULL, "model is NULL");
  m->prof_on = on != 0;
  m->sites.clear();
  m->pend.clear();
  m->ev_used = 0;
  return GPT_OK;
}

int gpt_profile_sites(gpt_model* m, int* n) {
  if (!m || !n) return fail(GPT_ENULL, "NULL argument");
  *n = (int)m->sites.size();
  return GPT_OK;
}

int gpt_profile_get(gpt_model* m, int i, char* name, int name_len, char* kernel, int kernel_len, int64_t* launches,
                    double* total_ms, double* work, int* work_kind) {
  if (!m || !name || !kernel || !launches || !total_ms || !work || !work_kind) return fail(GPT_ENULL, "NULL argument");
  if (i < 0 || i >= (int)m->sites.size()) return fail(GPT_EINVAL, "site index out of range");
  const auto& st = m->sites[i];
  snprintf(name, name_len, "%s", st.name.c_str());
  snprintf(kernel, kernel_len, "%s", st.kernel.c_str());
  *launches = st.launches;
  *total_ms = st.ms;
  *work = st.work;
  *work_kind = st.work_kind;
  return GPT_OK;
}

const char* gpt_strerror(int code) {
  switch (code) {
    case GPT_OK: return "ok";
    case GPT_EINVAL: return "invalid configuration or argument";
    case GPT_ENULL: return "NULL pointer";
    case GPT_ETOKEN: return "token id out of range";
    case GPT_EHIP: return "HIP runtime error";
    case GPT_ENONFINITE: return "non-finite loss";
    case GPT_ESPACE: return "workspace too small";
    case GPT_EALIGN: return "misaligned pointer";
    default: return "unknown error";
  }
}

const char* gpt_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
