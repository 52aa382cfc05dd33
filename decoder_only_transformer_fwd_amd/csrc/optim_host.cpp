// Host side of the optimizer step: the state plan (pass tables, buffer
// offsets) and the launch sequence of one Muon + AdamW update.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "model.h"

using namespace gk;
using namespace gm;

namespace gm __attribute__((visibility("hidden"))) {

// ------------------------------------------------------------------ optimizer
// Muon on every projection matrix, AdamW on E and U (the state holds fp32
// master weights for bf16 parameters, Muon momenta, AdamW moments, the pass
// lists and the Newton-Schulz buffers).
void optim_plan(const Shape& s, const ParamOffsets& P, OptPlan& o) {
  o = OptPlan{};
  std::vector<OptSeg> tab;
  long mom = 0;   // floats of momentum / moment state so far
  auto close_list = [&](OptPlan::List& l, std::vector<OptSeg> entries) {
    l.seg0 = (int)tab.size();
    l.n = (int)entries.size();
    int blk = 0;
    for (auto& e : entries) {
      e.blk0 = blk;
      blk += (int)((e.n + OPT_CHUNK - 1) / OPT_CHUNK);
      tab.push_back(e);
    }
    OptSeg sentinel{};
    sentinel.blk0 = blk;
    tab.push_back(sentinel);
    l.nblk = blk;
    o.max_part = std::max(o.max_part, blk);
  };
  auto seg_of = [](const gpt_tensor_desc& t) {
    OptSeg e{};
    e.off = t.offset;
    e.n = (long)t.rows * t.cols;
    return e;
  };
  // every tensor: the global gradient norm
  {
    std::vector<OptSeg> v;
    for (auto& t : P.descs) v.push_back(seg_of(t));
    close_list(o.all, v);
  }
  // Muon groups by shape, in layout order
  std::vector<std::pair<int, int>> shapes;
  for (auto& t : P.descs) {
    const bool mat = strcmp(t.name, "E") != 0 && strcmp(t.name, "U") != 0;
    if (mat && std::find(shapes.begin(), shapes.end(), std::make_pair(t.rows, t.cols)) == shapes.end())
      shapes.push_back({t.rows, t.cols});
  }
  size_t ns_need = 0;
  for (auto& sh : shapes) {
    OptPlan::Group g;
    g.rows = sh.first;
    g.cols = sh.second;
    std::vector<OptSeg> v;
    for (auto& t : P.descs) {
      if (!strcmp(t.name, "E") || !strcmp(t.name, "U") || t.rows != g.rows || t.cols != g.cols) continue;
      OptSeg e = seg_of(t);
      e.soff = mom;
      mom += e.n;
      e.xoff = (long)g.count * g.rows * g.cols;
      g.count++;
      v.push_back(e);
    }
    close_list(g.list, v);
    const long m = std::min(g.rows, g.cols);
    const size_t xbytes = align_up((size_t)g.count * g.rows * g.cols * 2);
    const size_t abytes = align_up((size_t)g.count * m * m * 2);
    ns_need = std::max(ns_need, 2 * xbytes + 2 * abytes);
    o.groups.push_back(g);
  }
  // AdamW: E (lr0), U (lr1)
  {
    std::vector<OptSeg> v;
    for (auto& t : P.descs) {
      if (strcmp(t.name, "E") && strcmp(t.name, "U")) continue;
      OptSeg e = seg_of(t);
      e.soff = mom;
      mom += 2 * e.n;
      e.which = strcmp(t.name, "U") == 0;
      v.push_back(e);
    }
    close_list(o.adam, v);
  }
  o.table_host = tab;
  o.has_master = s.dtype != DT_F32;
  size_t off = 0;
  o.hdr = off; off += ALIGN;
  o.table = off; off += align_up(tab.size() * sizeof(OptSeg));
  o.part = off; off += align_up((size_t)o.max_part * 4);
  o.master = off; off += o.has_master ? align_up((size_t)P.total * 4) : 0;
  o.mom = off; off += align_up((size_t)mom * 4);
  o.ns = off; off += ns_need;
  o.total = off;
}

// Newton-Schulz buffers of one group (byte offsets from the state base).
void ns_buffers(const OptPlan& o, const OptPlan::Group& g, size_t& xa, size_t& xb, size_t& ab, size_t& bb) {
  const long m = std::min(g.rows, g.cols);
  const size_t xbytes = align_up((size_t)g.count * g.rows * g.cols * 2);
  const size_t abytes = align_up((size_t)g.count * m * m * 2);
  xa = o.ns;
  xb = xa + xbytes;
  ab = xb + xbytes;
  bb = ab + abytes;
}

int ns_tile(int M, int N) { return M >= 256 && N >= 256 ? TILE_256x256_PP4 : TILE_128x128; }

// One batched bf16 product of the orthogonalisation: C = alpha * op(A, B)
// (+ beta * aux, aux laid out as C), `batch` members at element strides.
int ns_gemm(gpt_model& m, const char* site, int layout, int epi, int M, int N, int K, const void* A, long lda,
            long bsA, const void* B, long ldb, long bsB, void* C, long bsC, const void* aux, float alpha,
            float beta, int batch) {
  GemmArgs a{};
  a.A = A; a.B = B; a.C = C; a.aux = aux;
  a.M = M; a.N = N; a.K = K; a.lda = lda; a.ldb = ldb; a.ldc = N;
  a.alpha = alpha; a.beta = beta; a.k_split = K;
  a.bsA = bsA; a.bsB = bsB; a.bsC = bsC;
  const int tile = ns_tile(M, N);
  char label[128];
  gemm_kernel_label(DT_BF16, layout, epi, tile, label, sizeof label);
  std::string lab(label);
  lab.insert(lab.size() - 1, ", batched");
  // a symmetric product computes the tiles on and above the diagonal only
  const double t = (M + tile_bm(tile) - 1) / tile_bm(tile);
  const double frac = (epi == EPI_STORE_SYM || epi == EPI_AXPBY_SYM) ? (t + 1) / (2 * t) : 1.0;
  prof_begin(m, site, 2.0 * M * N * (double)K * batch * frac, 0, lab);
  if (gemm_launch_batched(a, layout, epi, tile, batch, m.st)) return fail(GPT_EINVAL, "batched gemm variant");
  prof_end(m);
  return GPT_OK;
}

// One optimizer step (enqueued on the model's stream).
int run_optim(gpt_model& m, char* state, const float* grads, const gpt_optim_params& hp, bool want_norm) {
  const OptPlan& o = m.opt;
  hipStream_t st = m.st;
  float* hdr = (float*)(state + o.hdr);
  const OptSeg* tab = (const OptSeg*)(state + o.table);
  float* part = (float*)(state + o.part);
  float* mom = (float*)(state + o.mom);
  // fp32 parameters are their own master copy; bf16 ones get a refreshed copy
  float* master = o.has_master ? (float*)(state + o.master) : (float*)m.W;
  void* w16 = o.has_master ? (void*)m.W : nullptr;
  const double n_all = (double)m.po.total;

  if (hp.grad_clip > 0.f || want_norm) {
    prof_begin(m, "optim_grad_norm", n_all * 4.0, 1, "opt_sumsq_kernel + opt_norm_kernel");
    opt_sumsq(grads, tab + o.all.seg0, o.all.n, o.all.nblk, part, st);
    opt_norm(part, o.all.nblk, hp.grad_clip, hdr, st);
    prof_end(m);
  } else {
    fill_f32(hdr + 1, 1, 1.f, st);   // clip coefficient 1
  }
  {
    AdamArgs a{};
    a.b1 = hp.beta1; a.b2 = hp.beta2; a.eps = hp.eps; a.wd = hp.weight_decay;
    a.ibc1 = (float)(1.0 / (1.0 - std::pow((double)hp.beta1, (double)hp.step)));
    a.ibc2 = (float)(1.0 / (1.0 - std::pow((double)hp.beta2, (double)hp.step)));
    a.lr0 = hp.embedding_lr;
    a.lr1 = hp.unembedding_lr;
    double n = 0;
    for (int i = 0; i < o.adam.n; ++i) n += (double)o.table_host[o.adam.seg0 + i].n;
    prof_begin(m, "optim_adamw", n * (o.has_master ? 30.0 : 28.0), 1, "opt_adamw_kernel");
    opt_adamw(master, mom, grads, w16, tab + o.adam.seg0, o.adam.n, o.adam.nblk, hdr, a, st);
    prof_end(m);
  }
  const float a_ns = 3.4445f, b_ns = -4.7750f, c_ns = 2.0315f;
  for (const auto& g : o.groups) {
    const int r = g.rows, c = g.cols, cnt = g.count;
    const bool tall = r > c;
    const int mm = tall ? c : r, kk = tall ? r : c;
    const long rc = (long)r * c, m2 = (long)mm * mm;
    size_t xa, xb, ab, bb;
    ns_buffers(o, g, xa, xb, ab, bb);
    char* X = state + xa;
    char* Y = state + xb;
    char* Am = state + ab;
    char* Bm = state + bb;
    const double n = (double)rc * cnt;
    prof_begin(m, "optim_muon_momentum", n * 12.0, 1, "opt_muon_momentum_kernel");
    opt_muon_momentum(grads, mom, tab + g.list.seg0, g.list.n, g.list.nblk, hdr, hp.momentum, hp.nesterov, part, st);
    prof_end(m);
    prof_begin(m, "optim_muon_normalise", n * 10.0, 1, "opt_muon_normalise_kernel");
    opt_muon_normalise(grads, mom, tab + g.list.seg0, g.list.n, g.list.nblk, hdr, hp.momentum, hp.nesterov, part, X,
                       st);
    prof_end(m);
    for (int it = 0; it < hp.ns_steps; ++it) {
      int rc2;
      // A = X X^T (wide) or X^T X (tall): [mm, mm], symmetric
      if (!tall)
        rc2 = ns_gemm(m, "ns_gram", LAYOUT_KK, EPI_STORE_SYM, mm, mm, kk, X, c, rc, X, c, rc, Am, m2, nullptr, 1.f,
                      0.f, cnt);
      else
        rc2 = ns_gemm(m, "ns_gram", LAYOUT_MN, EPI_STORE_SYM, mm, mm, kk, X, c, rc, X, c, rc, Am, m2, nullptr, 1.f,
                      0.f, cnt);
      if (rc2) return rc2;
      // B = b A + c A A (A symmetric, so A A = A A^T, and B is symmetric)
      if ((rc2 = ns_gemm(m, "ns_poly", LAYOUT_KK, EPI_AXPBY_SYM, mm, mm, mm, Am, mm, m2, Am, mm, m2, Bm, m2, Am,
                         c_ns, b_ns, cnt)))
        return rc2;
      // X' = a X + B X (wide) or a X + X B (tall; B symmetric)
      if (!tall)
        rc2 = ns_gemm(m, "ns_apply", LAYOUT_KN, EPI_AXPBY, r, c, r, Bm, mm, m2, X, c, rc, Y, rc, X, 1.f, a_ns, cnt);
      else
        rc2 = ns_gemm(m, "ns_apply", LAYOUT_KK, EPI_AXPBY, r, c, c, X, c, rc, Bm, mm, m2, Y, rc, X, 1.f, a_ns, cnt);
      if (rc2) return rc2;
      std::swap(X, Y);
    }
    const float scale = std::sqrt(std::max(1.0f, (float)r / (float)c));
    prof_begin(m, "optim_muon_update", n * (o.has_master ? 12.0 : 10.0), 1, "opt_muon_update_kernel");
    opt_muon_update(master, X, w16, tab + g.list.seg0, g.list.n, g.list.nblk, hp.matrix_lr, scale, hp.weight_decay,
                    st);
    prof_end(m);
  }
  HIP_TRY(hipGetLastError());
  return GPT_OK;
}

}  // namespace gm

extern "C" {

int gpt_optim_state_bytes(const gpt_config* cfg, size_t* bytes) {
  if (!bytes) return fail(GPT_ENULL, "bytes is NULL");
  Shape s;
  int rc = check_config(cfg, s);
  if (rc) return rc;
  ParamOffsets p;
  param_offsets(s, p);
  OptPlan o;
  optim_plan(s, p, o);
  *bytes = o.total;
  return GPT_OK;
}

int gpt_optim_init(gpt_model* m, void* state, size_t state_bytes) {
  if (!m || !state) return fail(GPT_ENULL, "gpt_optim_init: NULL argument");
  if ((uintptr_t)state & (ALIGN - 1)) return fail(GPT_EALIGN, "state must be 256-byte aligned");
  OptPlan o;
  optim_plan(m->s, m->po, o);
  if (state_bytes < o.total)
    return fail(GPT_ESPACE, "optimizer state too small: need " + std::to_string(o.total) + " bytes");
  char* st = (char*)state;
  m->opt_state = nullptr;
  HIP_TRY(hipMemcpyAsync(st + o.table, o.table_host.data(), o.table_host.size() * sizeof(OptSeg),
                         hipMemcpyHostToDevice, m->st));
  long nmom = 0;
  for (const auto& g : o.groups) nmom += (long)g.rows * g.cols * g.count;
  for (int i = 0; i < o.adam.n; ++i) nmom += 2 * o.table_host[o.adam.seg0 + i].n;
  fill_f32((float*)(st + o.mom), nmom, 0.f, m->st);
  fill_f32((float*)(st + o.hdr), ALIGN / 4, 0.f, m->st);
  if (o.has_master)
    opt_widen(m->W, (float*)(st + o.master), (const OptSeg*)(st + o.table) + o.all.seg0, o.all.n, o.all.nblk, m->st);
  HIP_TRY(hipGetLastError());
  HIP_TRY(hipStreamSynchronize(m->st));   // the table's host copy must outlive the transfer
  m->opt = o;
  m->opt_state = state;
  return GPT_OK;
}

int gpt_optim_master(gpt_model* m, float** master) {
  if (!m || !master) return fail(GPT_ENULL, "gpt_optim_master: NULL argument");
  if (!m->opt_state) return fail(GPT_EINVAL, "no optimizer state: call gpt_optim_init first");
  *master = m->opt.has_master ? (float*)((char*)m->opt_state + m->opt.master) : (float*)m->W;
  return GPT_OK;
}

int gpt_optim_step(gpt_model* m, void* state, const float* grads, const gpt_optim_params* hp, float* grad_norm) {
  if (!m || !state || !grads || !hp) return fail(GPT_ENULL, "gpt_optim_step: NULL argument");
  if (state != m->opt_state) return fail(GPT_EINVAL, "state was not prepared by gpt_optim_init for this model");
  if ((uintptr_t)grads & (ALIGN - 1)) return fail(GPT_EALIGN, "grads must be 256-byte aligned");
  const float f[] = {hp->matrix_lr, hp->momentum, hp->embedding_lr, hp->unembedding_lr, hp->beta1,
                     hp->beta2,     hp->eps,      hp->weight_decay, hp->grad_clip};
  for (float x : f)
    if (!std::isfinite(x)) return fail(GPT_EINVAL, "optimizer parameters must be finite");
  if (hp->momentum < 0.f || hp->momentum >= 1.f) return fail(GPT_EINVAL, "momentum must be in [0, 1)");
  if (hp->beta1 < 0.f || hp->beta1 >= 1.f || hp->beta2 < 0.f || hp->beta2 >= 1.f)
    return fail(GPT_EINVAL, "beta1 and beta2 must be in [0, 1)");
  if (!(hp->eps > 0.f)) return fail(GPT_EINVAL, "eps must be positive");
  if (hp->ns_steps < 1 || hp->ns_steps > 32) return fail(GPT_EINVAL, "ns_steps must be in [1, 32]");
  if (hp->nesterov != 0 && hp->nesterov != 1) return fail(GPT_EINVAL, "nesterov must be 0 or 1");
  if (hp->step < 1) return fail(GPT_EINVAL, "step must be >= 1");
  int rc = run_optim(*m, (char*)state, grads, *hp, grad_norm != nullptr);
  if (rc) return rc;
  if (grad_norm) {
    float v = 0.f;
    HIP_TRY(hipMemcpyAsync(&v, (char*)state + m->opt.hdr, 4, hipMemcpyDeviceToHost, m->st));
    HIP_TRY(hipStreamSynchronize(m->st));
    *grad_norm = v;
  }
  if (m->prof_on) {
    HIP_TRY(hipStreamSynchronize(m->st));
    prof_collect(*m);
  }
  return GPT_OK;
}

}  // extern "C"
