// Host side of KV-cache inference: prefill through the step's forward, and
// decoding steps (skinny products, add + norm, attention over the cache)
// captured once as a HIP graph and replayed.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <string>

#include "model.h"

using namespace gk;
using namespace gm;

namespace gm __attribute__((visibility("hidden"))) {

// ------------------------------------------------------------------ inference
size_t kv_layer_elems(const Shape& s) { return (size_t)s.B * s.Hkv * s.T * s.Dh; }

int check_infer(gpt_model& m) {
  if (m.s.dtype != DT_BF16) return fail(GPT_EINVAL, "inference runs on bf16 parameters (GPT_BF16 or GPT_FP8 models)");
  if (m.s.B > 32) return fail(GPT_EINVAL, "inference supports batch <= 32");
  if (m.s.Dh != 64 && m.s.Dh != 128) return fail(GPT_EINVAL, "inference supports head_dim 64 or 128");
  return GPT_OK;
}

// One skinny product of decoding, timed as a site like the step's products.
int dec_gemm(gpt_model& m, const char* site, int epi, const void* x, long ldx, int K, const void* Wt, int N, void* C,
             int ldc, void* C2 = nullptr, int ksplit = 1) {
  const int B = m.s.B;
  prof_begin(m, site, 2.0 * B * (double)N * K, 0, std::string("skinny_gemm_kernel<") + std::to_string(epi) + ">");
  if (skinny_gemm(epi, x, ldx, B, K, Wt, N, C, ldc, C2, ksplit, m.st)) return fail(GPT_EINVAL, "skinny gemm shape");
  prof_end(m);
  return GPT_OK;
}

// Prefill: the forward over n tokens per row (positions 0..n-1), the keys and
// values of every layer into the cache, and the next-token logits of the
// last position.
int run_prefill(gpt_model& m, const int32_t* tokens, int n, char* kv, float* logits) {
  Shape sp = m.s;
  sp.T = n;
  sp.BT = sp.B * n;
  sp.Tp = (n + 63) / 64 * 64;
  sp.fp8 = false;   // fp8 models decode with their bf16 weights
  for (auto& w : sp.win) w = std::min(w, n);
  int rc = run_step(m, tokens, tokens, nullptr, 1.f, 0, &sp, true);
  if (rc) return rc;
  const Shape& s = m.s;
  const size_t kvl = kv_layer_elems(s);
  prof_begin(m, "prefill_kv_fill", (double)sp.BT * 2.0 * s.dkv * 2.0 * 2.0, 1, "kv_fill_kernel");
  for (int l = 0; l < s.L; ++l) {
    uint16_t* kc = (uint16_t*)kv + (size_t)2 * l * kvl;
    kv_fill(m.ws + m.lay[l].qkv, kc, kc + kvl, s.B, n, s.H, s.Hkv, s.Dh, s.T, m.st);
  }
  prof_end(m);
  // rows b*n + n - 1 of the final normalised activations
  return dec_gemm(m, "prefill_lm_head", EPI_STORE_F32, m.ws + m.nL + (size_t)(n - 1) * s.d * 2, (long)n * s.d, s.d,
                  m.W + (size_t)m.po.U * 2, s.V, logits, s.V);
}

// One decoding step on the model's stream: token ids and position come from
// the decoder's device buffers (decode_stage fills them), so the launch
// sequence does not depend on them and can be captured once.  `pos` (host)
// only sizes the profiler's work accounting.
int run_decode(gpt_model& m, int pos, char* kv, float* logits) {
  const Shape& s = m.s;
  const ParamOffsets& P = m.po;
  const int B = s.B, d = s.d, F = s.F, V = s.V, H = s.H, Dh = s.Dh;
  hipStream_t st = m.st;
  auto wp = [&](long off) { return (const void*)(m.W + off * 2); };
  float* h = at<float>(m, m.h);
  int* flag = at<int>(m, m.flag);
  char* n1 = m.ws + m.lay[0].n1;
  char* qkv = m.ws + m.lay[0].qkv;
  char* o = m.ws + m.lay[0].o;
  char* u = m.ws + m.lay[0].u;
  char* g = m.ws + m.lay[0].g;
  float* dpart = at<float>(m, m.dpart);
  const int32_t* tokens = at<int32_t>(m, m.dtok);
  const int* posp = at<int>(m, m.dpos);
  const size_t kvl = kv_layer_elems(s);
  int rc;
  float* split = at<float>(m, m.dsplit);
  prof_begin(m, "decode_embed", (double)B * d * 6.0, 1, "embed_fwd_kernel<bf16>");
  embed_fwd(DT_BF16, tokens, tokens, wp(P.E), h, B, d, V, flag, st);
  prof_end(m);
  int pending = 0;   // K-split partials of the last product, added by the next norm
  auto addnorm = [&](void* y) {
    prof_begin(m, "decode_add_rmsnorm", (double)B * d * (4.0 * pending + 10.0), 1, "decode_add_rmsnorm_kernel");
    decode_add_rmsnorm(h, split, pending, B, d, y, s.eps, st);
    prof_end(m);
    pending = 0;
  };
  for (int l = 0; l < s.L; ++l) {
    uint16_t* kc = (uint16_t*)kv + (size_t)2 * l * kvl;
    uint16_t* vc = kc + kvl;
    addnorm(n1);
    if ((rc = dec_gemm(m, "decode_qkv", EPI_STORE, n1, d, d, wp(P.Wqkv[l]), s.Nqkv, qkv, s.Nqkv))) return rc;
    const int lo = std::max(0, pos - s.win[l] + 1);
    prof_begin(m, "decode_attention", (double)B * s.Hkv * (pos - lo + 1) * Dh * 4.0, 1,
               "attn_decode_split_kernel + attn_decode_combine_kernel");
    if (attn_decode(qkv, kc, vc, at<float>(m, m.cosb), at<float>(m, m.sinb), dpart, o, B, H, s.Hkv, Dh, s.T, posp,
                    s.win[l], s.eps, st))
      return fail(GPT_EINVAL, "decode attention head_dim");
    prof_end(m);
    if ((rc = dec_gemm(m, "decode_o", EPI_PARTIAL, o, d, d, wp(P.Wo[l]), d, split, d, nullptr, DEC_KSPLIT))) return rc;
    pending = DEC_KSPLIT;
    addnorm(n1);
    if ((rc = dec_gemm(m, "decode_w1_relu2", EPI_RELU2, n1, d, d, wp(P.W1[l]), F, u, F, g))) return rc;
    if ((rc = dec_gemm(m, "decode_w2", EPI_PARTIAL, g, F, F, wp(P.W2[l]), d, split, d, nullptr, DEC_KSPLIT))) return rc;
    pending = DEC_KSPLIT;
  }
  addnorm(m.ws + m.nL);
  if ((rc = dec_gemm(m, "decode_lm_head", EPI_STORE_F32, m.ws + m.nL, d, d, wp(P.U), V, logits, V))) return rc;
  HIP_TRY(hipGetLastError());
  return GPT_OK;
}

// Replays the captured decoding step (capturing it first, or again when the
// cache or logits buffer differs from the captured one).
int decode_graph_launch(gpt_model& m, int pos, void* kv, float* logits) {
  const int rc0 = graph_stream(m);
  if (rc0) return rc0;
  auto& g = m.dg;
  if (!g.exec || g.kv != kv || g.logits != logits) {
    if (g.exec) (void)hipGraphExecDestroy(g.exec);
    if (g.graph) (void)hipGraphDestroy(g.graph);
    g.exec = nullptr;
    g.graph = nullptr;
    HIP_TRY(hipStreamBeginCapture(g.cs, hipStreamCaptureModeThreadLocal));
    hipStream_t saved = m.st;
    m.st = g.cs;
    const int rc = run_decode(m, pos, (char*)kv, logits);
    m.st = saved;
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(g.cs, &graph);
    if (rc) {
      if (graph) (void)hipGraphDestroy(graph);
      return rc;
    }
    if (e != hipSuccess) return fail(GPT_EHIP, std::string("decode graph capture: ") + hipGetErrorString(e));
    g.graph = graph;
    HIP_TRY(hipGraphInstantiate(&g.exec, g.graph, nullptr, nullptr, 0));
    g.kv = kv;
    g.logits = logits;
  }
  HIP_TRY(hipEventRecord(g.before, m.st));
  HIP_TRY(hipStreamWaitEvent(g.cs, g.before, 0));
  HIP_TRY(hipGraphLaunch(g.exec, g.cs));
  HIP_TRY(hipEventRecord(g.after, g.cs));
  HIP_TRY(hipStreamWaitEvent(m.st, g.after, 0));
  return GPT_OK;
}

// Waits for the stream, then reports an out-of-range id.
int finish_infer(gpt_model& m) {
  int flag = 0;
  HIP_TRY(hipMemcpyAsync(&flag, m.ws + m.flag, 4, hipMemcpyDeviceToHost, m.st));
  HIP_TRY(hipStreamSynchronize(m.st));
  if (m.prof_on) prof_collect(m);
  if (flag) return fail(GPT_ETOKEN, "a token id is outside [0, vocab)");
  return GPT_OK;
}

}  // namespace gm

extern "C" {

int gpt_kv_cache_bytes(const gpt_config* cfg, size_t* bytes) {
  if (!bytes) return fail(GPT_ENULL, "bytes is NULL");
  Shape s;
  int rc = check_config(cfg, s);
  if (rc) return rc;
  *bytes = (size_t)2 * s.L * kv_layer_elems(s) * 2;
  return GPT_OK;
}

int gpt_prefill(gpt_model* m, const int32_t* tokens, int n_tokens, void* kv_cache, float* logits) {
  if (!m || !tokens || !kv_cache || !logits) return fail(GPT_ENULL, "gpt_prefill: NULL argument");
  int rc = check_infer(*m);
  if (rc) return rc;
  if (n_tokens < 1 || n_tokens > m->s.T) return fail(GPT_EINVAL, "n_tokens must be in [1, seq_len]");
  if (((uintptr_t)kv_cache | (uintptr_t)logits) & 15) return fail(GPT_EALIGN, "kv_cache and logits must be 16-byte aligned");
  if ((rc = run_prefill(*m, tokens, n_tokens, (char*)kv_cache, logits))) return rc;
  return finish_infer(*m);
}

int gpt_decode(gpt_model* m, const int32_t* tokens, int pos, void* kv_cache, float* logits) {
  if (!m || !tokens || !kv_cache || !logits) return fail(GPT_ENULL, "gpt_decode: NULL argument");
  int rc = check_infer(*m);
  if (rc) return rc;
  if (pos < 1 || pos >= m->s.T) return fail(GPT_EINVAL, "pos must be in [1, seq_len)");
  if (((uintptr_t)kv_cache | (uintptr_t)logits) & 15) return fail(GPT_EALIGN, "kv_cache and logits must be 16-byte aligned");
  decode_stage(tokens, m->s.B, pos, at<int32_t>(*m, m->dtok), at<int>(*m, m->dpos), at<int>(*m, m->flag), m->st);
  if (m->prof_on) {
    // profiled steps run eagerly, so that every launch is timed
    if ((rc = run_decode(*m, pos, (char*)kv_cache, logits))) return rc;
  } else {
    if ((rc = decode_graph_launch(*m, pos, kv_cache, logits))) return rc;
  }
  return finish_infer(*m);
}

}  // extern "C"
