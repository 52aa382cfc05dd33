// Internal declarations shared by the library's host sources (the step,
// the optimizer, inference): the model handle, shapes, parameter offsets,
// and the error and profiling helpers.  Not part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>

#include <string>
#include <vector>

#include "../../include/gpt.h"
#include "kernels.h"

namespace gm __attribute__((visibility("hidden"))) {
using namespace gk;

// Records msg as the thread's last error text and returns code.
int fail(int code, const std::string& msg);

}  // namespace gm

#define HIP_TRY(expr)                                                              \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess)                                                          \
      return gm::fail(GPT_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

namespace gm __attribute__((visibility("hidden"))) {

constexpr size_t ALIGN = 256;
// decoding: K splits of the products whose few weight rows would leave most
// CUs idle (output projection, W2); their partials go through the next norm
constexpr int DEC_KSPLIT = 8;
static_assert(DEC_KSPLIT <= 8, "the decoder's add + norm kernel adds at most 8 partials");
// micro-batches per gpt_step_micro call
constexpr int MAX_MICRO = 1024;
// The cross-entropy backward works on the vocabulary in chunks of at most
// this many columns: the logit gradient of one chunk is formed, consumed by
// the lm_head's input- and weight-gradient products, and overwritten by the
// next chunk's.
constexpr int VOCAB_CHUNK = 8192;
// fork / join events of the overlapped weight gradients per step (two per
// product: 4 per layer and 2 per vocabulary chunk)
// work-groups a weight-gradient product on the second stream aims for
constexpr long SIDE_WG_TARGET = 96;
constexpr int OV_EVENTS = 1024;
inline size_t align_up(size_t x, size_t a = ALIGN) { return (x + a - 1) / a * a; }

struct Shape {
  int L, d, H, Dh, F, V, T, B, BT, Tp, dtype, es;
  int Hkv, dkv, Nqkv;   // key/value heads, their width Hkv*Dh, and the fused QKV width d + 2*dkv
  bool fp8;   // linear layers (QKV, O, W1, W2) in fp8; everything else as bf16
  float eps, base;
  std::vector<int> win;   // keys visible per layer
};

int check_config(const gpt_config* c, Shape& s);

// Single products for gpt_gemm / gpt_gemm_noalloc: argument checks (host
// only), the split count after rounding K to whole steps, and the launch.
int gemm_check(int dtype, int layout, int M, int N, int K, const void* A, const void* B, const float* C, int splits,
               int tile, const char* who);
int gemm_real_splits(int dtype, int K, int splits, int* k_split);
int gemm_entry(int dtype, int layout, int M, int N, int K, const void* A, const void* B, float* C, float* workspace,
               int splits, int tile, void* stream, const char* who);

struct ParamOffsets {
  long E, U;
  std::vector<long> Wqkv, Wo, W1, W2;
  long total;
  std::vector<gpt_tensor_desc> descs;
};

void param_offsets(const Shape& s, ParamOffsets& p);

// Optimizer state plan: byte offsets into the caller's state buffer and the
// pass lists (each list ends with a sentinel entry).
struct OptPlan {
  struct List {
    int seg0 = 0, n = 0, nblk = 0;
  };
  struct Group {   // Muon matrices of one shape, orthogonalised as one batch
    List list;
    int rows = 0, cols = 0, count = 0;
  };
  size_t hdr = 0, table = 0, part = 0, master = 0, mom = 0, ns = 0, total = 0;
  size_t xa = 0, xb = 0, ab = 0, bb = 0;   // Newton-Schulz buffers (offsets from ns)
  bool has_master = false;
  List all, adam;
  std::vector<Group> groups;
  std::vector<OptSeg> table_host;
  int max_part = 0;
};

}  // namespace gm

struct gpt_model {
  gpt_config cfg;
  gm::Shape s;
  gm::ParamOffsets po;
  hipStream_t st;
  char* ws;
  const char* W;
  // workspace offsets (bytes)
  struct Layer {
    size_t n1, rstd1, qkv, rqk, qT, kT, vT, o, lse2, n2, rstd2, u, g;
    // fp8: transposed activation codes kept for the weight gradients, and the
    // step's weight codes (row-major and transposed) for QKV, O, W1, W2
    size_t n1T, oT, n2T, gT, wq[4], wqT[4];
  };
  std::vector<Layer> lay;
  size_t h, nL, rstdL, part, tgt, lse, rowloss, lossdev, flag, mloss, dpart, dtok, dpos, dsplit, dz, dm, dh, dhA, du, dO, dOT, Dv, dqkv, splitk,
      cosb, sinb, keys, emb_rank, emb_cnt, emb_tot, emb_start, emb_bsum, emb_heads, emb_part, total;
  size_t splitk_floats;
  size_t q8row, q8T, q8T2, amax, scales;   // fp8: transient codes, per-tensor amax / scale slots
  size_t f32w;   // fp8: transient fp32 [BT][F], du in the backward
  int n_slots;
  int xent_tile, xent_nblk;
  // optional per-launch-site timing with HIP events on the step's stream
  struct Site {
    std::string name;
    std::string kernel;   // template signature of the launched kernel
    long launches = 0;
    double ms = 0.0, work = 0.0;
    int work_kind = 0;  // 0 = flops, 1 = bytes
  };
  struct Pending {
    int site;
    double work;
    hipEvent_t a, b;
  };
  gm::OptPlan opt;
  void* opt_state = nullptr;   // the state buffer gpt_optim_init prepared
  // decoding: one step captured as a HIP graph (for the cache and logits
  // buffers it was captured with), replayed on a stream of its own that is
  // ordered after the model's stream by events
  struct DecodeGraph {
    hipStream_t cs = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    hipEvent_t before = nullptr, after = nullptr;
    const void* kv = nullptr;
    const void* logits = nullptr;
  } dg;
  // gpt_step_micro: the n micro-batch steps captured as one graph, for the
  // buffers and arguments it was captured with (replayed on dg.cs)
  struct MicroGraph {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    const void* tokens = nullptr;
    const void* targets = nullptr;
    const void* grads = nullptr;
    int n = 0, accumulate = 0;
    float scale = 0.f;
  } mg;
  bool prof_on = false;
  // Weight-gradient products of the backward run on a second stream of the
  // handle, overlapping the input-gradient chain (which alone feeds the next
  // layer): `side` is created by gpt_create (default priority), forks and
  // joins are events from the ring `ov_ev`.  Off with profiling (so that
  // every launch is timed alone) or by gpt_overlap_enable(m, 0).
  hipStream_t side = nullptr;
  std::vector<hipEvent_t> ov_ev;
  size_t ov_next = 0;
  bool overlap = true;
  bool rope_epilogue = true;   // the fused rotary epilogue where it applies (gpt_rope_epilogue_enable)
  size_t splitk2 = 0, splitk2_floats = 0;
  size_t dhA2 = 0, dz2 = 0;          // second copies of dhA and dz, alternated
  std::vector<Site> sites;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
  std::vector<Pending> pend;
  int cur_site = -1;
  double cur_work = 0.0;
  ~gpt_model() {
    for (hipEvent_t e : ev_pool) (void)hipEventDestroy(e);
    for (hipEvent_t e : ov_ev) (void)hipEventDestroy(e);
    if (side) (void)hipStreamDestroy(side);
    if (mg.exec) (void)hipGraphExecDestroy(mg.exec);
    if (mg.graph) (void)hipGraphDestroy(mg.graph);
    if (dg.exec) (void)hipGraphExecDestroy(dg.exec);
    if (dg.graph) (void)hipGraphDestroy(dg.graph);
    if (dg.before) (void)hipEventDestroy(dg.before);
    if (dg.after) (void)hipEventDestroy(dg.after);
    if (dg.cs) (void)hipStreamDestroy(dg.cs);
  }
};

namespace gm __attribute__((visibility("hidden"))) {

template <typename P>
P* at(gpt_model& m, size_t off) { return (P*)(m.ws + off); }

// Per-launch-site timing with HIP events on the model's stream (no-ops when
// profiling is off); prof_collect resolves the pairs after a synchronisation.
void prof_begin(gpt_model& m, const char* name, double work, int kind, const std::string& kernel);
void prof_end(gpt_model& m);
void prof_collect(gpt_model& m);

// One forward+backward pass enqueued on m.st (see the step source).
int run_step(gpt_model& m, const int32_t* tokens, const int32_t* targets, float* grads, float grad_scale,
             int accumulate, const Shape* shape = nullptr, bool forward_only = false, float* loss_out = nullptr,
             bool clear_flag = true, bool quant_weights = true);

// The handle's graph-replay stream and its two ordering events (created on
// first use).
int graph_stream(gpt_model& m);

}  // namespace gm
