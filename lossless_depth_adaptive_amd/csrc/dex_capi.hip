// Host side of the DEX lattice-step library: the C ABI declared in
// include/dex.h, workspace carving, weight packing, prefill, and the launch
// sequence of one lattice round ("Depth Exploration for LLM Decoding",
// Algorithm 1: expand -> DECS -> insert -> commit and collapse, or advance).
//
// The host owns the FSM counters of each sequence (state q, committed length
// C, commits made); the device owns everything that depends on token values
// (node map, candidates, KV, hidden states). A sequence in state q runs the
// 2^q new nodes of its tree: 2^(q-1-j) at explorer j < q and the anchor path's
// node at explorer q, so the row counts of a round are known on the host
// before launch, and the only device-to-host transfer per round is the commit
// records (at most one per sequence).
#include <algorithm>
#include <array>
#include <cstdint>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>
#include <type_traits>

#include "common.h"
#include "dex.h"
#include "plan.h"

namespace dex {
template <typename T>
hipError_t launch_pack(void*, const void*, const void*, const void*, int, int, int, int, int, int, int, hipStream_t);
template <typename T>
hipError_t launch_gemm(const GemmArgs&, int, hipStream_t);
hipError_t launch_gemm_wide(const GemmArgs&, int, int, hipStream_t);
hipError_t launch_head_reduce(const float*, int, int, int, const RowInfo*, int, int*, float*, hipStream_t);
template <typename T>
hipError_t launch_embed(const void*, const RowInfo*, int, int, float*, float*, float*, const float*, int, hipStream_t);
hipError_t launch_attention(const AttnItem*, int, const int*, int, int, int, const RowInfo*, int, const float*,
                            const bf16_t*,
                            const bf16_t*, float*, float*, float*, const ModelDims&, int, int, int, int, int, int,
                            bool, hipStream_t);
hipError_t launch_sched(const SeqPlan*, int, RowInfo*, int*, const int*, const int*, int*, const int*, int, int, int,
                        int, int, hipStream_t);
hipError_t launch_commit(const SeqPlan*, int, int*, const int*, const float*, int*, int*, int*, int*, int*, int*,
                         float*, const int*, int, int, int, int, hipStream_t);
hipError_t launch_promote(const SeqPlan*, int, const int*, const bf16_t*, bf16_t*, const ModelDims&, hipStream_t);
hipError_t launch_ar_rows(const SeqPlan*, int, RowInfo*, const int*, int, hipStream_t);
hipError_t launch_ar_commit(const SeqPlan*, int, const int*, const float*, int*, int*, int*, float*, int, int,
                            hipStream_t);
hipError_t launch_reset(int*, int*, int*, int*, const int*, int, int, hipStream_t);
}  // namespace dex

using namespace dex;

namespace {

thread_local std::string g_create_error;
constexpr size_t kMaxGraphs = 256;


}  // namespace

// Scratch of dex_step_noalloc, for callers that cannot allocate: a file-scope
// device array, one copy per GPU, held until the process ends. Its host-side
// name is not a device address; host code uses the address that
// hipGetSymbolAddress returns for the current device (g_scratch_ptr).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices] = {};
static std::mutex g_scratch_mu;

// Looks up the static scratch's device address on the current device, once
// per device. Returns the device index, or -1 with err set.
static int scratch_setup(std::string& err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    err = std::string("hipGetDevice: ") + hipGetErrorString(e);
    return -1;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev]) return dev;
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr) {
    err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
    return -1;
  }
  g_scratch_ptr[dev] = p;
  return dev;
}

struct dex_ctx {
  dex_model_config cfg;
  dex_options opt;
  ModelDims D;
  int N, S, L;
  std::vector<int> X;
  bool bf16;
  int device = -1;         // device the context was created on
  bool no_graphs = false;  // launch this round eagerly (dex_step_noalloc)
  hipStream_t st;
  char* ws;
  WsPlan wp;
  // device views
  float *ad_vec = nullptr, *xa = nullptr, *ssq_head = nullptr;
  std::vector<float> ad_alpha;    // inducing-adapter gates (host), one per non-final explorer
  float *norms, *cosT, *sinT, *hidden, *xn, *xh, *margin, *dbg_m, *dbg_logits, *q;
  float *attn_part, *attn_tail, *head_part, *ssq, *gemm_split;
  int *map, *cand, *freel, *cursor, *anchor, *anchors_in, *records, *promote, *dbg_u, *Xd;
  RowInfo* rows;
  SeqPlan* plans;
  AttnItem* items;
  int* item_list;   // attention block list: single items, then group leads (after the Rmax items)
  bf16_t *kvc, *exb;
  void *attn_out, *act, *embed, *head;
  // host state
  int nseq = 0;
  std::vector<int> q_, C_, commits_, plen_;
  int mode_used = 0;  // 0 none since prefill, 1 lattice, 2 autoregressive
  bool any_commit = false;
  bool poisoned = false;
  SeqPlan* h_plans = nullptr;
  int* h_records = nullptr;
  AttnItem* h_items = nullptr;
  int* h_item_list = nullptr;     // attention block list (after the Rmax items of h_items)
  RowInfo* h_rows = nullptr;
  std::string err;
  int last_rows[kMaxN] = {0};
  int last_total = 0;
  // optional per-class timing with HIP events on the context's stream
  struct Mark {
    hipEvent_t a = nullptr, b = nullptr;
    int cls = 0, launches = 0;
    double bytes = 0, flops = 0;
  };
  hipStream_t cap_st = nullptr;   // private stream that round graphs are captured on
  bool prof = false;
  int attn_umax = 1;              // most units in one attention item of the current round
  int attn_nj = 0;                // most chunks holding explore keys in one item of the round (0 to 2)
  int attn_single = 0;            // attention items of the current pass that form a group of their own
  int attn_groups = 0;            // attention items of the current pass that lead a group of several
  int attn_tails = 0;             // (item, 4-row quarter) entries of the per-row attention chunks
  std::vector<Mark> marks;
  size_t nmarks = 0;
  // HIP graphs of whole rounds, keyed by the round's plan
  std::unordered_map<std::string, hipGraphExec_t> graphs;
  std::unordered_map<std::string, int> graph_seen;
  dex_kernel_stats stats[DEX_PROF_NCLASS] = {};

  void* at(size_t off) { return ws + off; }
};

#define HIPCHK(expr)                                                              \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess) {                                                       \
      ctx->err = std::string(#expr) + ": " + hipGetErrorString(e_);               \
      ctx->poisoned = true;                                                       \
      return DEX_EHIP;                                                            \
    }                                                                             \
  } while (0)

namespace {

// The attention block lists of the context's first nitems host items.
void attn_block_list(dex_ctx* ctx, int nitems) {
  const BlockList b = attn_block_list(ctx->h_items, nitems, ctx->h_item_list);
  ctx->attn_single = b.single;
  ctx->attn_groups = b.groups;
  ctx->attn_tails = b.tails;
}

// Groups of at least this many rows go to the wide GEMM kernel, the others to
// the split-k kernel (both give a row the same bits). The split-k kernel
// re-reads every row's activations for each 16-column tile, so its time grows
// with the rows: on four 7B/13B-shaped weights it wins only below about 8 rows
// (at 16 rows the wide kernel is 1.4-2x faster). A wide launch that would
// have fewer than 384 blocks at 4 column tiles per wave runs 2 tiles per wave
// (7B gate/up and QKV: 8-15% faster), and one of fewer than 128 blocks (d x d
// and down projections) runs split by k range.
#ifndef DEX_WIDE_ROWS
#define DEX_WIDE_ROWS 8
#endif
constexpr int kWideRows = DEX_WIDE_ROWS;

// Launches grouped GEMMs over `groups` (kMaxGroups per launch, wide and
// split-k groups apart; wide ones only with bf16 weights); ga carries
// everything else. A wide launch that would have few blocks runs split by k
// range when its rows fit the scratch (split_cols: the scratch's row length).
// Unsplit wide launches may row-shard their groups over the XCDs (xcd_pays).
// Counts launches.
#ifndef DEX_XCD_ROWS
#define DEX_XCD_ROWS 1
#endif
constexpr int kXcdRows = DEX_XCD_ROWS;
// 8-wave blocks (64 rows x 512 columns, one block per CU) halve the
// activation re-reads of the 4-wave ones (each block reads its rows'
// activations once per K pass); a launch uses them when it still has this
// many blocks. Measured (three runs each, library variants): 13B-shaped batch
// 8 320.7 -> 342.5 tokens/s, GQA batch 16 179.4 -> 189.2, 7B sampled 209.2 ->
// 213.5, 7B greedy 270.2 -> 273.6; thresholds from 1 to 128 blocks measured
// the same, 256 and 512 less.
#ifndef DEX_W8_MIN_BLOCKS
#define DEX_W8_MIN_BLOCKS 128
#endif
constexpr int kW8MinBlocks = DEX_W8_MIN_BLOCKS;
#ifndef DEX_W8_HEAD
#define DEX_W8_HEAD 1
#endif
constexpr int kW8Head = DEX_W8_HEAD;
// Groups of fewer than kWideRows rows join the wide launch when they are few
// next to it (at most a quarter of its groups: batched rounds, where they
// would otherwise stream their stages' weights in a serial split-k launch of
// their own); 13B-shaped batch 8: 364 -> 373 tokens/s. Where they are many
// (the batch-1 lattice's small stages) the split-k kernel is much cheaper:
// merging them cost the 7B-shaped sampled workload 7%.
// 1: unsplit wide launches order their blocks weight by weight
// (GemmArgs.nrun). The 13B-shaped batch-8 layer GEMMs then fetch 1.14x their
// algorithmic bytes instead of 1.39x, but the workload ran 1-2% slower (200
// rounds, median of three: 356.4 -> 348.6 tokens/s; GQA batch 16 193.2 ->
// 188.8), so the column-block order stays the default.
#ifndef DEX_STAGE_MAJOR
#define DEX_STAGE_MAJOR 0
#endif
constexpr bool kStageMajor = DEX_STAGE_MAJOR != 0;
#ifndef DEX_MERGE_SMALL
#define DEX_MERGE_SMALL 1
#endif

// Whether a wide launch row-shards its groups over the XCDs (GemmArgs.xcd_rows):
// it saves the activation re-reads of the sharded groups (each column block
// after the first would read them again) and costs the weight reads of the
// XCDs that hold groups of the same stage (each of them streams that stage's
// weights). Taken when the saving is larger. Without the model, 13B-shaped
// batch 8 preferred never (364 vs 354 tokens/s; both its layer GEMMs and its
// exit head) and the GQA batch-16 exit head always (370 vs 403 ms per 60
// rounds). Two passes each, tokens/s with the model / never / always: 13B
// batch 8 373.9, 371.6 / 371.8, 372.6 / 369.0, 369.8; GQA batch 16 188.0,
// 185.8 / 184.1, 184.4 / 187.0, 187.3.
bool xcd_pays(const GemmArgs& ga, int bt, int es) {
  const int Q = ga.ngroups & ~7;
  if (Q == 0 || kXcdRows == 0) return false;
  if (kXcdRows == 2) return true;
  const int ncb = (ga.N / 16 + bt - 1) / bt;
  double rows = 0;
  for (int g = 0; g < Q; ++g) rows += ga.g[g].m;
  const double saving = rows * ga.K * 4.0 * (ncb - 1);
  const int gpx = Q / 8;
  int per_xcd = 0, overall = 0;
  for (int g = 0; g < Q; ++g) {
    if (g == 0 || ga.g[g].w != ga.g[g - 1].w) ++overall;   // groups of a weight are consecutive
    if (g % gpx == 0 || ga.g[g].w != ga.g[g - 1].w) ++per_xcd;
  }
  const double cost = (double)(per_xcd - overall) * ga.N * ga.K * es;
  return saving > cost;
}

template <typename T>
hipError_t launch_groups(GemmArgs& ga, const std::vector<GemmGroup>& groups, int epi, int split_cols,
                         hipStream_t st, int* launches) {
  int nwide = 0, nsmall = 0;
  for (const GemmGroup& g : groups) (g.m >= kWideRows ? nwide : nsmall)++;
  const bool merge = DEX_MERGE_SMALL && std::is_same<T, bf16_t>::value && nsmall > 0 && 4 * nsmall <= nwide;
  for (int wide = 0; wide < 2; ++wide) {
    ga.ngroups = 0;
    int rows = 0;
    for (size_t i = 0; i <= groups.size(); ++i) {
      const bool is_wide = std::is_same<T, bf16_t>::value && i < groups.size() &&
                           (groups[i].m >= kWideRows || merge);
      const bool mine = i < groups.size() && is_wide == (wide == 1);
      const bool flush = i == groups.size() || ga.ngroups == kMaxGroups;
      if (flush && ga.ngroups) {
        hipError_t e = hipSuccess;
        if (wide) {
          // blocks at 4 tiles per wave: many -> as they are; a medium launch
          // -> 2 tiles per wave (twice the blocks); few -> split by k range
          const int blocks4 = ga.ngroups * ((ga.N / 16 + 15) / 16);
          int shape = WIDE_T4;
          if (blocks4 < 128 && rows <= kSplitRows && ga.N <= split_cols) shape = WIDE_SPLIT;
          else if (blocks4 < 384) shape = WIDE_T2;
          if (shape != WIDE_SPLIT && (epi != EPI_HEAD || kW8Head) &&
              ga.ngroups * ((ga.N / 16 + 31) / 32) >= kW8MinBlocks)
            shape = WIDE_W8;
          ga.xcd_rows = shape != WIDE_SPLIT &&
                        xcd_pays(ga, shape == WIDE_W8 ? 32 : shape == WIDE_T2 ? 8 : 16, (int)sizeof(T));
          ga.nrun = 0;
          if (kStageMajor && shape != WIDE_SPLIT) {
            const int q0 = ga.xcd_rows ? ga.ngroups & ~7 : 0;
            for (int g = q0; g < ga.ngroups; ++g)
              if (g == q0 || ga.g[g].w != ga.g[g - 1].w) ga.run0[ga.nrun++] = g;
            ga.run0[ga.nrun] = ga.ngroups;
          }
          e = launch_gemm_wide(ga, epi, shape, st);
          *launches += shape == WIDE_SPLIT ? 2 : 1;
        } else {
          e = launch_gemm<T>(ga, epi, st);
          ++*launches;
        }
        if (e != hipSuccess) return e;
        ga.ngroups = 0;
        rows = 0;
      }
      if (mine) {
        ga.g[ga.ngroups] = groups[i];
        ga.g[ga.ngroups++].srow = rows;
        rows += groups[i].m;
      }
    }
  }
  return hipSuccess;
}

// Opens a timed region of class `cls`; returns its mark index or -1.
int prof_begin(dex_ctx* ctx, int cls) {
  if (!ctx->prof) return -1;
  if (ctx->nmarks == ctx->marks.size()) {
    dex_ctx::Mark m;
    if (hipEventCreate(&m.a) != hipSuccess || hipEventCreate(&m.b) != hipSuccess) return -1;
    ctx->marks.push_back(m);
  }
  dex_ctx::Mark& m = ctx->marks[ctx->nmarks];
  m.cls = cls;
  m.launches = 0;
  m.bytes = m.flops = 0;
  if (hipEventRecord(m.a, ctx->st) != hipSuccess) return -1;
  return (int)ctx->nmarks++;
}

void prof_end(dex_ctx* ctx, int idx, int launches, double bytes, double flops) {
  if (idx < 0) return;
  dex_ctx::Mark& m = ctx->marks[idx];
  m.launches = launches;
  m.bytes = bytes;
  m.flops = flops;
  (void)hipEventRecord(m.b, ctx->st);
}

// After the stream has been synchronised: fold the marks into the stats.
void prof_collect(dex_ctx* ctx) {
  for (size_t i = 0; i < ctx->nmarks; ++i) {
    dex_ctx::Mark& m = ctx->marks[i];
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, m.a, m.b) != hipSuccess) continue;
    dex_kernel_stats& st = ctx->stats[m.cls];
    st.ms += ms;
    st.launches += m.launches;
    st.bytes += m.bytes;
    st.flops += m.flops;
  }
  ctx->nmarks = 0;
}

template <typename T>
int pack_weights(dex_ctx* ctx, const dex_weights* w) {
  const int L = ctx->L, d = ctx->D.d, nq = ctx->D.nq, nkv = ctx->D.nkv, hd = ctx->D.hd, F = ctx->D.F, V = ctx->D.V;
  hipStream_t st = ctx->st;
  for (int l = 0; l < L; ++l) {
    HIPCHK(launch_pack<T>(ctx->at(ctx->wp.wqkv[l]), w->wq[l], w->wk[l], w->wv[l], nq * hd, nkv * hd, nkv * hd, d, 1,
                          (nq + 2 * nkv) * hd, hd, st));
    HIPCHK(launch_pack<T>(ctx->at(ctx->wp.wo[l]), w->wo[l], nullptr, nullptr, d, 0, 0, nq * hd, 0, d, hd, st));
    HIPCHK(launch_pack<T>(ctx->at(ctx->wp.wgu[l]), w->w_gate[l], w->w_up[l], nullptr, F, F, 0, d, 2, 2 * F, hd, st));
    HIPCHK(launch_pack<T>(ctx->at(ctx->wp.wdown[l]), w->w_down[l], nullptr, nullptr, d, 0, 0, F, 0, d, hd, st));
  }
  const void* hsrc = ctx->cfg.tied_head ? w->tok_embed : w->lm_head;
  HIPCHK(launch_pack<T>(ctx->head, hsrc, nullptr, nullptr, V, 0, 0, d, 0, V, hd, st));
  HIPCHK(hipMemcpyAsync(ctx->embed, w->tok_embed, (size_t)V * d * sizeof(T), hipMemcpyDeviceToDevice, st));
  // Norm weights to fp32, through the host (2L+1 vectors of d).
  std::vector<T> tmp(d);
  std::vector<float> nf((size_t)(2 * L + 1) * d);
  for (int i = 0; i < 2 * L + 1; ++i) {
    const void* src = i == 2 * L ? w->final_norm : (i % 2 == 0 ? w->attn_norm[i / 2] : w->ffn_norm[i / 2]);
    HIPCHK(hipMemcpy(tmp.data(), src, d * sizeof(T), hipMemcpyDeviceToHost));
    for (int k = 0; k < d; ++k) {
      float f;
      if (sizeof(T) == 2) {
        const unsigned u = ((unsigned)((const unsigned short*)tmp.data())[k]) << 16;
        std::memcpy(&f, &u, 4);
      } else {
        std::memcpy(&f, (const char*)tmp.data() + 4 * k, 4);
      }
      nf[(size_t)i * d + k] = f;
    }
  }
  HIPCHK(hipMemcpy(ctx->norms, nf.data(), nf.size() * 4, hipMemcpyHostToDevice));
  // Inducing adapters: W1, W2 packed like any layer matrix; b1, b2 and the
  // norm weight to fp32 through the host.
  const int m = ctx->cfg.adapter_hidden;
  for (int k = 0; m && k < ctx->N - 1; ++k) {
    HIPCHK(launch_pack<T>(ctx->at(ctx->wp.wad1[k]), w->adapter_w1[k], nullptr, nullptr, m, 0, 0, d, 0, m, hd, st));
    HIPCHK(launch_pack<T>(ctx->at(ctx->wp.wad2[k]), w->adapter_w2[k], nullptr, nullptr, d, 0, 0, m, 0, d, hd, st));
    const void* srcs[3] = {w->adapter_b1[k], w->adapter_b2[k], w->adapter_norm[k]};
    const int lens[3] = {m, d, d};
    std::vector<T> t2((size_t)m);
    std::vector<float> f2;
    for (int v = 0; v < 3; ++v) {
      HIPCHK(hipMemcpy(t2.data(), srcs[v], lens[v] * sizeof(T), hipMemcpyDeviceToHost));
      for (int i = 0; i < lens[v]; ++i) {
        float f;
        if (sizeof(T) == 2) {
          const unsigned u = ((unsigned)((const unsigned short*)t2.data())[i]) << 16;
          std::memcpy(&f, &u, 4);
        } else {
          std::memcpy(&f, (const char*)t2.data() + 4 * i, 4);
        }
        f2.push_back(f);
      }
    }
    HIPCHK(hipMemcpy(ctx->ad_vec + (size_t)k * (m + 2 * d), f2.data(), f2.size() * 4, hipMemcpyHostToDevice));
    ctx->ad_alpha.push_back(w->adapter_alpha[k]);
  }
  return DEX_OK;
}

// Adapter vectors of explorer k in the workspace: b1 [m], b2 [d], norm [d].
const float* ad_b1(dex_ctx* ctx, int k) { return ctx->ad_vec + (size_t)k * (ctx->cfg.adapter_hidden + 2 * ctx->D.d); }
const float* ad_b2(dex_ctx* ctx, int k) { return ad_b1(ctx, k) + ctx->cfg.adapter_hidden; }
const float* ad_norm(dex_ctx* ctx, int k) { return ad_b2(ctx, k) + ctx->D.d; }

// Inducing adapters on the exit rows of non-final explorers: `ranges` holds
// (explorer, first row, count). ADAPT1: SiLU(W1 (RMSNorm(h) * g) + b1) into
// the activation buffer; ADAPT2: h~ = h + alpha (W2 a + b2) becomes the exit
// head's input (xh, ssq_head).
template <typename T>
int run_adapters(dex_ctx* ctx, const std::vector<std::array<int, 3>>& ranges) {
  if (ranges.empty()) return DEX_OK;
  const ModelDims& D = ctx->D;
  hipStream_t st = ctx->st;
  const int m = ctx->cfg.adapter_hidden;
  GemmArgs ga;
  std::memset(&ga, 0, sizeof(ga));
  ga.rows = ctx->rows;
  ga.hidden = ctx->hidden;
  ga.ssq = ctx->ssq;
  ga.ssq_head = ctx->ssq_head;
  ga.xin = ctx->xa;
  ga.xh = ctx->xh;
  ga.gfinal = ctx->norms + (size_t)2 * ctx->L * D.d;
  ga.eps = D.eps;
  ga.act = ctx->act;
  ga.a = ctx->act;
  ga.split = ctx->gemm_split;
  const double es = sizeof(T);
  double bytes = 0, flops = 0;
  int nrows = 0;
  for (int pass = 0; pass < 2; ++pass) {
    std::vector<GemmGroup> groups;
    for (const auto& rg : ranges) {
      const int k = rg[0];
      for (int o = 0; o < rg[2]; o += 64) {
        GemmGroup g{ctx->at(pass ? ctx->wp.wad2[k] : ctx->wp.wad1[k]), nullptr, rg[1] + o, std::min(64, rg[2] - o),
                    0, 0, pass ? ad_b2(ctx, k) : ad_b1(ctx, k), ctx->ad_alpha[k], nullptr};
        groups.push_back(g);
      }
      if (pass == 0) nrows += rg[2];
    }
    ga.K = pass ? m : D.d;
    ga.N = pass ? D.d : m;
    const int mk = prof_begin(ctx, DEX_PROF_GEMM);
    int launches = 0;
    HIPCHK(launch_groups<T>(ga, groups, pass ? EPI_ADAPT2 : EPI_ADAPT1, ctx->wp.split_cols, st, &launches));
    bytes = (double)ranges.size() * m * D.d * es + (double)nrows * (m + D.d) * 4 * (pass ? 2 : 1);
    flops = 2.0 * nrows * m * D.d;
    prof_end(ctx, mk, launches, bytes, flops);
  }
  return DEX_OK;
}

// One pass of the layer stack over `nrows` rows already set up in ctx->rows.
// stage_rows: for each stage, [row0, count) of its rows; lam_count layer
// slots; lattice != 0 for lattice rows (stage j runs layers lfirst[j] ..
// lfirst[j+1] - 1, so it takes part in slots lam < its length), 0 for
// autoregressive and prefill rows (one stage, layer = lam). want_xh: rows
// write h * final-norm weight after their last layer (exit head input).
// attn_stage_bytes/flops: algorithmic attention traffic of one layer slot per
// stage. Per layer slot: QKV GEMM (fused RMSNorm, RoPE, K/V write) ->
// attention -> O GEMM (+ residual) -> gate/up GEMM (fused RMSNorm, SwiGLU) ->
// down GEMM (+ residual).
template <typename T>
int run_layers(dex_ctx* ctx, int nrows, const std::vector<std::pair<int, int>>& stage_rows, int lam_count,
               int lattice, int nitems, int max_keys, bool want_xh,
               const std::vector<double>& attn_stage_bytes = {}, const std::vector<double>& attn_stage_flops = {}) {
  const ModelDims& D = ctx->D;
  hipStream_t st = ctx->st;
  const int d = D.d, nq = D.nq, nkv = D.nkv, hd = D.hd, F = D.F;
  const double es = sizeof(T);
  auto len_of = [&](size_t j) { return lattice ? stage_len(D, (int)j) : lam_count; };
  // Groups are collected in a host list and launched kMaxGroups at a time.
  std::vector<GemmGroup> glist;
  // next_norm: RMSNorm weight the residual-add epilogue folds into xn for the
  // row's next consumer (1: this layer's FFN norm, 2: the next layer's
  // attention norm); xh_at_end: the rows' last layer also writes xh.
  auto groups_for = [&](int lam, const std::vector<size_t>& woff, int next_norm, bool xh_at_end) {
    glist.clear();
    for (size_t j = 0; j < stage_rows.size(); ++j) {
      const int r0 = stage_rows[j].first, cnt = stage_rows[j].second;
      if (lam >= len_of(j)) continue;
      const int layer = layer_of(D, lattice, (int)j, lam);
      const float* gamma = nullptr;
      if (next_norm == 1) gamma = ctx->norms + (size_t)layer * 2 * d + d;                    // this layer's FFN norm
      if (next_norm == 2 && layer + 1 < ctx->L) gamma = ctx->norms + (size_t)(layer + 1) * 2 * d;  // next attention norm
      const int xh = xh_at_end && lam == len_of(j) - 1;
      // rows of a non-final explorer that exits also feed its inducing adapter
      const bool adapted = xh && lattice && ctx->cfg.adapter_hidden > 0 && (int)j < ctx->N - 1 &&
                           (!ctx->opt.single_exit || j == 0);
      for (int o = 0; o < cnt; o += 64)
        glist.push_back(GemmGroup{ctx->at(woff[layer]), gamma, r0 + o, std::min(64, cnt - o), 0, xh, nullptr, 0.f,
                                  adapted ? ad_norm(ctx, (int)j) : nullptr});
    }
  };
  auto run_gemm = [&](GemmArgs& ga, int epi) -> hipError_t {
    // algorithmic traffic: each distinct weight matrix once, activations in and out
    double bytes = 0, flops = 0;
    const void* lastw = nullptr;
    for (const GemmGroup& g : glist) {
      if (g.w != lastw) bytes += (double)ga.N * ga.K * es;
      lastw = g.w;
      bytes += (double)g.m * ga.K * 4;
      bytes += epi == EPI_QKV ? (double)g.m * ga.N * 4 : epi == EPI_RESID ? 2.0 * g.m * ga.N * 4 : (double)g.m * ga.N / 2 * 4;
      flops += 2.0 * g.m * ga.N * ga.K;
    }
    const int mk = prof_begin(ctx, DEX_PROF_GEMM);
    int launches = 0;
    const hipError_t e = launch_groups<T>(ga, glist, epi, ctx->wp.split_cols, st, &launches);
    if (e != hipSuccess) return e;
    prof_end(ctx, mk, launches, bytes, flops);
    return hipSuccess;
  };
  GemmArgs ga;
  std::memset(&ga, 0, sizeof(ga));
  ga.rows = ctx->rows;
  ga.hidden = ctx->hidden;
  ga.ssq = ctx->ssq;
  ga.xn = ctx->xn;
  ga.xh = ctx->xh;
  ga.xa = ctx->xa;
  ga.ssq_head = ctx->ssq_head;
  ga.xin = ctx->xn;
  ga.gfinal = ctx->norms + (size_t)2 * ctx->L * d;
  ga.eps = D.eps;
  ga.dims = D;
  ga.cosT = ctx->cosT;
  ga.sinT = ctx->sinT;
  ga.qout = ctx->q;
  ga.kvc = ctx->kvc;
  ga.exb = ctx->exb;
  ga.lattice = lattice;
  ga.qscale = (float)(1.4426950408889634 / std::sqrt((double)hd));
  ga.split = ctx->gemm_split;
  ga.act = ctx->act;
  for (int lam = 0; lam < lam_count; ++lam) {
    ga.lam = lam;
    groups_for(lam, ctx->wp.wqkv, 0, false);
    ga.K = d;
    ga.N = (nq + 2 * nkv) * hd;
    HIPCHK(run_gemm(ga, EPI_QKV));
    double attn_bytes = 0, attn_flops = 0;
    for (size_t j = 0; j < attn_stage_bytes.size(); ++j)
      if (lam < len_of(j)) {
        attn_bytes += attn_stage_bytes[j];
        attn_flops += attn_stage_flops[j];
      }
    int mk = prof_begin(ctx, DEX_PROF_ATTN);
    HIPCHK(launch_attention(ctx->items, nitems, ctx->item_list, ctx->attn_single, ctx->attn_groups,
                            lattice != 0 ? ctx->attn_tails : 0, ctx->rows, nrows,
                            ctx->q, ctx->kvc, ctx->exb, ctx->attn_tail, ctx->attn_part, (float*)ctx->attn_out, D, lam,
                            lattice, ctx->wp.nchunk, max_keys, lattice != 0 ? ctx->attn_umax : 0,
                            lattice != 0 ? ctx->attn_nj : 0, (ctx->opt.debug & 4) != 0, st));
    prof_end(ctx, mk, 2, attn_bytes, attn_flops);
    groups_for(lam, ctx->wp.wo, 1, false);
    ga.K = nq * hd;
    ga.N = d;
    ga.a = ctx->attn_out;
    HIPCHK(run_gemm(ga, EPI_RESID));
    groups_for(lam, ctx->wp.wgu, 0, false);
    ga.K = d;
    ga.N = 2 * F;
    HIPCHK(run_gemm(ga, EPI_SWIGLU));
    groups_for(lam, ctx->wp.wdown, 2, want_xh);
    ga.K = F;
    ga.N = d;
    ga.a = ctx->act;
    HIPCHK(run_gemm(ga, EPI_RESID));
  }
  return DEX_OK;
}

// Exit head for the rows of `ranges` (first row, count): final RMSNorm
// (fused), LM head, DECS mask and Gumbel perturbation in the GEMM epilogue,
// then the per-row argmax reduce.
template <typename T>
int run_head(dex_ctx* ctx, const std::vector<std::pair<int, int>>& ranges) {
  const ModelDims& D = ctx->D;
  hipStream_t st = ctx->st;
  GemmArgs ga;
  std::memset(&ga, 0, sizeof(ga));
  ga.rows = ctx->rows;
  ga.xin = ctx->xh;
  ga.ssq = ctx->ssq_head;
  ga.eps = D.eps;
  ga.K = D.d;
  ga.N = D.V;
  ga.out = (ctx->opt.debug & 1) ? ctx->dbg_logits : nullptr;
  ga.mode = ctx->opt.mode;
  ga.tau = ctx->opt.temperature;
  ga.gumbel = ctx->opt.gumbel;
  ga.gumbel_rows = ctx->opt.gumbel_rows;
  ga.part = ctx->head_part;
  const double es = sizeof(T);
  const int mk = prof_begin(ctx, DEX_PROF_HEAD);
  int launches = 0, nrows = 0;
  std::vector<GemmGroup> groups;
  for (const auto& rg : ranges) {
    for (int o = 0; o < rg.second; o += 64)
      groups.push_back(GemmGroup{ctx->head, nullptr, rg.first + o, std::min(64, rg.second - o), 0});
    nrows += rg.second;
  }
  ga.split = ctx->gemm_split;
  HIPCHK(launch_groups<T>(ga, groups, EPI_HEAD, ctx->wp.split_cols, st, &launches));
  for (const auto& rg : ranges) {
    HIPCHK(launch_head_reduce(ctx->head_part, D.V / 16, rg.first, rg.second, ctx->rows, D.P, ctx->cand, ctx->margin,
                              st));
    ++launches;
  }
  prof_end(ctx, mk, launches, (double)D.V * D.d * es + (double)nrows * D.d * 4 + (double)nrows * (D.V / 16) * 12 * 2,
           2.0 * nrows * D.V * D.d);
  return DEX_OK;
}

// One round (lattice) or one autoregressive token for every live sequence.
template <typename T>
int run_step(dex_ctx* ctx, bool ar, dex_commit* out, int32_t cap, int32_t* n_out) {
  const int N = ctx->N, B = ctx->nseq;
  const int T_ = ctx->opt.max_new_tokens;
  const int ncap = node_cap(ctx->opt, N);
  // Host plan: rows per (sequence, stage) from the FSM state alone.
  RoundShape shape;
  round_rows(ctx->q_.data(), ctx->commits_.data(), B, N, T_, ar, ncap, shape);
  const std::vector<int>& live = shape.live;
  const std::vector<int>& rows_seq_stage = shape.rows;
  const int* stage_tot = shape.stage_tot;
  const int* stage_off = shape.stage_off;
  const int nlive = shape.nlive;
  if (nlive == 0) {
    ctx->err = "every sequence has reached max_new_tokens";
    return DEX_ESTATE;
  }
  if (cap < nlive) {
    ctx->err = "output capacity below the number of live sequences";
    return DEX_ENOSPC;
  }
  const int R = shape.R;
  const int ncommit = seq_plans(shape, ctx->q_.data(), ctx->C_.data(), ctx->plen_.data(), B, N, ar, ctx->h_plans);
  // Attention work items: rows of one (sequence, stage), at most kAttnUnits units each.
  const ItemStats is = round_items(shape, ctx->h_plans, ctx->q_.data(), ctx->C_.data(), B, N, ar,
                                   ctx->D.nq / ctx->D.nkv, ctx->h_items);
  const int nitems = is.nitems, max_keys = is.max_keys;
  ctx->attn_umax = is.umax;
  ctx->attn_nj = is.nj;
  attn_block_list(ctx, nitems);
  // Algorithmic attention traffic of one layer slot, per stage: each
  // (sequence, stage) group reads its committed K/V once, each row its
  // explore entries.
  std::vector<double> attn_bytes(N, 0.0), attn_flops(N, 0.0);
  if (ctx->prof) {
    const double kvrow = 2.0 * ctx->D.nkv * ctx->D.hd * 2 * ctx->D.kvp;   // K and V, stored bytes
    for (int s = 0; s < B; ++s) {
      if (!live[s]) continue;
      const int q = ar ? 0 : ctx->q_[s];
      const int C = ctx->C_[s] + (ar ? 1 : 0);
      for (int j = 0; j < N; ++j)
        if (rows_seq_stage[(size_t)s * N + j]) attn_bytes[j] += C * kvrow;
      for (int n = (1 << q) - 1; n <= (1 << (q + 1)) - 2; ++n) {
        if (!ar && ncap && !node_held(n + 1, ncap)) continue;
        const int anc = ar ? 0 : __builtin_popcount(n + 1);
        const int j = ar ? 0 : __builtin_ctz(n + 1);
        attn_bytes[j] += anc * kvrow + ctx->D.nq * ctx->D.hd * 8.0;
        attn_flops[j] += 4.0 * ctx->D.nq * ctx->D.hd * (C + anc);
      }
    }
  }
  hipStream_t st = ctx->st;
  // Everything the round enqueues; run eagerly, or captured into a HIP graph
  // and replayed when the same plan (FSM states, commit flags, attention chunk
  // count, explore-chunk slots, profiling) comes back. Plans, items and the
  // attention block lists are re-read from the pinned host buffers at every
  // replay.
  auto enqueue = [&]() -> int {
    hipStream_t st = ctx->st;
    int mk = prof_begin(ctx, DEX_PROF_LATTICE);
    HIPCHK(hipMemcpyAsync(ctx->plans, ctx->h_plans, B * sizeof(SeqPlan), hipMemcpyHostToDevice, st));
    HIPCHK(hipMemcpyAsync(ctx->items, ctx->h_items, nitems * sizeof(AttnItem), hipMemcpyHostToDevice, st));
    const int nlist = ctx->attn_single + ctx->attn_groups + ctx->attn_tails;
    if (nlist) HIPCHK(hipMemcpyAsync(ctx->item_list, ctx->h_item_list, nlist * sizeof(int), hipMemcpyHostToDevice, st));
    if (ar) {
      HIPCHK(launch_ar_rows(ctx->plans, B, ctx->rows, ctx->anchor, ctx->D.P, st));
      HIPCHK(launch_embed<T>(ctx->embed, ctx->rows, 0, R, ctx->hidden, ctx->xn, ctx->ssq, ctx->norms, ctx->D.d, st));
    } else {
      HIPCHK(launch_sched(ctx->plans, B, ctx->rows, ctx->map, ctx->cand, ctx->freel, ctx->cursor, ctx->anchor, N,
                          ctx->D.P, ctx->opt.decs, ctx->opt.single_exit, ncap, st));
      // explorer 0's rows (the round's first) start from their token's embedding
      HIPCHK(launch_embed<T>(ctx->embed, ctx->rows, 0, stage_tot[0], ctx->hidden, ctx->xn, ctx->ssq, ctx->norms,
                             ctx->D.d, st));
    }
    prof_end(ctx, mk, 2, (double)R * sizeof(RowInfo) + (double)stage_tot[0] * ctx->D.d * (4 + sizeof(T)), 0);
    std::vector<std::pair<int, int>> stage_rows;
    for (int j = 0; j < N; ++j) stage_rows.push_back({stage_off[j], stage_tot[j]});
    int rc = run_layers<T>(ctx, R, stage_rows, ar ? ctx->L : ctx->S, ar ? 0 : 1, nitems, max_keys, true,
                           attn_bytes, attn_flops);
    if (rc) return rc;
    // Inducing adapters on the exit rows of non-final explorers.
    if (!ar && ctx->cfg.adapter_hidden > 0) {
      std::vector<std::array<int, 3>> ad;
      for (int j = 0; j < N - 1; ++j)
        if (stage_tot[j] && (!ctx->opt.single_exit || j == 0)) ad.push_back({j, stage_off[j], stage_tot[j]});
      rc = run_adapters<T>(ctx, ad);
      if (rc) return rc;
    }
    // Every row exits, except intermediate explorers in the single-exit ablation.
    std::vector<std::pair<int, int>> exits;
    if (!ar && ctx->opt.single_exit && N > 1) {
      if (stage_tot[0]) exits.push_back({stage_off[0], stage_tot[0]});
      if (stage_tot[N - 1]) exits.push_back({stage_off[N - 1], stage_tot[N - 1]});
    } else {
      exits.push_back({0, R});
    }
    rc = run_head<T>(ctx, exits);
    if (rc) return rc;
    mk = prof_begin(ctx, DEX_PROF_LATTICE);
    if (ncommit) {
      if (ar) {
        HIPCHK(launch_ar_commit(ctx->plans, B, ctx->cand, ctx->margin, ctx->anchor, ctx->records, ctx->dbg_u,
                                ctx->dbg_m, ctx->D.P, ctx->L, st));
      } else {
        HIPCHK(launch_commit(ctx->plans, B, ctx->map, ctx->cand, ctx->margin, ctx->freel, ctx->cursor, ctx->anchor,
                             ctx->records, ctx->promote, ctx->dbg_u, ctx->dbg_m, ctx->Xd, N, ctx->D.P,
                             ctx->opt.single_exit, ncap, st));
        HIPCHK(launch_promote(ctx->plans, B, ctx->promote, ctx->exb, ctx->kvc, ctx->D, st));
      }
      HIPCHK(hipMemcpyAsync(ctx->h_records, ctx->records, (size_t)B * 5 * 4, hipMemcpyDeviceToHost, st));
    }
    prof_end(ctx, mk, ncommit ? (ar ? 1 : 2) : 0,
             ar ? 0.0 : 2.0 * ncommit * ctx->L * 2.0 * ctx->D.nkv * ctx->D.hd * 2 * ctx->D.kvp, 0);
    return DEX_OK;
  };
  // Timed rounds run eagerly: an event recorded inside a replayed graph does
  // not wait for the kernel before it, so it cannot time that kernel.
  const bool graphs = !(ctx->opt.debug & 2) && !ctx->prof && !ctx->no_graphs;
  const std::string key = graphs ? graph_key(ar, max_keys, ctx->attn_nj, shape, ctx->h_plans, B) : std::string();
  auto found = graphs ? ctx->graphs.find(key) : ctx->graphs.end();
  if (found != ctx->graphs.end()) {
    HIPCHK(hipGraphLaunch(found->second, st));
  } else if (graphs && ++ctx->graph_seen[key] >= 2 && ctx->graphs.size() < kMaxGraphs) {
    // Capture on the library's own stream (the caller's may be the legacy
    // default stream, which cannot be captured), launch on the caller's.
    HIPCHK(hipStreamBeginCapture(ctx->cap_st, hipStreamCaptureModeThreadLocal));
    ctx->st = ctx->cap_st;
    const int rc = enqueue();
    ctx->st = st;
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(ctx->cap_st, &g);
    if (rc != DEX_OK || e != hipSuccess) {
      if (g) (void)hipGraphDestroy(g);
      if (rc == DEX_OK) {
        ctx->err = std::string("hipStreamEndCapture: ") + hipGetErrorString(e);
        ctx->poisoned = true;
        return DEX_EHIP;
      }
      return rc;
    }
    hipGraphExec_t exec = nullptr;
    const hipError_t ei = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    HIPCHK(ei);
    ctx->graphs.emplace(key, exec);
    HIPCHK(hipGraphLaunch(exec, st));
  } else {
    const int rc = enqueue();
    if (rc) return rc;
  }
  HIPCHK(hipStreamSynchronize(st));
  prof_collect(ctx);
  int n = 0;
  for (int s = 0; s < B; ++s) {
    if (!live[s]) continue;
    if (ctx->h_plans[s].commit) {
      const int* r = ctx->h_records + s * 5;
      dex_commit c;
      c.seq = r[0];
      c.position = r[1];
      c.token = r[2];
      c.branch = r[3];
      c.layers = r[4];
      out[n++] = c;
      ctx->C_[s] += 1;
      ctx->commits_[s] += 1;
      ctx->q_[s] = next_q(ctx->q_[s], true, ar, ncap, c.branch, N);
    } else {
      ctx->q_[s] = next_q(ctx->q_[s], false, ar, ncap, 0, N);
    }
  }
  *n_out = n;
  ctx->any_commit = ctx->any_commit || n > 0;
  for (int j = 0; j < N; ++j) ctx->last_rows[j] = stage_tot[j];
  ctx->last_total = R;
  return DEX_OK;
}

template <typename T>
int run_prefill(dex_ctx* ctx, int n_seqs, const int32_t* tokens, const int32_t* lens) {
  hipStream_t st = ctx->st;
  std::vector<int> anchors(n_seqs);
  size_t off = 0;
  for (int s = 0; s < n_seqs; ++s) {
    anchors[s] = tokens[off + lens[s] - 1];
    off += lens[s];
  }
  HIPCHK(hipMemcpy(ctx->anchors_in, anchors.data(), n_seqs * 4, hipMemcpyHostToDevice));
  HIPCHK(launch_reset(ctx->map, ctx->freel, ctx->cursor, ctx->anchor, ctx->anchors_in, n_seqs, ctx->D.P, st));
  const int base_h = ctx->opt.max_batch * ctx->D.P;
  const int per_item = std::max(1, kAttnUnits / (ctx->D.nq / ctx->D.nkv));
  PrefillCursor cur;
  for (;;) {
    int nitems = 0, max_keys = 0;
    const int R = prefill_chunk(tokens, lens, n_seqs, base_h, per_item, cur, ctx->h_rows, ctx->h_items, nitems,
                                max_keys);
    if (R == 0) break;
    HIPCHK(hipMemcpyAsync(ctx->rows, ctx->h_rows, R * sizeof(RowInfo), hipMemcpyHostToDevice, st));
    attn_block_list(ctx, nitems);
    HIPCHK(hipMemcpyAsync(ctx->items, ctx->h_items, nitems * sizeof(AttnItem), hipMemcpyHostToDevice, st));
    HIPCHK(hipMemcpyAsync(ctx->item_list, ctx->h_item_list,
                          (ctx->attn_single + ctx->attn_groups + ctx->attn_tails) * sizeof(int),
                          hipMemcpyHostToDevice, st));
    HIPCHK(launch_embed<T>(ctx->embed, ctx->rows, 0, R, ctx->hidden, ctx->xn, ctx->ssq, ctx->norms, ctx->D.d, st));
    std::vector<std::pair<int, int>> stage_rows = {{0, R}};
    const int rc = run_layers<T>(ctx, R, stage_rows, ctx->L, 0, nitems, max_keys, false);
    if (rc) return rc;
    HIPCHK(hipStreamSynchronize(st));  // host row buffers are reused by the next chunk
  }
  HIPCHK(hipStreamSynchronize(st));
  return DEX_OK;
}

}  // namespace

extern "C" {

int dex_workspace_bytes(const dex_model_config* cfg, const int32_t* X, int32_t n_x, const dex_options* opt,
                        size_t* out_bytes) {
  std::string err;
  const int rc = validate(cfg, X, n_x, opt, err);
  if (rc) {
    g_create_error = err;
    return rc;
  }
  if (!out_bytes) {
    g_create_error = "null output";
    return DEX_EINVAL;
  }
  *out_bytes = plan_workspace(cfg, X, n_x, opt).total;
  return DEX_OK;
}

int dex_create(const dex_model_config* cfg, const dex_weights* w, const int32_t* X, int32_t n_x, int32_t L,
               const dex_options* opt, void* d_workspace, size_t ws_bytes, void* stream, dex_ctx** out) {
  std::string err;
  int rc = validate(cfg, X, n_x, opt, err);
  if (!rc && (!w || !d_workspace || !out)) { err = "null weights, workspace or output"; rc = DEX_EINVAL; }
  if (!rc && L != cfg->n_layers) { err = "L must equal cfg->n_layers"; rc = DEX_EINVAL; }
  if (!rc) {
    const bool tied = cfg->tied_head != 0;
    bool ok = w->tok_embed && w->final_norm && (tied || w->lm_head) && w->attn_norm && w->wq && w->wk && w->wv &&
              w->wo && w->ffn_norm && w->w_gate && w->w_up && w->w_down;
    for (int l = 0; ok && l < cfg->n_layers; ++l)
      ok = w->attn_norm[l] && w->wq[l] && w->wk[l] && w->wv[l] && w->wo[l] && w->ffn_norm[l] && w->w_gate[l] &&
           w->w_up[l] && w->w_down[l];
    if (ok && cfg->adapter_hidden > 0) {
      ok = w->adapter_w1 && w->adapter_b1 && w->adapter_w2 && w->adapter_b2 && w->adapter_norm && w->adapter_alpha;
      for (int k = 0; ok && k < n_x - 1; ++k)
        ok = w->adapter_w1[k] && w->adapter_b1[k] && w->adapter_w2[k] && w->adapter_b2[k] && w->adapter_norm[k];
    }
    if (!ok) { err = "null weight pointer"; rc = DEX_EINVAL; }
  }
  WsPlan wp;
  if (!rc) {
    wp = plan_workspace(cfg, X, n_x, opt);
    if (ws_bytes < wp.total) {
      char buf[160];
      snprintf(buf, sizeof buf, "workspace too small: %zu < %zu bytes", ws_bytes, wp.total);
      err = buf;
      rc = DEX_ENOSPC;
    }
  }
  // the static scratch of dex_step_noalloc, looked up once per device
  const int device = rc ? -1 : scratch_setup(err);
  if (!rc && device < 0) rc = DEX_EHIP;
  if (rc) {
    g_create_error = err;
    return rc;
  }
  dex_ctx* ctx = new dex_ctx();
  ctx->device = device;
  ctx->cfg = *cfg;
  ctx->opt = *opt;
  ctx->N = n_x;
  ctx->L = cfg->n_layers;
  ctx->S = longest_stage(X, n_x);
  ctx->X.assign(X, X + n_x);
  ctx->bf16 = cfg->dtype == DEX_DTYPE_BF16;
  ctx->st = (hipStream_t)stream;
  ctx->ws = (char*)d_workspace;
  ctx->wp = wp;
  ModelDims& D = ctx->D;
  D.L = cfg->n_layers;
  D.d = cfg->d_model;
  D.nq = cfg->n_heads;
  D.nkv = cfg->n_kv_heads;
  D.hd = cfg->head_dim;
  D.F = cfg->d_ffn;
  D.V = cfg->vocab;
  D.S = ctx->S;
  D.lfirst[0] = 0;
  for (int j = 0; j < n_x; ++j) D.lfirst[j + 1] = X[j];
  D.N = n_x;
  D.P = (1 << n_x) - 1;
  D.B = opt->max_batch;
  D.Cmax = opt->max_context;
  D.Cs = (D.Cmax + kKvTile - 1) / kKvTile * kKvTile;
  D.kvp = kv_planes(cfg->dtype);
  D.eps = cfg->rms_eps;
  ctx->embed = ctx->at(wp.embed);
  ctx->head = ctx->at(wp.head);
  ctx->norms = (float*)ctx->at(wp.norms);
  ctx->cosT = (float*)ctx->at(wp.cosT);
  ctx->sinT = (float*)ctx->at(wp.sinT);
  ctx->kvc = (bf16_t*)ctx->at(wp.kvc);
  ctx->exb = (bf16_t*)ctx->at(wp.exb);
  ctx->hidden = (float*)ctx->at(wp.hidden);
  ctx->xn = (float*)ctx->at(wp.xn);
  ctx->xh = (float*)ctx->at(wp.xh);
  ctx->xa = (float*)ctx->at(wp.xa);
  ctx->ssq_head = (float*)ctx->at(wp.ssq_head);
  ctx->ad_vec = (float*)ctx->at(wp.ad_vec);
  ctx->map = (int*)ctx->at(wp.map);
  ctx->cand = (int*)ctx->at(wp.cand);
  ctx->margin = (float*)ctx->at(wp.margin);
  ctx->freel = (int*)ctx->at(wp.freel);
  ctx->cursor = (int*)ctx->at(wp.cursor);
  ctx->anchor = (int*)ctx->at(wp.anchor);
  ctx->anchors_in = (int*)ctx->at(wp.anchors_in);
  ctx->records = (int*)ctx->at(wp.records);
  ctx->promote = (int*)ctx->at(wp.promote);
  ctx->dbg_u = (int*)ctx->at(wp.dbg_u);
  ctx->dbg_m = (float*)ctx->at(wp.dbg_m);
  ctx->Xd = (int*)ctx->at(wp.Xd);
  ctx->dbg_logits = (opt->debug & 1) ? (float*)ctx->at(wp.dbg_logits) : nullptr;
  ctx->rows = (RowInfo*)ctx->at(wp.rows);
  ctx->plans = (SeqPlan*)ctx->at(wp.plans);
  ctx->items = (AttnItem*)ctx->at(wp.items);
  ctx->item_list = (int*)(ctx->items + wp.Rmax);
  ctx->q = (float*)ctx->at(wp.q);
  ctx->ssq = (float*)ctx->at(wp.ssq);
  ctx->attn_out = ctx->at(wp.attn_out);
  ctx->act = ctx->at(wp.act);
  ctx->attn_part = (float*)ctx->at(wp.attn_part);
  ctx->attn_tail = (float*)ctx->at(wp.attn_tail);
  ctx->gemm_split = (float*)ctx->at(wp.gemm_split);
  ctx->head_part = (float*)ctx->at(wp.head_part);
  auto fail = [&](int code) {
    g_create_error = ctx->err;
    dex_destroy(ctx);
    return code;
  };
  if (hipStreamCreateWithFlags(&ctx->cap_st, hipStreamNonBlocking) != hipSuccess ||
      hipHostMalloc((void**)&ctx->h_plans, sizeof(SeqPlan) * D.B) != hipSuccess ||
      hipHostMalloc((void**)&ctx->h_records, 5 * 4 * D.B) != hipSuccess ||
      hipHostMalloc((void**)&ctx->h_items, (sizeof(AttnItem) + 12) * wp.Rmax) != hipSuccess ||
      hipHostMalloc((void**)&ctx->h_rows, sizeof(RowInfo) * wp.Rmax) != hipSuccess) {
    ctx->err = "stream creation or hipHostMalloc failed";
    return fail(DEX_EHIP);
  }
  ctx->h_item_list = (int*)(ctx->h_items + wp.Rmax);
  rc = ctx->bf16 ? pack_weights<bf16_t>(ctx, w) : pack_weights<float>(ctx, w);
  if (rc) return fail(rc);
  // RoPE table: angle pos * base^(-2i/hd) in double, cos/sin rounded to float.
  const int half = D.hd / 2;
  std::vector<float> cs((size_t)D.Cmax * half), sn((size_t)D.Cmax * half);
  for (int p = 0; p < D.Cmax; ++p)
    for (int i = 0; i < half; ++i) {
      const double ang = (double)p * std::pow((double)cfg->rope_base, -2.0 * i / D.hd);
      cs[(size_t)p * half + i] = (float)std::cos(ang);
      sn[(size_t)p * half + i] = (float)std::sin(ang);
    }
  int xd[kMaxN] = {0};
  for (int k = 0; k < n_x; ++k) xd[k] = X[k];
  if (hipMemcpy(ctx->cosT, cs.data(), cs.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(ctx->sinT, sn.data(), sn.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(ctx->Xd, xd, sizeof(xd), hipMemcpyHostToDevice) != hipSuccess ||
      hipStreamSynchronize(ctx->st) != hipSuccess) {
    ctx->err = "upload of tables failed";
    return fail(DEX_EHIP);
  }
  *out = ctx;
  return DEX_OK;
}

int dex_prefill(dex_ctx* ctx, int32_t n_seqs, const int32_t* tokens, const int32_t* lens) {
  if (!ctx) return DEX_EINVAL;
  if (ctx->poisoned) return DEX_EHIP;
  if (n_seqs < 1 || n_seqs > ctx->opt.max_batch || !tokens || !lens) {
    ctx->err = "n_seqs must be 1..max_batch with non-null tokens and lens";
    return DEX_EINVAL;
  }
  size_t total = 0;
  for (int s = 0; s < n_seqs; ++s) {
    if (lens[s] < 1) { ctx->err = "prompt length must be >= 1"; return DEX_EINVAL; }
    if ((long long)lens[s] + ctx->opt.max_new_tokens + ctx->N > ctx->opt.max_context) {
      ctx->err = "prompt length + max_new_tokens + N exceeds max_context";
      return DEX_ENOSPC;
    }
    total += lens[s];
  }
  for (size_t i = 0; i < total; ++i)
    if (tokens[i] < 0 || tokens[i] >= ctx->D.V) { ctx->err = "token id outside [0, vocab)"; return DEX_EINVAL; }
  const int rc = ctx->bf16 ? run_prefill<bf16_t>(ctx, n_seqs, tokens, lens) : run_prefill<float>(ctx, n_seqs, tokens, lens);
  if (rc) return rc;
  ctx->nseq = n_seqs;
  ctx->q_.assign(n_seqs, 0);
  ctx->C_.assign(n_seqs, 0);
  ctx->commits_.assign(n_seqs, 0);
  ctx->plen_.assign(n_seqs, 0);
  for (int s = 0; s < n_seqs; ++s) {
    ctx->C_[s] = lens[s] - 1;
    ctx->plen_[s] = lens[s];
  }
  ctx->mode_used = 0;
  ctx->any_commit = false;
  return DEX_OK;
}

static int step_common(dex_ctx* ctx, bool ar, dex_commit* out, int32_t cap, int32_t* n_out) {
  if (!ctx) return DEX_EINVAL;
  if (ctx->poisoned) return DEX_EHIP;
  if (!out || !n_out) { ctx->err = "null output"; return DEX_EINVAL; }
  if (ctx->nseq == 0) { ctx->err = "no prefill"; return DEX_ESTATE; }
  const int want = ar ? 2 : 1;
  if (ctx->mode_used && ctx->mode_used != want) {
    ctx->err = "lattice and autoregressive steps cannot be mixed after one prefill";
    return DEX_ESTATE;
  }
  const int rc = ctx->bf16 ? run_step<bf16_t>(ctx, ar, out, cap, n_out) : run_step<float>(ctx, ar, out, cap, n_out);
  if (rc == DEX_OK) ctx->mode_used = want;
  return rc;
}

int dex_step(dex_ctx* ctx, dex_commit* out, int32_t cap, int32_t* n_out) { return step_common(ctx, false, out, cap, n_out); }

int dex_ar_step(dex_ctx* ctx, dex_commit* out, int32_t cap, int32_t* n_out) { return step_common(ctx, true, out, cap, n_out); }

int dex_step_noalloc(dex_ctx* ctx, dex_commit* out, int32_t cap, int32_t* n_out) {
  if (!ctx) return DEX_EINVAL;
  if (ctx->poisoned) return DEX_EHIP;
  const WsPlan& wp = ctx->wp;
  size_t need = 0;
  for (int r = 0; r < SC_N; ++r) need += (wp.sstep[r] + 255) & ~(size_t)255;
  if (need > kStaticScratchBytes) {
    char buf[200];
    snprintf(buf, sizeof buf, "per-round scratch of this context (%zu bytes) exceeds the static scratch (%zu bytes)",
             need, kStaticScratchBytes);
    ctx->err = buf;
    return DEX_ENOSPC;
  }
  char* base = (char*)g_scratch_ptr[ctx->device];
  if (base == nullptr) {
    ctx->err = "static scratch not set up on the context's device";
    return DEX_EHIP;
  }
  size_t off[SC_N];
  size_t o = 0;
  for (int r = 0; r < SC_N; ++r) {
    off[r] = o;
    o += (wp.sstep[r] + 255) & ~(size_t)255;
  }
  // the round's scratch regions point into the static array for this call only
  RowInfo* rows = ctx->rows;
  SeqPlan* plans = ctx->plans;
  AttnItem* items = ctx->items;
  int* item_list = ctx->item_list;
  float *q = ctx->q, *attn_part = ctx->attn_part, *attn_tail = ctx->attn_tail, *gemm_split = ctx->gemm_split,
        *head_part = ctx->head_part;
  void *attn_out = ctx->attn_out, *act = ctx->act;
  const bool prof = ctx->prof;
  ctx->rows = (RowInfo*)(base + off[SC_ROWS]);
  ctx->plans = (SeqPlan*)(base + off[SC_PLANS]);
  ctx->items = (AttnItem*)(base + off[SC_ITEMS]);
  ctx->item_list = (int*)(ctx->items + wp.Rstep);
  ctx->q = (float*)(base + off[SC_Q]);
  ctx->attn_out = base + off[SC_ATTN_OUT];
  ctx->act = base + off[SC_ACT];
  ctx->attn_part = (float*)(base + off[SC_ATTN_PART]);
  ctx->attn_tail = (float*)(base + off[SC_ATTN_TAIL]);
  ctx->gemm_split = (float*)(base + off[SC_GEMM_SPLIT]);
  ctx->head_part = (float*)(base + off[SC_HEAD_PART]);
  ctx->no_graphs = true;    // no graph capture or instantiation
  ctx->prof = false;        // no timing events
  const int rc = step_common(ctx, false, out, cap, n_out);
  ctx->rows = rows;
  ctx->plans = plans;
  ctx->items = items;
  ctx->item_list = item_list;
  ctx->q = q;
  ctx->attn_out = attn_out;
  ctx->act = act;
  ctx->attn_part = attn_part;
  ctx->attn_tail = attn_tail;
  ctx->gemm_split = gemm_split;
  ctx->head_part = head_part;
  ctx->no_graphs = false;
  ctx->prof = prof;
  return rc;
}

int dex_debug_anchor(dex_ctx* ctx, int32_t seq, int32_t* u, float* margins, float* logits) {
  if (!ctx) return DEX_EINVAL;
  if (ctx->poisoned) return DEX_EHIP;
  if (seq < 0 || seq >= ctx->nseq) { ctx->err = "seq out of range"; return DEX_EINVAL; }
  if (logits && !(ctx->opt.debug & 1)) { ctx->err = "logits need options.debug bit 0"; return DEX_EINVAL; }
  if (ctx->commits_[seq] == 0) { ctx->err = "sequence has no commit yet"; return DEX_ESTATE; }
  const int n = ctx->mode_used == 2 ? 1 : ctx->N;
  if (u) HIPCHK(hipMemcpy(u, ctx->dbg_u + seq * kMaxN, n * 4, hipMemcpyDeviceToHost));
  if (margins) HIPCHK(hipMemcpy(margins, ctx->dbg_m + seq * kMaxN, n * 4, hipMemcpyDeviceToHost));
  if (logits) HIPCHK(hipMemcpy(logits, ctx->dbg_logits + (size_t)seq * ctx->D.V, (size_t)ctx->D.V * 4, hipMemcpyDeviceToHost));
  return DEX_OK;
}

int dex_last_step_rows(const dex_ctx* ctx, int32_t* rows_per_stage, int32_t* total_rows) {
  if (!ctx) return DEX_EINVAL;
  if (rows_per_stage)
    for (int j = 0; j < ctx->N; ++j) rows_per_stage[j] = ctx->last_rows[j];
  if (total_rows) *total_rows = ctx->last_total;
  return DEX_OK;
}

int dex_profile(dex_ctx* ctx, int32_t enable, dex_kernel_stats* out, int32_t n) {
  if (!ctx) return DEX_EINVAL;
  if (ctx->poisoned) return DEX_EHIP;
  if (out && (n < 0 || n > DEX_PROF_NCLASS)) {
    ctx->err = "n must be 0..DEX_PROF_NCLASS";
    return DEX_EINVAL;
  }
  if (out) {
    for (int i = 0; i < n; ++i) out[i] = ctx->stats[i];
    for (int i = 0; i < DEX_PROF_NCLASS; ++i) ctx->stats[i] = dex_kernel_stats{};
  }
  ctx->prof = enable != 0;
  return DEX_OK;
}

void dex_destroy(dex_ctx* ctx) {
  if (!ctx) return;
  for (auto& kv : ctx->graphs) (void)hipGraphExecDestroy(kv.second);
  if (ctx->cap_st) (void)hipStreamDestroy(ctx->cap_st);
  for (auto& m : ctx->marks) {
    if (m.a) (void)hipEventDestroy(m.a);
    if (m.b) (void)hipEventDestroy(m.b);
  }
  if (ctx->h_plans) (void)hipHostFree(ctx->h_plans);
  if (ctx->h_records) (void)hipHostFree(ctx->h_records);
  if (ctx->h_items) (void)hipHostFree(ctx->h_items);
  if (ctx->h_rows) (void)hipHostFree(ctx->h_rows);
  delete ctx;
}

const char* dex_last_error(const dex_ctx* ctx) {
  if (!ctx) return g_create_error.c_str();
  return ctx->err.c_str();
}

}  // extern "C"
