// Host plan of the DEX lattice step: the configuration checks, the workspace
// layout, and what one round runs -- rows per (sequence, explorer), the
// per-sequence plans, the attention work items and block lists, the HIP-graph
// key and the FSM update after the round. Pure functions of host state with
// no device calls: dex_capi.hip runs them, and the host tests build this
// header alone (DEX_HD empty) under AddressSanitizer.
//
// The lattice is numbered as a heap (Depth Exploration for LLM Decoding,
// Section 3.2, Figure 2 and "Finite-state control and collapse"): round q of
// a tree runs heap level q, the nodes 2^q - 1 .. 2^(q+1) - 2; node n belongs
// to explorer ctz(n + 1) and reads popcount(n + 1) - 1 explore-buffer
// ancestors. After a commit with branch b the kept subtree has done N - 1 - b
// rounds (Algorithm 1's collapse).
#pragma once
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "dex.h"
#include "types.h"

namespace dex {

// Rows of one prefill chunk (positions of one or more sequences). 2048
// against 512: the GQA workload's sixteen 8192-token prompts 7.39 -> 5.20 s,
// the 13B-shaped batch's eight 1024-token prompts 618 -> 505 ms.
#ifndef DEX_PREFILL_ROWS
#define DEX_PREFILL_ROWS 2048
#endif
constexpr int kPrefillRows = DEX_PREFILL_ROWS;

struct Layout {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  }
};

// Every buffer of the workspace, as byte offsets.
struct WsPlan {
  size_t embed, head, norms, cosT, sinT, kvc, exb, hidden, xn, xh, xa, ssq_head, ad_vec;
  std::vector<size_t> wad1, wad2;  // packed inducing adapters, one per non-final explorer
  size_t map, cand, margin, freel, cursor, anchor, anchors_in, records, promote, dbg_u, dbg_m, Xd, dbg_logits;
  size_t rows, plans, items, q, attn_out, act, attn_part, attn_tail, head_part, ssq, gemm_split;
  std::vector<size_t> wqkv, wo, wgu, wdown;
  size_t total;
  int Rmax, nchunk, split_cols;
  size_t sbytes[10];   // bytes of the per-round scratch regions (ScratchRegion order)
  // The same regions sized for lattice and autoregressive rounds only (Rstep
  // rows: no prefill chunk), which is all dex_step_noalloc needs.
  int Rstep;
  size_t sstep[10];
};

// Per-round scratch regions of the workspace: written by a round before they
// are read and never carried to the next round (plan staging, attention and
// GEMM partial results, exit-head tile summaries). dex_step_noalloc takes
// them from the static device array instead.
enum ScratchRegion { SC_ROWS, SC_PLANS, SC_ITEMS, SC_Q, SC_ATTN_OUT, SC_ACT, SC_ATTN_PART, SC_ATTN_TAIL, SC_GEMM_SPLIT,
                     SC_HEAD_PART, SC_N };

inline size_t esize(int dtype) { return dtype == DEX_DTYPE_BF16 ? 2 : 4; }
// 16-bit planes per cached K or V value: fp16 for bfloat16 models, a bfloat16
// (hi, lo) pair for fp32 models.
inline int kv_planes(int dtype) { return dtype == DEX_DTYPE_BF16 ? 1 : 2; }

inline int validate(const dex_model_config* c, const int32_t* X, int32_t n_x, const dex_options* o, std::string& err) {
  if (!c || !X || !o) { err = "null argument"; return DEX_EINVAL; }
  if (c->n_layers < 1 || c->d_model < 16 || c->n_heads < 1 || c->n_kv_heads < 1 || c->d_ffn < 8 || c->vocab < 16) {
    err = "non-positive model dimension"; return DEX_EINVAL;
  }
  if (c->dtype != DEX_DTYPE_F32 && c->dtype != DEX_DTYPE_BF16) { err = "dtype must be F32 or BF16"; return DEX_EINVAL; }
  if (c->head_dim != 64 && c->head_dim != 128) { err = "head_dim must be 64 or 128"; return DEX_EINVAL; }
  if (c->n_heads % c->n_kv_heads) { err = "n_heads must be a multiple of n_kv_heads"; return DEX_EINVAL; }
  if (c->n_heads / c->n_kv_heads > kAttnUnits) { err = "too many query heads per kv head"; return DEX_EINVAL; }
  const int kstep = c->dtype == DEX_DTYPE_BF16 ? 32 : 16;
  if (c->d_model % kstep || (c->n_heads * c->head_dim) % kstep || c->d_ffn % kstep) {
    err = "d_model, n_heads*head_dim and d_ffn must be multiples of the MFMA k-step (32 bf16, 16 fp32)";
    return DEX_EINVAL;
  }
  if (c->d_model % 16 || c->vocab % 16 || c->d_ffn % 8) { err = "d_model and vocab must be multiples of 16, d_ffn of 8"; return DEX_EINVAL; }
  if (!(c->rms_eps > 0) || !(c->rope_base > 1)) { err = "rms_eps and rope_base must be positive"; return DEX_EINVAL; }
  if (n_x < 1 || n_x > kMaxN) { err = "number of exploration depths must be 1..10"; return DEX_EINVAL; }
  if (c->adapter_hidden < 0 || c->adapter_hidden % (c->dtype == DEX_DTYPE_BF16 ? 32 : 16)) {
    err = "adapter_hidden must be 0 or a positive multiple of the MFMA k-step (32 bf16, 16 fp32)";
    return DEX_EINVAL;
  }
  for (int k = 0; k < n_x; ++k) {
    if (X[k] < 1 || (k > 0 && X[k] <= X[k - 1])) { err = "exploration set must be strictly increasing within [1, L]"; return DEX_EINVAL; }
  }
  if (X[n_x - 1] != c->n_layers) { err = "the last exploration depth must equal L"; return DEX_EINVAL; }
  if (o->max_batch < 1 || o->max_batch > 64) { err = "max_batch must be 1..64"; return DEX_EINVAL; }
  if (o->max_context < 2) { err = "max_context must be at least 2"; return DEX_EINVAL; }
  if (o->max_new_tokens < 1) { err = "max_new_tokens must be positive"; return DEX_EINVAL; }
  if (o->mode != DEX_GREEDY && o->mode != DEX_SAMPLE) { err = "mode must be GREEDY or SAMPLE"; return DEX_EINVAL; }
  if (o->single_exit != 0 && o->single_exit != 1) { err = "single_exit must be 0 or 1"; return DEX_EINVAL; }
  if (o->branch_cap < 0 || o->branch_cap > n_x) { err = "branch_cap must be 0..N"; return DEX_EINVAL; }
  if (o->single_exit && o->branch_cap) { err = "branch_cap and single_exit cannot be combined"; return DEX_EINVAL; }
  if (o->mode == DEX_SAMPLE) {
    if (!(o->temperature > 0)) { err = "temperature must be positive"; return DEX_EINVAL; }
    if (!o->gumbel) { err = "sampling needs Gumbel rows"; return DEX_EINVAL; }
    if (((uintptr_t)o->gumbel & 15) != 0) { err = "gumbel must be 16-byte aligned"; return DEX_EINVAL; }
    if (o->gumbel_rows < o->max_new_tokens + n_x - 1) { err = "gumbel_rows must be >= max_new_tokens + N - 1"; return DEX_EINVAL; }
  }
  return DEX_OK;
}

// Layers of the longest stage: max over j of d_j - d_{j-1} (d_{-1} = 0).
inline int longest_stage(const int32_t* X, int n_x) {
  int s = 0;
  for (int j = 0; j < n_x; ++j) s = std::max(s, X[j] - (j ? X[j - 1] : 0));
  return s;
}

inline WsPlan plan_workspace(const dex_model_config* c, const int32_t* X, int n_x, const dex_options* o) {
  WsPlan w;
  Layout lay;
  const size_t es = esize(c->dtype);
  const size_t L = c->n_layers, d = c->d_model, nq = c->n_heads, nkv = c->n_kv_heads, hd = c->head_dim,
               F = c->d_ffn, V = c->vocab, B = o->max_batch, Cmax = o->max_context;
  const int N = n_x, S = longest_stage(X, n_x), P = (1 << N) - 1;
  w.Rmax = std::max(std::max((int)B << (N - 1), kPrefillRows), (int)B);
  w.nchunk = (int)((Cmax + kAttnSCKeys - 1) / kAttnSCKeys);
  const size_t Cs = (Cmax + kKvTile - 1) / kKvTile * kKvTile;
  const size_t R = w.Rmax;
  w.embed = lay.take(V * d * es);
  w.head = lay.take(V * d * es);
  for (size_t l = 0; l < L; ++l) {
    w.wqkv.push_back(lay.take((nq + 2 * nkv) * hd * d * es));
    w.wo.push_back(lay.take(d * nq * hd * es));
    w.wgu.push_back(lay.take(2 * F * d * es));
    w.wdown.push_back(lay.take(d * F * es));
  }
  w.norms = lay.take((2 * L + 1) * d * 4);
  const size_t m = c->adapter_hidden;
  for (int k = 0; m && k < N - 1; ++k) {
    w.wad1.push_back(lay.take(m * d * es));
    w.wad2.push_back(lay.take(d * m * es));
  }
  w.ad_vec = lay.take(m ? (size_t)(N - 1) * (m + 2 * d) * 4 : 0);   // per adapter: b1 [m], b2 [d], norm [d]
  w.cosT = lay.take(Cmax * (hd / 2) * 4);
  w.sinT = lay.take(Cmax * (hd / 2) * 4);
  const size_t kvb = 2 * 2 * (size_t)kv_planes(c->dtype);   // bytes of a position's K and V per dim
  w.kvc = lay.take(B * L * nkv * Cs * hd * kvb);
  w.exb = lay.take(B * P * S * nkv * hd * kvb);
  w.hidden = lay.take((B * P + kPrefillRows) * d * 4);
  w.xn = lay.take((B * P + kPrefillRows) * d * 4);
  w.xh = lay.take((B * P + kPrefillRows) * d * 4);
  w.xa = lay.take(m ? (B * P + kPrefillRows) * d * 4 : 0);
  w.ssq_head = lay.take((B * P + kPrefillRows) * (d / 16) * 4);
  w.map = lay.take(B * P * 4);
  w.cand = lay.take(B * P * 4);
  w.margin = lay.take(B * P * 4);
  w.freel = lay.take(B * P * 4);
  w.cursor = lay.take(B * 4);
  w.anchor = lay.take(B * 4);
  w.anchors_in = lay.take(B * 4);
  w.records = lay.take(B * 5 * 4);
  w.promote = lay.take(B * kMaxN * 4);
  w.dbg_u = lay.take(B * kMaxN * 4);
  w.dbg_m = lay.take(B * kMaxN * 4);
  w.Xd = lay.take(kMaxN * 4);
  w.dbg_logits = lay.take((o->debug & 1) ? B * V * 4 : 0);
  w.split_cols = (int)std::max(std::max((nq + 2 * nkv) * hd, 2 * F), d);
  auto scratch_sizes = [&](size_t R, size_t* sb) {
    sb[SC_ROWS] = R * sizeof(RowInfo);
    sb[SC_PLANS] = B * sizeof(SeqPlan);
    sb[SC_ITEMS] = R * (sizeof(AttnItem) + 12);   // items, then the attention block lists (3 R ints)
    sb[SC_Q] = R * nq * hd * 4;
    sb[SC_ATTN_OUT] = R * nq * hd * 4;
    sb[SC_ACT] = R * std::max(F, m) * 4;
    sb[SC_ATTN_PART] = R * nq * w.nchunk * (hd + 4) * 4;
    sb[SC_ATTN_TAIL] = R * nq * kMixSlots * (hd + 4) * 4;
    // the split-range partials serve the wide (bf16) GEMM only
    sb[SC_GEMM_SPLIT] = c->dtype == DEX_DTYPE_BF16 ? (size_t)kKSplit * kSplitRows * w.split_cols * 4 : 0;
    sb[SC_HEAD_PART] = R * (V / 16) * 3 * 4;
  };
  w.Rstep = std::max((int)B << (N - 1), (int)B);
  scratch_sizes(R, w.sbytes);
  scratch_sizes(w.Rstep, w.sstep);
  w.rows = lay.take(w.sbytes[SC_ROWS]);
  w.plans = lay.take(w.sbytes[SC_PLANS]);
  w.items = lay.take(w.sbytes[SC_ITEMS]);
  w.q = lay.take(w.sbytes[SC_Q]);
  w.ssq = lay.take((B * P + kPrefillRows) * (d / 16) * 4);
  w.attn_out = lay.take(w.sbytes[SC_ATTN_OUT]);
  w.act = lay.take(w.sbytes[SC_ACT]);
  w.attn_part = lay.take(w.sbytes[SC_ATTN_PART]);
  w.attn_tail = lay.take(w.sbytes[SC_ATTN_TAIL]);
  w.gemm_split = lay.take(w.sbytes[SC_GEMM_SPLIT]);
  w.head_part = lay.take(w.sbytes[SC_HEAD_PART]);
  w.total = lay.off;
  return w;
}

// Node cap of the lattice (node_held): 1 for the single-exit ablation, the
// pruned lattice's branch_cap below N, else 0 (every node).
inline int node_cap(const dex_options& o, int N) {
  if (o.single_exit) return 1;
  return o.branch_cap > 0 && o.branch_cap < N ? o.branch_cap : 0;
}

// Attention blocks: the items of one (sequence, stage) are covered in groups of
// up to kAttnGroup consecutive items; item i of n leads a group of this size (0:
// inside a group).
inline int attn_lead(int i, int n) { return i % kAttnGroup ? 0 : std::min(kAttnGroup, n - i); }

// Rows of one round: which sequences are live (fewer than T commits), and
// the rows of sequence s at explorer j (rows[s N + j]), from the FSM states q
// alone: the nodes of heap level q of each tree (2^(q-1-j) at explorer j < q,
// one at explorer q; with a node cap, the level's held nodes), or one row at
// explorer 0 per sequence for an autoregressive step. stage_tot and
// stage_off: the rows of explorer j over the batch, and where they start
// (rows of one explorer are contiguous, sequences in order within it).
struct RoundShape {
  std::vector<int> live, rows;
  int stage_tot[kMaxN + 1] = {0};
  int stage_off[kMaxN + 1] = {0};
  int nlive = 0, R = 0;
};

inline void round_rows(const int* q, const int* commits, int B, int N, int T, bool ar, int ncap, RoundShape& r) {
  r.live.assign(B, 0);
  r.rows.assign((size_t)B * N, 0);
  std::fill(r.stage_tot, r.stage_tot + kMaxN + 1, 0);
  r.nlive = 0;
  for (int s = 0; s < B; ++s) {
    r.live[s] = commits[s] < T;
    if (!r.live[s]) continue;
    ++r.nlive;
    const int qs = ar ? 0 : q[s];
    if (!ar && ncap) {   // pruned lattice (single-exit: one node per explorer 0..q)
      for (int n = (1 << qs) - 1; n <= (1 << (qs + 1)) - 2; ++n)
        if (node_held(n + 1, ncap)) ++r.rows[(size_t)s * N + __builtin_ctz(n + 1)];
    }
    for (int j = 0; j < N; ++j) {
      int& c = r.rows[(size_t)s * N + j];
      if (ar) c = j == 0 ? 1 : 0;
      else if (!ncap) c = j < qs ? 1 << (qs - 1 - j) : (j == qs ? 1 : 0);   // full lattice
      r.stage_tot[j] += c;
    }
  }
  r.stage_off[0] = 0;
  for (int j = 0; j < N; ++j) r.stage_off[j + 1] = r.stage_off[j] + r.stage_tot[j];
  r.R = r.stage_off[N];
}

// Per-sequence plans of the round (plans[0..B)); returns the sequences that
// commit this round (those whose round reaches the final explorer, every live
// one for an autoregressive step).
inline int seq_plans(const RoundShape& r, const int* q, const int* C, const int* plen, int B, int N, bool ar,
                     SeqPlan* plans) {
  int cursor[kMaxN];
  std::copy(r.stage_off, r.stage_off + N, cursor);
  int ncommit = 0;
  for (int s = 0; s < B; ++s) {
    SeqPlan& p = plans[s];
    std::memset(&p, 0, sizeof(p));
    p.live = r.live[s];
    p.q = ar ? 0 : q[s];
    p.C = C[s];
    p.commit = r.live[s] && (ar || p.q + 1 == N);
    p.prompt_len = plen[s];
    ncommit += p.commit;
    for (int j = 0; j < N; ++j) {
      p.base[j] = cursor[j];
      cursor[j] += r.rows[(size_t)s * N + j];
    }
  }
  return ncommit;
}

// Attention work items of a round: the rows of one (sequence, explorer), cut
// into items of at most kAttnUnits (row, query head) units; rep = n_heads /
// n_kv_heads. Lattice rows read the committed keys [0, C) plus their explore
// keys at [C, C + q - j + 1), which lie in at most two 32-key chunks.
struct ItemStats {
  int nitems = 0, max_keys = 0;
  int umax = 1;   // most units in one item
  int nj = 0;     // most chunks holding explore keys in one item (lattice rows)
};

inline ItemStats round_items(const RoundShape& r, const SeqPlan* plans, const int* q, const int* C, int B, int N,
                             bool ar, int rep, AttnItem* items) {
  ItemStats st;
  const int per_item = std::max(1, kAttnUnits / rep);
  for (int j = 0; j < N; ++j)
    for (int s = 0; s < B; ++s) {
      const int cnt = r.rows[(size_t)s * N + j];
      const int mk = C[s] + (ar ? 1 : (q[s] - j + 1));
      for (int o = 0; o < cnt; o += per_item) {
        AttnItem& it = items[st.nitems++];
        it.seq = s;
        it.row0 = plans[s].base[j] + o;
        it.nrows = std::min(per_item, cnt - o);
        it.stage = j;
        it.max_keys = mk;
        it.xc0 = ar ? -1 : C[s] / kKvTile;
        it.xc1 = ar ? -1 : (mk - 1) / kKvTile;
        if (!ar) st.nj = std::max(st.nj, it.xc1 - it.xc0 + 1);
        it.lead = attn_lead(o / per_item, (cnt + per_item - 1) / per_item);
        st.max_keys = std::max(st.max_keys, mk);
        st.umax = std::max(st.umax, it.nrows * rep);
      }
    }
  return st;
}

// Attention block lists of the first nitems items: the items that form a
// group of their own (the shared-role blocks of attn_kernel), then the items
// that lead a group of several (attn_group_kernel), then, for items whose rows
// read explore keys, one entry 4 item + q per run q of kTailRows of the item's
// rows (the per-row chunk blocks of attn_kernel; an item has at most
// kAttnUnits rows, so q < 4), so that no launch has blocks without work. list
// receives at most nitems plus the sum over items with explore keys of
// ceil(nrows / kTailRows) entries.
struct BlockList {
  int single = 0, groups = 0, tails = 0;
};

inline BlockList attn_block_list(const AttnItem* items, int nitems, int* list) {
  BlockList b;
  for (int i = 0; i < nitems; ++i)
    if (items[i].lead == 1) list[b.single++] = i;
  for (int i = 0; i < nitems; ++i)
    if (items[i].lead > 1) list[b.single + b.groups++] = i;
  for (int i = 0; i < nitems; ++i)
    if (items[i].xc0 >= 0)
      for (int qt = 0; qt * kTailRows < items[i].nrows; ++qt) list[b.single + b.groups + b.tails++] = 4 * i + qt;
  return b;
}

// Key of a round's HIP graph: everything the enqueued work depends on beyond
// the pinned host buffers it re-reads at replay (autoregressive or lattice,
// attention super-chunk count, explore-chunk slots, each sequence's FSM state
// and commit flag).
inline std::string graph_key(bool ar, int max_keys, int nj, const RoundShape& r, const SeqPlan* plans, int B) {
  std::string key;
  key.reserve(16 + 3 * B);
  key += ar ? 'A' : 'D';
  key += std::to_string((max_keys + kAttnSCKeys - 1) / kAttnSCKeys);
  key += ':';
  key += (char)('0' + nj);
  for (int s = 0; s < B; ++s) {
    key += (char)('a' + (r.live[s] ? plans[s].q : 31));
    key += plans[s].commit ? 'c' : '.';
  }
  return key;
}

// Prefill: every prompt position but the last of each sequence goes into the
// committed cache (the last one is the first round's anchor input), through
// the layer stack in chunks of at most kPrefillRows rows. A chunk takes the
// positions in order, sequence after sequence, so one chunk can hold the end
// of one prompt and the start of the next. cursor: the next (sequence,
// position); tok_off: where that sequence's tokens start in the concatenated
// prompts.
struct PrefillCursor {
  int seq = 0, pos = 0;
  size_t tok_off = 0;
};

// Fills rows[0..R) (hidden rows base_h + i) and the chunk's attention items
// (per sequence segment, at most per_item rows each, led in groups of up to
// kAttnGroup; a group's first item carries the group's largest key count,
// since its blocks stop at that item's max_keys). Returns R, 0 when every
// position is done; max_keys: the most keys any row reads.
inline int prefill_chunk(const int32_t* tokens, const int32_t* lens, int n_seqs, int base_h, int per_item,
                         PrefillCursor& c, RowInfo* rows, AttnItem* items, int& nitems, int& max_keys) {
  int R = 0;
  nitems = 0;
  max_keys = 0;
  while (R < kPrefillRows && c.seq < n_seqs) {
    const int npos = lens[c.seq] - 1;
    if (c.pos >= npos) {
      c.tok_off += lens[c.seq];
      ++c.seq;
      c.pos = 0;
      continue;
    }
    const int take = std::min(kPrefillRows - R, npos - c.pos);
    for (int i = 0; i < take; ++i) {
      RowInfo& r = rows[R + i];
      std::memset(&r, 0, sizeof(r));
      r.seq = c.seq;
      r.hrow = base_h + R + i;
      r.pos = c.pos + i;
      r.tok = tokens[c.tok_off + c.pos + i];
      r.ncommit = c.pos + i + 1;
      r.kv_commit = 1;
    }
    const int first = nitems, nseg = (take + per_item - 1) / per_item;
    for (int o = 0; o < take; o += per_item) {
      AttnItem& it = items[nitems++];
      std::memset(&it, 0, sizeof(it));
      it.seq = c.seq;
      it.row0 = R + o;
      it.nrows = std::min(per_item, take - o);
      it.max_keys = c.pos + o + it.nrows;
      it.xc0 = it.xc1 = -1;
      it.lead = attn_lead(o / per_item, nseg);
    }
    for (int i = first; i < nitems; ++i)
      for (int k = 1; k < items[i].lead; ++k) items[i].max_keys = std::max(items[i].max_keys, items[i + k].max_keys);
    max_keys = std::max(max_keys, c.pos + take);
    R += take;
    c.pos += take;
  }
  return R;
}

// FSM state of a sequence after a round: one more level of the same tree, or
// after a commit with branch b the N - 1 - b rounds its kept subtree has done
// (none for an autoregressive step, or when a pruned lattice did not hold that
// branch's subtree).
inline int next_q(int q, bool committed, bool ar, int ncap, int branch, int N) {
  if (!committed) return q + 1;
  return ar || (ncap && branch >= ncap) ? 0 : N - 1 - branch;
}

}  // namespace dex
