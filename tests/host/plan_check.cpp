// Host checks of the lattice step's plan (csrc/plan.h), built by g++ alone with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_plan.py):
// configuration checks, workspace carving, rows per round against a brute
// enumeration of the heap level, per-sequence plans, attention items and block
// lists, the HIP-graph key, the FSM over scripted commits, the prefill
// chunks (every prompt position once, in order) and the K/V tile layout that
// the cache writers and the attention kernels share. Every buffer is
// sized exactly as the library sizes its host buffers, so a write past one is
// an ASan report. Prints "plan checks ok" and exits 0 when every check holds.
//
// Facts checked (Depth Exploration for LLM Decoding, Section 3.2, Figure 2,
// "Finite-state control and collapse" and "Commit process"; Algorithm 1):
// round q of a tree runs heap level q (nodes 2^q - 1 .. 2^(q+1) - 2, explorer
// ctz(n + 1)); a tree commits in the round that reaches the final explorer;
// after a commit with branch b the next commit comes b + 1 rounds later, so K
// commits take N + sum over the first K - 1 commits of (b + 1) rounds.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <string>
#include <vector>

#include "plan.h"

using namespace dex;

static int g_fail = 0;
#define CHECK(cond)                                                           \
  do {                                                                        \
    if (!(cond)) {                                                            \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      if (++g_fail > 20) std::exit(1);                                        \
    }                                                                         \
  } while (0)

static dex_model_config model(int L, int d, int nq, int nkv, int hd, int F, int V, int dtype) {
  dex_model_config c{};
  c.n_layers = L;
  c.d_model = d;
  c.n_heads = nq;
  c.n_kv_heads = nkv;
  c.head_dim = hd;
  c.d_ffn = F;
  c.vocab = V;
  c.rope_base = 10000.f;
  c.rms_eps = 1e-5f;
  c.dtype = dtype;
  return c;
}

static dex_options options(int B, int Cmax, int T) {
  dex_options o{};
  o.mode = DEX_GREEDY;
  o.temperature = 1.f;
  o.max_batch = B;
  o.max_context = Cmax;
  o.max_new_tokens = T;
  return o;
}

static std::vector<int32_t> uniform_x(int L, int N) {
  std::vector<int32_t> X;
  for (int k = 1; k <= N; ++k) X.push_back(L * k / N);
  return X;
}

// --- configuration checks ----------------------------------------------------
static void check_validate() {
  std::string err;
  const dex_model_config good[] = {model(4, 64, 4, 2, 64, 128, 512, DEX_DTYPE_F32),
                                    model(32, 4096, 32, 32, 128, 11008, 32000, DEX_DTYPE_BF16),
                                    model(40, 5120, 40, 40, 128, 13824, 32000, DEX_DTYPE_BF16),
                                    model(36, 4096, 32, 8, 128, 12288, 151936, DEX_DTYPE_BF16)};
  for (const auto& c : good) {
    const auto X = uniform_x(c.n_layers, 4);
    dex_options o = options(8, 2048, 64);
    CHECK(validate(&c, X.data(), 4, &o, err) == DEX_OK);
  }
  // one field wrong at a time
  auto bad = [&](auto mutate) {
    dex_model_config c = model(32, 4096, 32, 8, 128, 11008, 32000, DEX_DTYPE_BF16);
    auto X = uniform_x(32, 4);
    dex_options o = options(8, 2048, 64);
    int n_x = 4;
    mutate(c, X, o, n_x);
    err.clear();
    const int rc = validate(&c, X.data(), n_x, &o, err);
    CHECK(rc == DEX_EINVAL);
    CHECK(!err.empty());
  };
  bad([](auto& c, auto&, auto&, int&) { c.head_dim = 96; });
  bad([](auto& c, auto&, auto&, int&) { c.n_kv_heads = 5; });
  bad([](auto& c, auto&, auto&, int&) { c.n_heads = 64; c.n_kv_heads = 2; });   // 32 query heads per kv head
  bad([](auto& c, auto&, auto&, int&) { c.d_model = 4080; });                   // not a multiple of 32 (bf16)
  bad([](auto& c, auto&, auto&, int&) { c.vocab = 32001; });
  bad([](auto& c, auto&, auto&, int&) { c.dtype = 7; });
  bad([](auto& c, auto&, auto&, int&) { c.adapter_hidden = 48; });
  bad([](auto& c, auto&, auto&, int&) { c.rms_eps = 0.f; });
  bad([](auto&, auto& X, auto&, int&) { X[1] = X[0]; });                         // not increasing
  bad([](auto&, auto& X, auto&, int&) { X[3] = 31; });                           // last depth != L
  bad([](auto&, auto&, auto&, int& n) { n = 0; });
  bad([](auto&, auto&, auto&, int& n) { n = kMaxN + 1; });
  bad([](auto&, auto&, auto& o, int&) { o.max_batch = 0; });
  bad([](auto&, auto&, auto& o, int&) { o.max_batch = 65; });
  bad([](auto&, auto&, auto& o, int&) { o.mode = 2; });
  bad([](auto&, auto&, auto& o, int&) { o.branch_cap = 5; });
  bad([](auto&, auto&, auto& o, int&) { o.single_exit = 1; o.branch_cap = 2; });
  bad([](auto&, auto&, auto& o, int&) { o.mode = DEX_SAMPLE; });                 // no Gumbel rows
  bad([](auto&, auto&, auto& o, int&) {
    o.mode = DEX_SAMPLE;
    o.gumbel = (const float*)(uintptr_t)0x1004;                                  // misaligned
    o.gumbel_rows = 128;
  });
  bad([](auto&, auto&, auto& o, int&) {
    o.mode = DEX_SAMPLE;
    o.gumbel = (const float*)(uintptr_t)0x1000;
    o.gumbel_rows = 66;                                                          // < T + N - 1
  });
  // valid small configurations with up to two fields set to random values:
  // validate never crashes, and what it accepts carves cleanly
  std::mt19937 rng(7);
  auto pick = [&](std::initializer_list<int> v) { return *(v.begin() + rng() % v.size()); };
  int accepted = 0, rejected = 0;
  for (int t = 0; t < 4000; ++t) {
    const int L = pick({1, 3, 8, 12});
    dex_model_config c = model(L, pick({64, 128, 256}), 4, pick({1, 2, 4}), pick({64, 128}), pick({128, 256}),
                               pick({256, 1040, 4096}), pick({0, 1}));
    int n_x = 1 + rng() % std::min(L, 4);
    std::vector<int32_t> X = uniform_x(L, n_x);
    X.resize(kMaxN + 2, L);
    dex_options o = options(1 + rng() % 8, 64 + rng() % 512, 1 + rng() % 32);
    o.branch_cap = rng() % 3 == 0 ? (int)(rng() % (n_x + 1)) : 0;
    for (int m = rng() % 3; m > 0; --m) {
      const int v = pick({-7, -1, 0, 1, 3, 16, 31, 32, 48, 96, 1 << 30});
      switch (rng() % 14) {
        case 0: c.n_layers = v; break;
        case 1: c.d_model = v; break;
        case 2: c.n_heads = v; break;
        case 3: c.n_kv_heads = v; break;
        case 4: c.head_dim = v; break;
        case 5: c.d_ffn = v; break;
        case 6: c.vocab = v; break;
        case 7: c.adapter_hidden = v; break;
        case 8: n_x = std::max(0, std::min(v, kMaxN + 2)); break;
        case 9: X[rng() % X.size()] = v; break;
        case 10: o.max_batch = v; break;
        case 11: o.max_context = v; break;
        case 12: o.branch_cap = v; break;
        default: o.single_exit = v; break;
      }
    }
    if (validate(&c, X.data(), n_x, &o, err) != DEX_OK) {
      ++rejected;
      continue;
    }
    ++accepted;
    if (c.d_model > 4096 || c.vocab > 1 << 20 || c.d_ffn > 1 << 16 || o.max_context > 1 << 16 ||
        c.n_layers > 64 || c.adapter_hidden > 4096)
      continue;   // accepted, but too large to carve here
    const WsPlan w = plan_workspace(&c, X.data(), n_x, &o);
    CHECK(w.total % 256 == 0);
    CHECK(w.head_part + w.sbytes[SC_HEAD_PART] <= w.total);
    CHECK(w.Rmax >= (o.max_batch << (n_x - 1)));
  }
  CHECK(accepted > 200 && rejected > 200);
}

// --- workspace carving ---------------------------------------------------------
static void check_workspace() {
  struct Case { dex_model_config c; int N, B, Cmax, T, m; };
  const Case cases[] = {{model(4, 64, 4, 2, 64, 128, 512, DEX_DTYPE_F32), 4, 3, 200, 32, 0},
                        {model(32, 4096, 32, 32, 128, 11008, 32000, DEX_DTYPE_BF16), 4, 1, 1024, 256, 0},
                        {model(40, 5120, 40, 40, 128, 13824, 32000, DEX_DTYPE_BF16), 8, 8, 1300, 256, 0},
                        {model(36, 4096, 32, 8, 128, 12288, 151936, DEX_DTYPE_BF16), 9, 16, 8340, 128, 0},
                        {model(8, 256, 4, 4, 64, 512, 1024, DEX_DTYPE_BF16), 4, 2, 300, 40, 64}};
  for (const Case& k : cases) {
    dex_model_config c = k.c;
    c.adapter_hidden = k.m;
    const auto X = uniform_x(c.n_layers, k.N);
    const dex_options o = options(k.B, k.Cmax, k.T);
    std::string err;
    CHECK(validate(&c, X.data(), k.N, &o, err) == DEX_OK);
    const WsPlan w = plan_workspace(&c, X.data(), k.N, &o);
    // every region is 256-byte aligned, in the order it was taken, inside the total
    std::vector<size_t> off = {w.embed, w.head};
    for (int l = 0; l < c.n_layers; ++l) {
      off.push_back(w.wqkv[l]);
      off.push_back(w.wo[l]);
      off.push_back(w.wgu[l]);
      off.push_back(w.wdown[l]);
    }
    off.push_back(w.norms);
    for (size_t a = 0; a < w.wad1.size(); ++a) {
      off.push_back(w.wad1[a]);
      off.push_back(w.wad2[a]);
    }
    for (size_t v : {w.ad_vec, w.cosT, w.sinT, w.kvc, w.exb, w.hidden, w.xn, w.xh, w.xa, w.ssq_head, w.map, w.cand,
                     w.margin, w.freel, w.cursor, w.anchor, w.anchors_in, w.records, w.promote, w.dbg_u, w.dbg_m,
                     w.Xd, w.dbg_logits, w.rows, w.plans, w.items, w.q, w.ssq, w.attn_out, w.act, w.attn_part,
                     w.attn_tail, w.gemm_split, w.head_part})
      off.push_back(v);
    for (size_t i = 0; i < off.size(); ++i) {
      CHECK(off[i] % 256 == 0);
      if (i) CHECK(off[i] >= off[i - 1]);
      CHECK(off[i] <= w.total);
    }
    const size_t es = c.dtype == DEX_DTYPE_BF16 ? 2 : 4;
    const size_t L = c.n_layers, d = c.d_model, nkv = c.n_kv_heads, hd = c.head_dim, V = c.vocab;
    const size_t P = (1u << k.N) - 1, Cs = (k.Cmax + kKvTile - 1) / kKvTile * kKvTile;
    // sizes the kernels rely on, from the shapes (not from the plan)
    CHECK(w.head - w.embed >= V * d * es);
    // K and V: fp16 for bf16 models, (hi, lo) bf16 pairs for fp32 models
    const size_t kvb = c.dtype == DEX_DTYPE_BF16 ? 4 : 8;
    CHECK(w.exb - w.kvc >= (size_t)k.B * L * nkv * Cs * hd * kvb);
    CHECK(w.xn - w.hidden >= ((size_t)k.B * P + kPrefillRows) * d * 4);
    // the widest round: heap level N - 1 of every sequence, or a prefill chunk
    const int widest = std::max(k.B << (k.N - 1), kPrefillRows);
    CHECK(w.Rmax >= widest);
    CHECK(w.sbytes[SC_ROWS] >= (size_t)widest * sizeof(RowInfo));
    CHECK(w.sbytes[SC_HEAD_PART] >= (size_t)widest * (V / 16) * 12);
    CHECK(w.plans + w.sbytes[SC_PLANS] <= w.items);
    // the allocation-free step's regions: decode rounds only, never larger
    CHECK(w.Rstep >= k.B << (k.N - 1) && w.Rstep <= w.Rmax);
    for (int r = 0; r < SC_N; ++r) CHECK(w.sstep[r] <= w.sbytes[r]);
    CHECK(w.sstep[SC_HEAD_PART] >= (size_t)(k.B << (k.N - 1)) * (V / 16) * 12);
    CHECK(w.head_part + w.sbytes[SC_HEAD_PART] <= w.total);
    // the K/V addressing the kernels use stays inside the carved regions: the
    // last (sequence, layer, kv head) run of committed tiles, and the last
    // explore entry (16-bit elements)
    ModelDims D{};
    D.L = c.n_layers;
    D.nkv = c.n_kv_heads;
    D.hd = c.head_dim;
    D.S = longest_stage(X.data(), k.N);
    D.N = k.N;
    D.P = (int)P;
    D.B = k.B;
    D.Cs = (int)Cs;
    D.kvp = kv_planes(c.dtype);
    CHECK(kv_head_base(D, k.B - 1, D.L - 1, D.nkv - 1) + (size_t)D.Cs * D.hd * 2 * D.kvp <= (w.exb - w.kvc) / 2);
    CHECK(kv_head_base(D, 0, 0, 1) == (size_t)D.Cs * D.hd * 2 * D.kvp || D.nkv == 1);
    CHECK(ex_base(D, k.B - 1, D.P - 1, D.S - 1, D.nkv - 1) + 2 * (size_t)D.kvp * D.hd <= (w.hidden - w.exb) / 2);
  }
}

// K/V tile layout: kv_elem (the writers: QKV epilogues, promotion) maps the
// 64 kvp hd values of a 32-position tile one to one onto the tile, and the
// attention kernels' own operand addressing reads the same element: K lane
// (g, n) of MFMA row block t and 32-dim step s takes 16 bytes at
// (4 s + g) 256 + (16 t + n) 8 (position 8 (n / 4) + 4 t + n % 4, dims
// 8 (4 s + g) ..), V^T lane (g, n) of output block b takes 16 bytes at
// 32 kvp hd + (16 b + n) 32 + 8 g (dim 16 b + n, positions 8 g ..); the lo
// plane of a pair sits 32 hd further.
static void check_kv_layout() {
  for (int kvp : {1, 2})
    for (int hd : {64, 128}) {
      const size_t tile = (size_t)64 * kvp * hd;
      std::vector<int> seen(tile, 0);
      for (int pos = 0; pos < kKvTile; ++pos)
        for (int kv = 0; kv < 2; ++kv)
          for (int pl = 0; pl < kvp; ++pl)
            for (int d = 0; d < hd; ++d) {
              const size_t e = kv_elem(hd, kvp, pos, kv, pl, d);
              CHECK(e < tile);
              if (e < tile) ++seen[e];
              CHECK(kv_elem(hd, kvp, pos + 3 * kKvTile, kv, pl, d) == e + 3 * tile);
            }
      for (size_t e = 0; e < tile; ++e) CHECK(seen[e] == 1);
      for (int lane = 0; lane < 64; ++lane) {
        const int g = lane >> 4, n = lane & 15;
        for (int pl = 0; pl < kvp; ++pl)
          for (int i = 0; i < 8; ++i) {
            for (int t = 0; t < 2; ++t)
              for (int st = 0; st < hd / 32; ++st)
                CHECK((size_t)(4 * st + g) * 256 + (16 * t + n) * 8 + (size_t)pl * 32 * hd + i ==
                      kv_elem(hd, kvp, 8 * (n >> 2) + 4 * t + (n & 3), 0, pl, 8 * (4 * st + g) + i));
            for (int b = 0; b < hd / 16; ++b)
              CHECK((size_t)32 * kvp * hd + (16 * b + n) * 32 + 8 * g + (size_t)pl * 32 * hd + i ==
                    kv_elem(hd, kvp, 8 * g + i, 1, pl, 16 * b + n));
          }
      }
    }
}

// --- one round's plan ------------------------------------------------------------
static void check_round(std::mt19937& rng, int N, int B, int rep, int ncap, bool ar) {
  const int T = 50;
  std::vector<int> q(B), C(B), commits(B), plen(B);
  for (int s = 0; s < B; ++s) {
    q[s] = ar ? 0 : rng() % N;
    plen[s] = 1 + rng() % 300;
    commits[s] = rng() % 4 == 0 ? T : rng() % T;   // some sequences finished
    C[s] = plen[s] + commits[s];
  }
  RoundShape r;
  round_rows(q.data(), commits.data(), B, N, T, ar, ncap, r);
  // brute enumeration of each live sequence's heap level
  int R = 0, nlive = 0;
  for (int s = 0; s < B; ++s) {
    const bool live = commits[s] < T;
    CHECK(r.live[s] == (int)live);
    nlive += live;
    std::vector<int> want(N, 0);
    if (live) {
      if (ar) {
        want[0] = 1;
      } else {
        for (unsigned n = (1u << q[s]) - 1; n <= (1u << (q[s] + 1)) - 2; ++n) {
          // held: every run of depth moves (0 bits of n + 1 after its leading 1)
          // that a position move (1 bit) ends is shorter than the cap
          bool held = true;
          if (ncap) {
            const int top = 31 - __builtin_clz(n + 1);
            int run = 0;
            for (int bit = top - 1; bit >= 0; --bit) {
              if ((n + 1) >> bit & 1) {
                if (run >= ncap) held = false;
                run = 0;
              } else {
                ++run;
              }
            }
          }
          if (held) ++want[__builtin_ctz(n + 1)];
        }
        if (!ncap) {   // the full level: 2^(q-1-j) nodes at explorer j < q, one at q
          for (int j = 0; j < N; ++j)
            CHECK(want[j] == (j < q[s] ? 1 << (q[s] - 1 - j) : (j == q[s] ? 1 : 0)));
        }
        if (ncap == 1)   // single exit: one node per explorer 0..q
          for (int j = 0; j < N; ++j) CHECK(want[j] == (j <= q[s] ? 1 : 0));
      }
    }
    for (int j = 0; j < N; ++j) {
      CHECK(r.rows[(size_t)s * N + j] == want[j]);
      R += want[j];
    }
  }
  CHECK(r.nlive == nlive);
  CHECK(r.R == R);
  CHECK(R <= B << (N - 1));
  for (int j = 0; j < N; ++j) CHECK(r.stage_off[j + 1] - r.stage_off[j] == r.stage_tot[j]);
  if (nlive == 0) return;

  // per-sequence plans: each (sequence, explorer) block lies in its explorer's
  // range, blocks do not overlap, and every row of the round is in one
  std::vector<SeqPlan> plans(B);
  const int ncommit = seq_plans(r, q.data(), C.data(), plen.data(), B, N, ar, plans.data());
  std::vector<int> owner(R, -1);
  int want_commit = 0;
  for (int s = 0; s < B; ++s) {
    want_commit += r.live[s] && (ar || q[s] + 1 == N);
    CHECK(plans[s].commit == (r.live[s] && (ar || q[s] + 1 == N)));
    for (int j = 0; j < N; ++j) {
      const int cnt = r.rows[(size_t)s * N + j];
      for (int i = 0; i < cnt; ++i) {
        const int row = plans[s].base[j] + i;
        CHECK(row >= r.stage_off[j] && row < r.stage_off[j + 1]);
        if (row >= 0 && row < R) {
          CHECK(owner[row] == -1);
          owner[row] = s * N + j;
        }
      }
    }
  }
  CHECK(ncommit == want_commit);
  for (int row = 0; row < R; ++row) CHECK(owner[row] >= 0);

  // attention items in a buffer of exactly the library's size (Rmax items,
  // then 3 Rmax list entries)
  const int Rmax = std::max(B << (N - 1), kPrefillRows);
  std::vector<AttnItem> items(Rmax);
  std::vector<int> list(3 * (size_t)Rmax);
  const ItemStats st = round_items(r, plans.data(), q.data(), C.data(), B, N, ar, rep, items.data());
  CHECK(st.nitems <= R);
  std::vector<int> covered(R, 0);
  int maxk = 0, umax = 1, nj = 0, tails = 0;
  for (int i = 0; i < st.nitems; ++i) {
    const AttnItem& it = items[i];
    CHECK(it.nrows >= 1 && it.nrows * rep <= std::max(kAttnUnits, rep));
    for (int k = 0; k < it.nrows; ++k) {
      const int row = it.row0 + k;
      CHECK(row >= 0 && row < R);
      if (row >= 0 && row < R) {
        ++covered[row];
        CHECK(owner[row] == it.seq * N + it.stage);
      }
    }
    const int mk = C[it.seq] + (ar ? 1 : q[it.seq] - it.stage + 1);
    CHECK(it.max_keys == mk);
    maxk = std::max(maxk, mk);
    umax = std::max(umax, it.nrows * rep);
    if (!ar) {
      // the explore keys [C, mk) lie in chunks xc0..xc1, at most two of them
      CHECK(it.xc0 * kKvTile <= C[it.seq] && (it.xc1 + 1) * kKvTile >= mk);
      CHECK(it.xc1 - it.xc0 <= 1);
      nj = std::max(nj, it.xc1 - it.xc0 + 1);
      tails += (it.nrows + kTailRows - 1) / kTailRows;
    } else {
      CHECK(it.xc0 == -1);
    }
    // a group leads up to kAttnGroup items of its own (sequence, explorer)
    if (it.lead > 0) {
      CHECK(it.lead <= kAttnGroup);
      for (int k = 1; k < it.lead; ++k) {
        CHECK(i + k < st.nitems);
        if (i + k < st.nitems) {
          CHECK(items[i + k].lead == 0);
          CHECK(items[i + k].seq == it.seq && items[i + k].stage == it.stage);
        }
      }
    } else {
      CHECK(i > 0 && items[i - 1].seq == it.seq && items[i - 1].stage == it.stage);
    }
  }
  for (int row = 0; row < R; ++row) CHECK(covered[row] == 1);
  CHECK(st.max_keys == maxk && st.umax == umax && st.nj == nj);

  const BlockList b = attn_block_list(items.data(), st.nitems, list.data());
  int singles = 0, leads = 0;
  for (int i = 0; i < st.nitems; ++i) {
    singles += items[i].lead == 1;
    leads += items[i].lead > 1;
  }
  CHECK(b.single == singles && b.groups == leads && b.tails == tails);
  for (int e = 0; e < b.single + b.groups; ++e) CHECK(list[e] >= 0 && list[e] < st.nitems);
  std::set<int> tail_entries;
  for (int e = b.single + b.groups; e < b.single + b.groups + b.tails; ++e) {
    const int i = list[e] / 4, qt = list[e] % 4;
    CHECK(i < st.nitems && qt * kTailRows < items[i].nrows);
    CHECK(tail_entries.insert(list[e]).second);
  }
}

// --- the graph key tells plans apart ------------------------------------------------
static void check_graph_key(std::mt19937& rng) {
  const int N = 4, B = 3, T = 10;
  std::map<std::string, std::vector<int>> seen;
  for (int t = 0; t < 3000; ++t) {
    std::vector<int> q(B), C(B), commits(B), plen(B, 5);
    for (int s = 0; s < B; ++s) {
      q[s] = rng() % N;
      commits[s] = rng() % 3 == 0 ? T : rng() % T;
      C[s] = 5 + commits[s] + (rng() % 2) * 40;
    }
    const bool ar = rng() % 5 == 0;
    RoundShape r;
    round_rows(q.data(), commits.data(), B, N, T, ar, 0, r);
    if (!r.nlive) continue;
    std::vector<SeqPlan> plans(B);
    seq_plans(r, q.data(), C.data(), plen.data(), B, N, ar, plans.data());
    std::vector<AttnItem> items(kPrefillRows);
    const ItemStats st = round_items(r, plans.data(), q.data(), C.data(), B, N, ar, 1, items.data());
    const std::string key = graph_key(ar, st.max_keys, st.nj, r, plans.data(), B);
    // what the recorded work depends on beyond the re-read host buffers
    std::vector<int> sig = {ar, (st.max_keys + kAttnSCKeys - 1) / kAttnSCKeys, st.nj};
    for (int s = 0; s < B; ++s) {
      sig.push_back(r.live[s] ? plans[s].q : -1);
      sig.push_back(plans[s].commit);
    }
    auto it = seen.find(key);
    if (it == seen.end()) seen.emplace(key, sig);
    else CHECK(it->second == sig);
  }
  CHECK(seen.size() > 50);
}

// --- the FSM over scripted commits --------------------------------------------------
static void check_fsm(std::mt19937& rng) {
  for (int N = 1; N <= kMaxN; ++N)
    for (int ncap = 0; ncap < N; ++ncap)
      for (int t = 0; t < 20; ++t) {
        const int K = 1 + rng() % 30;
        int q = 0, rounds = 0, commits = 0, want = N;   // the first commit comes after N rounds
        while (commits < K) {
          ++rounds;
          if (q + 1 == N) {
            int b = rng() % N;
            if (ncap == 1) b = rng() % 2 ? 0 : N - 1;   // single exit keeps branch 0 or N - 1
            ++commits;
            CHECK(rounds == want);
            q = next_q(q, true, false, ncap, b, N);
            // b + 1 more rounds, or a fresh tree of N when the pruned lattice held no subtree
            want += ncap && b >= ncap ? N : b + 1;
          } else {
            q = next_q(q, false, false, ncap, 0, N);
          }
          CHECK(q >= 0 && q < N);
        }
      }
  CHECK(next_q(0, true, true, 0, 0, 4) == 0);
}

// --- prefill chunks ----------------------------------------------------------------
static void check_prefill(std::mt19937& rng) {
  for (int t = 0; t < 300; ++t) {
    const int n = 1 + rng() % 16;
    std::vector<int32_t> lens(n);
    size_t total = 0;
    for (int s = 0; s < n; ++s) {
      lens[s] = 1 + (rng() % 3 == 0 ? rng() % 9000 : rng() % 700);
      total += lens[s];
    }
    std::vector<int32_t> tokens(total);
    std::vector<size_t> start(n);
    for (int s = 0, o = 0; s < n; o += lens[s], ++s) {
      start[s] = o;
      for (int p = 0; p < lens[s]; ++p) tokens[o + p] = s * 10000 + p;
    }
    const int per_item = 16 >> (rng() % 4);
    const int base_h = (int)(rng() % 1000);
    const int Rmax = kPrefillRows;   // the library's host buffers hold at least this many rows and items
    std::vector<RowInfo> rows(Rmax);
    std::vector<AttnItem> items(Rmax);
    std::vector<int> list(3 * (size_t)Rmax);
    PrefillCursor cur;
    int next_seq = 0, next_pos = 0, chunks = 0;
    for (;;) {
      int nitems = -1, maxk = -1;
      const int R = prefill_chunk(tokens.data(), lens.data(), n, base_h, per_item, cur, rows.data(), items.data(),
                                  nitems, maxk);
      if (R == 0) break;
      ++chunks;
      CHECK(R <= kPrefillRows && nitems <= R);
      int want_maxk = 0;
      for (int i = 0; i < R; ++i) {
        // positions in order, sequence after sequence, skipping each prompt's last token
        while (next_seq < n && next_pos >= lens[next_seq] - 1) {
          ++next_seq;
          next_pos = 0;
        }
        CHECK(next_seq < n);
        const RowInfo& r = rows[i];
        CHECK(r.seq == next_seq && r.pos == next_pos);
        CHECK(r.tok == next_seq * 10000 + next_pos);
        CHECK(r.hrow == base_h + i && r.ncommit == r.pos + 1 && r.kv_commit == 1 && r.stage == 0);
        want_maxk = std::max(want_maxk, r.ncommit);
        ++next_pos;
      }
      CHECK(maxk == want_maxk);
      // items: every row once, one sequence each, at most per_item rows
      std::vector<int> cover(R, 0);
      for (int i = 0; i < nitems; ++i) {
        const AttnItem& it = items[i];
        CHECK(it.nrows >= 1 && it.nrows <= per_item && it.xc0 == -1 && it.stage == 0);
        int own = 0;
        for (int k = 0; k < it.nrows; ++k) {
          const int row = it.row0 + k;
          CHECK(row >= 0 && row < R);
          if (row < 0 || row >= R) continue;
          ++cover[row];
          CHECK(rows[row].seq == it.seq);
          own = std::max(own, rows[row].ncommit);
        }
        if (it.lead > 1) {   // the group's first item carries its largest key count
          int g = own;
          for (int k = 1; k < it.lead; ++k) {
            CHECK(i + k < nitems && items[i + k].lead == 0 && items[i + k].seq == it.seq);
            const AttnItem& o = items[i + k];
            g = std::max(g, rows[o.row0 + o.nrows - 1].ncommit);
          }
          CHECK(it.max_keys == g);
        } else {
          CHECK(it.max_keys == own);
        }
      }
      for (int row = 0; row < R; ++row) CHECK(cover[row] == 1);
      const BlockList b = attn_block_list(items.data(), nitems, list.data());
      CHECK(b.tails == 0 && b.single + b.groups <= nitems);
    }
    while (next_seq < n && next_pos >= lens[next_seq] - 1) {
      ++next_seq;
      next_pos = 0;
    }
    CHECK(next_seq == n);   // every position went through exactly one chunk
    size_t rows_total = 0;
    for (int s = 0; s < n; ++s) rows_total += lens[s] - 1;
    CHECK(chunks == (int)((rows_total + kPrefillRows - 1) / kPrefillRows));
  }
}

int main() {
  check_validate();
  check_workspace();
  check_kv_layout();
  std::mt19937 rng(11);
  for (int N = 1; N <= kMaxN; ++N)
    for (int rep : {1, 2, 4, 8})
      for (int t = 0; t < 12; ++t) {
        const int B = 1 + rng() % (N >= 8 ? 8 : 64);
        check_round(rng, N, B, rep, 0, false);
        check_round(rng, N, B, rep, 0, true);
        if (N > 1) check_round(rng, N, B, rep, 1 + rng() % (N - 1), false);
      }
  check_graph_key(rng);
  check_fsm(rng);
  check_prefill(rng);
  if (g_fail) {
    std::fprintf(stderr, "%d plan checks failed\n", g_fail);
    return 1;
  }
  std::printf("plan checks ok\n");
  return 0;
}
