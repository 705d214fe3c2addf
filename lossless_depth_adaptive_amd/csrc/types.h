// Plain constants and structures of the DEX lattice-step library that both
// the kernels and the host plan use. No device code: the host plan
// (plan.h) compiles with any C++17 compiler when DEX_HD is defined empty.
#pragma once
#include <stddef.h>
#include <stdint.h>

#ifndef DEX_HD
#define DEX_HD __host__ __device__
#endif

namespace dex {

constexpr int kMaxN = 10;            // explorers supported (2^10 - 1 lattice nodes)
constexpr int kWave = 64;
constexpr int kGemmThreads = 512;    // 8 waves: fixed 8-way split of K
constexpr int kKSplit = 8;
constexpr int kMaxMB = 4;            // 16-row MFMA blocks per GEMM group (<= 64 rows)
constexpr int kMaxGroups = 48;       // GEMM groups per launch
constexpr int kSplitRows = 512;      // rows of one split-range wide GEMM launch
// Wide GEMM launch shapes: 4-wave blocks with 4 column tiles per wave
// (unsplit or split by k range) or 2 tiles per wave (unsplit); 8-wave blocks
// of 4 tiles per wave (512 columns, unsplit).
enum WideShape { WIDE_T4 = 0, WIDE_SPLIT = 1, WIDE_T2 = 2, WIDE_W8 = 3 };
constexpr int kAttnUnits = 16;       // (row, query head) units per attention work item (one MFMA tile)
constexpr int kKvTile = 32;          // positions per K/V cache tile = keys per attention chunk
#ifndef DEX_ATTN_SC
#define DEX_ATTN_SC 4
#endif
constexpr int kAttnSC = DEX_ATTN_SC;  // chunks per attention super-chunk (= waves per attention block)
constexpr int kAttnGroup = 4;        // unit tiles (items) of one sequence and stage per grouped attention block
constexpr int kAttnSCKeys = kKvTile * kAttnSC;
constexpr int kMixSlots = 2 * kAttnSC;   // chunk slots of the (at most two) mixed super-chunks
// Rows of an item whose explore keys one per-row attention block computes:
// kTailRowsPerWave rows in each of its kAttnSC waves.
#ifndef DEX_TAIL_RPW
#define DEX_TAIL_RPW 2
#endif
constexpr int kTailRowsPerWave = DEX_TAIL_RPW;
constexpr int kTailRows = kAttnSC * kTailRowsPerWave;
static_assert(kAttnUnits <= 4 * kTailRows, "a tail entry 4 item + q needs q < 4");

// One lattice (or autoregressive, or prefill) row of a step.
struct RowInfo {
  int seq;          // sequence index
  int phys;         // physical node slot of the sequence (token, margin, explore KV)
  int hrow;         // row of the fp32 hidden pool holding this row's residual stream
  int stage;        // explorer index j (layer j*S + lambda at layer slot lambda)
  int pos;          // absolute position of the row's input token
  int tok;          // token id to embed, or -1 when the row continues a hidden state
  int ncommit;      // keys read from the committed cache: positions [0, ncommit)
  int n_anc;        // explore-buffer keys at positions ncommit .. ncommit+n_anc-1
  int anc[kMaxN];   // physical slots holding those keys (same stage)
  int n_mask;       // tokens masked by depth-coupled sampling
  int mask[kMaxN];  // the masked token ids
  int final_;       // 1 for the final-depth reference node
  int grow;         // Gumbel row: target position minus the prompt length
  int kv_commit;    // 1: write this row's K/V into the committed cache at pos
};

// Per-sequence plan of one lattice step, written by the host.
struct SeqPlan {
  int live;         // sequence takes part in this step
  int q;            // FSM state: rounds completed by the current tree
  int C;            // committed KV length
  int commit;       // the round reaches the final explorer (q + 1 == N)
  int prompt_len;
  int base[kMaxN];  // first row index of this sequence's rows at each stage
};

struct ModelDims {
  int L, d, nq, nkv, hd, F, V;
  int S;            // layers of the longest stage (explore-buffer layer slots per node)
  int N;            // explorers
  int P;            // lattice node slots per sequence (2^N - 1)
  int B;            // max sequences
  int Cmax;         // max context
  int Cs;           // committed-cache positions per (sequence, layer, kv head): Cmax rounded up to kKvTile
  int kvp;          // 16-bit planes per K or V value: 1 (fp16, bf16 models) or 2 (bf16 hi, lo: fp32 models)
  float eps;
  int lfirst[kMaxN + 1];   // explorer j runs layers [lfirst[j], lfirst[j+1]) (d_{j-1} .. d_j - 1); lfirst[N] = L
};

// Layer of slot lam for a row of explorer `stage`: lattice rows run their
// stage's layers, autoregressive and prefill rows (lattice = 0) every layer.
DEX_HD inline int layer_of(const ModelDims& D, int lattice, int stage, int lam) {
  return lattice ? D.lfirst[stage] + lam : lam;
}
DEX_HD inline int stage_len(const ModelDims& D, int j) { return D.lfirst[j + 1] - D.lfirst[j]; }

struct GemmGroup {
  const void* w;        // packed weights of this group
  const float* gamma;   // EPI_RESID: RMSNorm weight of the row's next consumer (null: none)
  int row0;             // first row (activations A[row0 ...], row info rows[row0 ...])
  int m;                // rows, 1..64
  int srow;             // split-range wide GEMM: the group's first row in the partial-sum scratch
  int xh;               // EPI_RESID: also write h * final-norm weight (the rows end their stage here)
  const float* bias;    // EPI_ADAPT1 / EPI_ADAPT2: b1 / b2 of the group's adapter
  float alpha;          // EPI_ADAPT2: the adapter's gate
  const float* anorm;   // EPI_RESID: also write h * this adapter norm weight (null: none)
};

enum Epilogue { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_HEAD = 3, EPI_ADAPT1 = 4, EPI_ADAPT2 = 5 };
// Epilogues whose A operand is a normalised residual (h * g, scaled by rstd).
constexpr bool epi_norm(int e) { return e == EPI_QKV || e == EPI_SWIGLU || e == EPI_HEAD || e == EPI_ADAPT1; }

struct AttnItem {
  int seq;          // sequence of the rows
  int row0;         // first row
  int nrows;        // rows (all of one sequence and one layer), nrows * (nq / nkv) <= kAttnUnits
  int stage;        // explorer of the rows; layer = layer_of(D, lattice, stage, lam)
  int max_keys;     // max over the rows of ncommit + n_anc
  int xc0, xc1;     // chunks [xc0, xc1] may hold explore keys of some row (xc0 = -1: none);
                    // every row's explore keys lie in them
  int lead;         // items (this one and the next lead - 1, same sequence and stage) the
                    // attention block of this item covers; 0: covered by an earlier item
};

// K/V storage. Values are stored in kvp 16-bit planes, all rounded to nearest
// even: kvp = 1 for bfloat16 models, one fp16 value (11 significant bits,
// three more than the model's bfloat16; 2 bytes, the K/V stream of a bf16
// cache); kvp = 2 for fp32 models, a bfloat16 pair hi = bf16(x),
// lo = bf16(x - hi) (about 2^-17 relative, 4 bytes). Either way attention runs
// on 16-bit MFMA operands.
// Committed cache: per (sequence, layer, kv head) a run of Cs / kKvTile tiles
// of 32 positions, 64 kvp hd values each:
//   K plane pl: [hd / 8][slot][8] at offset pl * 32 hd, with position k of the
//     tile at slot 16 ((k >> 2) & 1) + 4 (k >> 3) + (k & 3);
//   V plane pl: [hd][32 positions] at offset 32 kvp hd + pl * 32 hd.
// Explore entry of one (sequence, node slot, layer slot, kv head): 2 kvp hd
//   values, the K planes then the V planes, each [hd].
DEX_HD inline int kv_slot(int k) { return 16 * ((k >> 2) & 1) + 4 * (k >> 3) + (k & 3); }
DEX_HD inline size_t kv_head_base(const ModelDims& D, int seq, int layer, int h) {
  return (((size_t)seq * D.L + layer) * D.nkv + h) * (size_t)D.Cs * D.hd * 2 * D.kvp;
}
DEX_HD inline size_t kv_elem(int hd, int kvp, int pos, int kv, int plane, int d) {
  const size_t tile = (size_t)(pos / kKvTile) * 64 * kvp * hd;
  const int k = pos % kKvTile;
  return kv == 0 ? tile + (size_t)plane * 32 * hd + (d >> 3) * 256 + kv_slot(k) * 8 + (d & 7)
                 : tile + (size_t)(kvp + plane) * 32 * hd + (size_t)d * 32 + k;
}
DEX_HD inline size_t ex_base(const ModelDims& D, int seq, int phys, int lam, int h) {
  return ((((size_t)seq * D.P + phys) * D.S + lam) * D.nkv + h) * 2 * D.kvp * (size_t)D.hd;
}

// Pruned lattice: whether heap node n (n1 = n + 1) is created when only nodes
// of explorers below `cap` spawn position children (cap 0: every node). The
// bits of n1 after its leading 1 are the node's path from the root (0 = depth
// move, 1 = position move); a position move leaves a node whose explorer is
// the number of depth moves since the previous position move (or the root),
// so the node exists when every run of 0s followed by a 1 is shorter than cap.
// The trailing 0s (the node's own explorer) are not constrained. cap = 1 gives
// the single-exit node set n1 = (2^(a+1) - 1) 2^b.
DEX_HD inline bool node_held(unsigned n1, int cap) {
  if (cap <= 0) return true;
  unsigned t = n1 >> __builtin_ctz(n1);   // odd: ends with the last position move
  while (t > 1) {
    t >>= 1;                              // that move
    const int z = __builtin_ctz(t);       // depth moves before it
    if (z >= cap) return false;
    t >>= z;
  }
  return true;
}

}  // namespace dex
