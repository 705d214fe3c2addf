// Lattice bookkeeping on the device: the round's row schedule (expand), the
// commit rule with collapse, and promotion of the anchor path's KV into the
// committed cache ("Depth Exploration for LLM Decoding", Algorithm 1 and
// Section 3.2).
//
// Nodes of a sequence's tree use heap numbering: node i has depth child 2i+1
// and position child 2i+2, so ETK_0's children are ETK_1 (depth) and ETK_2
// (position) and state q holds nodes 0 .. 2^q - 2, as the paper's four-explorer
// example states. The bits of i+1 after its leading 1 are the path from the
// root (0 = depth move, 1 = position move), hence
//   explorer (stage) = trailing zeros of i+1,
//   position offset  = popcount(i+1) - 1,
//   slot-chain root  = ((i+1) >> stage) - 1,  chain member at depth m = ((root+1) << m) - 1.
// A node's data (candidate token, margin, explore KV) lives in a physical slot
// of its sequence, reached through map[seq][heap index]; collapse re-points
// the map instead of moving data.
#include "common.h"

namespace dex {

// Expand: one workgroup per live sequence builds the row of every node the
// round creates (2^q of them at state q). The rows that start a slot
// (explorer 0, the first rows of the round) take their token's embedding in a
// launch of their own (embed_kernel, a workgroup per row).
// Pruned lattice (cap > 0): only the nodes node_held keeps are created; each
// takes the next free slot in heap order and the next row of its explorer.
// The single-exit ablation ("Depth Exploration for LLM Decoding", Section 4,
// Figure 4 right-top) has the cap-1 node set, n + 1 = (2^(a+1) - 1) 2^(q-a)
// for a = 0..q (one per explorer), and no masks.
__global__ void sched_kernel(const SeqPlan* __restrict__ plans, RowInfo* __restrict__ rows,
                             int* __restrict__ map, const int* __restrict__ cand,
                             const int* __restrict__ freel, int* __restrict__ cursor,
                             const int* __restrict__ anchor_tok, int N, int P, int decs, int single_exit,
                             int cap) {
  const int s = blockIdx.x;
  const SeqPlan pl = plans[s];
  if (!pl.live) return;
  const int q = pl.q, first = (1 << q) - 1, total = 1 << q;
  int nnew = total;
  if (cap) {
    nnew = 0;
    for (int t = 0; t < total; ++t) nnew += node_held(first + t + 1, cap);
  }
  const int cur = cursor[s];
  int* mp = map + (size_t)s * P;
  const int* cd = cand + (size_t)s * P;
  for (int t = threadIdx.x; t < total; t += blockDim.x) {
    const int n = first + t, n1 = n + 1;
    if (cap && !node_held(n1, cap)) continue;
    const int depth = __builtin_ctz(n1);
    const int posoff = __popc(n1) - 1;
    // rank: kept nodes of the round before n; idx: those of n's explorer
    int rank = t, idx = depth >= q ? 0 : (((n1 >> depth) - (1 << (q - depth)) - 1) >> 1);
    if (cap) {
      rank = idx = 0;
      for (int t2 = 0; t2 < t; ++t2) {
        const unsigned m1 = first + t2 + 1;
        if (node_held(m1, cap)) {
          ++rank;
          idx += __builtin_ctz(m1) == depth;
        }
      }
    }
    const int phys = freel[(size_t)s * P + cur + rank];
    mp[n] = phys;
    RowInfo R;
    R.seq = s;
    R.phys = phys;
    R.stage = depth;
    R.pos = pl.C + posoff;
    R.ncommit = pl.C;
    R.kv_commit = 0;
    R.final_ = depth == N - 1;
    R.grow = pl.C + posoff + 1 - pl.prompt_len;
    const int root = (n1 >> depth) - 1;
    R.hrow = s * P + (depth == 0 ? phys : mp[root]);
    R.tok = depth != 0 ? -1 : (n == 0 ? anchor_tok[s] : cd[mp[(n - 1) >> 1]]);
    // Slot roots on the path (the tree root and every position move), in
    // position order; their chain members at this stage hold the keys.
    const int level = 31 - __builtin_clz(n1);
    int cnt = 0;
    for (int sh = level; sh >= 0; --sh) {
      const int pfx = n1 >> sh;
      if (pfx == 1 || (pfx & 1)) {
        const int node = (pfx << depth) - 1;
        R.anc[cnt++] = node == n ? phys : mp[node];
      }
    }
    R.n_anc = cnt;
    // Depth-coupled sampling: candidates of shallower members of the chain.
    R.n_mask = 0;
    if (decs && !single_exit && depth < N - 1) {
      for (int m = 0; m < depth; ++m) R.mask[m] = cd[mp[((root + 1) << m) - 1]];
      R.n_mask = depth;
    }
    rows[pl.base[depth] + idx] = R;
  }
  if (threadIdx.x == 0) cursor[s] = cur + nnew;
}

// Commit and collapse for every sequence whose round reached the final
// explorer. u_j = candidate of anchor node 2^j - 1; the token is u_{N-1}; the
// branch is the smallest j with u_j == u_{N-1}. The subtree under the branch's
// position child (heap 2^(k+1)) becomes the new tree: relative node j at level
// lv maps to old node (2^(k+1) + 1) 2^lv - 1 + (j + 1 - 2^lv), for the
// 2^(N-1-k) - 1 nodes it holds. Free slots are rebuilt in increasing order.
// Pruned lattice (cap > 0): only the kept subtree's nodes that node_held keeps
// hold slots (the subtree's own numbering gives the same answer as the old
// tree's, since its root's path is k < cap depth moves and one position
// move), and a branch k >= cap had no position child: nothing is kept.
// Single-exit ablation (cap 1): only u_0 and u_{N-1} exist (branch 0 or N-1).
__global__ void commit_kernel(const SeqPlan* __restrict__ plans, int* __restrict__ map,
                              const int* __restrict__ cand, const float* __restrict__ margin,
                              int* __restrict__ freel, int* __restrict__ cursor,
                              int* __restrict__ anchor_tok, int* __restrict__ records,
                              int* __restrict__ promote_src, int* __restrict__ dbg_u,
                              float* __restrict__ dbg_m, const int* __restrict__ Xd, int N, int P,
                              int single_exit, int cap) {
  const int s = blockIdx.x;
  const SeqPlan pl = plans[s];
  if (!pl.live || !pl.commit) return;
  __shared__ int u[kMaxN];
  __shared__ int ksh;
  __shared__ int nm[1 << (kMaxN - 1)];
  __shared__ unsigned char used[1 << kMaxN];
  int* mp = map + (size_t)s * P;
  const int tid = threadIdx.x;
  if (tid < N) {
    const int p = mp[(1 << tid) - 1];
    const bool exits = !single_exit || tid == 0 || tid == N - 1;
    u[tid] = exits ? cand[(size_t)s * P + p] : -1;
    promote_src[s * kMaxN + tid] = p;
    dbg_u[s * kMaxN + tid] = u[tid];
    dbg_m[s * kMaxN + tid] = exits ? margin[(size_t)s * P + p] : 0.f;
  }
  for (int p = tid; p < P; p += blockDim.x) used[p] = 0;
  __syncthreads();
  if (tid == 0) {
    const int y = u[N - 1];
    int k = N - 1;
    for (int j = 0; j < N; ++j)
      if (u[j] == y) {
        k = j;
        break;
      }
    int* rec = records + s * 5;
    rec[0] = s;
    rec[1] = pl.C + 1;
    rec[2] = y;
    rec[3] = k;
    rec[4] = Xd[k];
    anchor_tok[s] = y;
    ksh = k;
  }
  __syncthreads();
  const int k = ksh;
  const int nk = cap && k >= cap ? 0 : (1 << (N - 1 - k)) - 1;
  const int root = 1 << (k + 1);
  for (int j = tid; j < nk; j += blockDim.x) {
    const int lv = 31 - __builtin_clz(j + 1);
    nm[j] = node_held(j + 1, cap) ? mp[((root + 1) << lv) - 1 + (j + 1 - (1 << lv))] : -1;
  }
  __syncthreads();
  for (int j = tid; j < nk; j += blockDim.x) {
    mp[j] = nm[j];
    if (nm[j] >= 0) used[nm[j]] = 1;
  }
  __syncthreads();
  if (tid == 0) {
    int c = 0;
    for (int p = 0; p < P; ++p)
      if (!used[p]) freel[(size_t)s * P + c++] = p;
    cursor[s] = 0;
  }
}

// Copy the anchor path's K/V (node 2^j - 1 holds stage j) into the committed
// cache at position C. grid = (sequences, layers, kv heads).
__global__ void promote_kernel(const SeqPlan* __restrict__ plans, const int* __restrict__ promote_src,
                               const bf16_t* __restrict__ exb, bf16_t* __restrict__ kvc, ModelDims D) {
  const int s = blockIdx.x, layer = blockIdx.y, h = blockIdx.z;
  const SeqPlan pl = plans[s];
  if (!pl.live || !pl.commit) return;
  int j = 0;
  while (D.lfirst[j + 1] <= layer) ++j;
  const int lam = layer - D.lfirst[j];
  const int phys = promote_src[s * kMaxN + j];
  const bf16_t* src = exb + ex_base(D, s, phys, lam, h);
  bf16_t* dst = kvc + kv_head_base(D, s, layer, h);
  const int kvp = D.kvp;
  for (int t = threadIdx.x; t < 2 * kvp * D.hd; t += blockDim.x) {   // the K planes, then the V planes, each [hd]
    const int kv = t / (kvp * D.hd), plane = (t / D.hd) % kvp, i = t % D.hd;
    dst[kv_elem(D.hd, kvp, pl.C, kv, plane, i)] = src[t];
  }
}

// Plain autoregressive rows: one full-depth row per live sequence.
__global__ void ar_rows_kernel(const SeqPlan* __restrict__ plans, int nseq, RowInfo* __restrict__ rows,
                               const int* __restrict__ anchor_tok, int P) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= nseq) return;
  const SeqPlan pl = plans[s];
  if (!pl.live) return;
  RowInfo R;
  R.seq = s;
  R.phys = 0;
  R.hrow = s * P;
  R.stage = 0;
  R.pos = pl.C;
  R.tok = anchor_tok[s];
  R.ncommit = pl.C + 1;
  R.n_anc = 0;
  R.n_mask = 0;
  R.final_ = 1;
  R.grow = pl.C + 1 - pl.prompt_len;
  R.kv_commit = 1;
  rows[pl.base[0]] = R;
}

__global__ void ar_commit_kernel(const SeqPlan* __restrict__ plans, int nseq, const int* __restrict__ cand,
                                 const float* __restrict__ margin, int* __restrict__ anchor_tok,
                                 int* __restrict__ records, int* __restrict__ dbg_u,
                                 float* __restrict__ dbg_m, int P, int L) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= nseq) return;
  const SeqPlan pl = plans[s];
  if (!pl.live) return;
  const int y = cand[(size_t)s * P];
  int* rec = records + s * 5;
  rec[0] = s;
  rec[1] = pl.C + 1;
  rec[2] = y;
  rec[3] = 0;
  rec[4] = L;
  anchor_tok[s] = y;
  dbg_u[s * kMaxN] = y;
  dbg_m[s * kMaxN] = margin[(size_t)s * P];
}

// Reset one sequence's lattice: empty map, all slots free, anchor token.
__global__ void reset_seq_kernel(int* __restrict__ map, int* __restrict__ freel, int* __restrict__ cursor,
                                 int* __restrict__ anchor_tok, const int* __restrict__ anchors, int nseq,
                                 int P) {
  const int s = blockIdx.x;
  if (s >= nseq) return;
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    freel[(size_t)s * P + p] = p;
    map[(size_t)s * P + p] = -1;
  }
  if (threadIdx.x == 0) {
    cursor[s] = 0;
    anchor_tok[s] = anchors[s];
  }
}

// ----------------------------------------------------------------------------
hipError_t launch_sched(const SeqPlan* plans, int nseq, RowInfo* rows, int* map, const int* cand,
                        const int* freel, int* cursor, const int* anchor_tok, int N, int P, int decs,
                        int single_exit, int cap, hipStream_t st) {
  hipLaunchKernelGGL(sched_kernel, dim3(nseq), dim3(256), 0, st, plans, rows, map, cand, freel, cursor,
                     anchor_tok, N, P, decs, single_exit, cap);
  return hipGetLastError();
}

hipError_t launch_commit(const SeqPlan* plans, int nseq, int* map, const int* cand, const float* margin,
                         int* freel, int* cursor, int* anchor_tok, int* records, int* promote_src,
                         int* dbg_u, float* dbg_m, const int* Xd, int N, int P, int single_exit, int cap,
                         hipStream_t st) {
  hipLaunchKernelGGL(commit_kernel, dim3(nseq), dim3(256), 0, st, plans, map, cand, margin, freel, cursor,
                     anchor_tok, records, promote_src, dbg_u, dbg_m, Xd, N, P, single_exit, cap);
  return hipGetLastError();
}

hipError_t launch_promote(const SeqPlan* plans, int nseq, const int* promote_src, const bf16_t* exb, bf16_t* kvc,
                          const ModelDims& D, hipStream_t st) {
  hipLaunchKernelGGL(promote_kernel, dim3(nseq, D.L, D.nkv), dim3(256), 0, st, plans, promote_src, exb, kvc, D);
  return hipGetLastError();
}

hipError_t launch_ar_rows(const SeqPlan* plans, int nseq, RowInfo* rows, const int* anchor_tok, int P,
                          hipStream_t st) {
  hipLaunchKernelGGL(ar_rows_kernel, dim3((nseq + 63) / 64), dim3(64), 0, st, plans, nseq, rows, anchor_tok, P);
  return hipGetLastError();
}

hipError_t launch_ar_commit(const SeqPlan* plans, int nseq, const int* cand, const float* margin,
                            int* anchor_tok, int* records, int* dbg_u, float* dbg_m, int P, int L,
                            hipStream_t st) {
  hipLaunchKernelGGL(ar_commit_kernel, dim3((nseq + 63) / 64), dim3(64), 0, st, plans, nseq, cand, margin,
                     anchor_tok, records, dbg_u, dbg_m, P, L);
  return hipGetLastError();
}

hipError_t launch_reset(int* map, int* freel, int* cursor, int* anchor_tok, const int* anchors, int nseq, int P,
                        hipStream_t st) {
  hipLaunchKernelGGL(reset_seq_kernel, dim3(nseq), dim3(256), 0, st, map, freel, cursor, anchor_tok, anchors,
                     nseq, P);
  return hipGetLastError();
}

}  // namespace dex
