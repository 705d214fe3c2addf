// Weight packing and the grouped, batch-invariant MFMA GEMM of the lattice step,
// with RMSNorm fused in front and RoPE/K-V write, residual add, SwiGLU or the
// DECS exit head fused behind.
//
// Every projection of a decoder layer (QKV, O, gate/up, down) and the shared
// LM head is Y[m, n] = sum_k A[m, k] W[n, k] with W row-major [N, K]
// ("Depth Exploration for LLM Decoding", Section 3.1: each explorer runs its
// stage, Layers(d_{k-1}, d_k], on its node batch; here one launch runs layer
// slot lambda of every stage that has rows, one weight group per stage).
//
// Activations A are fp32. For bf16 weights each A fragment is split in
// registers into a bf16 high part and a bf16 remainder (a = hi + lo up to
// 2^-16 relative), and both go through v_mfma_f32_16x16x32_bf16 against the
// same weight fragment: products are as exact as fp32 activations would
// give, at no extra weight traffic. fp32 weights use v_mfma_f32_16x16x4_f32.
//
// Fused RMSNorm: the producer of a residual row (embedding or a residual-add
// epilogue) writes, per 16-column tile, the residual h, h * g for the row's
// next normalising consumer (g its RMSNorm weight), and the tile's sum of
// squares. The consumer streams h * g as its A operand and multiplies each
// output by rstd = 1/sqrt(sum_t ssq[t] / d + eps), the sum taken lane-strided
// in tile order and closed by a fixed butterfly.
//
// Batch invariance: the value of output (m, n) depends only on row m of A and
// column n of W, never on how many rows share the launch or where the row
// sits. The reduction order is fixed by K alone:
//   * K is cut into k-steps of 32 (bf16) or 16 (fp32) elements;
//   * the k-steps are split into 8 contiguous ranges, [KS*w/8, KS*(w+1)/8)
//     for wave w, each accumulated from zero in increasing order;
//   * the 8 partial sums are added in wave order 0..7.
// So plain autoregressive decoding (one row) and a 2048-row lattice stage give
// bit-identical rows.
//
// Memory layout: weights are repacked once (dex_create) into MFMA fragments.
// Fragment (nb, ks) holds output columns 16nb..16nb+15 and k-step ks as 64
// lanes x 16 bytes, lane l carrying column l%16 and elements
// [ks*KSTEP + (l/16)*EPL, +EPL). A wave streaming its k range therefore reads
// one contiguous 1 KiB per instruction. Column order inside a 16-column tile is
// chosen for the epilogue: SwiGLU tiles hold 8 gate and the matching 8 up
// columns; query/key tiles hold 8 rotary pairs (i, i + hd/2).
#include "common.h"

namespace dex {

// Per k-step: A fragment of a lane (fp32 activations) and the weight fragment
// (16 bytes) -> accumulate into acc.
template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  static constexpr int KSTEP = 32;
  static constexpr int EPL = 8;      // elements per lane per k-step
  __device__ __forceinline__ static void mma(f32x4_t& acc, const float* f, const u32x4_t& b) {
    unsigned h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_bf2(f[2 * i], f[2 * i + 1], h[i], l[i]);
    bf16x8_t hi, lo, bv;
    __builtin_memcpy(&hi, h, 16);
    __builtin_memcpy(&lo, l, 16);
    __builtin_memcpy(&bv, &b, 16);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, bv, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, bv, acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int KSTEP = 16;
  static constexpr int EPL = 4;
  // Lane l supplies elements kbase + 4*(l/16) + i for i = 0..3; MFMA i reduces
  // over the four lane groups, so the four MFMAs cover the 16 elements.
  __device__ __forceinline__ static void mma(f32x4_t& acc, const float* f, const u32x4_t& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f[0], __uint_as_float(b[0]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f[1], __uint_as_float(b[1]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f[2], __uint_as_float(b[2]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f[3], __uint_as_float(b[3]), acc, 0, 0, 0);
  }
};

// Sum of squares of 16 consecutive values, in order.
__device__ __forceinline__ float ssq16(const float* v) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) s = fmaf(v[c], v[c], s);
  return s;
}

// ---------------------------------------------------------------------------
// Packing. mode 0: one source [N][K]. mode 1: QKV, rows of src0 (queries),
// src1 (keys), src2 (values) with n0, n1, n2 rows; query and key heads are
// permuted so that tile u of a head holds dims 8u..8u+7 in columns 0..7 and
// their rotary partners 8u+hd/2.. in columns 8..15 (hd = head_dim). mode 2:
// SwiGLU, gate (src0) and up (src1), each [n0][K]: packed tile nb holds gate
// rows 8nb..8nb+7 in columns 0..7 and up rows 8nb..8nb+7 in columns 8..15.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void pack_kernel(u32x4_t* __restrict__ dst, const T* __restrict__ s0, const T* __restrict__ s1,
                            const T* __restrict__ s2, int n0, int n1, int n2, int K, int mode, int hd,
                            long long total) {
  constexpr int KSTEP = Mfma<T>::KSTEP, EPL = Mfma<T>::EPL;
  const int KS = K / KSTEP;
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    const long long t = idx >> 6;
    const int ks = (int)(t % KS);
    const long long nb = t / KS;
    const int c = lane & 15;
    const int k0 = ks * KSTEP + (lane >> 4) * EPL;
    const T* src;
    if (mode == 2) {
      const long long r = nb * 8 + (c & 7);
      src = (c < 8 ? s0 : s1) + r * K;
    } else {
      long long r = nb * 16 + c;
      if (mode == 1 && r < (long long)n0 + n1) {
        const long long head = r / hd;
        const int within = (int)(r - head * hd), u = within >> 4;
        const int dim = c < 8 ? 8 * u + c : 8 * u + (c - 8) + hd / 2;
        r = head * hd + dim;
      }
      if (r < n0) src = s0 + r * K;
      else if (r < (long long)n0 + n1) src = s1 + (r - n0) * K;
      else src = s2 + (r - n0 - n1) * K;
    }
    dst[idx] = *(const u32x4_t*)(src + k0);
  }
}

// Rotary rotation of the pair (x1, x2) by the angle of cosine cs and sine sn,
// with its roundings spelled out (a product, then a fused multiply-add), so
// that every epilogue form gives the same bits whatever the compiler would
// contract.
__device__ __forceinline__ void rope_pair(float x1, float x2, float cs, float sn, float& o1, float& o2) {
  o1 = fmaf(x1, cs, -(x2 * sn));
  o2 = fmaf(x2, cs, x1 * sn);
}

// Exact merge of two (best, index, second) summaries: ties keep the lower id.
// The merge only compares and selects, so any order of merges gives the same
// summary: the rule's token and margin do not depend on how the tiles are
// grouped or which block reduces them.
__device__ __forceinline__ void top2_merge(float& b, int& i, float& s, float b2, int i2, float s2) {
  if (b2 > b || (b2 == b && i2 < i)) {
    s = fmaxf(s2, b);
    b = b2;
    i = i2;
  } else {
    s = fmaxf(s, b2);
  }
}

// ---------------------------------------------------------------------------
// Epilogue of one 16-column output tile for rows [0, G.m) of group G. val(rl, c)
// is the GEMM output of row rl, tile column c (before rstd); rs[rl] the row's
// rstd (normalising epilogues); scr is LDS scratch of ROWS x 17 floats. All NT
// threads of the block call it (it synchronises).
template <int EPI, int NT, int ROWS, typename Val>
__device__ __forceinline__ void epilogue_tile(const GemmArgs& args, const GemmGroup& G, int tile, Val val,
                                              const float* rs, float (*scr)[17]) {
  const int ntiles = args.N >> 4;
  constexpr int E = ROWS * 16;
  if constexpr (EPI == EPI_RESID) {
    // h += y for the tile's 16 columns; h * g for the next consumer (and the
    // exit head at a stage's end); then the tile's sum of squares.
    for (int e = threadIdx.x; e < E; e += NT) {
      const int rl = e >> 4, c = e & 15;
      if (rl >= G.m) continue;
      const size_t o = (size_t)args.rows[G.row0 + rl].hrow * args.N + tile * 16 + c;
      const float nv = args.hidden[o] + val(rl, c);
      args.hidden[o] = nv;
      if (G.gamma) args.xn[o] = nv * G.gamma[tile * 16 + c];
      if (G.xh) args.xh[o] = nv * args.gfinal[tile * 16 + c];
      if (G.anorm) args.xa[o] = nv * G.anorm[tile * 16 + c];
      scr[rl][c] = nv;
    }
    __syncthreads();
    for (int rl = threadIdx.x; rl < G.m; rl += NT) {
      const size_t so = (size_t)args.rows[G.row0 + rl].hrow * ntiles + tile;
      const float v = ssq16(scr[rl]);
      args.ssq[so] = v;
      if (G.xh) args.ssq_head[so] = v;
    }
  } else if constexpr (EPI == EPI_ADAPT1) {
    // Inducing adapter, first layer: SiLU(W1 (RMSNorm(h) * g) + b1).
    for (int e = threadIdx.x; e < E; e += NT) {
      const int rl = e >> 4, c = e & 15;
      if (rl >= G.m) continue;
      const float u = val(rl, c) * rs[rl] + G.bias[tile * 16 + c];
      ((float*)args.act)[(size_t)(G.row0 + rl) * args.N + tile * 16 + c] = u / (1.0f + expf(-u));
    }
  } else if constexpr (EPI == EPI_ADAPT2) {
    // Inducing adapter, second layer: h~ = h + alpha (W2 a + b2) is the exit
    // head's input (times the final-norm weight) and its tile sums of squares;
    // the residual stream keeps h.
    for (int e = threadIdx.x; e < E; e += NT) {
      const int rl = e >> 4, c = e & 15;
      if (rl >= G.m) continue;
      const size_t o = (size_t)args.rows[G.row0 + rl].hrow * args.N + tile * 16 + c;
      const float ht = args.hidden[o] + G.alpha * (val(rl, c) + G.bias[tile * 16 + c]);
      args.xh[o] = ht * args.gfinal[tile * 16 + c];
      scr[rl][c] = ht;
    }
    __syncthreads();
    for (int rl = threadIdx.x; rl < G.m; rl += NT)
      args.ssq_head[(size_t)args.rows[G.row0 + rl].hrow * ntiles + tile] = ssq16(scr[rl]);
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int e = threadIdx.x; e < ROWS * 8; e += NT) {
      const int rl = e >> 3, c = e & 7;
      if (rl >= G.m) continue;
      const float g = val(rl, c) * rs[rl], u = val(rl, c + 8) * rs[rl];
      const float s = g / (1.0f + expf(-g));
      ((float*)args.act)[(size_t)(G.row0 + rl) * (args.N >> 1) + tile * 8 + c] = s * u;
    }
  } else if constexpr (EPI == EPI_QKV) {
    // RoPE on query/key pairs (columns c, c+8), K/V into the committed cache
    // (autoregressive and prefill rows) or the node's explore slot.
    const ModelDims& D = args.dims;
    const int hd = D.hd, tph = hd >> 4;
    const int head = tile / tph, u = tile - head * tph;
    for (int e = threadIdx.x; e < ROWS * 8; e += NT) {
      const int rl = e >> 3, c = e & 7;
      if (rl >= G.m) continue;
      const int row = G.row0 + rl;
      const RowInfo& R = args.rows[row];
      const float x1 = val(rl, c) * rs[rl], x2 = val(rl, c + 8) * rs[rl];
      const int layer = layer_of(D, args.lattice, R.stage, args.lam);
      // K/V go out in the cache's format (fp16, or (hi, lo) bf16 pairs):
      // committed tile or explore entry.
      bf16_t* kvbase = nullptr;
      int kv = 0;
      const int kvp = D.kvp;
      if (head >= D.nq) {
        kv = head < D.nq + D.nkv ? 0 : 1;
        const int hh = head - D.nq - kv * D.nkv;
        kvbase = R.kv_commit ? args.kvc + kv_head_base(D, R.seq, layer, hh)
                             : args.exb + ex_base(D, R.seq, R.phys, args.lam, hh) + (size_t)kv * kvp * hd;
      }
      auto put = [&](int dd, float v) {
        unsigned hi, lo = 0;
        if (kvp == 1) hi = f2h2(v, 0.f);
        else split_bf2(v, 0.f, hi, lo);
        if (R.kv_commit) {
          kvbase[kv_elem(hd, kvp, R.pos, kv, 0, dd)] = (bf16_t)hi;
          if (kvp == 2) kvbase[kv_elem(hd, kvp, R.pos, kv, 1, dd)] = (bf16_t)lo;
        } else {
          kvbase[dd] = (bf16_t)hi;
          if (kvp == 2) kvbase[hd + dd] = (bf16_t)lo;
        }
      };
      if (kv == 1) {                         // values: natural column order
        put(16 * u + c, x1);
        put(16 * u + c + 8, x2);
        continue;
      }
      const int i = 8 * u + c;
      const float cs = args.cosT[(size_t)R.pos * (hd >> 1) + i], sn = args.sinT[(size_t)R.pos * (hd >> 1) + i];
      float o1, o2;
      rope_pair(x1, x2, cs, sn, o1, o2);
      if (head < D.nq) {
        float* qd = args.qout + ((size_t)row * D.nq + head) * hd;
        qd[i] = o1 * args.qscale;
        qd[i + (hd >> 1)] = o2 * args.qscale;
      } else {
        put(i, o1);
        put(i + (hd >> 1), o2);
      }
    }
  } else {  // EPI_HEAD
    for (int e = threadIdx.x; e < E; e += NT) {
      const int rl = e >> 4, c = e & 15;
      if (rl >= G.m) continue;
      const float z = val(rl, c) * rs[rl];
      const int row = G.row0 + rl;
      const int n = tile * 16 + c;
      const RowInfo& ri = args.rows[row];
      if (args.out != nullptr && ri.final_) args.out[(size_t)ri.seq * args.N + n] = z;
      float s = z;
      if (!ri.final_) {
        for (int i = 0; i < ri.n_mask; ++i)
          if (ri.mask[i] == n) s = -INFINITY;
      }
      if (args.mode == 1)
        s = s / args.tau + args.gumbel[((size_t)ri.seq * args.gumbel_rows + ri.grow) * args.N + n];
      scr[rl][c] = s;
    }
    __syncthreads();
    for (int rl = threadIdx.x; rl < ROWS; rl += NT) {
      if (rl >= G.m) continue;
      float best = scr[rl][0], second = -INFINITY;
      int bi = 0;
      for (int c = 1; c < 16; ++c) {
        const float s = scr[rl][c];
        if (s > best) {
          second = best;
          best = s;
          bi = c;
        } else if (s > second) {
          second = s;
        }
      }
      float* p = args.part + ((size_t)(G.row0 + rl) * ntiles + tile) * 3;
      p[0] = best;
      p[1] = __int_as_float(tile * 16 + bi);
      p[2] = second;
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM. grid = (N/(16 NB) tile blocks, groups), block = 512 (8 waves =
// the 8 k ranges). A workgroup covers NB adjacent 16-column tiles and reuses
// each activation fragment for all of them.
// ---------------------------------------------------------------------------
#ifndef DEX_GEMM_U
#define DEX_GEMM_U 4
#endif
// Blocks of one row block (the decode-bound shape) are held to 64 VGPRs, so a
// CU keeps four blocks (32 waves) and their loads in flight instead of three.
template <typename T, int MB, int NB, int EPI>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(MB == 1 ? 8 : 1))) void gemm_kernel(
    const GemmArgs args) {
  constexpr int KSTEP = Mfma<T>::KSTEP;
  constexpr int EPL = Mfma<T>::EPL;
  constexpr int AW = EPL / 4;          // 16-byte A loads per lane per k-step (fp32 activations)
  constexpr int U = DEX_GEMM_U;        // k-steps of loads in flight per wave
  constexpr bool NORM = epi_norm(EPI);
  const int gi = blockIdx.y;
  if (gi >= args.ngroups) return;
  const GemmGroup G = args.g[gi];
  const int tile0 = blockIdx.x * NB;
  const int ntiles = args.N >> 4;
  const int K = args.K;
  const int KS = K / KSTEP;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int kb = (KS * w) / kKSplit, ke = (KS * (w + 1)) / kKSplit;
  const int col16 = lane & 15;
  const int kq = (lane >> 4) * EPL;

  __shared__ float red[kKSplit][NB][MB * 256];
  __shared__ float rs_sh[MB * 16];
  __shared__ float scr[MB * 16][17];

  const u32x4_t* wp = (const u32x4_t*)G.w + (size_t)tile0 * KS * 64 + lane;
  f32x4_t acc[MB][NB];
  // Rows past the group's end are not loaded (masked lanes fetch nothing).
  const u32x4_t* ap[MB];
  bool av[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int r = mb * 16 + col16;
    av[mb] = r < G.m;
    const int rr = av[mb] ? r : 0;
    const float* base = NORM ? args.xin + (size_t)args.rows[G.row0 + rr].hrow * K
                             : (const float*)args.a + (size_t)(G.row0 + rr) * K;
    ap[mb] = (const u32x4_t*)(base + kq);
  }
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  auto load_a = [&](int k, int mb, float* f) {
#pragma unroll
    for (int x = 0; x < AW; ++x) {
      const u32x4_t v = av[mb] ? ap[mb][k * (KSTEP / 4) + x] : zero;
#pragma unroll
      for (int e = 0; e < 4; ++e) f[4 * x + e] = __uint_as_float(v[e]);
    }
  };
  auto load_b = [&](int k, int nb) { return __builtin_nontemporal_load(wp + ((size_t)nb * KS + k) * 64); };

  // Every load of U k-steps is issued before the MFMAs that consume them.
  int ks = kb;
  for (; ks + U <= ke; ks += U) {
    u32x4_t bv[U][NB];
    float a[U][MB][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) bv[u][nb] = load_b(ks + u, nb);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) load_a(ks + u, mb, a[u][mb]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) Mfma<T>::mma(acc[mb][nb], a[u][mb], bv[u][nb]);
  }
  for (; ks < ke; ++ks) {
    u32x4_t b[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) b[nb] = load_b(ks, nb);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float a[EPL];
      load_a(ks, mb, a);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) Mfma<T>::mma(acc[mb][nb], a, b[nb]);
    }
  }

  // rstd of each row of a normalising GEMM, from the producer's tile sums.
  if constexpr (NORM) {
    const int nt = K >> 4;
    for (int rl = w; rl < G.m; rl += kKSplit) {
      const float* sq = args.ssq + (size_t)args.rows[G.row0 + rl].hrow * nt;
      float s = 0.f;
      for (int t = lane; t < nt; t += 64) s += sq[t];
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0) rs_sh[rl] = 1.0f / sqrtf(s / (float)K + args.eps);
    }
  }

  // Partial tiles of the 8 k ranges, then their sum in wave order.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[w][nb][(mb * 16 + (lane >> 4) * 4 + r) * 16 + col16] = acc[mb][nb][r];
  __syncthreads();
  for (int nb = 0; nb < NB; ++nb) {
    auto total = [&](int rl, int c) {
      const int e = rl * 16 + c;
      float v = red[0][nb][e];
#pragma unroll
      for (int q = 1; q < kKSplit; ++q) v += red[q][nb][e];
      return v;
    };
    epilogue_tile<EPI, kGemmThreads, MB * 16>(args, G, tile0 + nb, total, rs_sh, scr);
    if (NB > 1) __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Wide GEMM for groups of many rows (bf16 weights). 1-D grid of (group, column
// block[, k range]) blocks, block = NWV waves (4, or 8 for one block of 512
// columns per CU); a block computes 64 rows x NWV WT column tiles, wave w the
// WT tiles from WT w (WT and NWV do not change any output's bits, only the
// block count). Each k-step's activations (64 rows x 32, fp32) are split once
// into bf16 (hi, lo) by the first four waves and stored in LDS in MFMA operand
// order, shared by all waves, so a block reads its rows' activations once per
// K pass whatever its width; global loads run three k-steps ahead in
// registers. Each output is reduced exactly as in
// gemm_kernel: the 8 k ranges [KS r/8, KS (r+1)/8) are accumulated from zero
// by the same MFMA chain (hi then lo per k-step), in order, and summed in
// range order, so a row gets the same bits from either kernel and from any
// grouping. SPLIT: the block takes one k range only and leaves its partial in
// args.split for gemm_split_reduce_kernel.
// Blocks that read the same weight tile (the row groups of one column block)
// are given consecutive logical ids on one XCD, so the tile is fetched into
// that XCD's L2 once.
// ---------------------------------------------------------------------------
constexpr int kWideThreads = 256;

// Exit-head epilogue of a wide block: t holds the block's BT tiles for its 64
// rows (before rstd). Lane l of each of the NW waves takes row l, and wave w
// the tiles w, w + NW, ...: the row's data is read once, and each tile's 16
// columns are scanned in column order exactly as in epilogue_tile (same mask,
// noise and top-2 arithmetic, so the summaries carry the same bits). With a
// row per lane and a row pitch of 4 banks, the 16-byte LDS reads of a wave
// fall on distinct banks.
template <int BT, int NW>
__device__ __forceinline__ void head_epilogue_wide(const GemmArgs& args, const GemmGroup& G, int tb0,
                                                   const float (*t)[BT * 16 + 4], const float* rs) {
  const int ntiles = args.N >> 4;
  const int rl = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (rl >= G.m) return;
  const RowInfo& ri = args.rows[G.row0 + rl];
  const bool fin = ri.final_ != 0;
  const float rsl = rs[rl];
  float* outp = args.out != nullptr && fin ? args.out + (size_t)ri.seq * args.N : nullptr;
  const float* gum = args.mode == 1 ? args.gumbel + ((size_t)ri.seq * args.gumbel_rows + ri.grow) * args.N : nullptr;
  // Whether a masked token falls in the block's columns at all (a row masks at
  // most N - 1 tokens, so nearly every block has none).
  const int nm = fin ? 0 : ri.n_mask;
  bool hit = false;
  for (int i = 0; i < nm; ++i) hit |= ri.mask[i] >= tb0 * 16 && ri.mask[i] < (tb0 + BT) * 16;
  float* part = args.part + ((size_t)(G.row0 + rl) * ntiles) * 3;
  for (int tl = w; tl < BT && tb0 + tl < ntiles; tl += NW) {
    const int n0 = (tb0 + tl) * 16;
    float s[16];
#pragma unroll
    for (int c = 0; c < 16; c += 4) {
      const float4 v = *(const float4*)&t[rl][tl * 16 + c];
      s[c] = v.x * rsl;
      s[c + 1] = v.y * rsl;
      s[c + 2] = v.z * rsl;
      s[c + 3] = v.w * rsl;
    }
    if (outp != nullptr) {
#pragma unroll
      for (int c = 0; c < 16; c += 4) *(float4*)(outp + n0 + c) = float4{s[c], s[c + 1], s[c + 2], s[c + 3]};
    }
    if (hit) {
      for (int i = 0; i < nm; ++i) {
        const int m = ri.mask[i] - n0;
#pragma unroll
        for (int c = 0; c < 16; ++c)
          if (m == c) s[c] = -INFINITY;
      }
    }
    if (gum != nullptr) {
#pragma unroll
      for (int c = 0; c < 16; c += 4) {
        const float4 g = *(const float4*)(gum + n0 + c);
        s[c] = s[c] / args.tau + g.x;
        s[c + 1] = s[c + 1] / args.tau + g.y;
        s[c + 2] = s[c + 2] / args.tau + g.z;
        s[c + 3] = s[c + 3] / args.tau + g.w;
      }
    }
    float best = s[0], second = -INFINITY;
    int bi = 0;
#pragma unroll
    for (int c = 1; c < 16; ++c) {
      const bool gt = s[c] > best;
      second = gt ? best : (s[c] > second ? s[c] : second);
      bi = gt ? c : bi;
      best = gt ? s[c] : best;
    }
    float* p = part + (size_t)(tb0 + tl) * 3;
    p[0] = best;
    p[1] = __int_as_float(n0 + bi);
    p[2] = second;
  }
}

// Residual epilogue of a wide block, in the same lane layout: lane l of wave w
// adds row l's outputs of tiles w, w + NW, ... into the residual stream. The
// residual reads of all of the lane's tiles go out before the first is used
// (one memory latency per block instead of one per tile). Per element and per
// tile sum of squares the arithmetic is epilogue_tile's, so the bits are too.
// Query/key/value epilogue of a wide block, in the same lane layout: lane l of
// wave w takes row l's tiles w, w + NW, ... (a tile lies in one head), with
// the row's data read once. Per element the arithmetic is epilogue_tile's;
// key and explore-buffer runs of 8 or 16 dims go out as 16-byte stores.
template <int BT, int NW>
__device__ __forceinline__ void qkv_epilogue_wide(const GemmArgs& args, const GemmGroup& G, int tb0,
                                                  const float (*t)[BT * 16 + 4], const float* rs) {
  const ModelDims& D = args.dims;
  const int hd = D.hd, tph = hd >> 4, half = hd >> 1;
  const int ntiles = args.N >> 4;
  const int rl = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (rl >= G.m) return;
  const int row = G.row0 + rl;
  const RowInfo& R = args.rows[row];
  const int seq = R.seq, phys = R.phys, pos = R.pos;
  const bool commit = R.kv_commit != 0;
  const int layer = layer_of(D, args.lattice, R.stage, args.lam);
  const float rsl = rs[rl];
  const float* cosr = args.cosT + (size_t)pos * half;
  const float* sinr = args.sinT + (size_t)pos * half;
  // 8 consecutive values in the cache's format: fp16 at hp (kvp = 1), or
  // (hi, lo) bf16 runs at hp and lp (16-byte aligned).
  const int kvp = D.kvp;
  auto put8 = [kvp](bf16_t* hp, bf16_t* lp, const float* v) {
    u32x4_t h, l;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      unsigned hk, lk;
      if (kvp == 1) hk = f2h2(v[2 * k], v[2 * k + 1]), lk = 0;
      else split_bf2(v[2 * k], v[2 * k + 1], hk, lk);
      h[k] = hk;
      l[k] = lk;
    }
    *(u32x4_t*)hp = h;
    if (kvp == 2) *(u32x4_t*)lp = l;
  };
  for (int tl = w; tl < BT && tb0 + tl < ntiles; tl += NW) {
    const int tile = tb0 + tl;
    const int head = tile / tph, u = tile - head * tph;
    float x[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = *(const float4*)&t[rl][tl * 16 + 4 * q];
      x[4 * q] = v.x * rsl;
      x[4 * q + 1] = v.y * rsl;
      x[4 * q + 2] = v.z * rsl;
      x[4 * q + 3] = v.w * rsl;
    }
    if (head >= D.nq + D.nkv) {   // values: dims 16u .. 16u + 15 in column order
      const int hh = head - D.nq - D.nkv;
      if (commit) {
        bf16_t* base = args.kvc + kv_head_base(D, seq, layer, hh);
#pragma unroll
        for (int c = 0; c < 16; c += 2) {
          unsigned hi, lo = 0;
          if (kvp == 1) hi = f2h2(x[c], x[c + 1]);
          else split_bf2(x[c], x[c + 1], hi, lo);
          base[kv_elem(hd, kvp, pos, 1, 0, 16 * u + c)] = (bf16_t)hi;
          base[kv_elem(hd, kvp, pos, 1, 0, 16 * u + c + 1)] = (bf16_t)(hi >> 16);
          if (kvp == 2) {
            base[kv_elem(hd, kvp, pos, 1, 1, 16 * u + c)] = (bf16_t)lo;
            base[kv_elem(hd, kvp, pos, 1, 1, 16 * u + c + 1)] = (bf16_t)(lo >> 16);
          }
        }
      } else {
        bf16_t* base = args.exb + ex_base(D, seq, phys, args.lam, hh) + (size_t)kvp * hd + 16 * u;
        put8(base, base + hd, x);
        put8(base + 8, base + hd + 8, x + 8);
      }
      continue;
    }
    float o1[8], o2[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) rope_pair(x[c], x[c + 8], cosr[8 * u + c], sinr[8 * u + c], o1[c], o2[c]);
    if (head < D.nq) {   // 16-byte stores: dims 8u .. 8u + 7 and half + 8u .. half + 8u + 7
      float* qd = args.qout + ((size_t)row * D.nq + head) * hd + 8 * u;
      const float qs = args.qscale;
      *(f32x4_t*)qd = f32x4_t{o1[0] * qs, o1[1] * qs, o1[2] * qs, o1[3] * qs};
      *(f32x4_t*)(qd + 4) = f32x4_t{o1[4] * qs, o1[5] * qs, o1[6] * qs, o1[7] * qs};
      *(f32x4_t*)(qd + half) = f32x4_t{o2[0] * qs, o2[1] * qs, o2[2] * qs, o2[3] * qs};
      *(f32x4_t*)(qd + half + 4) = f32x4_t{o2[4] * qs, o2[5] * qs, o2[6] * qs, o2[7] * qs};
    } else {
      const int hh = head - D.nq;
      if (commit) {
        bf16_t* base = args.kvc + kv_head_base(D, seq, layer, hh);
        put8(base + kv_elem(hd, kvp, pos, 0, 0, 8 * u), base + kv_elem(hd, kvp, pos, 0, 1, 8 * u), o1);
        put8(base + kv_elem(hd, kvp, pos, 0, 0, 8 * u + half), base + kv_elem(hd, kvp, pos, 0, 1, 8 * u + half), o2);
      } else {
        bf16_t* base = args.exb + ex_base(D, seq, phys, args.lam, hh) + 8 * u;
        put8(base, base + hd, o1);
        put8(base + half, base + hd + half, o2);
      }
    }
  }
}

template <int BT, int NW>
__device__ __forceinline__ void resid_epilogue_wide(const GemmArgs& args, const GemmGroup& G, int tb0,
                                                    const float (*t)[BT * 16 + 4]) {
  constexpr int TPW = BT / NW;   // tiles per wave
  const int ntiles = args.N >> 4;
  const int rl = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (rl >= G.m) return;
  const size_t rbase = (size_t)args.rows[G.row0 + rl].hrow * args.N;
  float4 h[TPW][4];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int tile = tb0 + w + j * NW;
    if (tile < ntiles) {
#pragma unroll
      for (int q = 0; q < 4; ++q) h[j][q] = *(const float4*)(args.hidden + rbase + tile * 16 + 4 * q);
    }
  }
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int tl = w + j * NW, tile = tb0 + tl;
    if (tile >= ntiles) break;
    float v[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 y = *(const float4*)&t[rl][tl * 16 + 4 * q];
      v[4 * q] = h[j][q].x + y.x;
      v[4 * q + 1] = h[j][q].y + y.y;
      v[4 * q + 2] = h[j][q].z + y.z;
      v[4 * q + 3] = h[j][q].w + y.w;
    }
    const size_t o = rbase + tile * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q) *(float4*)(args.hidden + o + 4 * q) = float4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
    auto scaled = [&](float* dst, const float* g) {
      float u[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) u[c] = v[c] * g[tile * 16 + c];
#pragma unroll
      for (int q = 0; q < 4; ++q) *(float4*)(dst + o + 4 * q) = float4{u[4 * q], u[4 * q + 1], u[4 * q + 2], u[4 * q + 3]};
    };
    if (G.gamma) scaled(args.xn, G.gamma);
    if (G.xh) scaled(args.xh, args.gfinal);
    if (G.anorm) scaled(args.xa, G.anorm);
    const float s = ssq16(v);
    const size_t so = (size_t)args.rows[G.row0 + rl].hrow * ntiles + tile;
    args.ssq[so] = s;
    if (G.xh) args.ssq_head[so] = s;
  }
}

template <int EPI, bool SPLIT, int WT, int NWV>
__global__ __launch_bounds__(NWV * 64) void gemm_wide_kernel(const GemmArgs args) {
  constexpr int NT = NWV * 64;  // threads: NWV waves, each WT column tiles of the block's 64 rows
  constexpr int BT = NWV * WT;  // 16-column tiles per block
  constexpr int MBLK = 4;      // 16-row blocks per block (the first four waves stage them)
  static_assert(NWV == 4 || (NWV == 8 && !SPLIT), "4 waves, or 8 unsplit");
  constexpr int ROWS = 16 * MBLK;
  constexpr int DEPTH = 3;     // k-steps of loads in flight
  constexpr int KSTEP = 32;
  constexpr bool NORM = epi_norm(EPI);
  const int ntiles = args.N >> 4;
  const int ncb = (ntiles + BT - 1) / BT;
  const int nblk = args.ngroups * ncb * (SPLIT ? kKSplit : 1);
  // Block order. The hardware hands blocks to the 8 XCDs round-robin.
  //  * Row-sharded part (xcd_rows, the first Q = ngroups - ngroups % 8
  //    groups): XCD x takes groups [x Q/8, (x + 1) Q/8) for every column
  //    block, column block slowest, so the activations of its rows stay in its
  //    L2 while the weight tiles stream through (a weight tile is read by the
  //    XCDs whose groups need it).
  //  * The other groups: the blocks that read one weight tile (the row groups
  //    of a column block) get consecutive logical ids on one XCD, so the tile
  //    is fetched into that XCD's L2 once. With runs (nrun > 0), the groups
  //    of one weight take all their column blocks before the next weight's
  //    groups start, so an XCD works on one or two weights at a time and
  //    keeps only their groups' activations in flight, not every group's.
  const int Q = !SPLIT && args.xcd_rows ? args.ngroups & ~7 : 0;
  int gi, cb, z = 0;
  if ((int)blockIdx.x < Q * ncb) {
    const int x = blockIdx.x & 7, kk = blockIdx.x >> 3, gpx = Q >> 3;
    gi = x * gpx + kk % gpx;
    cb = kk / gpx;
  } else {
    const int R = args.ngroups - Q;
    const int lb = xcd_block(blockIdx.x - Q * ncb, nblk - Q * ncb);
    if (!SPLIT && args.nrun > 0) {
      int r = 0;
      while (r + 1 < args.nrun && lb >= ncb * (args.run0[r + 1] - Q)) ++r;
      const int g0 = args.run0[r], len = args.run0[r + 1] - g0, local = lb - ncb * (g0 - Q);
      gi = g0 + local % len;
      cb = local / len;
    } else {
      gi = Q + lb % R;
      cb = (lb / R) % ncb;
      z = SPLIT ? lb / (R * ncb) : 0;
    }
  }
  const GemmGroup G = args.g[gi];
  const int tb0 = cb * BT;
  const int K = args.K, KS = K / KSTEP;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col16 = lane & 15, kg = lane >> 4;
  const int t0 = tb0 + w * WT;

  // f[buf][slot][part][mb][lane]: part 0 (hi) / 1 (lo) of row 16 mb +
  // (lane & 15), k 8 (lane >> 4) .. +7 of k-step `slot` of the KPB k-steps
  // staged between two barriers, the A operand of lane `lane`.
  constexpr int KPB = SPLIT || NWV != 8 ? 1 : kWideKPB;
  struct Stage { u32x4_t f[2][KPB][2][MBLK][64]; };
  struct Out { float t[SPLIT ? 1 : ROWS][BT * 16 + 4]; };   // the split form stores from registers
  __shared__ union { Stage s; Out o; } sm;
  __shared__ float rs_sh[ROWS];
  __shared__ float scr[SPLIT || EPI != EPI_ADAPT2 ? 1 : ROWS][17];

  // Thread (w, lane) of the first four waves converts the fragment that lane
  // `lane` of row block w reads. Rows past the group's end repeat its first
  // row and tiles past N the last tile: their outputs are never stored.
  const bool conv = w < MBLK;
  const int ar = 16 * (conv ? w : 0) + col16;
  const int rr = ar < G.m ? ar : 0;
  const float* asrc = (NORM ? args.xin + (size_t)args.rows[G.row0 + rr].hrow * K
                            : (const float*)args.a + (size_t)(G.row0 + rr) * K) + 8 * kg;
  // weight fragments: a lane offset on the group's base, and per tile a
  // uniform offset (the tile index is the same for the whole wave)
  const u32x4_t* bbase = (const u32x4_t*)G.w + lane;
  int btile[WT];
#pragma unroll
  for (int nb = 0; nb < WT; ++nb) btile[nb] = t0 + nb < ntiles ? t0 + nb : ntiles - 1;

  struct Pre {
    f32x4_t a[2];
    u32x4_t b[WT];
  };
  auto load_a = [&](int ks, Pre& p) {
    ks = ks < KS ? ks : KS - 1;
    const f32x4_t* ap = (const f32x4_t*)(asrc + (size_t)ks * KSTEP);
    p.a[0] = ap[0];
    p.a[1] = ap[1];
  };
  auto load_b = [&](int ks, Pre& p) {
    ks = ks < KS ? ks : KS - 1;
#pragma unroll
    for (int nb = 0; nb < WT; ++nb) p.b[nb] = bbase[((size_t)btile[nb] * KS + ks) * 64];
  };
  // One k-step from the registers of p, which then take k-step ks + DEPTH
  // (three register sets, so each load has two k-steps of MFMAs to land in;
  // a fourth set measured no faster): the activation loads go out once p.a is
  // staged, the weight loads once the MFMAs have read p.b. stage() before the
  // barrier, compute() after it.
  auto stage = [&](int ks, Pre& p, int buf, int slot) {
    if (conv) {
      u32x4_t hv, lv;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        unsigned h0, l0, h1, l1;
        split_bf2(p.a[x][0], p.a[x][1], h0, l0);
        split_bf2(p.a[x][2], p.a[x][3], h1, l1);
        hv[2 * x] = h0;
        hv[2 * x + 1] = h1;
        lv[2 * x] = l0;
        lv[2 * x + 1] = l1;
      }
      sm.s.f[buf][slot][0][w][lane] = hv;
      sm.s.f[buf][slot][1][w][lane] = lv;
      load_a(ks + DEPTH, p);
    }
  };
  auto compute = [&](int ks, Pre& p, int buf, int slot, f32x4_t (&acc)[MBLK][WT]) {
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb) {
      const u32x4_t ahu = sm.s.f[buf][slot][0][mb][lane], alu = sm.s.f[buf][slot][1][mb][lane];
      bf16x8_t ah, al;
      __builtin_memcpy(&ah, &ahu, 16);
      __builtin_memcpy(&al, &alu, 16);
#pragma unroll
      for (int nb = 0; nb < WT; ++nb) {
        bf16x8_t bv;
        __builtin_memcpy(&bv, &p.b[nb], 16);
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bv, acc[mb][nb], 0, 0, 0);
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bv, acc[mb][nb], 0, 0, 0);
      }
    }
    load_b(ks + DEPTH, p);
  };

  // The k ranges in order: acc takes one range, tot the range sums (the first
  // as it is, the next ones added in order); the loop walks every k-step of
  // the block's ranges with the three register sets in turn.
  f32x4_t tot[MBLK][WT], acc[MBLK][WT];
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
    for (int nb = 0; nb < WT; ++nb) acc[mb][nb] = tot[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int r0 = SPLIT ? z : 0, r1 = SPLIT ? z + 1 : kKSplit;
  int ks = (KS * r0) / kKSplit;
  const int kend = (KS * r1) / kKSplit;
  int r = r0, rend = (KS * (r0 + 1)) / kKSplit;
  Pre p[DEPTH];
#pragma unroll
  for (int i = 0; i < DEPTH; ++i) {
    if (conv) load_a(ks + i, p[i]);
    load_b(ks + i, p[i]);
  }
  auto close = [&](int k) {
    if (k + 1 == rend) {
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
        for (int nb = 0; nb < WT; ++nb) {
          tot[mb][nb] = r == r0 ? acc[mb][nb] : tot[mb][nb] + acc[mb][nb];
          acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      ++r;
      rend = (KS * (r + 1)) / kKSplit;
    }
  };
  if constexpr (KPB == 1) {
    auto step = [&](int k, Pre& pk) {
      stage(k, pk, k & 1, 0);
      __syncthreads();
      compute(k, pk, k & 1, 0, acc);
      close(k);
    };
    for (; ks + DEPTH <= kend; ks += DEPTH) {
#pragma unroll
      for (int i = 0; i < DEPTH; ++i) step(ks + i, p[i]);
    }
#pragma unroll
    for (int i = 0; i < DEPTH - 1; ++i) {
      if (ks < kend) {
        step(ks, p[i]);
        ++ks;
      }
    }
  } else {
    // Two k-steps per barrier: k-steps k and k + 1 (when below kend) staged
    // into buffer pi & 1, then computed in order. The register sets still
    // take k-steps in turn (six k-steps walk the three sets twice).
    static_assert(KPB == 2 && DEPTH == 3, "pairs of k-steps over three register sets");
    int pi = 0;
    auto pair = [&](int k, Pre& pa, Pre& pb) {
      const int buf = pi & 1;
      const bool two = k + 1 < kend;
      stage(k, pa, buf, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (two) stage(k + 1, pb, buf, 1);
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
      compute(k, pa, buf, 0, acc);
      close(k);
      if (two) {
        // keep the second k-step's LDS reads below the first one's MFMAs:
        // hoisted, they need 32 more VGPRs and spill
        __builtin_amdgcn_sched_barrier(0);
        compute(k + 1, pb, buf, 1, acc);
        close(k + 1);
      }
      ++pi;
    };
    for (; ks + 2 * DEPTH <= kend; ks += 2 * DEPTH) {
      pair(ks, p[0], p[1]);
      pair(ks + 2, p[2], p[0]);
      pair(ks + 4, p[1], p[2]);
    }
    if (ks < kend) pair(ks, p[0], p[1]);
    if (ks + 2 < kend) pair(ks + 2, p[2], p[0]);
    if (ks + 4 < kend) pair(ks + 4, p[1], p[2]);
  }

  if constexpr (SPLIT) {
    float* dst = args.split + ((size_t)z * kSplitRows + G.srow) * args.N;
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
      for (int nb = 0; nb < WT; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rl = mb * 16 + kg * 4 + r;
          if (rl < G.m && t0 + nb < ntiles) dst[(size_t)rl * args.N + (t0 + nb) * 16 + col16] = tot[mb][nb][r];
        }
    return;
  }
  if constexpr (NORM) {
    const int nt = K >> 4;
    for (int rl = w; rl < G.m; rl += NWV) {
      const float* sq = args.ssq + (size_t)args.rows[G.row0 + rl].hrow * nt;
      float s = 0.f;
      for (int t = lane; t < nt; t += 64) s += sq[t];
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0) rs_sh[rl] = 1.0f / sqrtf(s / (float)K + args.eps);
    }
  }
  __syncthreads();   // the last k-step's LDS reads are done before the outputs overwrite them
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
    for (int nb = 0; nb < WT; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.o.t[mb * 16 + kg * 4 + r][(w * WT + nb) * 16 + col16] = tot[mb][nb][r];
  __syncthreads();
  if constexpr (EPI == EPI_HEAD) {
    head_epilogue_wide<BT, NWV>(args, G, tb0, sm.o.t, rs_sh);
  } else if constexpr (EPI == EPI_RESID) {
    resid_epilogue_wide<BT, NWV>(args, G, tb0, sm.o.t);
  } else if constexpr (EPI == EPI_QKV) {
    qkv_epilogue_wide<BT, NWV>(args, G, tb0, sm.o.t, rs_sh);
  } else {
    // Only the adapter's second layer uses scr, so only it waits between tiles.
    for (int tl = 0; tl < BT && tb0 + tl < ntiles; ++tl) {
      epilogue_tile<EPI, NT, ROWS>(args, G, tb0 + tl, [&](int rl, int c) { return sm.o.t[rl][tl * 16 + c]; },
                                           rs_sh, scr);
      if constexpr (EPI == EPI_ADAPT2) __syncthreads();
    }
  }
}

// Sum of a split-range wide GEMM's 8 range partials, in range order, then the
// epilogue. grid = (groups, N/16 tiles), block = 256.
template <int EPI>
__global__ __launch_bounds__(kWideThreads) void gemm_split_reduce_kernel(const GemmArgs args) {
  constexpr bool NORM = epi_norm(EPI);
  const GemmGroup G = args.g[blockIdx.x];
  const int tile = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __shared__ float val[64][17];
  __shared__ float rs_sh[64];
  __shared__ float scr[64][17];
  const size_t rstride = (size_t)kSplitRows * args.N;
  for (int e = threadIdx.x; e < G.m * 16; e += kWideThreads) {
    const int rl = e >> 4, c = e & 15;
    const float* p = args.split + (size_t)(G.srow + rl) * args.N + tile * 16 + c;
    float v = p[0];
#pragma unroll
    for (int q = 1; q < kKSplit; ++q) v += p[q * rstride];
    val[rl][c] = v;
  }
  if constexpr (NORM) {
    const int K = args.K, nt = K >> 4;
    for (int rl = w; rl < G.m; rl += kWideThreads / 64) {
      const float* sq = args.ssq + (size_t)args.rows[G.row0 + rl].hrow * nt;
      float s = 0.f;
      for (int t = lane; t < nt; t += 64) s += sq[t];
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0) rs_sh[rl] = 1.0f / sqrtf(s / (float)K + args.eps);
    }
  }
  __syncthreads();
  epilogue_tile<EPI, kWideThreads, 64>(args, G, tile, [&](int rl, int c) { return val[rl][c]; }, rs_sh, scr);
}

// One workgroup of four waves per row of [row0, row0 + nrows): reduce the
// per-tile summaries to the row's token and margin (the merge is exact, so
// how the tiles are split among the threads does not change the result).
__global__ void head_reduce_kernel(const float* __restrict__ part, int ntiles, int row0,
                                   const RowInfo* __restrict__ rows, int P, int* __restrict__ cand,
                                   float* __restrict__ margin) {
  const int row = row0 + blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float b = -INFINITY, s = -INFINITY;
  int i = 0x7fffffff;
  for (int t = threadIdx.x; t < ntiles; t += blockDim.x) {
    const float* p = part + ((size_t)row * ntiles + t) * 3;
    top2_merge(b, i, s, p[0], __float_as_int(p[1]), p[2]);
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const float b2 = __shfl_xor(b, off);
    const int i2 = __shfl_xor(i, off);
    const float s2 = __shfl_xor(s, off);
    top2_merge(b, i, s, b2, i2, s2);
  }
  __shared__ float wb[4], ws[4];
  __shared__ int wi[4];
  if (lane == 0) {
    wb[w] = b;
    wi[w] = i;
    ws[w] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < (int)(blockDim.x >> 6); ++k) top2_merge(b, i, s, wb[k], wi[k], ws[k]);
    const RowInfo& ri = rows[row];
    if (i < 0 || i >= ntiles * 16) i = 0;  // unreachable for finite logits; keeps token ids in range
    cand[ri.seq * P + ri.phys] = i;
    margin[ri.seq * P + ri.phys] = b - s;
  }
}

// Embedding gather for rows with tok >= 0 (explorer 0 of a lattice round, prefill and
// autoregressive rows):
// h = E[tok] in fp32, xn = h * g0 (first layer's attention-norm weight) and the
// per-16-column sums of squares.
template <typename T>
__global__ void embed_kernel(const T* __restrict__ E, const RowInfo* __restrict__ rows, int row0,
                             float* __restrict__ hidden, float* __restrict__ xn, float* __restrict__ ssq,
                             const float* __restrict__ g0, int d) {
  const RowInfo& r = rows[row0 + blockIdx.x];
  if (r.tok < 0) return;
  const T* e = E + (size_t)r.tok * d;
  const size_t base = (size_t)r.hrow * d;
  for (int t = threadIdx.x; t < d / 16; t += blockDim.x) {
    float v[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) v[c] = to_f<T>(e[16 * t + c]);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      hidden[base + 16 * t + c] = v[c];
      xn[base + 16 * t + c] = v[c] * g0[16 * t + c];
    }
    ssq[(size_t)r.hrow * (d / 16) + t] = ssq16(v);
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <typename T>
hipError_t launch_pack(void* dst, const void* s0, const void* s1, const void* s2, int n0, int n1,
                       int n2, int K, int mode, int Npacked, int hd, hipStream_t st) {
  const long long total = (long long)(Npacked / 16) * (K / Mfma<T>::KSTEP) * 64;
  const int threads = 256;
  long long blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_kernel<T>, dim3((unsigned)blocks), dim3(threads), 0, st, (u32x4_t*)dst,
                     (const T*)s0, (const T*)s1, (const T*)s2, n0, n1, n2, K, mode, hd, total);
  return hipGetLastError();
}
template hipError_t launch_pack<float>(void*, const void*, const void*, const void*, int, int, int,
                                       int, int, int, int, hipStream_t);
template hipError_t launch_pack<bf16_t>(void*, const void*, const void*, const void*, int, int, int,
                                        int, int, int, int, hipStream_t);

#ifndef DEX_GEMM_NB
#define DEX_GEMM_NB 1
#endif
template <typename T, int NB, int EPI>
static hipError_t launch_gemm_mb(const GemmArgs& a, int mb, hipStream_t st) {
  dim3 grid(a.N / (16 * NB), a.ngroups);
  switch (mb) {
    case 1: hipLaunchKernelGGL((gemm_kernel<T, 1, NB, EPI>), grid, dim3(kGemmThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((gemm_kernel<T, 2, NB, EPI>), grid, dim3(kGemmThreads), 0, st, a); break;
    case 3: hipLaunchKernelGGL((gemm_kernel<T, 3, NB, EPI>), grid, dim3(kGemmThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((gemm_kernel<T, 4, NB, EPI>), grid, dim3(kGemmThreads), 0, st, a); break;
  }
  return hipGetLastError();
}

template <typename T, int EPI>
static hipError_t launch_gemm_nb(const GemmArgs& a, int mb, hipStream_t st) {
  if (DEX_GEMM_NB > 1 && (a.N / 16) % DEX_GEMM_NB == 0) return launch_gemm_mb<T, DEX_GEMM_NB, EPI>(a, mb, st);
  return launch_gemm_mb<T, 1, EPI>(a, mb, st);
}

template <int EPI, bool SPLIT, int WT, int NWV = 4>
static void wide_launch(const GemmArgs& a, hipStream_t st) {
  const int ncb = (a.N / 16 + NWV * WT - 1) / (NWV * WT);
  const dim3 grid(a.ngroups * ncb * (SPLIT ? kKSplit : 1));
  hipLaunchKernelGGL((gemm_wide_kernel<EPI, SPLIT, WT, NWV>), grid, dim3(NWV * 64), 0, st, a);
  if (SPLIT) {
    hipLaunchKernelGGL((gemm_split_reduce_kernel<EPI>), dim3(a.ngroups, a.N / 16), dim3(kWideThreads), 0, st, a);
  }
}

// Runs one grouped GEMM with bf16 weights on the wide kernel (every group has
// many rows). split: one block per k range, partial sums through args.split
// (groups' srow set, rows < kSplitRows), then their in-order sum and the
// epilogue.
// Launch shapes of the wide kernel: 4 tiles per wave, unsplit or split by k
// range, or 2 tiles per wave unsplit (twice the blocks for medium launches).
template <int EPI>
static void wide_launch_shape(const GemmArgs& a, int shape, hipStream_t st) {
  if (shape == WIDE_SPLIT) wide_launch<EPI, true, 4>(a, st);
  else if (shape == WIDE_T2) wide_launch<EPI, false, 2>(a, st);
  else if (shape == WIDE_W8) wide_launch<EPI, false, 4, 8>(a, st);
  else wide_launch<EPI, false, 4>(a, st);
}

hipError_t launch_gemm_wide(const GemmArgs& a, int epi, int shape, hipStream_t st) {
  switch (epi) {
    case EPI_QKV: wide_launch_shape<EPI_QKV>(a, shape, st); break;
    case EPI_RESID: wide_launch_shape<EPI_RESID>(a, shape, st); break;
    case EPI_SWIGLU: wide_launch_shape<EPI_SWIGLU>(a, shape, st); break;
    case EPI_ADAPT1: wide_launch_shape<EPI_ADAPT1>(a, shape, st); break;
    case EPI_ADAPT2: wide_launch_shape<EPI_ADAPT2>(a, shape, st); break;
    default: wide_launch_shape<EPI_HEAD>(a, shape, st); break;
  }
  return hipGetLastError();
}

// Runs one grouped GEMM; the MFMA row-block count is the largest group's.
template <typename T>
hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t st) {
  int mmax = 1;
  for (int i = 0; i < a.ngroups; ++i) mmax = a.g[i].m > mmax ? a.g[i].m : mmax;
  const int mb = (mmax + 15) / 16;
  switch (epi) {
    case EPI_QKV: return launch_gemm_nb<T, EPI_QKV>(a, mb, st);
    case EPI_RESID: return launch_gemm_nb<T, EPI_RESID>(a, mb, st);
    case EPI_SWIGLU: return launch_gemm_nb<T, EPI_SWIGLU>(a, mb, st);
    case EPI_ADAPT1: return launch_gemm_nb<T, EPI_ADAPT1>(a, mb, st);
    case EPI_ADAPT2: return launch_gemm_nb<T, EPI_ADAPT2>(a, mb, st);
    default: return launch_gemm_nb<T, EPI_HEAD>(a, mb, st);
  }
}
template hipError_t launch_gemm<float>(const GemmArgs&, int, hipStream_t);
template hipError_t launch_gemm<bf16_t>(const GemmArgs&, int, hipStream_t);

hipError_t launch_head_reduce(const float* part, int ntiles, int row0, int nrows, const RowInfo* rows, int P,
                              int* cand, float* margin, hipStream_t st) {
  if (nrows == 0) return hipSuccess;
  hipLaunchKernelGGL(head_reduce_kernel, dim3(nrows), dim3(256), 0, st, part, ntiles, row0, rows, P, cand, margin);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_embed(const void* E, const RowInfo* rows, int row0, int nrows, float* hidden, float* xn,
                        float* ssq, const float* g0, int d, hipStream_t st) {
  if (nrows == 0) return hipSuccess;
  hipLaunchKernelGGL(embed_kernel<T>, dim3(nrows), dim3(256), 0, st, (const T*)E, rows, row0, hidden, xn, ssq, g0, d);
  return hipGetLastError();
}
template hipError_t launch_embed<float>(const void*, const RowInfo*, int, int, float*, float*, float*, const float*,
                                        int, hipStream_t);
template hipError_t launch_embed<bf16_t>(const void*, const RowInfo*, int, int, float*, float*, float*, const float*,
                                         int, hipStream_t);

}  // namespace dex
