// Lattice attention of the lattice step.
//
// Every row is computed from that row's own inputs in a fixed order, so a node
// of the depth-position lattice and the same context decoded autoregressively
// produce identical bits.
#include <type_traits>

#include "common.h"

namespace dex {

// ----------------------------------------------------------------------------
// Lattice attention ("Depth Exploration for LLM Decoding", Section 3.2: the
// binary expansion lets ancestry, KV entries and attention masks be indexed
// consistently). A row attends to the committed cache [0, ncommit) and to the
// explore-buffer entries of its ancestors at positions ncommit.. (its own
// entry last). All rows of a work item share one sequence and layer.
//
// Products run on 16-bit MFMA in the cache's format (common.h). fp16 K/V
// (bfloat16 models): v_mfma_f32_16x16x32_f16 with the fp32 query and softmax
// weights split into an fp16 pair, k.q taken as k.q_hi + k.q_lo (and p.v the
// same way). bfloat16 (hi, lo) K/V (fp32 models): v_mfma_f32_16x16x32_bf16
// with both operands split, a.b taken as hi.hi + hi.lo + lo.hi.
// A work item is one MFMA tile of up to 16 units (row, query head) of one kv
// head. Scores come out transposed, S^T = K Q^T: lane (g, n) = (lane / 16,
// lane % 16) holds unit n's scores for keys 8g .. 8g+7 of a 32-key chunk, which
// is exactly the B operand of the value product O^T = V^T P^T. The K tile
// layout (see common.h) puts those keys in MFMA row order, the V planes are
// stored transposed, so every operand is one 16-byte load and each load
// instruction of the wave covers whole contiguous runs.
//
// Reduction order, a function of key positions only (so a lattice node and
// the same context decoded autoregressively agree bit for bit):
//   chunk       = 32 positions [32c, 32c + 32): scores by the MFMA chain over
//                 32-dim steps in order; m = max; p = 2^(s - m); l = sum of
//                 p (each lane's eight in key order, then lanes g^1, g^2 by
//                 butterfly); acc = V^T P^T by one MFMA chain;
//   super-chunk = kAttnSC chunks folded left to right (fold below);
//   span        = kAttnSpan super-chunks folded left to right (by a grouped
//                 block, or by attn_combine_kernel from super-chunk states);
//   row         = spans folded left to right by attn_combine_kernel.
// Queries arrive pre-multiplied by log2(e)/sqrt(hd).
//
// A chunk in which some row reads explore entries (positions it does not share
// with the tile's other rows; the host marks them as chunks xc0..xc1 of the
// item, at most two since a row has at most N explore keys) is computed once
// per row, with that row's keys gathered into the same operand layout and its
// query heads of the kv head as the MFMA columns; every other chunk is computed
// once for the whole tile with keys past a unit's limit masked. Both give a
// unit the same operand values in the same MFMA order, hence the same bits.
// The per-row chunks are latency-bound, so they run as extra blocks of the same
// launch, overlapping the bandwidth-bound shared chunks; the super-chunks that
// hold them are folded by the combine kernel.
// ----------------------------------------------------------------------------

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) {
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}
__device__ __forceinline__ f16x8_t as_f16x8(const u32x4_t& v) {
  f16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// acc += A B^T over one 32-element k step, operands split into (hi, lo).
__device__ __forceinline__ f32x4_t mma3(f32x4_t acc, const u32x4_t& ah, const u32x4_t& al, const u32x4_t& bh,
                                        const u32x4_t& bl) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah), as_bf16x8(bh), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ah), as_bf16x8(bl), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(al), as_bf16x8(bh), acc, 0, 0, 0);
  return acc;
}

// acc += A B^T over one 32-element k step in the format of KVP planes: A
// (the cached operand) fp16 and B split into an fp16 (hi, lo) pair (KVP = 1):
// A.B_hi, then A.B_lo; or both bfloat16 pairs (KVP = 2), mma3.
template <int KVP>
__device__ __forceinline__ f32x4_t mma_kv(f32x4_t acc, const u32x4_t& ah, const u32x4_t& al, const u32x4_t& bh,
                                          const u32x4_t& bl) {
  if constexpr (KVP == 1) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(ah), as_f16x8(bh), acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(ah), as_f16x8(bl), acc, 0, 0, 0);
  } else {
    return mma3(acc, ah, al, bh, bl);
  }
}

// Eight fp32 values as (hi, lo) pairs in the 16-bit format of KVP planes
// (SAT as for f2h2).
template <int KVP, bool SAT = true>
__device__ __forceinline__ void split8(const float* x, u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    unsigned h, l;
    split16<KVP, SAT>(x[2 * i], x[2 * i + 1], h, l);
    hi[i] = h;
    lo[i] = l;
  }
}

// 2^x by the hardware instruction (v_exp_f32): results below 2^-126 come out
// as zero rather than subnormal, which saves the range fix-up exp2f adds
// around it. Every softmax weight and fold factor takes this one path.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Fold partial (m, l, a) into state (M, L, A); both describe non-empty key sets.
template <int NA>
__device__ __forceinline__ void fold(float& M, float& L, float* A, float m, float l, const float* a) {
  const float Mn = fmaxf(M, m);
  const float al = exp2_hw(M - Mn), be = exp2_hw(m - Mn);
  L = fmaf(l, be, L * al);
#pragma unroll
  for (int k = 0; k < NA; ++k) A[k] = fmaf(a[k], be, A[k] * al);
  M = Mn;
}

// Bits 0 .. min(max(nv, 0), 8) - 1 set: the keys of a lane's eight that lie
// below its unit's limit (nv = limit - first key of the eight).
__device__ __forceinline__ unsigned key_bits(int nv) {
  nv = nv < 0 ? 0 : (nv > 8 ? 8 : nv);
  return (1u << nv) - 1u;
}

// One 32-key chunk for the tile. qsrc(s, hi, lo): this lane's query operand
// (unit n, dims 32s + 8g .. 32s + 8g + 7); ksrc(t, s, hi, lo): its K operand for
// row block t (0, 1) and 32-dim step s; vsrc(b, hi, lo): its V^T operand for
// output dims [16b, 16b + 16), as loaded; vpost(b, hi, lo) then fixes it up
// (masks, gathered values). The lo operands are read only with KVP = 2.
// valid8 bit i: key 8g + i counts for this lane's unit; `full` (the same in
// every lane): every key of the chunk counts for every unit of the tile, which
// skips the selects (same values). Out: acc[b][r] = the
// unit's unnormalised output at dim 16b + 4g + r, and the chunk's m and l
// (m = -inf when no key counts).
template <int HD, int KVP, typename QSrc, typename KSrc, typename VSrc, typename VPost>
__device__ __forceinline__ void chunk_partial(QSrc qsrc, KSrc ksrc, VSrc vsrc, VPost vpost, unsigned valid8, bool full,
                                              f32x4_t* acc, float& m, float& l) {
  constexpr int NS = HD / 32, NB = HD / 16;
  u32x4_t kh[2][NS], kl[2][NS], vh[NB], vl[NB];
  f32x4_t st[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    st[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4_t qh, ql;
      ksrc(t, s, kh[t][s], kl[t][s]);
      qsrc(s, qh, ql);
      st[t] = mma_kv<KVP>(st[t], kh[t][s], kl[t][s], qh, ql);
    }
  }
  // The chunk's max and softmax weights, in a masked and an unmasked copy
  // (a branch on `full`, not a select per key).
  float p[8], mx;
  auto weights = [&](auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    float sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = !MASKED || (valid8 >> i) & 1 ? st[i >> 2][i & 3] : -INFINITY;
    mx = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float msafe = mx == -INFINITY ? 0.f : mx;
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = !MASKED || (valid8 >> i) & 1 ? exp2_hw(sv[i] - msafe) : 0.f;
  };
  if (full) weights(std::false_type{});
  else weights(std::true_type{});
  float ls = p[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) ls += p[i];
  ls += __shfl_xor(ls, 16);
  ls += __shfl_xor(ls, 32);
  m = mx;
  l = ls;
  u32x4_t ph, pl;
  split8<KVP, false>(p, ph, pl);   // softmax weights lie in [0, 1]
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    vsrc(b, vh[b], vl[b]);
    vpost(b, vh[b], vl[b]);
    acc[b] = mma_kv<KVP>(f32x4_t{0.f, 0.f, 0.f, 0.f}, vh[b], vl[b], ph, pl);
  }
}

// V^T operand fix-up of the shared chunks: positions at or past vlim (the
// largest key limit of the tile) may hold stale or never-written values; their
// elements are zeroed so that p = 0 contributes exact zeros.
template <int KVP>
__device__ __forceinline__ void mask_v(u32x4_t& vh, u32x4_t& vl, int nv) {
  if (nv < 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned keep = (2 * i + 1 < nv ? 0xFFFF0000u : 0u) | (2 * i < nv ? 0xFFFFu : 0u);
      vh[i] &= keep;
      if constexpr (KVP == 2) vl[i] &= keep;
    }
  }
}

// Super-chunks per span: a row's super-chunk states are folded left to right
// within each span of kAttnSpan, and the span states left to right.
constexpr int kAttnSpan = 16;
constexpr int kSpanBlocks = 512;   // grouped blocks that fill the chip (two per CU)
constexpr int kSpreadBlocks = 4096;   // attn_kernel launches that spread their per-row blocks
// Super-chunks a single-item block of attn_kernel runs in turn (each one's
// state written as a block of its own would), so that its item, rows and
// query tile are read once for all of them.
#ifndef DEX_ATTN_SCPB
#define DEX_ATTN_SCPB 2
#endif
constexpr int kSingleSC = DEX_ATTN_SCPB;
// The same for a grouped block that runs super-chunks (not whole spans).
#ifndef DEX_GROUP_SCPB
#define DEX_GROUP_SCPB 2
#endif
constexpr int kGroupSC = DEX_GROUP_SCPB;

// Whether super-chunk sc of the item holds a per-row (explore) chunk.
__device__ __forceinline__ bool sc_mixed(const AttnItem& it, int sc) {
  return it.xc0 >= 0 && (sc == it.xc0 / kAttnSC || sc == it.xc1 / kAttnSC);
}

// Store the chunk partial of unit n held by lanes (g, n) to dst[hd + 2].
template <int HD>
__device__ __forceinline__ void store_partial(float* dst, const f32x4_t* acc, float m, float l, int g) {
#pragma unroll
  for (int b = 0; b < HD / 16; ++b) *(f32x4_t*)(dst + 16 * b + 4 * g) = acc[b];
  if (g == 0) {
    dst[HD] = m;
    dst[HD + 1] = l;
  }
}

// LDS of one attention block: the shared-chunk role's query tiles (up to
// MAXT) and chunk partials, or the per-row role's explore values.
template <int HD, int MAXT> struct AttnSmem {
  union {
    struct {
      alignas(16) float red[kAttnSC][kAttnUnits][HD + 4];   // chunk partials; rows 16-byte aligned
      bf16_t qsh[MAXT][2][kAttnUnits][HD + 8];   // queries as (hi, lo), rows padded by 16 bytes
    } m;
    bf16_t ev[kAttnSC][kMaxN][2 * HD];      // per wave: the V planes of the unit's explore entries
  };
};

// Queries of a tile of `units` units from row row0 on, split into (hi, lo),
// into LDS rows padded by 16 bytes. Threads t0, t0 + step, ... share the work.
template <int HD, int KVP>
__device__ __forceinline__ void load_q_tile(bf16_t (*dst)[kAttnUnits][HD + 8], int row0, int units, int h,
                                            const float* __restrict__ q, const ModelDims& D, int t0, int step) {
  const int rep = D.nq / D.nkv;
  for (int t = t0; t < kAttnUnits * HD / 8; t += step) {
    const int u = t / (HD / 8), d8 = 8 * (t % (HD / 8));
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (u < units) {
      const float* qr = q + ((size_t)(row0 + u / rep) * D.nq + h * rep + u % rep) * HD + d8;
      const f32x4_t a = *(const f32x4_t*)qr, b = *(const f32x4_t*)(qr + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = a[i];
        x[4 + i] = b[i];
      }
    }
    u32x4_t hi, lo;
    split8<KVP>(x, hi, lo);
    *(u32x4_t*)&dst[0][u][d8] = hi;
    *(u32x4_t*)&dst[1][u][d8] = lo;
  }
}

// Per-row role: the block takes rows rbase .. rbase + kTailRows - 1 of the
// item, wave w rows rbase + w + kAttnSC r (r < kTailRowsPerWave). For each it
// computes chunk c (one of xc0, xc1) with that row's own keys, for all
// rep = nq / nkv query heads of kv head h at once (MFMA column n carries query
// head h rep + n; the others repeat a query and are not stored), into
// mix[row][qh][c - kAttnSC (xc0 / kAttnSC)]. A column's result depends only on
// its own query, so each unit gets the bits it gets in a shared tile. The rows
// of an item that reads explore keys are lattice rows of one sequence, which
// share ncommit = C: the chunk's committed keys and values are the same for all
// of them, so a wave loads those once and, per row, the row's explore keys, its
// query and its explore values (gathered into the wave's own LDS slice), all
// issued together so that a row waits for memory once.
template <int HD, int KVP>
__device__ void attn_unit_rows(AttnSmem<HD, 1>& sm, const AttnItem& it, int h, int c, int rbase,
                               const RowInfo* __restrict__ rows, const float* __restrict__ q,
                               const bf16_t* __restrict__ kvc, const bf16_t* __restrict__ exb,
                               float* __restrict__ mix, const ModelDims& D, int lam, int lattice) {
  constexpr int NB = HD / 16, NS = HD / 32, HP = HD + 4;
  const int rep = D.nq / D.nkv;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
  const int p0 = c * kKvTile;
  const int r0 = rbase + w;
  if (r0 >= it.nrows || c > it.xc1) return;
  const int ncu = rows[it.row0 + r0].ncommit;
  const size_t eslot = (size_t)D.S * D.nkv * 2 * KVP * HD;  // 16-bit values between node slots
  const bf16_t* eb = exb + ex_base(D, it.seq, 0, lam, h);
  bf16_t (*ev)[2 * HD] = sm.ev[w];
  const int layer = layer_of(D, lattice, it.stage, lam);
  const bf16_t* tb = kvc + kv_head_base(D, it.seq, layer, h) + (size_t)c * 64 * KVP * HD;
  // The committed operands of the chunk (zero at and past ncu).
  u32x4_t kh[2][NS], kl[2][NS], vh[NB], vl[NB];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int p = p0 + 8 * (n >> 2) + 4 * t + (n & 3);
      kh[t][s] = kl[t][s] = u32x4_t{0u, 0u, 0u, 0u};
      if (p < ncu) {
        const bf16_t* kp = tb + (4 * s + g) * 256 + (16 * t + n) * 8;
        kh[t][s] = *(const u32x4_t*)kp;
        if constexpr (KVP == 2) kl[t][s] = *(const u32x4_t*)(kp + 32 * HD);
      }
    }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int pb = p0 + 8 * g, dd = 16 * b + n;
    vh[b] = vl[b] = u32x4_t{0u, 0u, 0u, 0u};
    if (pb < ncu) {
      const bf16_t* vp = tb + 32 * KVP * HD + dd * 32 + 8 * g;
      vh[b] = *(const u32x4_t*)vp;
      if constexpr (KVP == 2) vl[b] = *(const u32x4_t*)(vp + 32 * HD);
    }
  }
  for (int r = 0; r < kTailRowsPerWave; ++r) {
    const int rr = r0 + kAttnSC * r;
    if (rr >= it.nrows) break;
    const int row = it.row0 + rr;
    const RowInfo& Ru = rows[row];
    const int limu = ncu + Ru.n_anc;
    if (p0 >= limu) continue;   // no key of this row in chunk c
    // K of this row: the lanes of positions from ncu on take its explore
    // entries, zero past its limit (the committed lanes keep their operand)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int p = p0 + 8 * (n >> 2) + 4 * t + (n & 3);
        if (p >= ncu) {
          kh[t][s] = kl[t][s] = u32x4_t{0u, 0u, 0u, 0u};
          if (p < limu) {
            const bf16_t* kp = eb + Ru.anc[p - ncu] * eslot + 8 * (4 * s + g);
            kh[t][s] = *(const u32x4_t*)kp;
            if constexpr (KVP == 2) kl[t][s] = *(const u32x4_t*)(kp + HD);
          }
        }
      }
    const float* qr = q + ((size_t)row * D.nq + h * rep + min(n, rep - 1)) * HD;
    f32x4_t qa[NS][2];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qa[s][0] = *(const f32x4_t*)(qr + 32 * s + 8 * g);
      qa[s][1] = *(const f32x4_t*)(qr + 32 * s + 8 * g + 4);
    }
    // the V planes (KVP HD values) of each explore entry, 16 bytes a lane; the
    // slice belongs to this wave, whose LDS accesses take effect in order
    constexpr int PIECES = KVP * HD / 8;
    for (int t = lane; t < (limu - ncu) * PIECES; t += 64) {
      const int j = t / PIECES, o = 8 * (t % PIECES);
      *(u32x4_t*)&ev[j][o] = *(const u32x4_t*)(eb + Ru.anc[j] * eslot + KVP * HD + o);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    auto qsrc = [&](int s, u32x4_t& qh, u32x4_t& ql) {
      const float x[8] = {qa[s][0][0], qa[s][0][1], qa[s][0][2], qa[s][0][3],
                          qa[s][1][0], qa[s][1][1], qa[s][1][2], qa[s][1][3]};
      split8<KVP>(x, qh, ql);
    };
    // V of this row: positions from ncu on take its explore entry's value,
    // or 0 past its limit (every such element is rewritten for each row)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int pb = p0 + 8 * g, dd = 16 * b + n;
      if (pb + 7 < ncu) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int p = pb + i;
        if (p < ncu) continue;
        const unsigned hv = p < limu ? ev[p - ncu][dd] : 0u;
        const int sh = 16 * (i & 1);
        const unsigned keep = ~(0xFFFFu << sh);
        vh[b][i >> 1] = (vh[b][i >> 1] & keep) | (hv << sh);
        if constexpr (KVP == 2) {
          const unsigned lv = p < limu ? ev[p - ncu][HD + dd] : 0u;
          vl[b][i >> 1] = (vl[b][i >> 1] & keep) | (lv << sh);
        }
      }
    }
    auto ksrc = [&](int t, int s, u32x4_t& a, u32x4_t& b) {
      a = kh[t][s];
      b = kl[t][s];
    };
    auto vsrc = [&](int b, u32x4_t& a, u32x4_t& bb) {
      a = vh[b];
      bb = vl[b];
    };
    auto vpost = [&](int, u32x4_t&, u32x4_t&) {};
    const unsigned valid8 = key_bits(limu - (p0 + 8 * g));
    f32x4_t acc[NB];
    float m, l;
    chunk_partial<HD, KVP>(qsrc, ksrc, vsrc, vpost, valid8, p0 + kKvTile <= limu, acc, m, l);
    if (n < rep)
      store_partial<HD>(mix + (((size_t)row * D.nq + h * rep + n) * kMixSlots + c - kAttnSC * (it.xc0 / kAttnSC)) * HP,
                        acc, m, l, g);
    // the next row's gather writes the slice only after this row's reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Shared role over super-chunks sc0 .. sc1 - 1, in order: for each, wave w
// takes chunk kAttnSC * sc + w for the `count` unit tiles (items first,
// first + 1, ...) of one sequence and stage, loading its K/V once for all of
// them. Per tile, in a super-chunk without per-row chunks the block folds the
// chunks per unit into the super-chunk state (acc[hd], m, l); in one with them,
// the tile's chunks go to the mix slots for the combine kernel to fold. SPAN
// false: each super-chunk's state written to part[row][qh][sc]. SPAN true:
// the super-chunks of span `span` (kAttnSpan of them from sc0 = kAttnSpan
// span); the fold threads fold the states into the span state in registers
// (the first as it is, each later one that holds keys of the unit by the fold)
// and write it to part[row][qh][span]. Super-chunks with per-row chunks come
// last in a row's keys, so the span state covers the ones before them.
template <int HD, int MAXT, bool SPAN, int KVP>
__device__ void attn_shared_chunks(AttnSmem<HD, MAXT>& sm, const AttnItem* __restrict__ items, int first, int count,
                                   int h, int sc0, int sc1, int span, const RowInfo* __restrict__ rows,
                                   const float* __restrict__ q, const bf16_t* __restrict__ kvc,
                                   float* __restrict__ mix, float* __restrict__ part, const ModelDims& D, int lam,
                                   int lattice, int nsc_max) {
  constexpr int NB = HD / 16, NS = HD / 32, HP = HD + 4;
  auto& red = sm.m.red;
  const int rep = D.nq / D.nkv;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, g = lane >> 4,
            n = lane & 15;
  const AttnItem it0 = items[first];   // the tiles share sequence, stage and explore chunks
  const int layer = layer_of(D, lattice, it0.stage, lam);
  // Every tile's rows and key limits up front: lane n's unit (lim) and fold
  // thread fu's unit (flim). Loads of one kind are issued together.
  const int fu = threadIdx.x >> 4, fs = threadIdx.x & 15;
  int row0[MAXT], units[MAXT], lim[MAXT], flim[MAXT];
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    row0[t] = t < count ? items[first + t].row0 : 0;
    units[t] = t < count ? items[first + t].nrows * rep : 0;
  }
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    lim[t] = 0;
    flim[t] = 0;
    if (n < units[t]) {
      const RowInfo& R = rows[row0[t] + n / rep];
      lim[t] = R.ncommit + R.n_anc;
    }
    if (fu < units[t]) {
      const RowInfo& R = rows[row0[t] + fu / rep];
      flim[t] = R.ncommit + R.n_anc;
    }
  }
#pragma unroll
  for (int t = 0; t < MAXT; ++t)
    if (t < count) load_q_tile<HD, KVP>(sm.m.qsh[t], row0[t], units[t], h, q, D, threadIdx.x, 64 * kAttnSC);
  // Positions past every unit's limit may hold stale or never-written values:
  // their V elements are zeroed so that p = 0 contributes exact zeros. (Below
  // that limit every position holds a written key, so a unit with a smaller
  // limit gets exact zeros there as well.)
  int vlim = 0;
#pragma unroll
  for (int t = 0; t < MAXT; ++t) vlim = max(vlim, lim[t]);
  for (int off = 32; off >= 1; off >>= 1) vlim = max(vlim, __shfl_xor(vlim, off));
  vlim = __builtin_amdgcn_readfirstlane(vlim);   // the same in every lane
  // the smallest limit of each tile's units (the same in every lane)
  int tmin[MAXT];
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    int v = n < units[t] ? lim[t] : 0x7fffffff;
    for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off));
    tmin[t] = __builtin_amdgcn_readfirstlane(v);
  }
  __syncthreads();

  // Span state of fold thread fu's unit per tile (elements 4 fs + 64 q + e).
  constexpr int NA = HD / 16, NQ = NA / 4;
  float PM[MAXT], PL[MAXT], PA[MAXT][NA];
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    PM[t] = PL[t] = 0.f;
#pragma unroll
    for (int e = 0; e < NA; ++e) PA[t][e] = 0.f;
  }

  for (int sc = sc0; sc < sc1; ++sc) {
  const int c = sc * kAttnSC + w, p0 = c * kKvTile;
  const bool unit_chunk = it0.xc0 >= 0 && c >= it0.xc0 && c <= it0.xc1;
  const bool to_mix = sc_mixed(it0, sc);
  const bool work = !unit_chunk && p0 < vlim;

  // The chunk's K and V operands, every load issued before the first use.
  const bf16_t* tb = kvc + kv_head_base(D, it0.seq, layer, h) + (size_t)c * 64 * KVP * HD;
  u32x4_t kh[2][NS], kl[2][NS], vh[NB], vl[NB];
  if (work) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16_t* kp = tb + (4 * s + g) * 256 + (16 * t + n) * 8;
        kh[t][s] = *(const u32x4_t*)kp;
        if constexpr (KVP == 2) kl[t][s] = *(const u32x4_t*)(kp + 32 * HD);
      }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const bf16_t* vp = tb + 32 * KVP * HD + (16 * b + n) * 32 + 8 * g;
      vh[b] = *(const u32x4_t*)vp;
      if constexpr (KVP == 2) vl[b] = *(const u32x4_t*)(vp + 32 * HD);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (p0 + kKvTile > vlim)   // only a chunk that reaches past every limit needs the V mask
#pragma unroll
      for (int b = 0; b < NB; ++b) mask_v<KVP>(vh[b], vl[b], vlim - (p0 + 8 * g));
  }

#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    if (t >= count) break;
    if (work) {
      auto qsrc = [&](int s, u32x4_t& qh, u32x4_t& ql) {
        qh = *(const u32x4_t*)&sm.m.qsh[t][0][n][32 * s + 8 * g];
        ql = *(const u32x4_t*)&sm.m.qsh[t][1][n][32 * s + 8 * g];
      };
      auto ksrc = [&](int tt, int s, u32x4_t& a, u32x4_t& b) {
        a = kh[tt][s];
        b = kl[tt][s];
      };
      auto vsrc = [&](int b, u32x4_t& a, u32x4_t& bb) {
        a = vh[b];
        bb = vl[b];
      };
      auto vpost = [&](int, u32x4_t&, u32x4_t&) {};
      const unsigned valid8 = key_bits(lim[t] - (p0 + 8 * g));
      f32x4_t acc[NB];
      float m, l;
      chunk_partial<HD, KVP>(qsrc, ksrc, vsrc, vpost, valid8, p0 + kKvTile <= tmin[t], acc, m, l);
      if (n < units[t] && p0 < lim[t]) {
        if (to_mix) {
          const int row = row0[t] + n / rep, qhd = h * rep + n % rep;
          store_partial<HD>(mix + (((size_t)row * D.nq + qhd) * kMixSlots + c - kAttnSC * (it0.xc0 / kAttnSC)) * HP,
                            acc, m, l, g);
        } else {
          float* rd = red[w][n];
#pragma unroll
          for (int b = 0; b < NB; ++b) *(f32x4_t*)(rd + 16 * b + 4 * g) = acc[b];
          if (g == 0) {
            rd[HD] = m;
            rd[HD + 1] = l;
          }
        }
      }
    }
    if (to_mix) continue;
    __syncthreads();

    // Fold the super-chunk's chunks per unit: thread (unit, fs) takes the
    // element quads 4 fs + 64 q (the fold is element-wise, so the split does
    // not change any bits), which keeps a wave's 16-byte LDS reads on distinct
    // banks.
    if (fu < units[t]) {
      const int row = row0[t] + fu / rep, qhd = h * rep + fu % rep;
      const int cb = sc * kAttnSC;
      if (cb * kKvTile < flim[t]) {
        float M = red[0][fu][HD], L = red[0][fu][HD + 1], A[NA];
#pragma unroll
        for (int q4 = 0; q4 < NQ; ++q4) {
          const f32x4_t v = *(const f32x4_t*)&red[0][fu][4 * fs + 64 * q4];
#pragma unroll
          for (int e = 0; e < 4; ++e) A[4 * q4 + e] = v[e];
        }
        for (int ww = 1; ww < kAttnSC && (cb + ww) * kKvTile < flim[t]; ++ww) {
          float a[NA];
#pragma unroll
          for (int q4 = 0; q4 < NQ; ++q4) {
            const f32x4_t v = *(const f32x4_t*)&red[ww][fu][4 * fs + 64 * q4];
#pragma unroll
            for (int e = 0; e < 4; ++e) a[4 * q4 + e] = v[e];
          }
          fold<NA>(M, L, A, red[ww][fu][HD], red[ww][fu][HD + 1], a);
        }
        if constexpr (SPAN) {
          // Selects, not branches, keep the span state in one set of registers.
          float Mf = PM[t], Lf = PL[t], Af[NA];
#pragma unroll
          for (int e = 0; e < NA; ++e) Af[e] = PA[t][e];
          fold<NA>(Mf, Lf, Af, M, L, A);
          const bool firstsc = sc == sc0;
          PM[t] = firstsc ? M : Mf;
          PL[t] = firstsc ? L : Lf;
#pragma unroll
          for (int e = 0; e < NA; ++e) PA[t][e] = firstsc ? A[e] : Af[e];
        } else {
          float* dst = part + (((size_t)row * D.nq + qhd) * nsc_max + sc) * HP;
#pragma unroll
          for (int q4 = 0; q4 < NQ; ++q4)
            *(f32x4_t*)(dst + 4 * fs + 64 * q4) = f32x4_t{A[4 * q4], A[4 * q4 + 1], A[4 * q4 + 2], A[4 * q4 + 3]};
          if (fs == 0) {
            dst[HD] = M;
            dst[HD + 1] = L;
          }
        }
      }
    }
    if (SPAN || t + 1 < count || sc + 1 < sc1) __syncthreads();   // the fold has read red before it is written again
  }
  }

  if constexpr (SPAN) {
    if (!sc_mixed(it0, sc0)) {
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
        if (t >= count) break;
        if (fu < units[t] && sc0 * kAttnSCKeys < flim[t]) {
          const int row = row0[t] + fu / rep, qhd = h * rep + fu % rep;
          float* dst = part + (((size_t)row * D.nq + qhd) * nsc_max + span) * HP;
#pragma unroll
          for (int q4 = 0; q4 < NQ; ++q4)
            *(f32x4_t*)(dst + 4 * fs + 64 * q4) =
                f32x4_t{PA[t][4 * q4], PA[t][4 * q4 + 1], PA[t][4 * q4 + 2], PA[t][4 * q4 + 3]};
          if (fs == 0) {
            dst[HD] = PM[t];
            dst[HD + 1] = PL[t];
          }
        }
      }
    }
  }
}

// One launch, block = kAttnSC waves. Logical blocks [0, ntail): per-row
// chunks, index = (e * nkv + h) * nj + j for tail entry tlist[e] = 4 item +
// q -> chunk xc0 + j, rows kTailRows q .. kTailRows (q + 1) - 1 (nj: the most
// chunks with explore keys in one item). Logical blocks from ntail: index = (k * nkv + h)
// * nscb + i, shared role over super-chunks kSingleSC i .. kSingleSC (i + 1) - 1
// of item list[k], the k-th of the items that form a group of their own
// (nscb: the widest item's super-chunks in blocks of kSingleSC).
template <int HD, int KVP>
__global__ __launch_bounds__(64 * kAttnSC) void attn_kernel(
    const AttnItem* __restrict__ items, const int* __restrict__ list, const RowInfo* __restrict__ rows,
    const float* __restrict__ q, const bf16_t* __restrict__ kvc, const bf16_t* __restrict__ exb,
    float* __restrict__ mix, float* __restrict__ part, ModelDims D, int lam, int lattice, int nsc_max, int ntail,
    const int* __restrict__ tlist, int nj, int nscb) {
  __shared__ AttnSmem<HD, 1> sm;
  // Hardware block x -> logical index b. In a launch of kSpreadBlocks blocks
  // or more the per-row blocks are spread evenly among the shared ones (x
  // takes per-row block floor(x ntail / grid) when that count steps at x), so
  // that latency-bound and streaming blocks share the CUs for the whole
  // launch; a smaller launch, a few blocks per CU, keeps the per-row blocks
  // first, so its longest blocks start first.
  const int total = gridDim.x;
  const int t0 = (int)((long long)blockIdx.x * ntail / total);
  const int t1 = (int)((long long)(blockIdx.x + 1) * ntail / total);
  int b = total < kSpreadBlocks ? (int)blockIdx.x : (t1 > t0 ? t0 : ntail + (blockIdx.x - t0));
  if (b < ntail) {
    const int j = b % nj;
    b /= nj;
    const int e = tlist[b / D.nkv];
    const AttnItem it = items[e >> 2];
    if (it.xc0 < 0 || (lattice && lam >= stage_len(D, it.stage))) return;
    attn_unit_rows<HD, KVP>(sm, it, b % D.nkv, it.xc0 + j, kTailRows * (e & 3), rows, q, kvc, exb, mix, D, lam,
                            lattice);
    return;
  }
  b -= ntail;
  const int sc0 = (b % nscb) * kSingleSC;
  b /= nscb;
  const int ii = list[b / D.nkv];
  const AttnItem it = items[ii];
  if (it.lead != 1 || sc0 * kAttnSCKeys >= it.max_keys || (lattice && lam >= stage_len(D, it.stage))) return;
  const int sc1 = min(sc0 + kSingleSC, (it.max_keys + kAttnSCKeys - 1) / kAttnSCKeys);
  attn_shared_chunks<HD, 1, false, KVP>(sm, items, ii, 1, b % D.nkv, sc0, sc1, 0, rows, q, kvc, mix, part, D, lam,
                                        lattice, nsc_max);
}

// Groups of several items: the shared role over up to kAttnGroup tiles. SPAN:
// block (group, h, span) runs the super-chunks of one span and writes span
// states; otherwise block (group, h, b) runs super-chunks kGroupSC b ..
// kGroupSC (b + 1) - 1 and writes each one's state, and the combine kernel
// folds those into span states in the same order (the launch picks SPAN when
// it has blocks enough to fill the chip).
// 1-D grid, logical index (xcd_block) = (k * nkv + h) * nb + b for the group
// led by item list[k]: each XCD walks consecutive super-chunks or spans of one
// (group, kv head), so the blocks in flight stream a few contiguous K/V
// regions. (The single-item launch keeps the hardware order: there the remap
// made the per-row blocks pile up on the first XCDs.)
template <int HD, bool SPAN, int KVP>
__global__ __launch_bounds__(64 * kAttnSC) __attribute__((amdgpu_waves_per_eu(2))) void attn_group_kernel(
    const AttnItem* __restrict__ items, const int* __restrict__ list, const RowInfo* __restrict__ rows,
    const float* __restrict__ q, const bf16_t* __restrict__ kvc, float* __restrict__ mix, float* __restrict__ part,
    ModelDims D, int lam, int lattice, int nsc_max, int nb) {
  __shared__ AttnSmem<HD, kAttnGroup> sm;
  const int lb = xcd_block(blockIdx.x, gridDim.x);
  const int bi = lb % nb, ih = lb / nb;
  const int ii = list[ih / D.nkv], h = ih % D.nkv;
  const AttnItem it = items[ii];
  const int nsc = (it.max_keys + kAttnSCKeys - 1) / kAttnSCKeys;
  const int sc0 = SPAN ? bi * kAttnSpan : bi * kGroupSC, sc1 = min(sc0 + (SPAN ? kAttnSpan : kGroupSC), nsc);
  if (it.lead < 2 || sc0 >= nsc || (lattice && lam >= stage_len(D, it.stage))) return;
  attn_shared_chunks<HD, kAttnGroup, SPAN, KVP>(sm, items, ii, it.lead, h, sc0, sc1, bi, rows, q, kvc, mix, part, D, lam,
                                           lattice, nsc_max);
}

// Fold the states of each (row, query head) of an item and normalise: within
// each span of kAttnSpan super-chunks the super-chunk states left to right,
// then the span states left to right. An item of a group (lead != 1) has its
// span states from attn_group_kernel when it ran spans (span_states),
// covering each span's super-chunks up to the first one with per-row chunks;
// otherwise an item has one state per super-chunk (from attn_kernel or
// attn_group_kernel), folded here the same way. Super-chunks with
// per-row chunks (the last ones of a row) are folded here from their chunk
// partials, exactly as attn_kernel folds the others, and join their span's
// fold in order. grid = (items, kv heads, kAttnUnits / 4), block = 4 waves,
// one unit per wave (the units of an item are independent, and each one's
// folds are a chain of dependent loads, so they run side by side).
template <int HD>
__global__ void attn_combine_kernel(const AttnItem* __restrict__ items, const RowInfo* __restrict__ rows,
                                    const float* __restrict__ mix, const float* __restrict__ part,
                                    float* __restrict__ out, ModelDims D, int lam, int lattice, int nsc_max,
                                    int span_states) {
  constexpr int HS = HD / 64, HP = HD + 4;
  const AttnItem it = items[blockIdx.x];
  if (lattice && lam >= stage_len(D, it.stage)) return;
  const int nq = D.nq, h = blockIdx.y, rep = nq / D.nkv, units = it.nrows * rep;
  const bool grouped = span_states && it.lead != 1;
  const int lane = threadIdx.x & 63;
  {
    const int u = blockIdx.z * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (u >= units) return;
    const int row = it.row0 + u / rep, qh = h * rep + u % rep;
    const RowInfo& R = rows[row];
    const int lim = R.ncommit + R.n_anc;
    const int nsc = (lim + kAttnSCKeys - 1) / kAttnSCKeys;
    const float* base = part + ((size_t)row * nq + qh) * nsc_max * HP;
    const float* mbase = mix + ((size_t)row * nq + qh) * kMixSlots * HP;
    float M = 0.f, L = 0.f, A[HS];
    for (int k = 0; k * kAttnSpan < nsc; ++k) {
      const int lo = k * kAttnSpan, hi = min(lo + kAttnSpan, nsc);
      float ms = 0.f, ls = 0.f, as[HS];
      bool have = false;
      // Folds state (m, l, a) into the span state.
      auto join = [&](float m, float l, const float* a) {
        if (have) {
          fold<HS>(ms, ls, as, m, l, a);
        } else {
          ms = m;
          ls = l;
#pragma unroll
          for (int e = 0; e < HS; ++e) as[e] = a[e];
          have = true;
        }
      };
      if (grouped) {
        if (!sc_mixed(it, lo)) {
          const float* pc = base + k * HP;
          float a[HS];
#pragma unroll
          for (int e = 0; e < HS; ++e) a[e] = pc[lane * HS + e];
          join(pc[HD], pc[HD + 1], a);
        }
      } else {
        // The super-chunk states up to the first mixed one, read four at a
        // time ahead of their (in-order) folds.
        int end = lo;
        while (end < hi && !sc_mixed(it, end)) ++end;
        int sc = lo;
        for (; sc + 4 <= end; sc += 4) {
          float a4[4][HS], m4[4], l4[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float* pc = base + (sc + j) * HP;
#pragma unroll
            for (int e = 0; e < HS; ++e) a4[j][e] = pc[lane * HS + e];
            m4[j] = pc[HD];
            l4[j] = pc[HD + 1];
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) join(m4[j], l4[j], a4[j]);
        }
        for (; sc < end; ++sc) {
          const float* pc = base + sc * HP;
          float a[HS];
#pragma unroll
          for (int e = 0; e < HS; ++e) a[e] = pc[lane * HS + e];
          join(pc[HD], pc[HD + 1], a);
        }
      }
      for (int sc = lo; sc < hi; ++sc) {
        if (!sc_mixed(it, sc)) continue;
        const int cb = sc * kAttnSC;
        const float* pc = mbase + (cb - kAttnSC * (it.xc0 / kAttnSC)) * HP;
        float mm = pc[HD], lm = pc[HD + 1], am[HS];
#pragma unroll
        for (int e = 0; e < HS; ++e) am[e] = pc[lane * HS + e];
        for (int ww = 1; ww < kAttnSC && (cb + ww) * kKvTile < lim; ++ww) {
          const float* pw = pc + ww * HP;
          float a[HS];
#pragma unroll
          for (int e = 0; e < HS; ++e) a[e] = pw[lane * HS + e];
          fold<HS>(mm, lm, am, pw[HD], pw[HD + 1], a);
        }
        join(mm, lm, am);
      }
      if (k == 0) {
        M = ms;
        L = ls;
#pragma unroll
        for (int e = 0; e < HS; ++e) A[e] = as[e];
      } else {
        fold<HS>(M, L, A, ms, ls, as);
      }
    }
    const float inv = 1.0f / L;
    float* dst = out + ((size_t)row * nq + qh) * HD;
#pragma unroll
    for (int e = 0; e < HS; ++e) dst[lane * HS + e] = A[e] * inv;
  }
}

// ----------------------------------------------------------------------------
// Host launcher
// ----------------------------------------------------------------------------

// list: the nsingle items that form a group of their own, then the ngroups
// items that lead a group of several, then ntails entries 4 item + q of the
// runs of kTailRows rows of items whose rows read explore keys (0 when none
// do).
// umax: most units of an item whose rows
// read explore-buffer keys (lattice rows), 0 when no row does; nj: the most
// chunks holding explore keys in one item (xc1 - xc0 + 1, at most 2). span:
// grouped blocks run whole spans whatever their count.
template <int HD, int KVP>
static hipError_t launch_attention_t(const AttnItem* items, int nitems, const int* list, int nsingle, int ngroups,
                                     int ntails, const RowInfo* rows, const float* q, const bf16_t* kvc,
                                     const bf16_t* exb, float* mix, float* part, float* out, const ModelDims& D,
                                     int lam, int lattice, int nsc_max, int nsc, int nj, bool span, hipStream_t st) {
  const int ntail = ntails * D.nkv * nj;
  const int nscb = (nsc + kSingleSC - 1) / kSingleSC;
  const dim3 grid(ntail + nsingle * D.nkv * nscb);
  hipError_t e = hipSuccess;
  if (grid.x > 0) {
    hipLaunchKernelGGL((attn_kernel<HD, KVP>), grid, dim3(64 * kAttnSC), 0, st, items, list, rows, q, kvc, exb, mix,
                       part, D, lam, lattice, nsc_max, ntail, list + nsingle + ngroups, nj, nscb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // Grouped blocks run whole spans when that still gives the chip a block for
  // every slot (two per CU), else one super-chunk each.
  const int nspan = (nsc + kAttnSpan - 1) / kAttnSpan;
  const int span_states = ngroups > 0 && (span || ngroups * D.nkv * nspan >= kSpanBlocks);
  if (ngroups > 0 && nsc > 0) {
    const int nb = span_states ? nspan : (nsc + kGroupSC - 1) / kGroupSC;
    const dim3 ggrid(ngroups * D.nkv * nb);
    if (span_states)
      hipLaunchKernelGGL((attn_group_kernel<HD, true, KVP>), ggrid, dim3(64 * kAttnSC), 0, st, items,
                         list + nsingle, rows, q, kvc, mix, part, D, lam, lattice, nsc_max, nb);
    else
      hipLaunchKernelGGL((attn_group_kernel<HD, false, KVP>), ggrid, dim3(64 * kAttnSC), 0, st, items,
                         list + nsingle, rows, q, kvc, mix, part, D, lam, lattice, nsc_max, nb);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 cgrid(nitems, D.nkv, kAttnUnits / 4);
  hipLaunchKernelGGL((attn_combine_kernel<HD>), cgrid, dim3(256), 0, st, items, rows, mix, part, out, D, lam,
                     lattice, nsc_max, span_states);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnItem* items, int nitems, const int* list, int nsingle, int ngroups, int ntails,
                            const RowInfo* rows, int nrows, const float* q, const bf16_t* kvc, const bf16_t* exb,
                            float* mix, float* part, float* out, const ModelDims& D, int lam, int lattice, int nsc_max,
                            int max_keys, int umax, int nj, bool span, hipStream_t st) {
  (void)nrows;
  if (nitems == 0) return hipSuccess;
  const int nsc = (max_keys + kAttnSCKeys - 1) / kAttnSCKeys;
  if (nsc > nsc_max || umax > kAttnUnits || nsingle < 0 || ngroups < 0 || nsingle + ngroups > nitems || nj < 0 ||
      nj > 2 || ntails < 0 || ntails > 4 * nitems || (ntails > 0 && nj == 0) || (D.hd != 64 && D.hd != 128) ||
      (D.kvp != 1 && D.kvp != 2))
    return hipErrorInvalidValue;
  auto go = [&](auto hd, auto kvp) {
    return launch_attention_t<decltype(hd)::value, decltype(kvp)::value>(
        items, nitems, list, nsingle, ngroups, ntails, rows, q, kvc, exb, mix, part, out, D, lam, lattice, nsc_max,
        nsc, nj, span, st);
  };
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  using K1 = std::integral_constant<int, 1>;
  using K2 = std::integral_constant<int, 2>;
  if (D.hd == 128) return D.kvp == 1 ? go(I128{}, K1{}) : go(I128{}, K2{});
  return D.kvp == 1 ? go(I64{}, K1{}) : go(I64{}, K2{});
}

}  // namespace dex
