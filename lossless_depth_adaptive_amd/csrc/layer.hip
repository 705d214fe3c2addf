// Lattice attention of the lattice step.
//
// Every row is computed from that row's own inputs in a fixed order, so a node
// of the depth-position lattice and the same context decoded autoregressively
// produce identical bits.
#include "common.h"

namespace dex {

// ----------------------------------------------------------------------------
// Lattice attention ("Depth Exploration for LLM Decoding", Section 3.2: the
// binary expansion lets ancestry, KV entries and attention masks be indexed
// consistently). A row attends to the committed cache [0, ncommit) and to the
// explore-buffer entries of its ancestors at positions ncommit.. (its own
// entry last). All rows of a work item share one sequence and layer. K and V
// are fp32.
//
// Reduction order, a function of key positions only (so a lattice node and
// the same context decoded autoregressively agree bit for bit). With
// HS = hd/64 lane groups per key and TK = 64/HS keys per tile:
//   tile  = TK absolute positions [TK t, TK t + TK): lane group g of key j
//           forms the partial dot product over dims [64g, 64g+64) with four
//           interleaved sums added as (s0+s1)+(s2+s3), the groups then added
//           in order; m = max; p_j = 2^(s_j - m); l = xor-butterfly sum of p_j;
//           acc = sum_j p_j v_j in j order (even and odd j in two chains);
//   chunk = 8 tiles, merged in tile order;
//   row   = chunks merged in chunk order by attn_combine_kernel.
// Queries arrive pre-multiplied by log2(e)/sqrt(hd).
//
// grid = (items, kv heads, chunks), block = 512: wave w owns tile 8c+w. The
// wave loads its committed K rows and V columns into registers once and reuses
// them for every (row, query head) unit of the item; explore entries are read
// from the node slots directly.
// ----------------------------------------------------------------------------
constexpr int kAttnWaves = kAttnThreads / 64;

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
// Sum over each group of `width` lanes (xor butterfly, fixed order).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int off = width >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int HD> struct AttnGeom {
  static constexpr int HS = HD / 64;              // lane groups per key
  static constexpr int TK = 64 / HS;              // keys per tile
  static constexpr int CHUNK = kAttnWaves * TK;   // keys per chunk
};

// Partial q . k over 64 dims held as 16 float4 words.
template <typename Fetch>
__device__ __forceinline__ float dot64(const float* __restrict__ qv, Fetch fetch) {
  float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const f32x4_t k = fetch(i);
    s[0] = fmaf(qv[4 * i], k[0], s[0]);
    s[1] = fmaf(qv[4 * i + 1], k[1], s[1]);
    s[2] = fmaf(qv[4 * i + 2], k[2], s[2]);
    s[3] = fmaf(qv[4 * i + 3], k[3], s[3]);
  }
  return (s[0] + s[1]) + (s[2] + s[3]);
}

template <int HD>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(
    const AttnItem* __restrict__ items, const RowInfo* __restrict__ rows,
    const float* __restrict__ q, const float* __restrict__ kvc, const float* __restrict__ exb,
    float* __restrict__ part, ModelDims D, int lam, int smul, int nchunk) {
  using G = AttnGeom<HD>;
  constexpr int HS = G::HS, TK = G::TK, HP = HD + 2;
  __shared__ float qs[kAttnUnits][HD];
  __shared__ float red[kAttnWaves][kAttnUnits][HP];

  const AttnItem it = items[blockIdx.x];
  const int h = blockIdx.y, c = blockIdx.z;
  const int pb = c * G::CHUNK;
  if (pb >= it.max_keys) return;
  const int rep = D.nq / D.nkv;
  const int units = it.nrows * rep;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int seq = rows[it.row0].seq;
  int maxc = 0;
  for (int i = 0; i < it.nrows; ++i) maxc = max(maxc, rows[it.row0 + i].ncommit);

  for (int t = threadIdx.x; t < units * HD; t += kAttnThreads) {
    const int u = t / HD, dd = t - u * HD;
    const int row = it.row0 + u / rep, qh = h * rep + u % rep;
    qs[u][dd] = q[((size_t)row * D.nq + qh) * HD + dd];
  }

  const int layer = it.stage * smul + lam;
  const size_t cstride = (size_t)D.Cmax * HD;
  const float* kc = kvc + (((size_t)seq * D.L + layer) * 2 + 0) * D.nkv * cstride + h * cstride;
  const float* vc = kvc + (((size_t)seq * D.L + layer) * 2 + 1) * D.nkv * cstride + h * cstride;
  const size_t xs_slot = (size_t)D.S * 2 * D.nkv * HD;   // explore floats per node slot
  const float* xk = exb + (size_t)seq * D.P * xs_slot + (size_t)lam * 2 * D.nkv * HD + (size_t)h * HD;
  const float* xv = xk + (size_t)D.nkv * HD;

  // This wave's tile: key j = lane % TK, dims [64 g, 64 g + 64) with g = lane / TK.
  const int p0 = pb + TK * w;
  const int j = lane % TK, g = lane / TK;
  const int p = p0 + j;
  f32x4_t kw[16];
  float vw[TK][HS];
  const int nk = max(0, min(TK, maxc - p0));
  if (j < nk) {
    const f32x4_t* kr = (const f32x4_t*)(kc + (size_t)p * HD + 64 * g);
#pragma unroll
    for (int i = 0; i < 16; ++i) kw[i] = kr[i];
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) kw[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int jj = 0; jj < TK; ++jj)
#pragma unroll
    for (int e = 0; e < HS; ++e) vw[jj][e] = jj < nk ? vc[(size_t)(p0 + jj) * HD + lane * HS + e] : 0.f;
  __syncthreads();

  for (int u = 0; u < units; ++u) {
    const RowInfo& R = rows[it.row0 + u / rep];
    const int lim = R.ncommit + R.n_anc;
    float* rd = red[w][u];
    if (p0 >= lim) {
      if (lane == 0) {
        rd[HD] = -INFINITY;
        rd[HD + 1] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < HS; ++e) rd[lane * HS + e] = 0.f;
      continue;
    }
    const float* qv = qs[u] + 64 * g;
    float sp = 0.f;
    if (p < R.ncommit) {
      sp = dot64(qv, [&](int i) { return kw[i]; });
    } else if (p < lim) {
      const f32x4_t* xr = (const f32x4_t*)(xk + (size_t)R.anc[p - R.ncommit] * xs_slot + 64 * g);
      sp = dot64(qv, [&](int i) { return xr[i]; });
    }
    float s = sp;
    if (HS == 2) {
      const float other = __shfl_xor(sp, 32);
      s = g == 0 ? sp + other : other + sp;
    }
    if (p >= lim) s = -INFINITY;
    const float m = wave_max(s);
    const float pj = p < lim ? exp2f(s - m) : 0.f;
    const float l = group_sum(pj, TK);
    float a0[HS], a1[HS];
#pragma unroll
    for (int e = 0; e < HS; ++e) a0[e] = a1[e] = 0.f;
    const int nv = min(TK, lim - p0);
#pragma unroll
    for (int jj = 0; jj < TK; ++jj) {
      if (jj < nv) {
        const float pv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj));
        const int pp = p0 + jj;
        float v[HS];
        if (pp < R.ncommit) {
#pragma unroll
          for (int e = 0; e < HS; ++e) v[e] = vw[jj][e];
        } else {
          const float* xr = xv + (size_t)R.anc[pp - R.ncommit] * xs_slot + lane * HS;
#pragma unroll
          for (int e = 0; e < HS; ++e) v[e] = xr[e];
        }
#pragma unroll
        for (int e = 0; e < HS; ++e) {
          if (jj & 1) a1[e] = fmaf(pv, v[e], a1[e]);
          else a0[e] = fmaf(pv, v[e], a0[e]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < HS; ++e) rd[lane * HS + e] = a0[e] + a1[e];
    if (lane == 0) {
      rd[HD] = m;
      rd[HD + 1] = l;
    }
  }
  __syncthreads();
  // Merge the chunk's tiles in tile order; wave w takes units w, w+8, ...
  for (int u = w; u < units; u += kAttnWaves) {
    const int row = it.row0 + u / rep, qh = h * rep + u % rep;
    const RowInfo& R = rows[row];
    if (pb >= R.ncommit + R.n_anc) continue;
    float M = -INFINITY;
#pragma unroll
    for (int t = 0; t < kAttnWaves; ++t) M = fmaxf(M, red[t][u][HD]);
    float Ls = 0.f, o[HS];
#pragma unroll
    for (int e = 0; e < HS; ++e) o[e] = 0.f;
#pragma unroll
    for (int t = 0; t < kAttnWaves; ++t) {
      const float f = exp2f(red[t][u][HD] - M);
      Ls = fmaf(red[t][u][HD + 1], f, Ls);
#pragma unroll
      for (int e = 0; e < HS; ++e) o[e] = fmaf(red[t][u][lane * HS + e], f, o[e]);
    }
    float* dst = part + (((size_t)row * D.nq + qh) * nchunk + c) * HP;
#pragma unroll
    for (int e = 0; e < HS; ++e) dst[lane * HS + e] = o[e];
    if (lane == 0) {
      dst[HD] = M;
      dst[HD + 1] = Ls;
    }
  }
}

// Combine the split-KV chunks of a (row, head) in chunk order; one wave each.
template <int HD>
__global__ void attn_combine_kernel(const RowInfo* __restrict__ rows, int nrows, const float* __restrict__ part,
                                    float* __restrict__ out, int nq, int nchunk) {
  using G = AttnGeom<HD>;
  constexpr int HS = G::HS, HP = HD + 2;
  const int unit = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (unit >= nrows * nq) return;
  const int row = unit / nq, qh = unit % nq;
  const RowInfo& R = rows[row];
  const int nc = (R.ncommit + R.n_anc + G::CHUNK - 1) / G::CHUNK;
  const float* base = part + ((size_t)row * nq + qh) * nchunk * HP;
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, base[c * HP + HD]);
  float Ls = 0.f, o[HS];
#pragma unroll
  for (int e = 0; e < HS; ++e) o[e] = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float* pc = base + c * HP;
    const float f = exp2f(pc[HD] - M);
    Ls = fmaf(pc[HD + 1], f, Ls);
#pragma unroll
    for (int e = 0; e < HS; ++e) o[e] = fmaf(pc[lane * HS + e], f, o[e]);
  }
  const float inv = 1.0f / Ls;
  float* dst = out + ((size_t)row * nq + qh) * HD;
#pragma unroll
  for (int e = 0; e < HS; ++e) dst[lane * HS + e] = o[e] * inv;
}

// ----------------------------------------------------------------------------
// Host launcher
// ----------------------------------------------------------------------------
int attn_chunk(int hd) { return hd == 128 ? AttnGeom<128>::CHUNK : AttnGeom<64>::CHUNK; }

hipError_t launch_attention(const AttnItem* items, int nitems, const RowInfo* rows, int nrows, const float* q,
                            const float* kvc, const float* exb, float* part, float* out, const ModelDims& D,
                            int lam, int smul, int nchunk, int max_keys, hipStream_t st) {
  if (nitems == 0) return hipSuccess;
  const int nc = (max_keys + attn_chunk(D.hd) - 1) / attn_chunk(D.hd);
  dim3 grid(nitems, D.nkv, nc);
  if (D.hd == 128)
    hipLaunchKernelGGL((attn_kernel<128>), grid, dim3(kAttnThreads), 0, st, items, rows, q, kvc, exb, part, D, lam,
                       smul, nchunk);
  else
    hipLaunchKernelGGL((attn_kernel<64>), grid, dim3(kAttnThreads), 0, st, items, rows, q, kvc, exb, part, D, lam,
                       smul, nchunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int units = nrows * D.nq, wpb = 4;
  if (D.hd == 128)
    hipLaunchKernelGGL((attn_combine_kernel<128>), dim3((units + wpb - 1) / wpb), dim3(64 * wpb), 0, st, rows,
                       nrows, part, out, D.nq, nchunk);
  else
    hipLaunchKernelGGL((attn_combine_kernel<64>), dim3((units + wpb - 1) / wpb), dim3(64 * wpb), 0, st, rows,
                       nrows, part, out, D.nq, nchunk);
  return hipGetLastError();
}

}  // namespace dex
