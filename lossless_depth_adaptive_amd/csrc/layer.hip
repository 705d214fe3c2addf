// Per-row layer kernels of the lattice step: embedding gather, RMSNorm,
// RoPE with the K/V write, and lattice attention with its split-KV combine.
//
// Every kernel computes a row from that row's own inputs in a fixed order, so a
// node of the depth-position lattice and the same context decoded
// autoregressively produce identical bits.
#include "common.h"

namespace dex {

// ----------------------------------------------------------------------------
// Embedding: rows that start a slot (explorer 0, "Depth Exploration for LLM
// Decoding", Section 3.2: a position expansion starts the next token position
// from E_0) load E[tok] into their fp32 residual stream.
// ----------------------------------------------------------------------------
template <typename T>
__global__ void embed_kernel(const T* __restrict__ E, const RowInfo* __restrict__ rows, int row0,
                             float* __restrict__ hidden, int d) {
  const RowInfo& r = rows[row0 + blockIdx.x];
  if (r.tok < 0) return;
  const T* e = E + (size_t)r.tok * d;
  float* h = hidden + (size_t)r.hrow * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) h[i] = to_f<T>(e[i]);
}

// ----------------------------------------------------------------------------
// RMSNorm: out = x / sqrt(mean(x^2) + eps) * g, rounded to the GEMM input type.
// The weight g belongs to layer stage*smul + lam (smul = 0 gives one layer for
// every row). Sum of squares: per-thread strided partials, a fixed xor
// butterfly per wave, then the four waves in order.
// ----------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ hidden,
                                                      const RowInfo* __restrict__ rows, int row0,
                                                      const float* __restrict__ gbase,
                                                      long long gstride, int smul, int lam,
                                                      T* __restrict__ out, int d, float eps) {
  const int row = row0 + blockIdx.x;
  const RowInfo& r = rows[row];
  const float* x = hidden + (size_t)r.hrow * d;
  const float* g = gbase + (size_t)(r.stage * smul + lam) * gstride;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) ss = fmaf(x[i], x[i], ss);
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  __shared__ float wsum[4];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float rs = 1.0f / sqrtf(tot / (float)d + eps);
  T* o = out + (size_t)row * d;
  for (int i = threadIdx.x; i < d; i += 256) o[i] = from_f<T>(x[i] * rs * g[i]);
}

// ----------------------------------------------------------------------------
// RoPE and K/V write. Input: the QKV projection [rows][(nq + 2nkv) * hd] in
// fp32. Rotation pairs (i, i + hd/2) by angle pos * base^(-2i/hd) from a
// host-built table. Queries go to qout pre-multiplied by qscale
// (log2(e)/sqrt(hd), so attention can use exp2). Keys and values are stored
// in the storage type: into the committed cache at the row's position for
// autoregressive and prefill rows, into the node's explore slot otherwise.
// ----------------------------------------------------------------------------
template <typename T>
__global__ void rope_kv_kernel(const float* __restrict__ qkv, const RowInfo* __restrict__ rows,
                               int row0, const float* __restrict__ cosT,
                               const float* __restrict__ sinT, float* __restrict__ qout,
                               T* __restrict__ kvc, T* __restrict__ exb, ModelDims D, int smul,
                               int lam, float qscale) {
  const int row = row0 + blockIdx.x;
  const RowInfo& r = rows[row];
  const int hd = D.hd, half = hd >> 1;
  const int nh = D.nq + 2 * D.nkv;
  const float* src = qkv + (size_t)row * nh * hd;
  const float* cs = cosT + (size_t)r.pos * half;
  const float* sn = sinT + (size_t)r.pos * half;
  const int layer = r.stage * smul + lam;
  for (int t = threadIdx.x; t < nh * half; t += blockDim.x) {
    const int h = t / half, i = t - h * half;
    const float x1 = src[h * hd + i], x2 = src[h * hd + i + half];
    if (h < D.nq) {
      const float c = cs[i], s = sn[i];
      float* q = qout + ((size_t)row * D.nq + h) * hd;
      q[i] = (x1 * c - x2 * s) * qscale;
      q[i + half] = (x2 * c + x1 * s) * qscale;
      continue;
    }
    const int kv = (h < D.nq + D.nkv) ? 0 : 1;
    const int hh = h - D.nq - kv * D.nkv;
    float o1 = x1, o2 = x2;
    if (kv == 0) {
      const float c = cs[i], s = sn[i];
      o1 = x1 * c - x2 * s;
      o2 = x2 * c + x1 * s;
    }
    T* dst;
    if (r.kv_commit)
      dst = kvc + ((((size_t)r.seq * D.L + layer) * 2 + kv) * D.nkv + hh) * (size_t)D.Cmax * hd +
            (size_t)r.pos * hd;
    else
      dst = exb + ((((size_t)r.seq * D.P + r.phys) * D.S + lam) * 2 + kv) * (size_t)D.nkv * hd +
            (size_t)hh * hd;
    dst[i] = from_f<T>(o1);
    dst[i + half] = from_f<T>(o2);
  }
}

// ----------------------------------------------------------------------------
// Lattice attention ("Depth Exploration for LLM Decoding", Section 3.2: the
// binary expansion lets ancestry, KV entries and attention masks be indexed
// consistently). A row attends to the committed cache [0, ncommit) and to the
// explore-buffer entries of its ancestors at positions ncommit.. (its own
// entry last). Keys are visited in absolute-position tiles of 64 and split-KV
// chunks of 512 positions, whichever buffer holds them, so the reduction order
// of a row depends only on its position. All rows of a work item share one
// sequence and layer: committed K/V tiles are staged in LDS once for all of
// them.
//
// Per (row, query head) unit and tile: s_j = q . k_j (sequential over the head
// dimension), running max m, p_j = 2^(s_j - m), l = l*2^(m_old - m) +
// butterfly-sum p, acc = acc*2^(m_old - m) + sum_j p_j v_j (j increasing).
// grid = (items, kv heads, chunks), block = 256 (4 waves).
// ----------------------------------------------------------------------------
template <typename T> struct Pair;
template <> struct Pair<bf16_t> {
  static constexpr int PAD = 2;
  __device__ __forceinline__ static void ld(const bf16_t* p, int d, float& a, float& b) {
    const unsigned w = *(const unsigned*)(p + d);
    a = __uint_as_float(w << 16);
    b = __uint_as_float(w & 0xFFFF0000u);
  }
};
template <> struct Pair<float> {
  static constexpr int PAD = 1;
  __device__ __forceinline__ static void ld(const float* p, int d, float& a, float& b) {
    a = p[d];
    b = p[d + 1];
  }
};

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <typename T, int HD>
__global__ __launch_bounds__(kAttnThreads) void attn_kernel(
    const AttnItem* __restrict__ items, const RowInfo* __restrict__ rows,
    const float* __restrict__ q, const T* __restrict__ kvc, const T* __restrict__ exb,
    float* __restrict__ part, ModelDims D, int lam, int smul, int nchunk) {
  constexpr int LD = HD + Pair<T>::PAD;           // LDS row stride (elements)
  constexpr int UPW = kAttnUnits / 4;            // units per wave
  constexpr int DPL = HD / 64;                   // output dims per lane
  __shared__ T Ks[kAttnTile * LD];
  __shared__ T Vs[kAttnTile * LD];
  __shared__ float qs[kAttnUnits][HD];

  const AttnItem it = items[blockIdx.x];
  const int h = blockIdx.y, c = blockIdx.z;
  const int pb = c * kAttnChunk;
  if (pb >= it.max_keys) return;
  const int pe = min(pb + kAttnChunk, it.max_keys);
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
  const T* kc = kvc + (((size_t)seq * D.L + layer) * 2 + 0) * D.nkv * cstride + h * cstride;
  const T* vc = kvc + (((size_t)seq * D.L + layer) * 2 + 1) * D.nkv * cstride + h * cstride;
  const size_t xs_slot = (size_t)D.S * 2 * D.nkv * HD;   // explore elements per node slot
  const T* xk = exb + (size_t)seq * D.P * xs_slot + (size_t)lam * 2 * D.nkv * HD + (size_t)h * HD;
  const T* xv = xk + (size_t)D.nkv * HD;

  float m[UPW], l[UPW], acc[UPW][DPL];
#pragma unroll
  for (int i = 0; i < UPW; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int t = 0; t < DPL; ++t) acc[i][t] = 0.f;
  }

  for (int p0 = pb; p0 < pe; p0 += kAttnTile) {
    __syncthreads();
    // Stage committed keys/values of this tile (32-bit words).
    const int nld = max(0, min(kAttnTile, maxc - p0));
    constexpr int WPR = HD * (int)sizeof(T) / 4;   // 32-bit words per row
    for (int t = threadIdx.x; t < nld * WPR; t += kAttnThreads) {
      const int j = t / WPR, wd = t - j * WPR;
      const unsigned* ks = (const unsigned*)(kc + (size_t)(p0 + j) * HD);
      const unsigned* vs = (const unsigned*)(vc + (size_t)(p0 + j) * HD);
      ((unsigned*)(Ks + j * LD))[wd] = ks[wd];
      ((unsigned*)(Vs + j * LD))[wd] = vs[wd];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      const int u = w + 4 * i;
      if (u >= units) continue;
      const RowInfo& R = rows[it.row0 + u / rep];
      const int lim = R.ncommit + R.n_anc;
      if (p0 >= lim) continue;
      const int p = p0 + lane;
      float s = -INFINITY;
      if (p < lim) {
        const T* kp = (p < R.ncommit) ? (Ks + lane * LD) : (xk + (size_t)R.anc[p - R.ncommit] * xs_slot);
        float acc_s = 0.f;
        for (int dd = 0; dd < HD; dd += 2) {
          float k0, k1;
          Pair<T>::ld(kp, dd, k0, k1);
          acc_s = fmaf(qs[u][dd], k0, acc_s);
          acc_s = fmaf(qs[u][dd + 1], k1, acc_s);
        }
        s = acc_s;
      }
      const float mt = wave_max(s);
      const float mn = fmaxf(m[i], mt);
      const float alpha = exp2f(m[i] - mn);
      const float pj = (p < lim) ? exp2f(s - mn) : 0.f;
      l[i] = l[i] * alpha + wave_sum(pj);
#pragma unroll
      for (int t = 0; t < DPL; ++t) acc[i][t] *= alpha;
      const int nv = min(kAttnTile, lim - p0);
      for (int jj = 0; jj < nv; ++jj) {
        const float pv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jj));
        const int pp = p0 + jj;
        const T* vp = (pp < R.ncommit) ? (Vs + jj * LD) : (xv + (size_t)R.anc[pp - R.ncommit] * xs_slot);
#pragma unroll
        for (int t = 0; t < DPL; ++t) acc[i][t] = fmaf(pv, to_f<T>(vp[lane + 64 * t]), acc[i][t]);
      }
      m[i] = mn;
    }
  }
#pragma unroll
  for (int i = 0; i < UPW; ++i) {
    const int u = w + 4 * i;
    if (u >= units) continue;
    const int row = it.row0 + u / rep, qh = h * rep + u % rep;
    const RowInfo& R = rows[row];
    if (pb >= R.ncommit + R.n_anc) continue;
    float* o = part + (((size_t)row * D.nq + qh) * nchunk + c) * (HD + 2);
#pragma unroll
    for (int t = 0; t < DPL; ++t) o[lane + 64 * t] = acc[i][t];
    if (lane == 0) {
      o[HD] = m[i];
      o[HD + 1] = l[i];
    }
  }
}

// Combine the split-KV chunks of a (row, head) in chunk order; one wave each.
template <typename T, int HD>
__global__ void attn_combine_kernel(const RowInfo* __restrict__ rows, int row0, int nrows,
                                    const float* __restrict__ part, T* __restrict__ out, int nq,
                                    int nchunk) {
  constexpr int DPL = HD / 64;
  const int unit = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (unit >= nrows * nq) return;
  const int row = row0 + unit / nq, qh = unit % nq;
  const RowInfo& R = rows[row];
  const int lim = R.ncommit + R.n_anc;
  const int nc = (lim + kAttnChunk - 1) / kAttnChunk;
  const float* base = part + ((size_t)row * nq + qh) * nchunk * (HD + 2);
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, base[c * (HD + 2) + HD]);
  float Lsum = 0.f, o[DPL];
#pragma unroll
  for (int t = 0; t < DPL; ++t) o[t] = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float* pc = base + c * (HD + 2);
    const float f = exp2f(pc[HD] - M);
    Lsum = fmaf(pc[HD + 1], f, Lsum);
#pragma unroll
    for (int t = 0; t < DPL; ++t) o[t] = fmaf(pc[lane + 64 * t], f, o[t]);
  }
  const float inv = 1.0f / Lsum;
  T* dst = out + ((size_t)row * nq + qh) * HD;
#pragma unroll
  for (int t = 0; t < DPL; ++t) dst[lane + 64 * t] = from_f<T>(o[t] * inv);
}

// ----------------------------------------------------------------------------
// Host launchers
// ----------------------------------------------------------------------------
template <typename T>
hipError_t launch_embed(const void* E, const RowInfo* rows, int row0, int nrows, float* hidden, int d,
                        hipStream_t st) {
  if (nrows == 0) return hipSuccess;
  hipLaunchKernelGGL(embed_kernel<T>, dim3(nrows), dim3(256), 0, st, (const T*)E, rows, row0, hidden, d);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rmsnorm(const float* hidden, const RowInfo* rows, int row0, int nrows,
                          const float* gbase, long long gstride, int smul, int lam, void* out, int d,
                          float eps, hipStream_t st) {
  if (nrows == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel<T>, dim3(nrows), dim3(256), 0, st, hidden, rows, row0, gbase,
                     gstride, smul, lam, (T*)out, d, eps);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_rope_kv(const float* qkv, const RowInfo* rows, int row0, int nrows, const float* cosT,
                          const float* sinT, float* qout, void* kvc, void* exb, const ModelDims& D,
                          int smul, int lam, float qscale, hipStream_t st) {
  if (nrows == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_kv_kernel<T>, dim3(nrows), dim3(256), 0, st, qkv, rows, row0, cosT, sinT,
                     qout, (T*)kvc, (T*)exb, D, smul, lam, qscale);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attention(const AttnItem* items, int nitems, const RowInfo* rows, int row0, int nrows,
                            const float* q, const void* kvc, const void* exb, float* part, void* out,
                            const ModelDims& D, int lam, int smul, int nchunk, int max_keys, hipStream_t st) {
  if (nitems == 0) return hipSuccess;
  const int nc = (max_keys + kAttnChunk - 1) / kAttnChunk;
  dim3 grid(nitems, D.nkv, nc);
  if (D.hd == 128)
    hipLaunchKernelGGL((attn_kernel<T, 128>), grid, dim3(kAttnThreads), 0, st, items, rows, q,
                       (const T*)kvc, (const T*)exb, part, D, lam, smul, nchunk);
  else
    hipLaunchKernelGGL((attn_kernel<T, 64>), grid, dim3(kAttnThreads), 0, st, items, rows, q,
                       (const T*)kvc, (const T*)exb, part, D, lam, smul, nchunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int units = nrows * D.nq, wpb = 4;
  if (D.hd == 128)
    hipLaunchKernelGGL((attn_combine_kernel<T, 128>), dim3((units + wpb - 1) / wpb), dim3(64 * wpb), 0,
                       st, rows, row0, nrows, part, (T*)out, D.nq, nchunk);
  else
    hipLaunchKernelGGL((attn_combine_kernel<T, 64>), dim3((units + wpb - 1) / wpb), dim3(64 * wpb), 0,
                       st, rows, row0, nrows, part, (T*)out, D.nq, nchunk);
  return hipGetLastError();
}

#define DEX_INST(T)                                                                                  \
  template hipError_t launch_embed<T>(const void*, const RowInfo*, int, int, float*, int, hipStream_t); \
  template hipError_t launch_rmsnorm<T>(const float*, const RowInfo*, int, int, const float*, long long, \
                                        int, int, void*, int, float, hipStream_t);                   \
  template hipError_t launch_rope_kv<T>(const float*, const RowInfo*, int, int, const float*,         \
                                        const float*, float*, void*, void*, const ModelDims&, int, int, \
                                        float, hipStream_t);                                          \
  template hipError_t launch_attention<T>(const AttnItem*, int, const RowInfo*, int, int, const float*, \
                                          const void*, const void*, float*, void*, const ModelDims&,  \
                                          int, int, int, int, hipStream_t);
DEX_INST(float)
DEX_INST(bf16_t)

}  // namespace dex
