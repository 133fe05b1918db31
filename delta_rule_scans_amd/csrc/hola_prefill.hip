// hola_prefill.hip -- the HOLA exact cache over a whole prompt, block by block.
//
// "A Hippocampus for Linear Attention", sec. 3.3 (the cache keeps the w tokens
// with the largest write score; the top-w of a set does not depend on the order
// its members arrive in), sec. 3.4 eq. (7) (a token reads over the cache, the
// causal tokens of its own block and an optional null sink, with RMS-normalised
// query and keys at 1/sqrt(d_k)), sec. 3.2 eq. (4) (softmax read).
//
// Block j's tokens read the cache as it stood before block j; then the block
// is inserted. Three kernels:
//  * select: one workgroup per head walks the blocks in order and records, for
//    every block, which tokens the cache holds when the block reads it, then
//    merges the block in: every candidate's rank among (cache, block) by score
//    descending, position ascending is counted directly, and the first w stay.
//  * read: one workgroup per (head, block, 64 queries), every block in
//    parallel: streaming softmax over 32-key tiles of (cache members, causal
//    block tokens) in float32.
//  * commit: one workgroup per head gathers the final members' keys and values
//    (from the old cache or the prompt), then writes the cache in rank order.
#include <math.h>

#include "kdn_internal.h"

namespace kdn {
namespace {

constexpr int NT = 256;
constexpr int QT = 64;   // queries per read workgroup
constexpr int KT = 32;   // keys per tile
constexpr int MAXD = 128;

// Score order: larger score first, then smaller position, then smaller
// candidate index (only reached when a caller repeats a position). NaN scores
// rank below every other score. Recency order: larger position first.
__device__ __forceinline__ bool before(float ma, int pa, int ia, float mb, int pb, int ib,
                                       bool recency) {
  if (recency) return pa != pb ? pa > pb : ia < ib;
  ma = ma == ma ? ma : -INFINITY;
  mb = mb == mb ? mb : -INFINITY;
  if (ma != mb) return ma > mb;
  if (pa != pb) return pa < pb;
  return ia < ib;
}

// Cache members are coded as src >= 0: prompt token src; src < 0: old slot -1 - src.
__global__ __launch_bounds__(NT) void select_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  const int cap = a.w + a.block;
  float* cm = reinterpret_cast<float*>(lds_raw);  // candidates [cap]
  int* cp = reinterpret_cast<int*>(cm + cap);
  int* cs = cp + cap;
  float* nm = reinterpret_cast<float*>(cs + cap);  // next cache [w]
  int* np_ = reinterpret_cast<int*>(nm + a.w);
  int* ns = np_ + a.w;
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int nblk = (a.L + a.block - 1) / a.block;
  int n = min(a.cache_count[bh], a.w);
  n = max(n, 0);
  for (int e = tid; e < n; e += NT) {
    nm[e] = a.cache_m[(size_t)bh * a.w + e];
    np_[e] = a.cache_pos[(size_t)bh * a.w + e];
    ns[e] = -1 - e;
  }
  __syncthreads();
  for (int j = 0; j < nblk; ++j) {
    const int j0 = j * a.block, nb = min(a.block, a.L - j0);
    // the cache this block reads
    int* mem = a.members + ((size_t)bh * nblk + j) * a.w;
    for (int e = tid; e < n; e += NT) mem[e] = ns[e];
    if (tid == 0) a.member_count[(size_t)bh * nblk + j] = n;
    const int nc = n + nb;
    for (int e = tid; e < nc; e += NT) {
      if (e < n) {
        cm[e] = nm[e];
        cp[e] = np_[e];
        cs[e] = ns[e];
      } else {
        const int i = j0 + e - n;
        cm[e] = a.m[(size_t)bh * a.L + i];
        cp[e] = a.t0 + i;
        cs[e] = i;
      }
    }
    __syncthreads();
    for (int x = tid; x < nc; x += NT) {
      const float mx = cm[x];
      const int px = cp[x];
      int rank = 0;
      for (int y = 0; y < nc; ++y) rank += before(cm[y], cp[y], y, mx, px, x, a.policy == 1) ? 1 : 0;
      if (rank < a.w) {
        nm[rank] = mx;
        np_[rank] = px;
        ns[rank] = cs[x];
      }
    }
    n = min(nc, a.w);
    __syncthreads();
  }
  int* fin = a.final_src + (size_t)bh * a.w;
  for (int e = tid; e < n; e += NT) {
    fin[e] = ns[e];
    a.final_m[(size_t)bh * a.w + e] = nm[e];
    a.final_pos[(size_t)bh * a.w + e] = np_[e];
  }
  if (tid == 0) a.final_count[bh] = n;
}

template <typename Tin>
__global__ __launch_bounds__(NT) void read_kernel(PrefillArgs a) {
  __shared__ float sQ[QT][MAXD + 1];
  __shared__ float sK[KT][MAXD + 1];
  __shared__ float sV[KT][MAXD];
  __shared__ float sP[QT][KT + 1];
  __shared__ int sSrc[KT];
  const int bh = blockIdx.x, j = blockIdx.y, qt = blockIdx.z, tid = threadIdx.x;
  const int dk = a.dk, dv = a.dv;
  const int nblk = (a.L + a.block - 1) / a.block;
  const int j0 = j * a.block, nb = min(a.block, a.L - j0);
  const int q0 = qt * QT;  // first query, relative to the block
  if (q0 >= nb) return;
  const int nq = min(QT, nb - q0);
  const Tin* qh = static_cast<const Tin*>(a.q) + (size_t)bh * a.L * dk;
  const Tin* kh = static_cast<const Tin*>(a.k) + (size_t)bh * a.L * dk;
  const Tin* vh = static_cast<const Tin*>(a.v) + (size_t)bh * a.L * dv;
  const float* ck = a.cache_k + (size_t)bh * a.w * dk;
  const float* cv = a.cache_v + (size_t)bh * a.w * dv;
  const int* mem = a.members + ((size_t)bh * nblk + j) * a.w;
  const int ncache = a.member_count[(size_t)bh * nblk + j];
  // keys: the cache members, then the block's tokens up to the last query here
  const int nkeys = ncache + q0 + nq;
  const float inv_sqrt_d = 1.f / sqrtf((float)dk);

  // queries, RMS-normalised (4 lanes per row)
  for (int idx = tid; idx < QT * dk; idx += NT) {
    const int r = idx / dk, c = idx - r * dk;
    sQ[r][c] = r < nq ? Elem<Tin>::load(qh, (size_t)(j0 + q0 + r) * dk + c) : 0.f;
  }
  __syncthreads();
  const int qi = tid >> 2, part = tid & 3;
  {
    float ss = 0.f;
    for (int c = part; c < dk; c += 4) ss = fmaf(sQ[qi][c], sQ[qi][c], ss);
    ss += __shfl_xor(ss, 1, 4);
    ss += __shfl_xor(ss, 2, 4);
    const float sc = inv_sqrt_d / sqrtf(ss / dk + a.rms_eps);  // folds the 1/sqrt(d_k)
    for (int c = part; c < dk; c += 4) sQ[qi][c] *= sc;
  }
  const int qtok = q0 + qi;  // this row's token, relative to the block
  float M, Z;
  if (a.sink_logit) {
    M = a.sink_logit[bh % a.H];
    Z = 1.f;
  } else {
    M = -INFINITY;
    Z = 0.f;
  }
  float acc[MAXD / 4];
#pragma unroll
  for (int u = 0; u < MAXD / 4; ++u) acc[u] = 0.f;

  for (int e0 = 0; e0 < nkeys; e0 += KT) {
    __syncthreads();
    if (tid < KT) {
      const int e = e0 + tid;
      sSrc[tid] = e < nkeys ? (e < ncache ? mem[e] : j0 + e - ncache) : 0x7fffffff;
    }
    __syncthreads();
    for (int idx = tid; idx < KT * dk; idx += NT) {
      const int r = idx / dk, c = idx - r * dk;
      const int src = sSrc[r];
      float x = 0.f;
      if (src != 0x7fffffff)
        x = src >= 0 ? Elem<Tin>::load(kh, (size_t)src * dk + c) : ck[(size_t)(-1 - src) * dk + c];
      sK[r][c] = x;
    }
    for (int idx = tid; idx < KT * dv; idx += NT) {
      const int r = idx / dv, c = idx - r * dv;
      const int src = sSrc[r];
      float x = 0.f;
      if (src != 0x7fffffff)
        x = src >= 0 ? Elem<Tin>::load(vh, (size_t)src * dv + c) : cv[(size_t)(-1 - src) * dv + c];
      sV[r][c] = x;
    }
    __syncthreads();
    {  // key norms, 8 lanes per key
      const int kr = tid >> 3, sub = tid & 7;
      float ss = 0.f;
      for (int c = sub; c < dk; c += 8) ss = fmaf(sK[kr][c], sK[kr][c], ss);
      ss += __shfl_xor(ss, 1, 8);
      ss += __shfl_xor(ss, 2, 8);
      ss += __shfl_xor(ss, 4, 8);
      const float sc = 1.f / sqrtf(ss / dk + a.rms_eps);
      for (int c = sub; c < dk; c += 8) sK[kr][c] *= sc;
    }
    __syncthreads();
    // logits of this row against keys 8 part .. 8 part + 7 of the tile
    float l[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) l[jj] = 0.f;
    for (int c = 0; c < dk; ++c) {
      const float qv = sQ[qi][c];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) l[jj] = fmaf(qv, sK[8 * part + jj][c], l[jj]);
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int e = e0 + 8 * part + jj;
      // cache members are always visible; block tokens up to the query itself
      const bool vis = qi < nq && e < nkeys && (e < ncache || e - ncache <= qtok);
      l[jj] = vis ? l[jj] : -INFINITY;
      tmax = fmaxf(tmax, l[jj]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 1, 4));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 2, 4));
    const float Mn = fmaxf(M, tmax);
    // rows with nothing visible yet keep M = -inf; their weights stay 0
    const float scale = Mn == -INFINITY ? 1.f : __expf(M - Mn);
    float psum = 0.f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const float p = l[jj] == -INFINITY ? 0.f : __expf(l[jj] - Mn);
      sP[qi][8 * part + jj] = p;
      psum += p;
    }
    psum += __shfl_xor(psum, 1, 4);
    psum += __shfl_xor(psum, 2, 4);
    Z = fmaf(Z, scale, psum);
    M = Mn;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < MAXD / 4; ++u) acc[u] *= scale;
    for (int e = 0; e < KT; ++e) {
      const float p = sP[qi][e];
#pragma unroll
      for (int u = 0; u < MAXD / 4; ++u) {
        const int c = part + 4 * u;
        if (c < dv) acc[u] = fmaf(p, sV[e][c], acc[u]);
      }
    }
  }
  if (qi < nq) {
    float* o = a.o_cache + ((size_t)bh * a.L + j0 + qtok) * dv;
    const float inv = 1.f / Z;
#pragma unroll
    for (int u = 0; u < MAXD / 4; ++u) {
      const int c = part + 4 * u;
      if (c < dv) o[c] = acc[u] * inv;
    }
  }
}

template <typename Tin>
__global__ __launch_bounds__(NT) void commit_kernel(PrefillArgs a) {
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int n = a.final_count[bh];
  const int* fin = a.final_src + (size_t)bh * a.w;
  const int row = a.dk + a.dv;
  float* stage = a.stage + (size_t)bh * a.w * row;
  const Tin* kh = static_cast<const Tin*>(a.k) + (size_t)bh * a.L * a.dk;
  const Tin* vh = static_cast<const Tin*>(a.v) + (size_t)bh * a.L * a.dv;
  float* ck = a.cache_k + (size_t)bh * a.w * a.dk;
  float* cv = a.cache_v + (size_t)bh * a.w * a.dv;
  // gather first: a member may come from an old slot that is rewritten below
  for (int idx = tid; idx < n * row; idx += NT) {
    const int e = idx / row, c = idx - e * row;
    const int src = fin[e];
    float x;
    if (c < a.dk)
      x = src >= 0 ? Elem<Tin>::load(kh, (size_t)src * a.dk + c) : ck[(size_t)(-1 - src) * a.dk + c];
    else
      x = src >= 0 ? Elem<Tin>::load(vh, (size_t)src * a.dv + c - a.dk)
                   : cv[(size_t)(-1 - src) * a.dv + c - a.dk];
    stage[idx] = x;
  }
  __syncthreads();
  for (int idx = tid; idx < n * row; idx += NT) {
    const int e = idx / row, c = idx - e * row;
    if (c < a.dk) ck[(size_t)e * a.dk + c] = stage[idx];
    else cv[(size_t)e * a.dv + c - a.dk] = stage[idx];
  }
  for (int e = tid; e < n; e += NT) {
    a.cache_m[(size_t)bh * a.w + e] = a.final_m[(size_t)bh * a.w + e];
    a.cache_pos[(size_t)bh * a.w + e] = a.final_pos[(size_t)bh * a.w + e];
  }
  if (tid == 0) a.cache_count[bh] = n;
}

template <typename Tin>
hipError_t prefill_typed(const PrefillArgs& a, hipStream_t s) {
  const int nblk = (a.L + a.block - 1) / a.block;
  const size_t sel_lds = (size_t)3 * (a.w + a.block) * 4 + (size_t)3 * a.w * 4;
  hipLaunchKernelGGL(select_kernel, dim3(a.BH), dim3(NT), sel_lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(read_kernel<Tin>, dim3(a.BH, nblk, (a.block + QT - 1) / QT), dim3(NT), 0, s,
                     a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(commit_kernel<Tin>, dim3(a.BH), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

size_t prefill_workspace_bytes(int BH, int L, int dk, int dv, int w, int block) {
  const size_t nblk = ((size_t)L + block - 1) / block;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return up((size_t)BH * nblk * w * 4) + up((size_t)BH * nblk * 4) + 3 * up((size_t)BH * w * 4) +
         up((size_t)BH * 4) + up((size_t)BH * w * (dk + dv) * 4);
}

void prefill_bind_workspace(PrefillArgs& a, void* ws) {
  const size_t nblk = ((size_t)a.L + a.block - 1) / a.block;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* p = static_cast<char*>(ws);
  a.members = reinterpret_cast<int*>(p);
  p += up((size_t)a.BH * nblk * a.w * 4);
  a.member_count = reinterpret_cast<int*>(p);
  p += up((size_t)a.BH * nblk * 4);
  a.final_src = reinterpret_cast<int*>(p);
  p += up((size_t)a.BH * a.w * 4);
  a.final_m = reinterpret_cast<float*>(p);
  p += up((size_t)a.BH * a.w * 4);
  a.final_pos = reinterpret_cast<int*>(p);
  p += up((size_t)a.BH * a.w * 4);
  a.final_count = reinterpret_cast<int*>(p);
  p += up((size_t)a.BH * 4);
  a.stage = reinterpret_cast<float*>(p);
}

hipError_t launch_prefill(const PrefillArgs& a, bool in_bf16, hipStream_t s) {
  const size_t sel_lds = (size_t)3 * (a.w + a.block) * 4 + (size_t)3 * a.w * 4;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)sel_lds);
  if (e != hipSuccess) return e;
  return in_bf16 ? prefill_typed<uint16_t>(a, s) : prefill_typed<float>(a, s);
}

}  // namespace kdn
