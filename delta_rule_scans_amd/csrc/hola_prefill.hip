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
//  * block top: one workgroup per (head, block), every block in parallel,
//    ranks the block's tokens by score descending, position ascending (or by
//    position descending for the recency control) and keeps the first w.
//  * merge: one workgroup per head walks the blocks in order, records for
//    every block which tokens the cache holds when the block reads it, then
//    merges the block's top list in.
//  * read: one workgroup per (head, block, 64 queries), every block in
//    parallel: streaming softmax over 32-key tiles of (cache members, causal
//    block tokens) in float32, register-tiled.
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
constexpr int kMaxW = 256;       // largest cache capacity
constexpr int kMaxBlock = 1024;  // largest prompt block

// NaN scores rank below every other score.
__device__ __forceinline__ float score_key(float m) { return m == m ? m : -INFINITY; }

// Block tops: the w best tokens of each block on its own, every block in
// parallel. Positions rise with the index inside a block, so the score order
// ties break on the index and the recency order is the reverse index order.
// Each token's rank is counted against the whole block.
__global__ __launch_bounds__(NT) void block_top_kernel(PrefillArgs a) {
  __shared__ __align__(16) float sm[kMaxBlock];
  const int bh = blockIdx.x, j = blockIdx.y, tid = threadIdx.x;
  const int nblk = (a.L + a.block - 1) / a.block;
  const int j0 = j * a.block, nb = min(a.block, a.L - j0);
  const float* mh = a.m + (size_t)bh * a.L + j0;
  for (int i = tid; i < nb; i += NT) sm[i] = score_key(mh[i]);
  for (int i = nb + tid; i < ((nb + 3) & ~3); i += NT) sm[i] = -INFINITY;
  __syncthreads();
  const size_t base = ((size_t)bh * nblk + j) * a.w;
  for (int x = tid; x < nb; x += NT) {
    int rank;
    if (a.policy == 1) {
      rank = nb - 1 - x;
    } else {
      const float mx = sm[x];
      rank = 0;
      // padding slots hold -inf and sit after x, so they never count
      for (int y = 0; y < nb; y += 4) {
        const float4 m4 = *reinterpret_cast<const float4*>(&sm[y]);
        rank += (m4.x > mx) | ((m4.x == mx) & (y < x));
        rank += (m4.y > mx) | ((m4.y == mx) & (y + 1 < x));
        rank += (m4.z > mx) | ((m4.z == mx) & (y + 2 < x));
        rank += (m4.w > mx) | ((m4.w == mx) & (y + 3 < x));
      }
    }
    if (rank < a.w) {
      a.top_m[base + rank] = mh[x];
      a.top_pos[base + rank] = a.t0 + j0 + x;
      a.top_src[base + rank] = j0 + x;
    }
  }
}

// Cache members are coded as src >= 0: prompt token src; src < 0: old slot -1 - src.
//
// The cache a block reads is the top-w of the old cache and every earlier
// block, and the top-w of a union is the top-w of the union of the parts'
// top-w lists, so one workgroup per head merges the block tops in order: two
// sorted lists, each entry's new rank is its own index plus the number of
// entries of the other list ahead of it (a binary search). On a full tie the
// cache entry goes first, as the earlier candidate.
__global__ __launch_bounds__(NT) void merge_kernel(PrefillArgs a) {
  __shared__ float cm[2][kMaxW];
  __shared__ int cp[2][kMaxW], cs[2][kMaxW];
  __shared__ float tm[kMaxW];
  __shared__ int tp[kMaxW];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int nblk = (a.L + a.block - 1) / a.block;
  const bool rec = a.policy == 1;
  int n = min(max(a.cache_count[bh], 0), a.w);
  // the old cache need not be in rank order: rank it by counting, ties by slot
  if (tid < n) {
    cm[1][tid] = a.cache_m[(size_t)bh * a.w + tid];
    cp[1][tid] = a.cache_pos[(size_t)bh * a.w + tid];
  }
  __syncthreads();
  if (tid < n) {
    const float mx = score_key(cm[1][tid]);
    const int px = cp[1][tid];
    int r = 0;
    for (int y = 0; y < n; ++y) {
      const float my = score_key(cm[1][y]);
      const int py = cp[1][y];
      const bool tie_first = y < tid;
      r += rec ? (py > px || (py == px && tie_first))
               : (my > mx || (my == mx && (py < px || (py == px && tie_first))));
    }
    cm[0][r] = cm[1][tid];
    cp[0][r] = px;
    cs[0][r] = -1 - tid;
  }
  int cur = 0;
  // the next block top, loaded a step ahead
  const size_t tbase = (size_t)bh * nblk * a.w;
  float nm = 0.f;
  int npos = 0, nsrc = 0;
  if (tid < min(a.block, a.L) && tid < a.w) {
    nm = a.top_m[tbase + tid];
    npos = a.top_pos[tbase + tid];
    nsrc = a.top_src[tbase + tid];
  }
  __syncthreads();
  for (int j = 0; j < nblk; ++j) {
    const int nt = min(min(a.block, a.L - j * a.block), a.w);
    int* mem = a.members + ((size_t)bh * nblk + j) * a.w;
    if (tid < n) mem[tid] = cs[cur][tid];
    if (tid == 0) a.member_count[(size_t)bh * nblk + j] = n;
    const float fm = nm;
    const int fp = npos, fs = nsrc;
    if (tid < nt) {
      tm[tid] = score_key(fm);
      tp[tid] = fp;
    }
    if (j + 1 < nblk && tid < min(min(a.block, a.L - (j + 1) * a.block), a.w)) {
      const size_t o = tbase + (size_t)(j + 1) * a.w + tid;
      nm = a.top_m[o];
      npos = a.top_pos[o];
      nsrc = a.top_src[o];
    }
    __syncthreads();
    const int nx = cur ^ 1;
    if (tid < n) {  // cache entry: block-top entries strictly ahead of it
      const float mx = score_key(cm[cur][tid]);
      const int px = cp[cur][tid];
      int lo = 0, hi = nt;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const bool ahead = rec ? tp[mid] > px : (tm[mid] > mx || (tm[mid] == mx && tp[mid] < px));
        if (ahead) lo = mid + 1;
        else hi = mid;
      }
      const int r = tid + lo;
      if (r < a.w) {
        cm[nx][r] = cm[cur][tid];
        cp[nx][r] = px;
        cs[nx][r] = cs[cur][tid];
      }
    }
    if (tid < nt) {  // block-top entry: cache entries ahead of it or tied with it
      const float mx = tm[tid];
      const int px = fp;
      int lo = 0, hi = n;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const float cmid = score_key(cm[cur][mid]);
        const int pmid = cp[cur][mid];
        const bool ahead = rec ? pmid >= px : (cmid > mx || (cmid == mx && pmid <= px));
        if (ahead) lo = mid + 1;
        else hi = mid;
      }
      const int r = tid + lo;
      if (r < a.w) {
        cm[nx][r] = fm;
        cp[nx][r] = fp;
        cs[nx][r] = fs;
      }
    }
    n = min(n + nt, a.w);
    cur = nx;
    __syncthreads();
  }
  if (tid < n) {
    a.final_src[(size_t)bh * a.w + tid] = cs[cur][tid];
    a.final_m[(size_t)bh * a.w + tid] = cm[cur][tid];
    a.final_pos[(size_t)bh * a.w + tid] = cp[cur][tid];
  }
  if (tid == 0) a.final_count[bh] = n;
}

// Read: 64 queries per workgroup against 32-key tiles, register-tiled so that
// every LDS read feeds several FMAs. Thread (qg, j) = (tid / 16, tid % 16)
// owns queries 4 qg .. 4 qg + 3; in the logits it takes keys 2 j, 2 j + 1 of
// the tile, in the weighted sum value columns 8 j .. 8 j + 7. Queries and
// keys are stored transposed ([d][query], [d][key]) and scaled by their RMS
// norm (the queries also by 1/sqrt(d_k)), so a logit is a plain dot product.
template <typename Tin>
__global__ __launch_bounds__(NT) void read_kernel(PrefillArgs a) {
  __shared__ float sQt[MAXD][QT + 4];
  __shared__ float sKt[MAXD][KT + 4];
  __shared__ float sV[KT][MAXD + 4];
  __shared__ float sPt[KT][QT + 4];
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

  {  // queries: 4 lanes per row, RMS-normalised, times 1/sqrt(d_k), transposed
    const int r = tid >> 2, part = tid & 3;
    float x[MAXD / 4];
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < MAXD / 4; ++u) {
      const int c = part + 4 * u;
      x[u] = (r < nq && c < dk) ? Elem<Tin>::load(qh, (size_t)(j0 + q0 + r) * dk + c) : 0.f;
      ss = fmaf(x[u], x[u], ss);
    }
    ss += __shfl_xor(ss, 1, 4);
    ss += __shfl_xor(ss, 2, 4);
    const float sc = inv_sqrt_d / sqrtf(ss / dk + a.rms_eps);
#pragma unroll
    for (int u = 0; u < MAXD / 4; ++u) sQt[part + 4 * u][r] = x[u] * sc;
  }
  const int qg = tid >> 4, jj = tid & 15;
  float M[4], Z[4], acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    M[i] = a.sink_logit ? a.sink_logit[bh % a.H] : -INFINITY;
    Z[i] = a.sink_logit ? 1.f : 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[i][c] = 0.f;
  }

  for (int e0 = 0; e0 < nkeys; e0 += KT) {
    __syncthreads();
    if (tid < KT) {
      const int e = e0 + tid;
      sSrc[tid] = e < nkeys ? (e < ncache ? mem[e] : j0 + e - ncache) : 0x7fffffff;
    }
    __syncthreads();
    {  // keys: 8 lanes per key, RMS-normalised, transposed
      const int kr = tid >> 3, part = tid & 7;
      const int src = sSrc[kr];
      float x[MAXD / 8];
      float ss = 0.f;
#pragma unroll
      for (int u = 0; u < MAXD / 8; ++u) {
        const int c = part + 8 * u;
        float v = 0.f;
        if (src != 0x7fffffff && c < dk)
          v = src >= 0 ? Elem<Tin>::load(kh, (size_t)src * dk + c) : ck[(size_t)(-1 - src) * dk + c];
        x[u] = v;
        ss = fmaf(v, v, ss);
      }
      ss += __shfl_xor(ss, 1, 8);
      ss += __shfl_xor(ss, 2, 8);
      ss += __shfl_xor(ss, 4, 8);
      const float sc = 1.f / sqrtf(ss / dk + a.rms_eps);
#pragma unroll
      for (int u = 0; u < MAXD / 8; ++u) sKt[part + 8 * u][kr] = x[u] * sc;
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
    // logits: 4 queries x 2 keys per thread
    float l[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) l[i][0] = l[i][1] = 0.f;
    for (int d = 0; d < dk; ++d) {
      const float4 qv = *reinterpret_cast<const float4*>(&sQt[d][4 * qg]);
      const float2 kv = *reinterpret_cast<const float2*>(&sKt[d][2 * jj]);
      const float qa[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        l[i][0] = fmaf(qa[i], kv.x, l[i][0]);
        l[i][1] = fmaf(qa[i], kv.y, l[i][1]);
      }
    }
    float p[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qtok = q0 + 4 * qg + i;  // relative to the block
      float tmax = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = e0 + 2 * jj + h;
        // cache members are always visible; block tokens up to the query itself
        const bool vis = 4 * qg + i < nq && e < nkeys && (e < ncache || e - ncache <= qtok);
        l[i][h] = vis ? l[i][h] : -INFINITY;
        tmax = fmaxf(tmax, l[i][h]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 1, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 2, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 4, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 8, 16));
      const float Mn = fmaxf(M[i], tmax);
      // rows with nothing visible yet keep M = -inf; their weights stay 0
      const float scale = Mn == -INFINITY ? 1.f : __expf(M[i] - Mn);
      float ps = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        p[i][h] = l[i][h] == -INFINITY ? 0.f : __expf(l[i][h] - Mn);
        ps += p[i][h];
      }
      ps += __shfl_xor(ps, 1, 16);
      ps += __shfl_xor(ps, 2, 16);
      ps += __shfl_xor(ps, 4, 16);
      ps += __shfl_xor(ps, 8, 16);
      Z[i] = fmaf(Z[i], scale, ps);
      M[i] = Mn;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[i][c] *= scale;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<float4*>(&sPt[2 * jj + h][4 * qg]) = make_float4(p[0][h], p[1][h], p[2][h], p[3][h]);
    __syncthreads();
    // weighted values: 4 queries x 8 value columns per thread
    for (int e = 0; e < KT; ++e) {
      const float4 pv = *reinterpret_cast<const float4*>(&sPt[e][4 * qg]);
      const float4 v0 = *reinterpret_cast<const float4*>(&sV[e][8 * jj]);
      const float4 v1 = *reinterpret_cast<const float4*>(&sV[e][8 * jj + 4]);
      const float pa[4] = {pv.x, pv.y, pv.z, pv.w};
      const float va[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[i][c] = fmaf(pa[i], va[c], acc[i][c]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qi = 4 * qg + i;
    if (qi < nq) {
      float* o = a.o_cache + ((size_t)bh * a.L + j0 + q0 + qi) * dv;
      const float inv = 1.f / Z[i];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (8 * jj + c < dv) o[8 * jj + c] = acc[i][c] * inv;
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
  if (a.w > kMaxW || a.block > kMaxBlock || a.w > NT) return hipErrorInvalidValue;
  hipLaunchKernelGGL(block_top_kernel, dim3(a.BH, nblk), dim3(NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(a.BH), dim3(NT), 0, s, a);
  e = hipGetLastError();
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
  return 4 * up((size_t)BH * nblk * w * 4) + up((size_t)BH * nblk * 4) +
         3 * up((size_t)BH * w * 4) + up((size_t)BH * 4) + up((size_t)BH * w * (dk + dv) * 4);
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
  p += up((size_t)a.BH * a.w * (a.dk + a.dv) * 4);
  a.top_m = reinterpret_cast<float*>(p);
  p += up((size_t)a.BH * nblk * a.w * 4);
  a.top_pos = reinterpret_cast<int*>(p);
  p += up((size_t)a.BH * nblk * a.w * 4);
  a.top_src = reinterpret_cast<int*>(p);
}

hipError_t launch_prefill(const PrefillArgs& a, bool in_bf16, hipStream_t s) {
  return in_bf16 ? prefill_typed<uint16_t>(a, s) : prefill_typed<float>(a, s);
}

}  // namespace kdn
