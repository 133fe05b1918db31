// hola.hip -- HOLA exact key/value cache for one decoding token per head.
//
// "A Hippocampus for Linear Attention", part 2/3:
//  sec. 3.3: keep the w tokens with the largest write score m seen so far;
//            the score is fixed at write time, so an online insert is exact.
//  sec. 3.4 eq. (7): read with RMS-normalised q, k at logit scale 1/sqrt(d)
//            (softmax over the visible set).
//  sec. 3.3 (visible set): cache + the current block's causal tokens (here the
//            current token) + one optional null sink.
// The read uses the cache as it stood before this token; then the insert.
//
// One workgroup (256 lanes) per head. Logits: 32 lanes per cached row (8 rows
// per pass), 16-byte loads. Weighted value sum: lane (rg, cg) accumulates
// columns of group cg over rows rg, rg + 8, ...; partial sums meet in LDS.
// With 16-byte rows and at most 64 slots, every key and value row a lane
// needs (8 of each) is loaded into registers before anything else, so the
// value reads are in flight while the logits and the softmax are formed.
// Eviction: one wavefront takes the lexicographic minimum of (m, -pos) with
// shuffles, so the choice is deterministic and uses no atomics. A NaN score
// ranks below every other score (ranked as -infinity, stored unchanged), as in
// the prompt cache. The recency control of sec. 4.5 evicts the smallest
// position instead.
#include "kdn_internal.h"

namespace kdn {
namespace {

constexpr int NT = 256;
constexpr int WMAX = 256;
constexpr int PF = 8;  // rows per lane held in registers (capacities up to 8 * PF)

// ranking key of a score: NaN ranks below every other score
__device__ __forceinline__ float rank_key(float m) { return m == m ? m : -INFINITY; }

__device__ __forceinline__ float sum32(float x) {
  for (int off = 16; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <bool VEC>
__device__ __forceinline__ void dot_row(const float* row, const float* sq, int d, int cg, float& qk,
                                        float& kk) {
  qk = 0.f;
  kk = 0.f;
  if (VEC) {
    if (4 * cg < d) {
      const float4 x = *reinterpret_cast<const float4*>(row + 4 * cg);
      qk = x.x * sq[4 * cg] + x.y * sq[4 * cg + 1] + x.z * sq[4 * cg + 2] + x.w * sq[4 * cg + 3];
      kk = x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
    }
  } else {
    for (int c = cg; c < d; c += 32) {
      const float x = row[c];
      qk = fmaf(x, sq[c], qk);
      kk = fmaf(x, x, kk);
    }
  }
}

template <bool VEC, bool REGS>
__global__ __launch_bounds__(NT) void hola_kernel(const float* __restrict__ q,
                                                  const float* __restrict__ k,
                                                  const float* __restrict__ v,
                                                  const float* __restrict__ m, int32_t t,
                                                  float* __restrict__ cache_k,
                                                  float* __restrict__ cache_v,
                                                  float* __restrict__ cache_m,
                                                  int32_t* __restrict__ cache_pos,
                                                  int32_t* __restrict__ cache_count,
                                                  const float* __restrict__ sink_logit,
                                                  float* __restrict__ o_cache, float rms_eps,
                                                  int H, int dk, int dv, int w, int recency) {
  // one entry per lane: every lane stores its element (0 past d_k, d_v)
  __shared__ __align__(16) float sq[NT], sk[NT], sv[NT];
  __shared__ float sl[WMAX + 2];
  __shared__ float red[8][128];
  __shared__ float sscal[4];
  __shared__ int sslot;
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, cg = tid & 31, rg = tid >> 5;
  const int n = min(max(cache_count[bh], 0), w);  // a corrupt count cannot index past the cache
  const float* ck = cache_k + (size_t)bh * w * dk;
  const float* cv = cache_v + (size_t)bh * w * dv;

  // the token's own rows, then (REGS: capacity at most 8 PF, 16-byte rows)
  // rows rg + 8 i of the cache, all without branches (buffer reads past the
  // n filled rows, or past the token's rows, return 0; columns past d_k or
  // d_v are never used), so that the first wait takes in only the token's rows
  const float xq = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
      make_rsrc(q + (size_t)bh * dk, dk * sizeof(float)), tid * 4, 0, 0));
  const float xk = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
      make_rsrc(k + (size_t)bh * dk, dk * sizeof(float)), tid * 4, 0, 0));
  const float xv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
      make_rsrc(v + (size_t)bh * dv, dv * sizeof(float)), tid * 4, 0, 0));
  constexpr bool regs = REGS;
  float4 kr[PF], vr[PF];
  if constexpr (REGS) {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(ck, (size_t)n * dk * sizeof(float));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(cv, (size_t)n * dv * sizeof(float));
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int j = rg + 8 * i;
      kr[i] = stream_load16(rk, (j * dk + 4 * cg) * (int)sizeof(float));
      vr[i] = stream_load16(rv, (j * dv + 4 * cg) * (int)sizeof(float));
    }
  }
  sq[tid] = xq;
  sk[tid] = xk;
  sv[tid] = xv;
  __syncthreads();
  if (tid < 64) {  // one wavefront: |q|^2
    float x = 0.f;
    for (int c = lane; c < dk; c += 64) x = fmaf(sq[c], sq[c], x);
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    if (lane == 0) sscal[0] = 1.f / sqrtf(x / dk + rms_eps) * (1.f / sqrtf((float)dk));
  }
  __syncthreads();
  const float qscale = sscal[0];

  // logits of the cached rows and of the current token (index n)
  if (regs) {
    auto logit = [&](int j, float4 x, bool cur) {
      float qk = 0.f, kk = 0.f;
      if (4 * cg < dk) {
        if (cur) x = *reinterpret_cast<const float4*>(sk + 4 * cg);
        const float4 y = *reinterpret_cast<const float4*>(sq + 4 * cg);
        qk = x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
        kk = x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
      }
      qk = sum32(qk);
      kk = sum32(kk);
      if (cg == 0) sl[j] = qk * qscale / sqrtf(kk / dk + rms_eps);
    };
#pragma unroll
    for (int i = 0; i < PF; ++i)
      if (rg + 8 * i < n) logit(rg + 8 * i, kr[i], false);
    if (rg == (n & 7)) logit(n, kr[0], true);
  } else {
    for (int j = rg; j <= n; j += 8) {
      float qk, kk;
      dot_row<VEC>(j < n ? ck + (size_t)j * dk : sk, sq, dk, cg, qk, kk);
      qk = sum32(qk);
      kk = sum32(kk);
      if (cg == 0) sl[j] = qk * qscale / sqrtf(kk / dk + rms_eps);
    }
  }
  const int nl = n + 1 + (sink_logit ? 1 : 0);
  if (sink_logit && tid == 0) sl[n + 1] = sink_logit[bh % H];
  __syncthreads();

  // softmax weights (one wavefront), in place
  if (tid < 64) {
    float mx = -INFINITY;
    for (int j = lane; j < nl; j += 64) mx = fmaxf(mx, sl[j]);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float den = 0.f;
    for (int j = lane; j < nl; j += 64) {
      const float p = expf(sl[j] - mx);
      sl[j] = p;
      den += p;
    }
    for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off, 64);
    if (lane == 0) sscal[1] = 1.f / den;
  }
  __syncthreads();

  // weighted value sum (the sink's value is 0)
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (regs) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int j = rg + 8 * i;
      if (j < n) {
        const float p = sl[j];
        acc[0] = fmaf(p, vr[i].x, acc[0]);
        acc[1] = fmaf(p, vr[i].y, acc[1]);
        acc[2] = fmaf(p, vr[i].z, acc[2]);
        acc[3] = fmaf(p, vr[i].w, acc[3]);
      }
    }
    if (rg == (n & 7) && 4 * cg < dv) {
      const float p = sl[n];
      const float4 x = *reinterpret_cast<const float4*>(sv + 4 * cg);
      acc[0] = fmaf(p, x.x, acc[0]);
      acc[1] = fmaf(p, x.y, acc[1]);
      acc[2] = fmaf(p, x.z, acc[2]);
      acc[3] = fmaf(p, x.w, acc[3]);
    }
  }
  for (int j = regs ? n + 1 : rg; j <= n; j += 8) {
    const float p = sl[j];
    const float* row = j < n ? cv + (size_t)j * dv : sv;
    if (VEC) {
      if (4 * cg < dv) {
        const float4 x = *reinterpret_cast<const float4*>(row + 4 * cg);
        acc[0] = fmaf(p, x.x, acc[0]);
        acc[1] = fmaf(p, x.y, acc[1]);
        acc[2] = fmaf(p, x.z, acc[2]);
        acc[3] = fmaf(p, x.w, acc[3]);
      }
    } else {
      for (int c = 0; c < 4; ++c) {
        const int col = cg + 32 * c;
        if (col < dv) acc[c] = fmaf(p, row[col], acc[c]);
      }
    }
  }
  for (int c = 0; c < 4; ++c) {
    const int col = VEC ? 4 * cg + c : cg + 32 * c;
    red[rg][col] = acc[c];
  }
  // eviction choice (wavefront 0) while the partial sums settle
  if (tid < 64) {
    const float mt = rank_key(m[bh]);
    int slot = -1;
    if (n < w) {
      slot = n;
    } else {
      float bm = INFINITY;
      int bp = -1, bs = -1;
      for (int j = lane; j < w; j += 64) {
        // recency: rank by position alone
        const float mj = recency ? 0.f : rank_key(cache_m[(size_t)bh * w + j]);
        const int pj = recency ? -cache_pos[(size_t)bh * w + j] : cache_pos[(size_t)bh * w + j];
        if (bs < 0 || mj < bm || (mj == bm && pj > bp)) {
          bm = mj;
          bp = pj;
          bs = j;
        }
      }
      for (int off = 32; off > 0; off >>= 1) {
        const float om = __shfl_xor(bm, off, 64);
        const int op = __shfl_xor(bp, off, 64);
        const int os = __shfl_xor(bs, off, 64);
        const bool take = (os >= 0) && (bs < 0 || om < bm || (om == bm && op > bp));
        if (take) {
          bm = om;
          bp = op;
          bs = os;
        }
      }
      if (recency || mt > bm) slot = bs;
    }
    if (lane == 0) sslot = slot;
  }
  __syncthreads();
  if (tid < dv) {
    float s = 0.f;
    for (int g = 0; g < 8; ++g) s += red[g][tid];
    o_cache[(size_t)bh * dv + tid] = s * sscal[1];
  }
  const int slot = sslot;
  if (slot >= 0) {
    if (tid < dk) cache_k[((size_t)bh * w + slot) * dk + tid] = sk[tid];
    if (tid < dv) cache_v[((size_t)bh * w + slot) * dv + tid] = sv[tid];
    if (tid == 0) {
      cache_m[(size_t)bh * w + slot] = m[bh];
      cache_pos[(size_t)bh * w + slot] = t;
      if (n < w) cache_count[bh] = n + 1;
    }
  }
}

}  // namespace

hipError_t launch_hola(const float* q, const float* k, const float* v, const float* m, int32_t t,
                       float* cache_k, float* cache_v, float* cache_m, int32_t* cache_pos,
                       int32_t* cache_count, const float* sink_logit, float* o_cache, float rms_eps,
                       int B, int H, int dk, int dv, int w, int policy, hipStream_t s) {
  const bool vec = dk % 4 == 0 && dv % 4 == 0 &&
                   ((reinterpret_cast<uintptr_t>(cache_k) | reinterpret_cast<uintptr_t>(cache_v)) &
                    15) == 0;
  const int nb = B * H;
  if (vec && w <= 8 * PF) {
    KDN_LAUNCH_NAMED("hola_kernel<true, true>", (hola_kernel<true, true>), dim3(nb), dim3(NT), 0,
                     s, q, k, v, m, t, cache_k, cache_v, cache_m, cache_pos, cache_count,
                     sink_logit, o_cache, rms_eps, H, dk, dv, w, policy);
  } else if (vec) {
    KDN_LAUNCH_NAMED("hola_kernel<true, false>", (hola_kernel<true, false>), dim3(nb), dim3(NT),
                     0, s, q, k, v, m, t, cache_k, cache_v, cache_m, cache_pos, cache_count,
                     sink_logit, o_cache, rms_eps, H, dk, dv, w, policy);
  } else {
    KDN_LAUNCH_NAMED("hola_kernel<false, false>", (hola_kernel<false, false>), dim3(nb), dim3(NT),
                     0, s, q, k, v, m, t, cache_k, cache_v, cache_m, cache_pos, cache_count,
                     sink_logit, o_cache, rms_eps, H, dk, dv, w, policy);
  }
  return hipGetLastError();
}

}  // namespace kdn
