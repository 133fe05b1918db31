// cov.hip -- covariance recursions of the Kalman writes and their per-token gains.
//
// "Kalman Delta Networks: Uncertainty-aware Associative Memory", abstract: the
// transition propagates the memory and its uncertainty; the Kalman gain
// weights each residual write. The covariance recursion never reads the
// state S, so the gains are computed here, before the state scan, and the scan
// consumes them as write vectors.
//
// Per token (process noise Q_t = (1 - alpha_t^2) sigma^2):
//   P-  = alpha^2 P + Q I,   u = P- k,   s = k^T u + r,   g = u / s,   P = P- - u u^T / s
// DIAG keeps p = diag(P) and projects after every step onto diagonal
// covariances by keeping the diagonal of the precision (mean-field):
//   p-_i = alpha^2 p_i + Q,  g_i = p-_i k_i / (sum_j p-_j k_j^2 + r),  p_i = p-_i r / (r + p-_i k_i^2).
// Each coordinate's map p -> p_new is a linear-fractional (Moebius) map, so a
// run of tokens composes into one 2x2 matrix (the abstract's "uncertainty
// recurrences are Mobius maps"). The DIAG path uses that: one pass composes the
// maps of every chunk in parallel, a short sequential pass over chunks applies
// them to get every chunk's starting variances, and a third pass recomputes the
// per-token values of every chunk in parallel.
#include <type_traits>

#include "kdn_internal.h"

namespace kdn {
namespace {

constexpr int kGainBatch = 16;  // tokens whose inputs are loaded together

// Map of one token on (p, 1), projectively: p_new = (m00 p + m01) / (m10 p + m11).
// From p- = a^2 p + Q and p_new = r p- / (k^2 p- + r). All entries are >= 0,
// so products never cancel.
__device__ __forceinline__ void token_map(float a, float qvar, float r, float kv, float& t00,
                                          float& t01, float& t10, float& t11) {
  const float a2 = a * a;
  const float Q = (1.f - a) * (1.f + a) * qvar;
  const float k2 = kv * kv;
  t00 = r * a2;
  t01 = r * Q;
  t10 = k2 * a2;
  t11 = fmaf(k2, Q, r);
}

template <typename Tk>
__global__ __launch_bounds__(128) void diag_maps_kernel(const Tk* k, const float* alpha,
                                                        const float* r, float qvar, float4* maps,
                                                        int L, int dk, int C, int nchunks) {
  __shared__ float sa[64], sr[64];
  const int bh = blockIdx.x, c = blockIdx.y, i = threadIdx.x;
  const int t0 = c * C, n = min(C, L - t0);
  if (i < n) {
    const size_t g = (size_t)bh * L + t0 + i;
    sa[i] = alpha ? alpha[g] : 1.f;
    sr[i] = r ? r[g] : 1.f;
  }
  __syncthreads();
  if (i >= dk) return;
  float m00 = 1.f, m01 = 0.f, m10 = 0.f, m11 = 1.f;
  // k of a batch of tokens loaded together (tokens past the chunk read token
  // n - 1 and are not used): one memory latency per batch
  for (int tb = 0; tb < n; tb += kGainBatch) {
    float kv[kGainBatch];
#pragma unroll
    for (int u = 0; u < kGainBatch; ++u)
      kv[u] = Elem<Tk>::load(k, ((size_t)bh * L + t0 + min(tb + u, n - 1)) * dk + i);
#pragma unroll
    for (int u = 0; u < kGainBatch; ++u) {
      // every token of the batch is formed (t < 64 stays inside sa, sr); only
      // those inside the chunk are applied, so the loads stay ahead of all uses
      const int t = tb + u;
      const bool in = t < n;
      float t00, t01, t10, t11;
      token_map(sa[t], qvar, sr[t], kv[u], t00, t01, t10, t11);
      const float n00 = fmaf(t00, m00, t01 * m10), n01 = fmaf(t00, m01, t01 * m11);
      const float n10 = fmaf(t10, m00, t11 * m10), n11 = fmaf(t10, m01, t11 * m11);
      // projective scale: any positive factor will do, so an approximate reciprocal
      const float sc = __builtin_amdgcn_rcpf(fmaxf(fmaxf(n00, n01), fmaxf(n10, n11)));
      m00 = in ? n00 * sc : m00;
      m01 = in ? n01 * sc : m01;
      m10 = in ? n10 * sc : m10;
      m11 = in ? n11 * sc : m11;
    }
  }
  maps[((size_t)bh * nchunks + c) * dk + i] = make_float4(m00, m01, m10, m11);
}

// One thread per (head, coordinate): the variance at every chunk start, by
// applying the chunk maps in order; stored over the map's first entry.
__global__ __launch_bounds__(128) void diag_prefix_kernel(const float* cov_in, float4* maps,
                                                          int BH, int dk, int nchunks) {
  const int idx = blockIdx.x * 128 + threadIdx.x;
  if (idx >= BH * dk) return;
  const int bh = idx / dk, i = idx - bh * dk;
  float p = cov_in[idx];
  float4* m = maps + (size_t)bh * nchunks * dk + i;
  for (int c0 = 0; c0 < nchunks; c0 += 8) {  // eight maps in flight at a time
    float4 M[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < nchunks) M[j] = m[(size_t)(c0 + j) * dk];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < nchunks) {
        m[(size_t)(c0 + j) * dk].x = p;
        p = fmaf(M[j].x, p, M[j].y) / fmaf(M[j].z, p, M[j].w);
      }
  }
}

// One wavefront per (head, chunk): lane l carries coordinates l and l + 64
// through the chunk's tokens in order; the sum over coordinates in
// s_t = r_t + sum_i p-_i k_i^2 is a wavefront reduction, so the gains of token
// t are written as soon as it is done. No LDS and no barriers, so many
// wavefronts per SIMD hide the memory latency.
// Sum over the 64 lanes, every lane gets it (all 64 lanes must be active):
// quad steps by DPP, 4-16 by swizzles within each half, the halves by one
// lane swap.
__device__ __forceinline__ float wave_sum64(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));  // ^1
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));  // ^2
  x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (4 << 10)));
  x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (8 << 10)));
  x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (16 << 10)));
  // after the swap, lanes 0-31 find the upper half's value in the second
  // result and lanes 32-63 the lower half's in the first
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return x + __uint_as_float(__lane_id() < 32 ? sw[1] : sw[0]);
}

template <typename Tk, typename Tg>
__global__ __launch_bounds__(256) void diag_gains_kernel(const Tk* k, const float* alpha,
                                                         const float* r, float* cov_out,
                                                         float qvar, const float4* maps,
                                                         Tg* gains, int BH, int L, int dk,
                                                         int C, int nchunks) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wave >= BH * nchunks) return;
  const int bh = wave / nchunks, c = wave - bh * nchunks;
  const int t0 = c * C, n = min(C, L - t0);
  const size_t tok = (size_t)bh * L + t0;
  const int i0 = lane, i1 = lane + 64;
  const bool ok0 = i0 < dk, ok1 = i1 < dk;
  const float4* mp = maps + ((size_t)bh * nchunks + c) * dk;
  float p0 = ok0 ? mp[i0].x : 0.f, p1 = ok1 ? mp[i1].x : 0.f;  // chunk-start variances
  for (int t = 0; t < n; ++t) {
    const size_t g = tok + t;
    const float a = alpha ? alpha[g] : 1.f, rt = r ? r[g] : 1.f;
    const float a2 = a * a, Q = (1.f - a) * (1.f + a) * qvar;
    const float k0 = ok0 ? Elem<Tk>::load(k, g * dk + i0) : 0.f;
    const float k1 = ok1 ? Elem<Tk>::load(k, g * dk + i1) : 0.f;
    const float pm0 = fmaf(a2, p0, Q), pm1 = fmaf(a2, p1, Q);
    const float pk0 = pm0 * k0, pk1 = pm1 * k1;
    // reciprocals by v_rcp_f32 (1 ulp): the kernel is bound by its
    // instruction count, and exact divisions are ten instructions each
    const float inv = __builtin_amdgcn_rcpf(rt + wave_sum64(fmaf(pk0, k0, pk1 * k1)));
    if (ok0) Elem<Tg>::store(gains, g * dk + i0, pk0 * inv);
    if (ok1) Elem<Tg>::store(gains, g * dk + i1, pk1 * inv);
    p0 = pm0 * rt * __builtin_amdgcn_rcpf(fmaf(pk0, k0, rt));
    p1 = pm1 * rt * __builtin_amdgcn_rcpf(fmaf(pk1, k1, rt));
  }
  if (c == nchunks - 1 && cov_out) {
    if (ok0) cov_out[(size_t)bh * dk + i0] = p0;
    if (ok1) cov_out[(size_t)bh * dk + i1] = p1;
  }
}

// Full covariance, one workgroup per head, sequential over tokens (d_k <= 64).
template <typename Tk, typename Tg>
__global__ __launch_bounds__(256) void full_gains_kernel(const Tk* k, const float* alpha,
                                                         const float* r, const float* cov_in,
                                                         float* cov_out, float qvar, Tg* gains,
                                                         int L, int dk) {
  __shared__ float sP[64 * 65];
  __shared__ float sU[64];
  __shared__ float sKv[64];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int PP = dk + 1;
  for (int idx = tid; idx < dk * dk; idx += 256) {
    const int i = idx / dk, j = idx - i * dk;
    sP[i * PP + j] = cov_in[(size_t)bh * dk * dk + idx];
  }
  for (int t = 0; t < L; ++t) {
    const size_t g = (size_t)bh * L + t;
    const float a = alpha ? alpha[g] : 1.f;
    const float rt = r ? r[g] : 1.f;
    const float Q = (1.f - a) * (1.f + a) * qvar;
    if (tid < dk) sKv[tid] = Elem<Tk>::load(k, g * dk + tid);
    __syncthreads();
    for (int idx = tid; idx < dk * dk; idx += 256) {
      const int i = idx / dk, j = idx - i * dk;
      sP[i * PP + j] = fmaf(a * a, sP[i * PP + j], i == j ? Q : 0.f);
    }
    __syncthreads();
    if (tid < dk) {
      float u = 0.f;
      for (int j = 0; j < dk; ++j) u = fmaf(sP[tid * PP + j], sKv[j], u);
      sU[tid] = u;
    }
    __syncthreads();
    float s = rt;
    for (int j = 0; j < dk; ++j) s = fmaf(sKv[j], sU[j], s);
    const float inv = 1.f / s;
    if (tid < dk) Elem<Tg>::store(gains, g * dk + tid, sU[tid] * inv);
    for (int idx = tid; idx < dk * dk; idx += 256) {
      const int i = idx / dk, j = idx - i * dk;
      sP[i * PP + j] -= sU[i] * sU[j] * inv;
    }
    __syncthreads();
  }
  if (cov_out) {
    for (int idx = tid; idx < dk * dk; idx += 256) {
      const int i = idx / dk, j = idx - i * dk;
      cov_out[(size_t)bh * dk * dk + idx] = sP[i * PP + j];
    }
  }
}

// ---------------------------------------------------------------- isotropic
// One variance p per head ("Kalman Delta Networks", abstract: the isotropic
// variant): p- = alpha^2 p + Q, gain p- k / (p- ||k||^2 + r) = beta_t k with
// beta_t = p- / (p- ||k||^2 + r), and the precision projected onto multiples
// of the identity, 1/p = 1/p- + ||k||^2 / (d_k r). The write is then the delta
// write with that beta. In p, one token is the Moebius map
// p -> (a^2 p + Q) / (c a^2 p + c Q + 1) with c = ||k||^2 / (d_k r).

// A token's map on p, projectively: p -> (a^2 p + Q) / (c a^2 p + c Q + 1), c =
// ||k||^2 / (d_k r), as the matrix [[a^2, Q], [c a^2, c Q + 1]].
struct Mob {
  float a, b, c, d;
};
__device__ __forceinline__ Mob mob_token(float al, float rt, float kk, float qvar, int dk) {
  const float a2 = al * al, Q = (1.f - al) * (1.f + al) * qvar, cc = kk / (dk * rt);
  return Mob{a2, Q, cc * a2, fmaf(cc, Q, 1.f)};
}
// x after y (x y), scaled so that the largest entry is 1 (any positive scale
// is the same map).
__device__ __forceinline__ Mob mob_mul(Mob x, Mob y) {
  Mob z{fmaf(x.a, y.a, x.b * y.c), fmaf(x.a, y.b, x.b * y.d), fmaf(x.c, y.a, x.d * y.c),
        fmaf(x.c, y.b, x.d * y.d)};
  const float sc = __builtin_amdgcn_rcpf(fmaxf(fmaxf(z.a, z.b), fmaxf(z.c, z.d)));
  return Mob{z.a * sc, z.b * sc, z.c * sc, z.d * sc};
}
__device__ __forceinline__ Mob mob_shfl_up(Mob x, int off, int lane) {
  Mob y{__shfl_up(x.a, off, 64), __shfl_up(x.b, off, 64), __shfl_up(x.c, off, 64),
        __shfl_up(x.d, off, 64)};
  return lane >= off ? y : Mob{1.f, 0.f, 0.f, 1.f};
}
// Inclusive scan over the wavefront in token order: lane t gets M_t ... M_0.
__device__ __forceinline__ Mob mob_scan(Mob m, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) m = mob_mul(m, mob_shfl_up(m, off, lane));
  return m;
}

// One wavefront per (head, chunk), lane t = token t: ||k_t||^2 (the wavefront
// reads each key row together, coalesced, and reduces it) and the chunk's map,
// the product of its token maps by a wavefront scan.
template <typename Tk>
__global__ __launch_bounds__(256) void iso_maps_kernel(const Tk* k, const float* alpha,
                                                       const float* r, float qvar, float* kk,
                                                       float4* maps, int BH, int L, int dk, int C,
                                                       int nchunks) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wave >= BH * nchunks) return;
  const int bh = wave / nchunks, c = wave - bh * nchunks;
  const int t0 = c * C, n = min(C, L - t0);
  const size_t g = (size_t)bh * L + t0 + lane;
  const size_t row0 = (size_t)bh * L + t0;
  float mine = 0.f;
  if constexpr (std::is_same<Tk, uint16_t>::value) {
    if (dk == 128) {
      // 16 lanes per row, 16-byte loads: rows 4 j + lane / 16 in pass j, all
      // 16 passes in flight; lane t then picks its row's sum
      const int q = lane >> 4, e = lane & 15;
      float part[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int t = 4 * j + q;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (t < n) u = *reinterpret_cast<const uint4*>(k + (row0 + t) * 128 + 8 * e);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
        float acc = 0.f;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float lo = __uint_as_float(w[h] << 16), hi = __uint_as_float(w[h] & 0xffff0000u);
          acc = fmaf(lo, lo, fmaf(hi, hi, acc));
        }
        part[j] = acc;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float x = part[j];
        x += __shfl_xor(x, 8, 16);
        x += __shfl_xor(x, 4, 16);
        x += __shfl_xor(x, 2, 16);
        x += __shfl_xor(x, 1, 16);
        const float v = __shfl(x, 16 * (lane & 3), 64);  // row 4 j + lane % 4
        if ((lane >> 2) == j) mine = v;
      }
      goto have_norms;
    }
  }
  for (int t = 0; t < n; ++t) {
    const float x0 = lane < dk ? Elem<Tk>::load(k, (row0 + t) * dk + lane) : 0.f;
    const float x1 = lane + 64 < dk ? Elem<Tk>::load(k, (row0 + t) * dk + lane + 64) : 0.f;
    const float sq = wave_sum64(fmaf(x0, x0, x1 * x1));
    if (lane == t) mine = sq;
  }
have_norms:
  Mob m{1.f, 0.f, 0.f, 1.f};
  if (lane < n) {
    kk[g] = mine;
    m = mob_token(alpha ? alpha[g] : 1.f, r ? r[g] : 1.f, mine, qvar, dk);
  }
  m = mob_scan(m, lane);
  const Mob tot{__shfl(m.a, n - 1, 64), __shfl(m.b, n - 1, 64), __shfl(m.c, n - 1, 64),
                __shfl(m.d, n - 1, 64)};
  if (lane == 0) maps[(size_t)bh * nchunks + c] = make_float4(tot.a, tot.b, tot.c, tot.d);
}

// One thread per head: the variance at every chunk start (over the map's
// first entry).
__global__ __launch_bounds__(64) void iso_prefix_kernel(const float* cov_in, float4* maps, int BH,
                                                        int nchunks) {
  const int bh = blockIdx.x * 64 + threadIdx.x;
  if (bh >= BH) return;
  float p = cov_in[bh];
  float4* m = maps + (size_t)bh * nchunks;
  for (int c0 = 0; c0 < nchunks; c0 += 8) {  // eight maps in flight at a time
    float4 M[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < nchunks) M[j] = m[c0 + j];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < nchunks) {
        m[c0 + j].x = p;
        p = fmaf(M[j].x, p, M[j].y) / fmaf(M[j].z, p, M[j].w);
      }
  }
}

// One wavefront per (head, chunk), lane t = token t: the variance before the
// token from the chunk's starting p (iso_prefix_kernel) and an exclusive scan
// of the token maps, then the write strength beta_t.
__global__ __launch_bounds__(256) void iso_beta_kernel(const float* alpha, const float* r,
                                                       const float* kk, float* cov_out, float qvar,
                                                       const float4* maps, float* beta, int BH,
                                                       int L, int dk, int C, int nchunks) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wave >= BH * nchunks) return;
  const int bh = wave / nchunks, c = wave - bh * nchunks;
  const int t0 = c * C, n = min(C, L - t0);
  const size_t g = (size_t)bh * L + t0 + lane;
  const float p0 = maps[(size_t)bh * nchunks + c].x;  // the chunk's starting variance
  float al = 1.f, rt = 1.f, kt = 0.f;
  Mob m{1.f, 0.f, 0.f, 1.f};
  if (lane < n) {
    al = alpha ? alpha[g] : 1.f;
    rt = r ? r[g] : 1.f;
    kt = kk[g];
    m = mob_token(al, rt, kt, qvar, dk);
  }
  const Mob e = mob_shfl_up(mob_scan(m, lane), 1, lane);  // M_{t-1} ... M_0
  const float p = fmaf(e.a, p0, e.b) / fmaf(e.c, p0, e.d);   // variance after token t - 1
  const float pm = fmaf(al * al, p, (1.f - al) * (1.f + al) * qvar);
  if (lane < n) beta[g] = pm / fmaf(pm, kt, rt);
  if (c == nchunks - 1 && cov_out && lane == n - 1)
    cov_out[bh] = pm * (dk * rt) / fmaf(pm, kt, dk * rt);
}

template <typename Tk, typename Tg>
hipError_t diag_typed(const void* k, const float* alpha, const float* r, const float* cov_in,
                      float* cov_out, float qvar, void* gains, float* maps, int BH, int L, int dk,
                      int C, hipStream_t s) {
  const int nchunks = (L + C - 1) / C;
  hipLaunchKernelGGL(diag_maps_kernel<Tk>, dim3(BH, nchunks), dim3(128), 0, s,
                     static_cast<const Tk*>(k), alpha, r, qvar, reinterpret_cast<float4*>(maps), L,
                     dk, C, nchunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(diag_prefix_kernel, dim3((BH * dk + 127) / 128), dim3(128), 0, s, cov_in,
                     reinterpret_cast<float4*>(maps), BH, dk, nchunks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int waves = BH * nchunks;
  hipLaunchKernelGGL((diag_gains_kernel<Tk, Tg>), dim3((waves + 3) / 4), dim3(256), 0, s,
                     static_cast<const Tk*>(k), alpha, r, cov_out, qvar,
                     reinterpret_cast<const float4*>(maps), static_cast<Tg*>(gains), BH, L, dk, C,
                     nchunks);
  return hipGetLastError();
}

template <typename Tk, typename Tg>
hipError_t full_typed(const void* k, const float* alpha, const float* r, const float* cov_in,
                      float* cov_out, float qvar, void* gains, int BH, int L, int dk,
                      hipStream_t s) {
  hipLaunchKernelGGL((full_gains_kernel<Tk, Tg>), dim3(BH), dim3(256), 0, s,
                     static_cast<const Tk*>(k), alpha, r, cov_in, cov_out, qvar,
                     static_cast<Tg*>(gains), L, dk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_diag_gains(const void* k, bool k_bf16, const float* alpha, const float* r,
                             const float* cov_in, float* cov_out, float q_noise_var, void* gains,
                             bool gains_f16, float* maps, int BH, int L, int dk, int chunk,
                             hipStream_t s) {
  if (k_bf16)
    return gains_f16 ? diag_typed<uint16_t, _Float16>(k, alpha, r, cov_in, cov_out, q_noise_var,
                                                       gains, maps, BH, L, dk, chunk, s)
                      : diag_typed<uint16_t, float>(k, alpha, r, cov_in, cov_out, q_noise_var,
                                                    gains, maps, BH, L, dk, chunk, s);
  return gains_f16 ? diag_typed<float, _Float16>(k, alpha, r, cov_in, cov_out, q_noise_var, gains,
                                                  maps, BH, L, dk, chunk, s)
                    : diag_typed<float, float>(k, alpha, r, cov_in, cov_out, q_noise_var, gains,
                                               maps, BH, L, dk, chunk, s);
}

hipError_t launch_iso_beta(const void* k, bool k_bf16, const float* alpha, const float* r,
                          const float* cov_in, float* cov_out, float q_noise_var, float* beta,
                          float* kk, float* maps, int BH, int L, int dk, int chunk,
                          hipStream_t s) {
  const int nchunks = (L + chunk - 1) / chunk;
  const int blocks = (BH * nchunks + 3) / 4;  // four wavefronts per workgroup
  if (k_bf16)
    hipLaunchKernelGGL(iso_maps_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(k), alpha, r, q_noise_var, kk,
                       reinterpret_cast<float4*>(maps), BH, L, dk, chunk, nchunks);
  else
    hipLaunchKernelGGL(iso_maps_kernel<float>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const float*>(k), alpha, r, q_noise_var, kk,
                       reinterpret_cast<float4*>(maps), BH, L, dk, chunk, nchunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(iso_prefix_kernel, dim3((BH + 63) / 64), dim3(64), 0, s, cov_in,
                     reinterpret_cast<float4*>(maps), BH, nchunks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(iso_beta_kernel, dim3(blocks), dim3(256), 0, s, alpha, r, kk, cov_out,
                     q_noise_var, reinterpret_cast<const float4*>(maps), beta, BH, L, dk, chunk,
                     nchunks);
  return hipGetLastError();
}

hipError_t launch_full_gains(const void* k, bool k_bf16, const float* alpha, const float* r,
                             const float* cov_in, float* cov_out, float q_noise_var, void* gains,
                             bool gains_f16, int BH, int L, int dk, hipStream_t s) {
  if (k_bf16)
    return gains_f16 ? full_typed<uint16_t, _Float16>(k, alpha, r, cov_in, cov_out, q_noise_var,
                                                       gains, BH, L, dk, s)
                      : full_typed<uint16_t, float>(k, alpha, r, cov_in, cov_out, q_noise_var,
                                                    gains, BH, L, dk, s);
  return gains_f16 ? full_typed<float, _Float16>(k, alpha, r, cov_in, cov_out, q_noise_var, gains,
                                                  BH, L, dk, s)
                    : full_typed<float, float>(k, alpha, r, cov_in, cov_out, q_noise_var, gains,
                                               BH, L, dk, s);
}

}  // namespace kdn
