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
// run of tokens composes into one 2x2 matrix ("Kalman Delta Networks:
// Uncertainty-aware Associative Memory", abstract, where the variance
// recursions are identified as Moebius maps). The DIAG path uses that: one pass composes the
// maps of every chunk in parallel, an associative scan over chunks turns them
// into every chunk's starting variances, and a third pass recomputes the
// per-token values of every chunk in parallel (on the matrix-core path the
// chunks are 32-token halves and the prepare kernel makes that third pass).
#include <type_traits>

#include "kdn_internal.h"

namespace kdn {
namespace {

constexpr int kGainBatch = 16;  // tokens whose inputs are loaded together

// One workgroup per (head, chunk), thread i = coordinate i: the composite of
// the chunk's token maps. The map of one token on (p, 1), projectively, is
// p_new = (m00 p + m01) / (m10 p + m11) with, from p- = a^2 p + Q and
// p_new = r p- / (k^2 p- + r): m00 = r a^2, m01 = r Q, m10 = k^2 a^2,
// m11 = k^2 Q + r. All entries are >= 0, so products never cancel.
template <typename Tk>
__global__ __launch_bounds__(128) void diag_maps_kernel(const Tk* k, const float* alpha,
                                                        const float* r, float qvar, float4* maps,
                                                        int L, int dk, int C, int nchunks) {
  // per token: r a^2, r Q, a^2, Q and r (what of the map does not depend on
  // the key); tokens past the sequence get the identity map
  __shared__ float4 sp[64];
  __shared__ float sr[64];
  const int bh = blockIdx.x, c = blockIdx.y, i = threadIdx.x;
  const int t0 = c * C, n = min(C, L - t0);
  if (i < 64) {
    const bool in = i < n;
    const size_t g = (size_t)bh * L + t0 + min(i, n - 1);
    const float a = in && alpha ? alpha[g] : 1.f, rt = in && r ? r[g] : 1.f;
    const float a2 = a * a, Q = (1.f - a) * (1.f + a) * qvar;
    sp[i] = in ? make_float4(rt * a2, rt * Q, a2, Q) : make_float4(1.f, 0.f, 0.f, 0.f);
    sr[i] = rt;
  }
  __syncthreads();
  if (i >= dk) return;
  float m00 = 1.f, m01 = 0.f, m10 = 0.f, m11 = 1.f;
  // k of a batch of tokens loaded together (tokens past the chunk read token
  // n - 1 and then count as zero: with their identity map they change nothing)
  for (int tb = 0; tb < n; tb += kGainBatch) {
    float kv[kGainBatch];
#pragma unroll
    for (int u = 0; u < kGainBatch; ++u)
      kv[u] = Elem<Tk>::load(k, ((size_t)bh * L + t0 + min(tb + u, n - 1)) * dk + i);
#pragma unroll
    for (int u = 0; u < kGainBatch; ++u) {
      const int t = tb + u;  // < 64: inside sp, sr
      const float4 tp = sp[t];
      const float k2 = t < n ? kv[u] * kv[u] : 0.f;
      const float t10 = k2 * tp.z, t11 = fmaf(k2, tp.w, sr[t]);
      const float n00 = fmaf(tp.x, m00, tp.y * m10), n01 = fmaf(tp.x, m01, tp.y * m11);
      const float n10 = fmaf(t10, m00, t11 * m10), n11 = fmaf(t10, m01, t11 * m11);
      // projective scale: any positive factor will do, so an approximate reciprocal
      const float sc = __builtin_amdgcn_rcpf(fmaxf(fmaxf(n00, n01), fmaxf(n10, n11)));
      m00 = n00 * sc;
      m01 = n01 * sc;
      m10 = n10 * sc;
      m11 = n11 * sc;
    }
  }
  maps[((size_t)bh * nchunks + c) * dk + i] = make_float4(m00, m01, m10, m11);
}

// Sum over the 64 lanes, every lane gets it (all 64 lanes must be active).
// DPP only, no trip through the LDS crossbar: the quad, half-row and row sums
// by lane permutations within each row of 16; then row 1 and row 3 add lane 15
// of the row before them, rows 2 and 3 add lane 31, and lane 63 holds the total.
template <int CTRL>
__device__ __forceinline__ float dpp_perm(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_sum64(float x) {
  x += dpp_perm<0xB1>(x);   // quad_perm 1,0,3,2
  x += dpp_perm<0x4E>(x);   // quad_perm 2,3,0,1
  x += dpp_perm<0x141>(x);  // row_half_mirror
  x += dpp_perm<0x140>(x);  // row_mirror
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xA, 0xF, false));  // row_bcast:15
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// One wavefront per (head, chunk): lane l carries coordinates l and l + 64
// through the chunk's tokens in order; the sum over coordinates in
// s_t = r_t + sum_i p-_i k_i^2 is a wavefront reduction, so the gains of token
// t are written as soon as it is done. No LDS and no barriers. (Any d_k and
// input type; the matrix-core path's shape uses diag_gains_rows_kernel.)

template <typename Tk, typename Tg>
__global__ __launch_bounds__(256) void diag_gains_kernel(const Tk* k, const float* alpha,
                                                         const float* r, float* cov_out,
                                                         float qvar, const float4* maps,
                                                         Tg* gains, int BH, int L, int dk,
                                                         int C, int nchunks, float* pprev,
                                                         float* sden) {
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
    if (pprev) {  // for the backward: the variance before the token
      if (ok0) pprev[g * dk + i0] = p0;
      if (ok1) pprev[g * dk + i1] = p1;
    }
    // reciprocals by v_rcp_f32 (1 ulp): exact divisions are ten instructions
    // each and sit on the chain from token to token
    const float sd = rt + wave_sum64(fmaf(pk0, k0, pk1 * k1));
    if (sden && lane == 0) sden[g] = sd;
    const float inv = __builtin_amdgcn_rcpf(sd);
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

// The same for bf16 keys, fp16 gains and d_k = 128: four chunks per
// wavefront, one per row of 16 lanes; lane j of a row carries coordinates
// 8 j .. 8 j + 7 of its chunk, so keys are read and gains written as 16-byte
// pieces (a row covers a token's 256-byte key row), and the sum over
// coordinates is a row reduction. The inputs of 8 tokens are loaded ahead.
typedef float f2v __attribute__((ext_vector_type(2)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_perm<0xB1>(x);   // quad_perm 1,0,3,2
  x += dpp_perm<0x4E>(x);   // quad_perm 2,3,0,1
  x += dpp_perm<0x141>(x);  // row_half_mirror
  return x + dpp_perm<0x140>(x);  // row_mirror
}
__global__ __launch_bounds__(256) void diag_gains_rows_kernel(const uint16_t* k, const float* alpha,
                                                              const float* r, float* cov_out,
                                                              float qvar, const float4* maps,
                                                              _Float16* gains, int BH, int L,
                                                              int C, int nchunks, float* pprev,
                                                              float* sden) {
  constexpr int DK = 128, NB = 8;
  const int lane = threadIdx.x & 63, cg = lane & 15;
  const int nitems = BH * nchunks;
  const int item0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  const bool live = item0 < nitems;  // rows past the last chunk repeat it and store nothing
  const int item = live ? item0 : nitems - 1;
  const int bh = item / nchunks, c = item - bh * nchunks;
  const int t0 = c * C, n = min(C, L - t0);
  const size_t tok = (size_t)bh * L + t0;
  float p[8];  // variances of coordinates 8 cg .. + 8, from the chunk start
  {
    const float4* mp = maps + (size_t)item * DK + 8 * cg;
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = mp[e].x;
  }
  for (int tb = 0; tb < C; tb += NB) {
    // tokens past the chunk read token n - 1 and are not applied
    uint4 kv[NB];
    float av[NB], rv[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const size_t g = tok + min(tb + u, n - 1);
      kv[u] = *reinterpret_cast<const uint4*>(k + g * DK + 8 * cg);
      av[u] = alpha ? alpha[g] : 1.f;
      rv[u] = r ? r[g] : 1.f;
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int t = tb + u;
      const bool in = live && t < n;
      const size_t g = tok + t;
      const uint32_t w[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
      float kf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = __uint_as_float(w[e] << 16);
        kf[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
      const float a = av[u], rt = rv[u];
      const float a2 = a * a, Q = (1.f - a) * (1.f + a) * qvar;
      float pm[8], pk[8], part = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pm[e] = fmaf(a2, p[e], Q);
        pk[e] = pm[e] * kf[e];
        part = fmaf(pk[e], kf[e], part);
      }
      // reciprocals by v_rcp_f32 (1 ulp), as in diag_gains_kernel
      const float sd = rt + row_sum16(part);
      const float inv = __builtin_amdgcn_rcpf(sd);
      if (in) {
        if (pprev) {  // for the backward: the variances before the token
          float4* pp = reinterpret_cast<float4*>(pprev + g * DK + 8 * cg);
          pp[0] = make_float4(p[0], p[1], p[2], p[3]);
          pp[1] = make_float4(p[4], p[5], p[6], p[7]);
        }
        if (sden && cg == 0) sden[g] = sd;
        uint32_t gh[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          gh[e] = __builtin_bit_cast(
              uint32_t, __builtin_convertvector(f2v{pk[2 * e] * inv, pk[2 * e + 1] * inv}, h2v));
        *reinterpret_cast<uint4*>(gains + g * DK + 8 * cg) = make_uint4(gh[0], gh[1], gh[2], gh[3]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        p[e] = in ? pm[e] * rt * __builtin_amdgcn_rcpf(fmaf(pk[e], kf[e], rt)) : p[e];
    }
  }
  if (live && c == nchunks - 1 && cov_out) {
    float4* co = reinterpret_cast<float4*>(cov_out + (size_t)bh * DK + 8 * cg);
    co[0] = make_float4(p[0], p[1], p[2], p[3]);
    co[1] = make_float4(p[4], p[5], p[6], p[7]);
  }
}

// Full covariance, one workgroup per head, sequential over tokens (d_k <= 64).
template <typename Tk, typename Tg>
__global__ __launch_bounds__(256) void full_gains_kernel(const Tk* k, const float* alpha,
                                                         const float* r, const float* cov_in,
                                                         float* cov_out, float qvar, Tg* gains,
                                                         int L, int dk) {
  // The token inputs of up to 64 tokens are staged together (keys [t][d_k],
  // alpha^2, Q, r), so the sequential loop reads only LDS. P holds the
  // predicted covariance of the token at hand; each token's update also
  // applies the next token's prediction, P <- a^2 (P - u u^T / s) + Q I, in
  // the same pass (the last token of a tile leaves the update alone and the
  // next tile predicts first), the same arithmetic as predicting separately.
  constexpr int TT = 64;
  __shared__ float sP[64 * 65];
  __shared__ float sU[64];
  __shared__ float sKt[TT * 64];
  __shared__ float sA2[TT], sQv[TT], sR[TT];
  __shared__ float sKu[4];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int PP = dk + 1;
  const int ri = tid >> 2, pq = tid & 3;  // row and quarter of P k
  for (int idx = tid; idx < dk * dk; idx += 256) {
    const int i = idx / dk, j = idx - i * dk;
    sP[i * PP + j] = cov_in[(size_t)bh * dk * dk + idx];
  }
  for (int t0 = 0; t0 < L; t0 += TT) {
    const int nt = min(TT, L - t0);
    __syncthreads();  // the previous tile's inputs are no longer read
    for (int idx = tid; idx < nt * dk; idx += 256)
      sKt[idx] = Elem<Tk>::load(k, ((size_t)bh * L + t0) * dk + idx);
    if (tid < nt) {
      const size_t g = (size_t)bh * L + t0 + tid;
      const float a = alpha ? alpha[g] : 1.f;
      sA2[tid] = a * a;
      sQv[tid] = (1.f - a) * (1.f + a) * qvar;
      sR[tid] = r ? r[g] : 1.f;
    }
    __syncthreads();
    // predict the tile's first token
    for (int idx = tid; idx < dk * dk; idx += 256) {
      const int i = idx / dk, j = idx - i * dk;
      sP[i * PP + j] = fmaf(sA2[0], sP[i * PP + j], i == j ? sQv[0] : 0.f);
    }
    __syncthreads();
    for (int tt = 0; tt < nt; ++tt) {
      const float* kt = sKt + tt * dk;
      // u = P k: four adjacent lanes per row (two interleaved sums each),
      // combined by lane shuffles; each wavefront's share of k^T u goes to LDS
      float u = 0.f;
      if (ri < dk) {
        float u0 = 0.f, u1 = 0.f;
        const float* pr_ = sP + ri * PP;
        for (int j = pq; j < dk; j += 8) {
          u0 = fmaf(pr_[j], kt[j], u0);
          if (j + 4 < dk) u1 = fmaf(pr_[j + 4], kt[j + 4], u1);
        }
        u = u0 + u1;
      }
      u += __shfl_xor(u, 1, 64);
      u += __shfl_xor(u, 2, 64);
      if (pq == 0 && ri < dk) sU[ri] = u;
      const float ku = wave_sum64(pq == 0 && ri < dk ? kt[ri] * u : 0.f);
      if ((tid & 63) == 0) sKu[tid >> 6] = ku;
      __syncthreads();
      const float s = sR[tt] + ((sKu[0] + sKu[1]) + (sKu[2] + sKu[3]));
      const float inv = 1.f / s;
      if (tid < dk) Elem<Tg>::store(gains, ((size_t)bh * L + t0 + tt) * dk + tid, sU[tid] * inv);
      const bool pred = tt + 1 < nt;
      const float a2 = pred ? sA2[tt + 1] : 1.f, Q = pred ? sQv[tt + 1] : 0.f;
      for (int idx = tid; idx < dk * dk; idx += 256) {
        const int i = idx / dk, j = idx - i * dk;
        const float p = sP[i * PP + j] - sU[i] * sU[j] * inv;
        sP[i * PP + j] = pred ? fmaf(a2, p, i == j ? Q : 0.f) : p;
      }
      __syncthreads();
    }
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

// The variance at every chunk start, by an associative scan over chunks: the
// chunk maps are Moebius maps, which compose associatively ("Kalman Delta
// Networks: Uncertainty-aware Associative Memory", abstract). One wavefront
// per sequence -- (head, coordinate) for the diagonal write, head for the
// isotropic one (dk = 1) -- with lanes as chunks, 64 at a time: an inclusive
// scan of the maps over the lanes in six doubling steps; each lane's
// exclusive composite takes the variance carried in from the chunks before to
// its chunk start, and the last lane's inclusive composite carries it on.
// Depth: six map products per 64 chunks, against 64 map applications one
// after the other. The result goes over each map's first entry.
__global__ __launch_bounds__(256) void prefix_scan_kernel(const float* cov_in, float4* maps,
                                                          int nseq, int dk, int nchunks) {
  const int seq = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (seq >= nseq) return;  // whole wavefronts
  const int bh = seq / dk, i = seq - bh * dk;
  float p = cov_in[seq];
  float4* m = maps + (size_t)bh * nchunks * dk + i;
  for (int c0 = 0; c0 < nchunks; c0 += 64) {
    const int c = c0 + lane;
    const bool ok = c < nchunks;
    Mob M{1.f, 0.f, 0.f, 1.f};  // lanes past the last chunk: the identity
    if (ok) {
      const float4 v = m[(size_t)c * dk];
      M = Mob{v.x, v.y, v.z, v.w};
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) M = mob_mul(M, mob_shfl_up(M, d, lane));
    const Mob X = mob_shfl_up(M, 1, lane);  // maps of the chunks before this one
    if (ok) m[(size_t)c * dk].x = fmaf(X.a, p, X.b) / fmaf(X.c, p, X.d);
    const int last = min(63, nchunks - 1 - c0);
    const float ta = __builtin_amdgcn_readlane(__float_as_int(M.a), last);
    const float tb = __builtin_amdgcn_readlane(__float_as_int(M.b), last);
    const float tc = __builtin_amdgcn_readlane(__float_as_int(M.c), last);
    const float td = __builtin_amdgcn_readlane(__float_as_int(M.d), last);
    p = fmaf(__int_as_float(ta), p, __int_as_float(tb)) / fmaf(__int_as_float(tc), p, __int_as_float(td));
  }
}

// The same scan for the diagonal write with d_k a multiple of 64, laid out for
// coalesced rows: one workgroup of kPfxWaves wavefronts per (head, 64
// coordinates), lane = coordinate, so each chunk's maps are one contiguous row
// of 64 float4. The chunks go in passes of kPfxWaves x kPfxRun: wavefront g
// composes the maps of its kPfxRun chunks, the composites meet in LDS, the
// wavefront carries the variance to its first chunk through the composites of
// the wavefronts before it and then through its own chunks, writing each
// chunk's starting variance over the map's first entry; the variance after
// the pass goes through all composites. With `starts` the starting variances
// go there instead, [BH, nchunks, dk] floats (coalesced rows, the maps left
// as they are).
constexpr int kPfxWaves = 16, kPfxRun = 8;
__device__ __forceinline__ float mob_apply(Mob x, float p) {
  return fmaf(x.a, p, x.b) / fmaf(x.c, p, x.d);
}
__global__ __launch_bounds__(64 * kPfxWaves) void prefix_rows_kernel(const float* cov_in, float4* maps,
                                                                    float* starts, int dk, int nchunks) {
  __shared__ Mob sAcc[kPfxWaves][64];
  const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int groups = dk / 64;
  const int bh = blockIdx.x / groups, i = (blockIdx.x - bh * groups) * 64 + lane;
  float p = cov_in[(size_t)bh * dk + i];
  float4* m = maps + (size_t)bh * nchunks * dk + i;
  float* st = starts ? starts + (size_t)bh * nchunks * dk + i : nullptr;
  for (int c0 = 0; c0 < nchunks; c0 += kPfxWaves * kPfxRun) {
    const int cb = c0 + g * kPfxRun;
    Mob run[kPfxRun];
#pragma unroll
    for (int j = 0; j < kPfxRun; ++j) {
      const float4 v = cb + j < nchunks ? m[(size_t)(cb + j) * dk] : make_float4(1.f, 0.f, 0.f, 1.f);
      run[j] = Mob{v.x, v.y, v.z, v.w};
    }
    Mob acc = run[0];
#pragma unroll
    for (int j = 1; j < kPfxRun; ++j) acc = mob_mul(run[j], acc);
    sAcc[g][lane] = acc;
    __syncthreads();
    float pg = p;
    for (int h = 0; h < g; ++h) pg = mob_apply(sAcc[h][lane], pg);
#pragma unroll
    for (int j = 0; j < kPfxRun; ++j) {
      if (cb + j < nchunks) {
        if (st) st[(size_t)(cb + j) * dk] = pg;
        else m[(size_t)(cb + j) * dk].x = pg;
      }
      pg = mob_apply(run[j], pg);
    }
#pragma unroll
    for (int h = 0; h < kPfxWaves; ++h) p = mob_apply(sAcc[h][lane], p);
    __syncthreads();
  }
}

hipError_t launch_prefix_diag(const float* cov_in, float* maps, int BH, int dk, int nchunks,
                              hipStream_t s, float* starts = nullptr) {
  if (dk % 64 == 0)
    KDN_LAUNCH(prefix_rows_kernel, dim3(BH * (dk / 64)), dim3(64 * kPfxWaves), 0, s, cov_in,
               reinterpret_cast<float4*>(maps), starts, dk, nchunks);
  else
    KDN_LAUNCH(prefix_scan_kernel, dim3((BH * dk + 3) / 4), dim3(256), 0, s, cov_in,
               reinterpret_cast<float4*>(maps), BH * dk, dk, nchunks);
  return hipGetLastError();
}

// One wavefront per (head, chunk), lane t = token t: the variance before the
// token from the chunk's starting p (prefix_scan_kernel) and an exclusive scan
// of the token maps, then the write strength beta_t.
__global__ __launch_bounds__(256) void iso_beta_kernel(const float* alpha, const float* r,
                                                       const float* kk, float* cov_out, float qvar,
                                                       const float4* maps, float* beta, int BH,
                                                       int L, int dk, int C, int nchunks,
                                                       float* pprev) {
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
  if (pprev && lane < n) pprev[g] = p;
  if (c == nchunks - 1 && cov_out && lane == n - 1)
    cov_out[bh] = pm * (dk * rt) / fmaf(pm, kt, dk * rt);
}

// ======================================================= covariance adjoints
// Gradients through the Kalman gains and the covariance recursion (the
// backward of the diagonal and isotropic writes). Given dL/db_t for the gain
// rows (DIAG) or dL/dbeta_t (ISO) from the state backward, and dL/dp_L, the
// reverse recursion over tokens carries dp = dL/dp_t per coordinate:
//   DIAG: ds = -(db . b) / s,  dpm_i = db_i k_i / s + ds k_i^2 + dp_i r^2 / D_i^2,
//         D_i = r + pm_i k_i^2,  dp_{t-1,i} = a^2 dpm_i,
//         dk_i += db_i pm_i / s + 2 ds pm_i k_i - 2 dp_i pm_i^2 r k_i / D_i^2,
//         dr = ds + sum_i dp_i pm_i^2 k_i^2 / D_i^2,  dalpha += 2 a sum_i dpm_i (p_i - sigma^2)
//   ISO:  dpm = dbeta r / s^2 + dp (d r)^2 / D^2,  D = d r + pm kk,  dp_{t-1} = a^2 dpm,
//         dkk = -dbeta pm^2 / s^2 - dp pm^2 d r / D^2 (dk += 2 dkk k),
//         dr = -dbeta pm / s^2 + dp pm^2 d kk / D^2,  dalpha += 2 a dpm (p - sigma^2)
// (pm = a^2 p + Q with p the variance before the token, s the gain's
// denominator). dp_{t-1} is affine in dp_t with coefficients that do not
// depend on dp, so, as in the forward, each chunk's tokens compose into one
// affine map (in parallel), a suffix scan over chunks carries dp to every chunk
// end, and a last pass runs each chunk's tokens in reverse from its carry.

constexpr int kAdjC = 64;  // tokens per adjoint chunk

// DIAG, one wavefront per (head, chunk), lane l: coordinates l and l + 64.
// Per token: the affine map dp_t -> dp_{t-1}; per chunk their composition.
__global__ __launch_bounds__(256) void diag_adj_maps_kernel(
    const float* k, const float* alpha, const float* r, float qvar, const float* pprev,
    const float* sden, const float* gains, const float* dgain, float2* amap, int BH, int L,
    int dk, int nchunks) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wave >= BH * nchunks) return;
  const int bh = wave / nchunks, c = wave - bh * nchunks;
  const int t0 = c * kAdjC, n = min(kAdjC, L - t0);
  const int i0 = lane, i1 = lane + 64;
  const bool ok0 = i0 < dk, ok1 = i1 < dk;
  float A0 = 1.f, C0 = 0.f, A1 = 1.f, C1 = 0.f;  // composed map, dp at chunk end -> start
  for (int t = 0; t < n; ++t) {
    const size_t g = (size_t)bh * L + t0 + t;
    const float a = alpha ? alpha[g] : 1.f, rt = r ? r[g] : 1.f, s = sden[g];
    const float a2 = a * a, Q = (1.f - a) * (1.f + a) * qvar;
    const float k0 = ok0 ? k[g * dk + i0] : 0.f, k1 = ok1 ? k[g * dk + i1] : 0.f;
    const float b0 = ok0 ? gains[g * dk + i0] : 0.f, b1 = ok1 ? gains[g * dk + i1] : 0.f;
    const float d0 = ok0 ? dgain[g * dk + i0] : 0.f, d1 = ok1 ? dgain[g * dk + i1] : 0.f;
    const float pm0 = fmaf(a2, ok0 ? pprev[g * dk + i0] : 0.f, Q);
    const float pm1 = fmaf(a2, ok1 ? pprev[g * dk + i1] : 0.f, Q);
    const float ds = -wave_sum64(fmaf(d0, b0, d1 * b1)) / s;
    const float D0 = fmaf(pm0 * k0, k0, rt), D1 = fmaf(pm1 * k1, k1, rt);
    const float c0 = a2 * fmaf(ds * k0, k0, d0 * k0 / s), c1 = a2 * fmaf(ds * k1, k1, d1 * k1 / s);
    const float e0 = a2 * (rt / D0) * (rt / D0), e1 = a2 * (rt / D1) * (rt / D1);
    // F <- F o f: x -> A (e x + c) + C
    C0 = fmaf(A0, c0, C0);
    A0 *= e0;
    C1 = fmaf(A1, c1, C1);
    A1 *= e1;
  }
  float2* m = amap + ((size_t)bh * nchunks + c) * dk;
  if (ok0) m[i0] = make_float2(A0, C0);
  if (ok1) m[i1] = make_float2(A1, C1);
}

// DIAG, one wavefront per (head, chunk): the chunk's tokens in reverse from the
// carried dp; adds the gain and covariance terms to dk and dalpha, writes dr.
__global__ __launch_bounds__(256) void diag_adj_out_kernel(
    const float* k, const float* alpha, const float* r, float qvar, const float* pprev,
    const float* sden, const float* gains, const float* dgain, const float* carry, float* dk_out,
    float* dalpha, float* dr, int BH, int L, int dk, int nchunks) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wave >= BH * nchunks) return;
  const int bh = wave / nchunks, c = wave - bh * nchunks;
  const int t0 = c * kAdjC, n = min(kAdjC, L - t0);
  const int i0 = lane, i1 = lane + 64;
  const bool ok0 = i0 < dk, ok1 = i1 < dk;
  const float* cr = carry + ((size_t)bh * nchunks + c) * dk;
  float dp0 = ok0 ? cr[i0] : 0.f, dp1 = ok1 ? cr[i1] : 0.f;
  for (int t = n - 1; t >= 0; --t) {
    const size_t g = (size_t)bh * L + t0 + t;
    const float a = alpha ? alpha[g] : 1.f, rt = r ? r[g] : 1.f, s = sden[g];
    const float a2 = a * a, Q = (1.f - a) * (1.f + a) * qvar;
    const float k0 = ok0 ? k[g * dk + i0] : 0.f, k1 = ok1 ? k[g * dk + i1] : 0.f;
    const float b0 = ok0 ? gains[g * dk + i0] : 0.f, b1 = ok1 ? gains[g * dk + i1] : 0.f;
    const float d0 = ok0 ? dgain[g * dk + i0] : 0.f, d1 = ok1 ? dgain[g * dk + i1] : 0.f;
    const float p0 = ok0 ? pprev[g * dk + i0] : 0.f, p1 = ok1 ? pprev[g * dk + i1] : 0.f;
    const float pm0 = fmaf(a2, p0, Q), pm1 = fmaf(a2, p1, Q);
    const float ds = -wave_sum64(fmaf(d0, b0, d1 * b1)) / s;
    const float D0 = fmaf(pm0 * k0, k0, rt), D1 = fmaf(pm1 * k1, k1, rt);
    const float q0 = pm0 / D0, q1 = pm1 / D1;   // pm / D
    const float dpm0 = d0 * k0 / s + ds * k0 * k0 + dp0 * (rt / D0) * (rt / D0);
    const float dpm1 = d1 * k1 / s + ds * k1 * k1 + dp1 * (rt / D1) * (rt / D1);
    if (ok0) dk_out[g * dk + i0] += d0 * pm0 / s + 2.f * ds * pm0 * k0 - 2.f * dp0 * q0 * q0 * rt * k0;
    if (ok1) dk_out[g * dk + i1] += d1 * pm1 / s + 2.f * ds * pm1 * k1 - 2.f * dp1 * q1 * q1 * rt * k1;
    const float drs = wave_sum64(fmaf(dp0 * q0 * q0 * k0, k0, dp1 * q1 * q1 * k1 * k1));
    const float das = wave_sum64(fmaf(dpm0, p0 - qvar, ok1 ? dpm1 * (p1 - qvar) : 0.f));
    if (lane == 0) {
      if (dr) dr[g] = ds + drs;
      if (dalpha) dalpha[g] += 2.f * a * (ok0 ? das : 0.f);
    }
    dp0 = a2 * dpm0;
    dp1 = a2 * dpm1;
  }
}

// ISO: one wavefront per (head, chunk), lane t = token t. Per token the affine
// map (e, c): dp_t -> dp_{t-1} = e dp_t + c, and the suffix compositions
// R_t = f_t o f_{t+1} o ... by a wavefront scan toward lane 0.
struct Aff {
  float e, c;
};
__device__ __forceinline__ Aff aff_after(Aff f, Aff g) {  // f o g
  return Aff{f.e * g.e, fmaf(f.e, g.c, f.c)};
}
__device__ __forceinline__ Aff aff_suffix(Aff m, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    Aff y{__shfl_down(m.e, off, 64), __shfl_down(m.c, off, 64)};
    if (lane + off >= 64) y = Aff{1.f, 0.f};
    m = aff_after(m, y);
  }
  return m;
}
// dp at every chunk end, from the last chunk back (dp at the start is
// dL/dp_0), by a suffix scan of the chunks' affine maps: one wavefront per
// (head, coordinate) (np coordinates per head), lanes as chunks, 64 at a time
// from the end; each lane applies the composite of the chunks after it to
// the dp carried in, and lane 0's composite carries it on.
__global__ __launch_bounds__(256) void adj_carry_kernel(const float* dcov_out, const float2* amap,
                                                        float* carry, float* dcov_in, int nseq,
                                                        int np, int nchunks) {
  const int seq = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (seq >= nseq) return;  // whole wavefronts
  const int bh = seq / np, i = seq - bh * np;
  float dp = dcov_out ? dcov_out[seq] : 0.f;
  for (int hi = nchunks - 1; hi >= 0; hi -= 64) {
    const int c = hi - 63 + lane;
    const bool ok = c >= 0;  // lanes before the first chunk: the identity
    const size_t o = ((size_t)bh * nchunks + (ok ? c : 0)) * np + i;
    Aff m{1.f, 0.f};
    if (ok) {
      const float2 v = amap[o];
      m = Aff{v.x, v.y};
    }
    m = aff_suffix(m, lane);  // this chunk's map after those of the later chunks
    Aff x{__shfl_down(m.e, 1, 64), __shfl_down(m.c, 1, 64)};
    if (lane == 63) x = Aff{1.f, 0.f};
    if (ok) carry[o] = fmaf(x.e, dp, x.c);
    const float e0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m.e), 0));
    const float c0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m.c), 0));
    dp = fmaf(e0, dp, c0);
  }
  if (dcov_in) dcov_in[seq] = dp;
}

struct IsoTok {
  float a, rt, p, pm, s, D, kk, db;
};
__device__ __forceinline__ IsoTok iso_tok(const float* alpha, const float* r, const float* kk,
                                          const float* pprev, const float* dbeta, float qvar,
                                          int dk, size_t g, bool in) {
  IsoTok x{1.f, 1.f, 0.f, 0.f, 1.f, 1.f, 0.f, 0.f};
  if (in) {
    x.a = alpha ? alpha[g] : 1.f;
    x.rt = r ? r[g] : 1.f;
    x.p = pprev[g];
    x.kk = kk[g];
    x.db = dbeta[g];
    x.pm = fmaf(x.a * x.a, x.p, (1.f - x.a) * (1.f + x.a) * qvar);
    x.s = fmaf(x.pm, x.kk, x.rt);
    x.D = fmaf(x.pm, x.kk, dk * x.rt);
  }
  return x;
}
__device__ __forceinline__ Aff iso_aff(const IsoTok& x, int dk, bool in) {
  if (!in) return Aff{1.f, 0.f};
  const float a2 = x.a * x.a, u = dk * x.rt / x.D;
  return Aff{a2 * u * u, a2 * x.db * x.rt / (x.s * x.s)};
}

__global__ __launch_bounds__(256) void iso_adj_maps_kernel(const float* alpha, const float* r,
                                                           float qvar, const float* kk,
                                                           const float* pprev, const float* dbeta,
                                                           float2* amap, int BH, int L, int dk,
                                                           int nchunks) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wave >= BH * nchunks) return;
  const int bh = wave / nchunks, c = wave - bh * nchunks;
  const int t0 = c * kAdjC, n = min(kAdjC, L - t0);
  const bool in = lane < n;
  const IsoTok x = iso_tok(alpha, r, kk, pprev, dbeta, qvar, dk, (size_t)bh * L + t0 + lane, in);
  const Aff m = aff_suffix(iso_aff(x, dk, in), lane);
  if (lane == 0) amap[(size_t)bh * nchunks + c] = make_float2(m.e, m.c);
}

__global__ __launch_bounds__(256) void iso_adj_out_kernel(const float* k, const float* alpha,
                                                          const float* r, float qvar,
                                                          const float* kk, const float* pprev,
                                                          const float* dbeta, const float* carry,
                                                          float* dk_out, float* dalpha, float* dr,
                                                          int BH, int L, int dk, int nchunks) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wave >= BH * nchunks) return;
  const int bh = wave / nchunks, c = wave - bh * nchunks;
  const int t0 = c * kAdjC, n = min(kAdjC, L - t0);
  const bool in = lane < n;
  const size_t g = (size_t)bh * L + t0 + lane;
  const IsoTok x = iso_tok(alpha, r, kk, pprev, dbeta, qvar, dk, g, in);
  const Aff incl = aff_suffix(iso_aff(x, dk, in), lane);       // f_t o ... o f_last
  Aff after{__shfl_down(incl.e, 1, 64), __shfl_down(incl.c, 1, 64)};  // f_{t+1} o ...
  if (lane == 63) after = Aff{1.f, 0.f};
  const float dpe = carry[(size_t)bh * nchunks + c];           // dp at the chunk end
  const float dp = fmaf(after.e, dpe, after.c);                 // dL/dp_t
  const float s2 = x.s * x.s, D2 = x.D * x.D, pm2 = x.pm * x.pm;
  const float dpm = x.db * x.rt / s2 + dp * (dk * x.rt) * (dk * x.rt) / D2;
  const float dkk = -x.db * pm2 / s2 - dp * pm2 * dk * x.rt / D2;
  if (in) {
    if (dr) dr[g] = -x.db * x.pm / s2 + dp * pm2 * dk * x.kk / D2;
    if (dalpha) dalpha[g] += 2.f * x.a * dpm * (x.p - qvar);
  }
  // dk += 2 dkk k, token by token, the wavefront over its coordinates
  const size_t row0 = (size_t)bh * L + t0;
  for (int t = 0; t < n; ++t) {
    const float f = 2.f * __shfl(dkk, t, 64);
    for (int i = lane; i < dk; i += 64) dk_out[(row0 + t) * dk + i] += f * k[(row0 + t) * dk + i];
  }
}

template <typename Tk, typename Tg>
hipError_t diag_typed(const void* k, const float* alpha, const float* r, const float* cov_in,
                      float* cov_out, float qvar, void* gains, float* maps, int BH, int L, int dk,
                      int C, hipStream_t s, float* pprev, float* sden) {
  const int nchunks = (L + C - 1) / C;
  KDN_LAUNCH(diag_maps_kernel<Tk>, dim3(BH, nchunks), dim3(128), 0, s,
                     static_cast<const Tk*>(k), alpha, r, qvar, reinterpret_cast<float4*>(maps), L,
                     dk, C, nchunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_prefix_diag(cov_in, maps, BH, dk, nchunks, s);
  if (e != hipSuccess) return e;
  if constexpr (std::is_same<Tk, uint16_t>::value && std::is_same<Tg, _Float16>::value) {
    if (dk == 128) {
      const int waves = (BH * nchunks + 3) / 4;  // four chunks per wavefront
      KDN_LAUNCH(diag_gains_rows_kernel, dim3((waves + 3) / 4), dim3(256), 0, s,
                         static_cast<const uint16_t*>(k), alpha, r, cov_out, qvar,
                         reinterpret_cast<const float4*>(maps), static_cast<_Float16*>(gains), BH,
                         L, C, nchunks, pprev, sden);
      return hipGetLastError();
    }
  }
  const int waves = BH * nchunks;
  KDN_LAUNCH((diag_gains_kernel<Tk, Tg>), dim3((waves + 3) / 4), dim3(256), 0, s,
                     static_cast<const Tk*>(k), alpha, r, cov_out, qvar,
                     reinterpret_cast<const float4*>(maps), static_cast<Tg*>(gains), BH, L, dk, C,
                     nchunks, pprev, sden);
  return hipGetLastError();
}

template <typename Tk, typename Tg>
hipError_t full_typed(const void* k, const float* alpha, const float* r, const float* cov_in,
                      float* cov_out, float qvar, void* gains, int BH, int L, int dk,
                      hipStream_t s) {
  KDN_LAUNCH((full_gains_kernel<Tk, Tg>), dim3(BH), dim3(256), 0, s,
                     static_cast<const Tk*>(k), alpha, r, cov_in, cov_out, qvar,
                     static_cast<Tg*>(gains), L, dk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_diag_gains(const void* k, bool k_bf16, const float* alpha, const float* r,
                             const float* cov_in, float* cov_out, float q_noise_var, void* gains,
                             bool gains_f16, float* maps, int BH, int L, int dk, int chunk,
                             hipStream_t s, float* pprev, float* sden) {
  if (k_bf16)
    return gains_f16 ? diag_typed<uint16_t, _Float16>(k, alpha, r, cov_in, cov_out, q_noise_var,
                                                       gains, maps, BH, L, dk, chunk, s, pprev, sden)
                      : diag_typed<uint16_t, float>(k, alpha, r, cov_in, cov_out, q_noise_var,
                                                    gains, maps, BH, L, dk, chunk, s, pprev, sden);
  return gains_f16 ? diag_typed<float, _Float16>(k, alpha, r, cov_in, cov_out, q_noise_var, gains,
                                                  maps, BH, L, dk, chunk, s, pprev, sden)
                    : diag_typed<float, float>(k, alpha, r, cov_in, cov_out, q_noise_var, gains,
                                               maps, BH, L, dk, chunk, s, pprev, sden);
}

hipError_t launch_diag_starts(const void* k, bool k_bf16, const float* alpha, const float* r,
                              const float* cov_in, float q_noise_var, float* maps, float* starts,
                              int BH, int L, int dk, int chunk, hipStream_t s) {
  if (dk % 64 != 0) return hipErrorInvalidValue;  // the compact starts need the row scan
  const int nchunks = (L + chunk - 1) / chunk;
  if (k_bf16)
    KDN_LAUNCH(diag_maps_kernel<uint16_t>, dim3(BH, nchunks), dim3(128), 0, s,
               static_cast<const uint16_t*>(k), alpha, r, q_noise_var,
               reinterpret_cast<float4*>(maps), L, dk, chunk, nchunks);
  else
    KDN_LAUNCH(diag_maps_kernel<float>, dim3(BH, nchunks), dim3(128), 0, s,
               static_cast<const float*>(k), alpha, r, q_noise_var, reinterpret_cast<float4*>(maps),
               L, dk, chunk, nchunks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_prefix_diag(cov_in, maps, BH, dk, nchunks, s, starts);
}

hipError_t launch_iso_beta(const void* k, bool k_bf16, const float* alpha, const float* r,
                          const float* cov_in, float* cov_out, float q_noise_var, float* beta,
                          float* kk, float* maps, int BH, int L, int dk, int chunk,
                          hipStream_t s, float* pprev) {
  const int nchunks = (L + chunk - 1) / chunk;
  const int blocks = (BH * nchunks + 3) / 4;  // four wavefronts per workgroup
  if (k_bf16)
    KDN_LAUNCH(iso_maps_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(k), alpha, r, q_noise_var, kk,
                       reinterpret_cast<float4*>(maps), BH, L, dk, chunk, nchunks);
  else
    KDN_LAUNCH(iso_maps_kernel<float>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const float*>(k), alpha, r, q_noise_var, kk,
                       reinterpret_cast<float4*>(maps), BH, L, dk, chunk, nchunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  KDN_LAUNCH(prefix_scan_kernel, dim3((BH + 3) / 4), dim3(256), 0, s, cov_in,
                     reinterpret_cast<float4*>(maps), BH, 1, nchunks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  KDN_LAUNCH(iso_beta_kernel, dim3(blocks), dim3(256), 0, s, alpha, r, kk, cov_out,
                     q_noise_var, reinterpret_cast<const float4*>(maps), beta, BH, L, dk, chunk,
                     nchunks, pprev);
  return hipGetLastError();
}

size_t cov_adj_scratch_floats(int BH, int L, int dk, bool diag) {
  const size_t nch = ((size_t)L + kAdjC - 1) / kAdjC, np = diag ? (size_t)dk : 1;
  return (size_t)BH * nch * np * 3;  // affine maps (2) and carries (1)
}

hipError_t launch_cov_adjoint(const CovAdjArgs& a, float* scratch, hipStream_t s) {
  const int nch = (a.L + kAdjC - 1) / kAdjC, np = a.diag ? a.dk : 1;
  float2* amap = reinterpret_cast<float2*>(scratch);
  float* carry = scratch + (size_t)a.BH * nch * np * 2;
  const int blocks = (a.BH * nch + 3) / 4;
  if (a.diag)
    KDN_LAUNCH(diag_adj_maps_kernel, dim3(blocks), dim3(256), 0, s, a.k, a.alpha, a.r,
                       a.qvar, a.pprev, a.sden, a.gains, a.dgain, amap, a.BH, a.L, a.dk, nch);
  else
    KDN_LAUNCH(iso_adj_maps_kernel, dim3(blocks), dim3(256), 0, s, a.alpha, a.r, a.qvar,
                       a.kk, a.pprev, a.dbeta, amap, a.BH, a.L, a.dk, nch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  KDN_LAUNCH(adj_carry_kernel, dim3((a.BH * np + 3) / 4), dim3(256), 0, s, a.dcov_out,
                     amap, carry, a.dcov_in, a.BH * np, np, nch);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.diag)
    KDN_LAUNCH(diag_adj_out_kernel, dim3(blocks), dim3(256), 0, s, a.k, a.alpha, a.r,
                       a.qvar, a.pprev, a.sden, a.gains, a.dgain, carry, a.dk_out, a.dalpha, a.dr,
                       a.BH, a.L, a.dk, nch);
  else
    KDN_LAUNCH(iso_adj_out_kernel, dim3(blocks), dim3(256), 0, s, a.k, a.alpha, a.r,
                       a.qvar, a.kk, a.pprev, a.dbeta, carry, a.dk_out, a.dalpha, a.dr, a.BH, a.L,
                       a.dk, nch);
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
