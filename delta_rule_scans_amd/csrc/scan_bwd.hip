// scan_bwd.hip -- gradients of the delta-write scan (reverse mode), chunkwise.
//
// Forward ("A Hippocampus for Linear Attention", sec. 3.3 eq. (5), sec. 3.5):
//   S_t = alpha_t S_{t-1} + b_t k_t e_t^T,  e_t = v_t - c_t S_{t-1}^T k_t,  o_t = S_t^T q_t,
// c_t = alpha_t (gated residual) or 0 (no erase). The plain residual (c_t = 1)
// is the gated one with b_t = beta_t / alpha_t and values alpha_t v_t, so it is
// run in that form and its gradients are mapped back at the end.
//
// Over a chunk of C tokens with incoming state S0, local decays
// g_t = prod_{l<=t} alpha_l, D_tl = g_t / g_l, Lambda_t = g_C / g_t and B = diag(b) K:
//   A = strict_lower((K B^T) * D),  Pm = lower_incl((Q B^T) * D),  T = (I + A)^-1,
//   E = T (V - diag(g) K S0),  O = diag(g) Q S0 + Pm E,  S_C = g_C S0 + (diag(Lambda) B)^T E.
// The pages give no backward pass. Differentiating the chunk form, with
// G = dL/dS_C and dO = dL/dO:
//   dE = Pm^T dO + diag(Lambda) B G,   dR = T^T dE (= dV),   dA = -strict_lower(dR E^T),
//   dS0 = g_C G + Q^T diag(g) dO - K^T diag(g) dR          (the chain to the previous chunk),
//   Xp = lower_incl(dO E^T) * D,  Xa = dA * D,
//   dQ = diag(g) dO S0^T + Xp B,
//   dB = Xp^T Q + Xa^T K + diag(Lambda) E G^T,
//   dK = Xa B - diag(g) dR S0^T + diag(b) dB,   db_t = dB_t . k_t,
// and the decays enter through log g: the row minus column sums of dPm * Pm and
// dA * A (the D factors), g_t q_t . (dO S0^T)_t, -g_t k_t . (dR S0^T)_t, and the
// state terms Lambda_t b_t k_t . (G e_t) (minus at t, plus at the chunk end) and
// g_C <G, S0>. Then d log alpha_t = sum_{t' >= t} d log g_t' within the chunk and
// dalpha_t = d log alpha_t / alpha_t (alpha must be positive). Without the erase
// term A = 0, T = I and the K S0 terms drop.
//
// Kernels (C = 64, float32 throughout, d_k, d_v <= 128):
//  * prep (head, chunk): A, Pm and T by blocked inversion (16 -> 32 -> 64).
//  * forward chain (head, 32 value columns): chunk-start states S0 and residuals E.
//  * reverse chain (head, 32 value columns): G at every chunk end, dR, dV, dS0.
//  * contractions over d_v (head, chunk, part): dO S0^T and dO E^T; dR S0^T and
//    dR E^T; E G^T and <G, S0>.
//  * gradients (head, chunk): dQ, dK, dbeta, dalpha.
// Products run on the fp32 matrix cores (v_mfma_f32_16x16x4f32) with operands read from LDS.
//
// Gain mode (a.gain set: the Kalman writes, "Kalman Delta Networks", abstract):
// the write vectors B are given rows g_t (the gains) instead of beta_t k_t, the
// residual is gated (c_t = alpha_t). The same formulas hold with diag(b) K
// replaced by the gain rows; dB is written out (a.dgain) for the covariance
// adjoint, dK keeps only the terms through the prediction K S0 and the Gram
// K B^T (Xa B - diag(g) dR S0^T), and the state terms of the decay use
// Lambda_t g_t . (G e_t). There is no dbeta.
#include "kdn_internal.h"

namespace kdn {
namespace {

constexpr int NT = 256;
constexpr int C = 64;       // tokens per chunk (one wavefront of scalars)
constexpr int TW = 32;      // value columns per chain workgroup
constexpr int DP = 128;     // d_k, padded
constexpr int LC = C + 1;   // row stride of [C][C] arrays


// Loads are split in two: fetch into registers (every load of a chunk in
// flight at once, or during the previous chunk's products), then put into LDS.
template <int N>
struct Frag {
  float x[N];
};

// [C][d] rows (n valid), zero padded to [C][DP]
template <int NTH>
__device__ __forceinline__ void fetch_rows(Frag<C * DP / NTH>& f, const float* src, int n, int d) {
#pragma unroll
  for (int u = 0; u < C * DP / NTH; ++u) {
    const int idx = threadIdx.x + u * NTH, t = idx >> 7, i = idx & (DP - 1);
    f.x[u] = (t < n && i < d) ? src[(size_t)t * d + i] : 0.f;
  }
}
template <int NTH, int LD>
__device__ __forceinline__ void put_rows(const Frag<C * DP / NTH>& f, float* dst) {
#pragma unroll
  for (int u = 0; u < C * DP / NTH; ++u) {
    const int idx = threadIdx.x + u * NTH;
    dst[(idx >> 7) * LD + (idx & (DP - 1))] = f.x[u];
  }
}
// a row-major [C][C] matrix
template <int NTH>
__device__ __forceinline__ void fetch_cc(Frag<C * C / NTH>& f, const float* src) {
#pragma unroll
  for (int u = 0; u < C * C / NTH; ++u) f.x[u] = src[threadIdx.x + u * NTH];
}
template <int NTH, int LD>
__device__ __forceinline__ void put_cc(const Frag<C * C / NTH>& f, float* dst) {
#pragma unroll
  for (int u = 0; u < C * C / NTH; ++u) {
    const int idx = threadIdx.x + u * NTH;
    dst[(idx >> 6) * LD + (idx & 63)] = f.x[u];
  }
}
// columns j0 .. j0 + W - 1 of [C][dv] rows (n valid), zero padded
template <int NTH, int W = TW>
__device__ __forceinline__ void fetch_tile(Frag<C * W / NTH>& f, const float* src, int n, int dv,
                                           int j0) {
#pragma unroll
  for (int u = 0; u < C * W / NTH; ++u) {
    const int idx = threadIdx.x + u * NTH, t = idx / W, j = idx % W;
    f.x[u] = (t < n && j0 + j < dv) ? src[(size_t)t * dv + j0 + j] : 0.f;
  }
}
// rows scaled by rs[t] when given
template <int NTH, int LD, int W = TW>
__device__ __forceinline__ void put_tile(const Frag<C * W / NTH>& f, float* dst, const float* rs) {
#pragma unroll
  for (int u = 0; u < C * W / NTH; ++u) {
    const int idx = threadIdx.x + u * NTH, t = idx / W, j = idx % W;
    dst[t * LD + j] = rs ? f.x[u] * rs[t] : f.x[u];
  }
}

// Chunk scalars (first wavefront): cumulative log decay, write scale b (beta,
// or beta / alpha for the plain residual), decay. Tokens past the end get
// alpha = 1 and b = 0, which leaves every product unchanged.
struct Scal {
  float al, be;
};
__device__ __forceinline__ Scal fetch_scalars(const BwdArgs& a, size_t tok, int n) {
  const int t = threadIdx.x;
  Scal r{1.f, 0.f};
  if (t < n && t < C) {
    r.al = a.alpha ? a.alpha[tok + t] : 1.f;
    r.be = a.beta ? a.beta[tok + t] : 1.f;  // no beta in gain mode: the gain rows are B
  }
  return r;
}
// The chunk-local prefix of log alpha is kept in float64: decay ratios are
// differences of prefixes, which reach about -1000 in a chunk of tokens with
// alpha near 1e-8, where float32 would keep only ~6e-5 of each ratio.
__device__ void put_scalars(const BwdArgs& a, Scal f, double* sLg, float* sB, float* sAl) {
  const int t = threadIdx.x;
  if (t < C) {
    const float b = a.resid == 1 ? f.be / f.al : f.be;
    double lg = logf(f.al);
#pragma unroll
    for (int off = 1; off < C; off <<= 1) {
      const double y = __shfl_up(lg, off, C);
      if (t >= off) lg += y;
    }
    sLg[t] = lg;
    sB[t] = b;
    sAl[t] = f.al;
  }
}


// ---------------------------------------------------------------------------
// Every product runs on the fp32 matrix cores in 16 x 16 blocks of
// v_mfma_f32_16x16x4f32: lane l holds A(m0 + l % 16, k) and B(k, n0 + l % 16)
// and the block's element (4 (l / 16) + i, l % 16) is accumulator i. The
// contraction runs in passes of 64; in step s of a pass, lane group l / 16
// takes k = 16 (l / 16) + s, so with LDS row strides of 1 mod 32 words the 32
// lanes of a read fall on distinct banks whether an operand is read along its
// rows or across them.
typedef float floatx4 __attribute__((ext_vector_type(4)));

// acc += sum_{k < K} A(m0 + i, k) B(k, n0 + j), A(m, k) = pa[m am + k ak],
// B(k, n) = pb[k bk + n bn]; K a multiple of 64. Even and odd steps go to two
// accumulators, so that two independent product chains are in flight.
__device__ __forceinline__ void mfma16(floatx4& acc, const float* pa, int am, int ak,
                                       const float* pb, int bk, int bn, int m0, int n0, int K) {
  const int l = threadIdx.x & 63, r = l & 15, q = l >> 4;
  floatx4 acc2 = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += 64) {
    const float* A = pa + (m0 + r) * am + (k0 + 16 * q) * ak;
    const float* B = pb + (k0 + 16 * q) * bk + (n0 + r) * bn;
#pragma unroll 4
    for (int s = 0; s < 16; s += 2) {
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[s * ak], B[s * bk], acc, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(A[(s + 1) * ak], B[(s + 1) * bk], acc2, 0, 0, 0);
    }
  }
  acc += acc2;
}

// A row of blocks (m0, 16 b), b < NB, sharing the A operand: acc[b] +=
// sum_{k < K} A(m0 + i, k) B(k, 16 b + j), A(m, k) = pa[m am + k ak] (times
// as[k] when given), B(k, n) = pb[k bk + n bn]; K a multiple of 64
template <int NB>
__device__ __forceinline__ void mfma_row(floatx4 (&acc)[NB], const float* pa, int am, int ak,
                                         const float* as, const float* pb, int bk, int bn, int m0,
                                         int K) {
  const int l = threadIdx.x & 63, r = l & 15, q = l >> 4;
  for (int k0 = 0; k0 < K; k0 += 64) {
    const float* A = pa + (m0 + r) * am + (k0 + 16 * q) * ak;
    const float* B = pb + (k0 + 16 * q) * bk + r * bn;
#pragma unroll 4
    for (int s = 0; s < 16; ++s) {
      float av = A[s * ak];
      if (as) av *= as[k0 + 16 * q + s];
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, B[s * bk + 16 * b * bn], acc[b], 0, 0, 0);
    }
  }
}

// Chain kernels: eight wavefronts; the 128 x 32 state (or state-gradient) tile
// stays in registers, two blocks per wavefront, mirrored into LDS as an operand.
constexpr int NTC = 512;      // threads of a chain workgroup
constexpr int LKC = DP + 1;   // [C][d_k] rows
constexpr int LCC = C + 1;    // [C][C] rows
constexpr int LOC = TW + 1;   // [C][TW] and [DP][TW] rows

__device__ __forceinline__ size_t cc_off(int bh, int nch, int c) {
  return ((size_t)bh * nch + c) * C * C;
}

// ---------------------------------------------------------------------------
// prep: A, Pm, T of one chunk
__global__ __launch_bounds__(NT) void bwd_prep_kernel(BwdArgs a) {
  extern __shared__ __align__(16) float lds[];
  constexpr int LP = DP + 1;
  // A, T and the block scratch reuse the K and Q tiles once both Grams are in
  // registers: 67 KB of LDS, two workgroups per CU
  static_assert(2 * C * LC + 32 * 33 <= 2 * C * LP, "A, T, Y fit over K and Q");
  float* sK = lds;                // [C][LP] (Grams)
  float* sQ = sK + C * LP;        // [C][LP] (Grams)
  float* sA = lds;                // [C][LC] (after the Grams)
  float* sT = sA + C * LC;        // [C][LC]
  float* sY = sT + C * LC;        // [32][33]
  double* sLg = reinterpret_cast<double*>(lds + 2 * C * LP);  // [C] (8-byte aligned)
  float* sB = reinterpret_cast<float*>(sLg + C);
  float* sAl = sB + C;
  float* sGn = sAl + C;           // [C][LP] gain rows (gain mode)
  const int bh = blockIdx.x, c = blockIdx.y, tid = threadIdx.x, nch = gridDim.y;
  const int n = min(C, a.L - c * C), dk = a.dk, dk64 = dk <= 64 ? 64 : DP;
  const size_t tok = (size_t)bh * a.L + (size_t)c * C;
  const bool erase = a.resid != 2, gain = a.gain != nullptr;
  {
    Frag<C * DP / NT> fk, fq, fg;
    fetch_rows<NT>(fk, a.k + tok * dk, n, dk);
    fetch_rows<NT>(fq, a.q + tok * dk, n, dk);
    if (gain) fetch_rows<NT>(fg, a.gain + tok * dk, n, dk);
    const Scal sc = fetch_scalars(a, tok, n);
    put_rows<NT, LP>(fk, sK);
    put_rows<NT, LP>(fq, sQ);
    if (gain) put_rows<NT, LP>(fg, sGn);
    put_scalars(a, sc, sLg, sB, sAl);
  }
  __syncthreads();
  const int w = tid >> 6, r = tid & 15, q = (tid & 63) >> 4;
  floatx4 kk[4] = {}, qk[4] = {};
  const float* sW = gain ? sGn : sK;  // the write vectors' direction: K B^T, Q B^T
  mfma_row<4>(kk, sK, LP, 1, nullptr, sW, 1, LP, 16 * w, dk64);
  mfma_row<4>(qk, sQ, LP, 1, nullptr, sW, 1, LP, 16 * w, dk64);
  __syncthreads();  // every wavefront is done with K and Q
  for (int idx = tid; idx < C * LC; idx += NT) sT[idx] = 0.f;
  float* Ag = a.Am + cc_off(bh, nch, c);
  float* Pg = a.Pm + cc_off(bh, nch, c);
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * w + 4 * q + i, l = 16 * b + r;
      const float f = l <= t ? sB[l] * expf((float)(sLg[t] - sLg[l])) : 0.f;
      const float av = (erase && l < t) ? kk[b][i] * f : 0.f;
      sA[t * LC + l] = av;
      Ag[t * C + l] = av;
      Pg[t * C + l] = qk[b][i] * f;
    }
  __syncthreads();
  // diagonal 16 x 16 blocks by substitution, one column per thread
  if (tid < 64) {
    const int o = 16 * (tid >> 4), col = tid & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = r == col ? 1.f : 0.f;
#pragma unroll
      for (int q = 0; q < r; ++q) s = fmaf(-sA[(o + r) * LC + o + q], x[q], s);
      x[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sT[(o + r) * LC + o + col] = x[r];
  }
  __syncthreads();
  // [[T1, 0], [X, T2]] inverts [[I + A11, 0], [A21, I + A22]] with X = -T2 A21 T1
  {
    const int p = tid >> 7, r = (tid >> 3) & 15, c2 = (tid & 7) * 2, o = 32 * p;
    float y0 = 0.f, y1 = 0.f;
    for (int s = 0; s < 16; ++s) {
      const float av = sA[(o + 16 + r) * LC + o + s];
      y0 = fmaf(av, sT[(o + s) * LC + o + c2], y0);
      y1 = fmaf(av, sT[(o + s) * LC + o + c2 + 1], y1);
    }
    sY[(16 * p + r) * 33 + c2] = y0;
    sY[(16 * p + r) * 33 + c2 + 1] = y1;
    __syncthreads();
    float x0 = 0.f, x1 = 0.f;
    for (int s = 0; s < 16; ++s) {
      const float tv = sT[(o + 16 + r) * LC + o + 16 + s];
      x0 = fmaf(-tv, sY[(16 * p + s) * 33 + c2], x0);
      x1 = fmaf(-tv, sY[(16 * p + s) * 33 + c2 + 1], x1);
    }
    sT[(o + 16 + r) * LC + o + c2] = x0;
    sT[(o + 16 + r) * LC + o + c2 + 1] = x1;
  }
  __syncthreads();
  {
    const int r = tid >> 3, c4 = (tid & 7) * 4;
    float y[4] = {};
    for (int s = 0; s < 32; ++s) {
      const float av = sA[(32 + r) * LC + s];
#pragma unroll
      for (int u = 0; u < 4; ++u) y[u] = fmaf(av, sT[s * LC + c4 + u], y[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) sY[r * 33 + c4 + u] = y[u];
    __syncthreads();
    float x[4] = {};
    for (int s = 0; s < 32; ++s) {
      const float tv = sT[(32 + r) * LC + 32 + s];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = fmaf(-tv, sY[s * 33 + c4 + u], x[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) sT[(32 + r) * LC + c4 + u] = x[u];
  }
  __syncthreads();
  float* Tg = a.Tm + cc_off(bh, nch, c);
  for (int idx = tid; idx < C * C; idx += NT) Tg[idx] = sT[(idx >> 6) * LC + (idx & 63)];
}

// forward chain: chunk-start states and residuals for 32 value columns
__global__ __launch_bounds__(NTC) void bwd_fwd_kernel(BwdArgs a) {
  extern __shared__ __align__(16) float lds[];
  float* sK = lds;              // [C][LKC]
  float* sT = sK + C * LKC;     // [C][LCC]
  float* sS = sT + C * LCC;     // [DP][LOC] state tile (operand copy)
  float* sR = sS + DP * LOC;    // [C][LOC] V - diag(g) K S0
  float* sE = sR + C * LOC;     // [C][LOC] diag(Lambda b) E
  double* sLg = reinterpret_cast<double*>(sE + C * LOC);  // [C] (8-byte aligned)
  float* sB = reinterpret_cast<float*>(sLg + C);
  float* sAl = sB + C;
  float* sGn = sAl + C;         // [C][LKC] gain rows (gain mode)
  const int bh = blockIdx.x, j0 = blockIdx.y * TW, tid = threadIdx.x;
  const int L = a.L, dk = a.dk, dv = a.dv, nch = (L + C - 1) / C, dk64 = dk <= 64 ? 64 : DP;
  const bool erase = a.resid != 2, gain = a.gain != nullptr;
  const int w = tid >> 6, l = tid & 63, r = l & 15, q = l >> 4;
  const int m0 = 16 * (w >> 1), n0 = 16 * (w & 1);  // this wavefront's [C][TW] block
  // state rows 16 w + 4 q + i, columns 16 h + r (h = 0, 1)
  floatx4 S[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 16 * w + 4 * q + i, j = 16 * h + r;
      S[h][i] = (a.state_in && d < dk && j0 + j < dv)
                    ? a.state_in[((size_t)bh * dk + d) * dv + j0 + j]
                    : 0.f;
      sS[d * LOC + j] = S[h][i];
    }
  Frag<C * DP / NTC> fk, fg;
  Frag<C * C / NTC> ft;
  Frag<C * TW / NTC> fv;
  Scal fs;
  auto fetch = [&](int c) {
    const int n = min(C, L - c * C);
    const size_t tok = (size_t)bh * L + (size_t)c * C;
    fetch_rows<NTC>(fk, a.k + tok * dk, n, dk);
    if (gain) fetch_rows<NTC>(fg, a.gain + tok * dk, n, dk);
    if (erase) fetch_cc<NTC>(ft, a.Tm + cc_off(bh, nch, c));
    fetch_tile<NTC>(fv, a.v + tok * dv, n, dv, j0);
    fs = fetch_scalars(a, tok, n);
  };
  fetch(0);
  for (int c = 0; c < nch; ++c) {
    const int n = min(C, L - c * C);
    __syncthreads();
    put_rows<NTC, LKC>(fk, sK);
    if (gain) put_rows<NTC, LKC>(fg, sGn);
    if (erase) put_cc<NTC, LCC>(ft, sT);
    put_scalars(a, fs, sLg, sB, sAl);
    {
      float* s0g = a.S0s + ((size_t)bh * nch + c) * dk * dv;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 16 * w + 4 * q + i, col = j0 + 16 * h + r;
          if (d < dk && col < dv) s0g[(size_t)d * dv + col] = S[h][i];
        }
    }
    __syncthreads();
    put_tile<NTC, LOC>(fv, sR, a.resid == 1 ? sAl : nullptr);
    if (c + 1 < nch) fetch(c + 1);
    __syncthreads();
    floatx4 e = {0.f, 0.f, 0.f, 0.f};
    if (erase) {
      floatx4 x = {0.f, 0.f, 0.f, 0.f};
      mfma16(x, sK, LKC, 1, sS, LOC, 1, m0, n0, dk64);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = m0 + 4 * q + i;
        sR[t * LOC + n0 + r] -= expf((float)sLg[t]) * x[i];
      }
      __syncthreads();
      mfma16(e, sT, LCC, 1, sR, LOC, 1, m0, n0, C);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = sR[(m0 + 4 * q + i) * LOC + n0 + r];
    }
    const double lgC = sLg[C - 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = m0 + 4 * q + i, col = j0 + n0 + r;
      if (t < n && col < dv) a.E[((size_t)bh * nch * C + (size_t)c * C + t) * dv + col] = e[i];
      sE[t * LOC + n0 + r] = e[i] * sB[t] * expf((float)(lgC - sLg[t]));
    }
    __syncthreads();
    const float gC = expf((float)lgC);
    floatx4 acc[2] = {S[0] * gC, S[1] * gC};
    mfma_row<2>(acc, gain ? sGn : sK, 1, LKC, nullptr, sE, LOC, 1, 16 * w, C);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      S[h] = acc[h];
#pragma unroll
      for (int i = 0; i < 4; ++i) sS[(16 * w + 4 * q + i) * LOC + 16 * h + r] = acc[h][i];
    }
  }
}

// reverse chain: state gradients at chunk ends, dR (= dV), dS0. GAIN is a
// template switch: a gain tile held in registers by every instantiation would
// push the delta-write chain past its register budget into scratch.
template <bool GAIN>
__global__ __launch_bounds__(NTC) void bwd_rev_kernel(BwdArgs a) {
  extern __shared__ __align__(16) float lds[];
  float* sK = lds;              // [C][LKC]
  float* sQ = sK + C * LKC;     // [C][LKC]
  float* sT = sQ + C * LKC;     // [C][LCC]
  float* sP = sT + C * LCC;     // [C][LCC]
  float* sG = sP + C * LCC;     // [DP][LOC] state gradient tile (operand copy)
  float* sO = sG + DP * LOC;    // [C][LOC] dO, then diag(g) dO
  float* sD = sO + C * LOC;     // [C][LOC] dE
  float* sX = sD + C * LOC;     // [C][LOC] -diag(g) dR
  double* sLg = reinterpret_cast<double*>(sX + C * LOC);  // [C] (8-byte aligned)
  float* sB = reinterpret_cast<float*>(sLg + C);
  float* sAl = sB + C;
  const int bh = blockIdx.x, j0 = blockIdx.y * TW, tid = threadIdx.x;
  const int L = a.L, dk = a.dk, dv = a.dv, nch = (L + C - 1) / C, dk64 = dk <= 64 ? 64 : DP;
  const bool erase = a.resid != 2;
  constexpr bool gain = GAIN;
  const int w = tid >> 6, l = tid & 63, r = l & 15, q = l >> 4;
  const int m0 = 16 * (w >> 1), n0 = 16 * (w & 1);
  floatx4 G[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 16 * w + 4 * q + i, j = 16 * h + r;
      G[h][i] = (a.dstate_out && d < dk && j0 + j < dv)
                    ? a.dstate_out[((size_t)bh * dk + d) * dv + j0 + j]
                    : 0.f;
      sG[d * LOC + j] = G[h][i];
    }
  // gain mode: the gain rows take the Q tile while dE is formed (no room for a
  // third [C][d_k] tile), and Q, loaded after that, replaces them before the
  // state-gradient update
  Frag<C * DP / NTC> fk, fq, fg;
  Frag<C * C / NTC> fp, ft;
  Frag<C * TW / NTC> fo;
  Scal fs;
  auto fetch_q = [&](int c) {
    const int n = min(C, L - c * C);
    fetch_rows<NTC>(fq, a.q + ((size_t)bh * L + (size_t)c * C) * dk, n, dk);
  };
  auto fetch = [&](int c) {
    const int n = min(C, L - c * C);
    const size_t tok = (size_t)bh * L + (size_t)c * C;
    fetch_rows<NTC>(fk, a.k + tok * dk, n, dk);
    if constexpr (GAIN) fetch_rows<NTC>(fg, a.gain + tok * dk, n, dk);
    else fetch_q(c);
    fetch_cc<NTC>(fp, a.Pm + cc_off(bh, nch, c));
    if (erase) fetch_cc<NTC>(ft, a.Tm + cc_off(bh, nch, c));
    fetch_tile<NTC>(fo, a.d_o + tok * dv, n, dv, j0);
    fs = fetch_scalars(a, tok, n);
  };
  fetch(nch - 1);
  if constexpr (GAIN) fetch_q(nch - 1);
  for (int c = nch - 1; c >= 0; --c) {
    const int n = min(C, L - c * C);
    const size_t tok = (size_t)bh * L + (size_t)c * C;
    __syncthreads();
    put_rows<NTC, LKC>(fk, sK);
    if constexpr (GAIN) put_rows<NTC, LKC>(fg, sQ);
    else put_rows<NTC, LKC>(fq, sQ);
    put_cc<NTC, LCC>(fp, sP);
    if (erase) put_cc<NTC, LCC>(ft, sT);
    put_tile<NTC, LOC>(fo, sO, nullptr);
    put_scalars(a, fs, sLg, sB, sAl);
    if (c > 0) fetch(c - 1);
    {
      float* gg = a.Gs + ((size_t)bh * nch + c) * dk * dv;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 16 * w + 4 * q + i, col = j0 + 16 * h + r;
          if (d < dk && col < dv) gg[(size_t)d * dv + col] = G[h][i];
        }
    }
    __syncthreads();
    const double lgC = sLg[C - 1];
    // dE = Pm^T dO + diag(Lambda b) K G
    floatx4 de;
    {
      floatx4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
      mfma16(x, sP, 1, LCC, sO, LOC, 1, m0, n0, C);
      mfma16(y, gain ? sQ : sK, LKC, 1, sG, LOC, 1, m0, n0, dk64);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = m0 + 4 * q + i;
        de[i] = fmaf(sB[t] * expf((float)(lgC - sLg[t])), y[i], x[i]);
        sD[t * LOC + n0 + r] = de[i];
      }
    }
    __syncthreads();
    if constexpr (GAIN) {  // every wavefront is done with the gain rows: Q takes the tile
      put_rows<NTC, LKC>(fq, sQ);
      if (c > 0) fetch_q(c - 1);
    }
    floatx4 dr = de;
    if (erase) {
      dr = floatx4{0.f, 0.f, 0.f, 0.f};
      mfma16(dr, sT, 1, LCC, sD, LOC, 1, m0, n0, C);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = m0 + 4 * q + i, col = j0 + n0 + r;
      if (t < n && col < dv) {
        a.dR[((size_t)bh * nch * C + (size_t)c * C + t) * dv + col] = dr[i];
        a.dv_out[(tok + t) * dv + col] = a.resid == 1 ? sAl[t] * dr[i] : dr[i];
      }
      const float g = expf((float)sLg[t]);
      sX[t * LOC + n0 + r] = -g * dr[i];
      sO[t * LOC + n0 + r] *= g;
    }
    __syncthreads();
    // G <- g_C G + Q^T diag(g) dO - K^T diag(g) dR
    const float gC = expf((float)lgC);
    floatx4 acc[2] = {G[0] * gC, G[1] * gC};
    mfma_row<2>(acc, sQ, 1, LKC, nullptr, sO, LOC, 1, 16 * w, C);
    if (erase) mfma_row<2>(acc, sK, 1, LKC, nullptr, sX, LOC, 1, 16 * w, C);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      G[h] = acc[h];
#pragma unroll
      for (int i = 0; i < 4; ++i) sG[(16 * w + 4 * q + i) * LOC + 16 * h + r] = acc[h][i];
    }
  }
  if (a.dstate_in) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 16 * w + 4 * q + i, col = j0 + 16 * h + r;
        if (d < dk && col < dv) a.dstate_in[((size_t)bh * dk + d) * dv + col] = G[h][i];
      }
  }
}

// ---------------------------------------------------------------------------
// contractions over the value columns. STATE = false (grid z = part 0, 1):
// part 0: dO S0^T, dO E^T; part 1: dR S0^T, dR E^T. STATE = true: E G^T and
// <G, S0>. Wavefront w takes rows 16 w .. 16 w + 15 of the products; the value
// columns stream through LDS 64 at a time.
constexpr int VW = 64;  // value columns per pass

template <bool STATE>
__global__ __launch_bounds__(NT) void bwd_contract_kernel(BwdArgs a) {
  extern __shared__ __align__(16) float lds[];
  constexpr int LJ = VW + 1;
  float* sL = lds;               // [C][LJ] left operand block
  float* sR = sL + C * LJ;       // [DP][LJ] S0 or G block
  float* sE = sR + DP * LJ;      // [C][LJ] E block
  float* sRed = sE + C * LJ;     // [NT / 64]
  const int bh = blockIdx.x, c = blockIdx.y, part = STATE ? 2 : blockIdx.z, tid = threadIdx.x;
  const int nch = gridDim.y, L = a.L, dk = a.dk, dv = a.dv;
  const int n = min(C, L - c * C);
  const size_t row0 = (size_t)bh * nch * C + (size_t)c * C;  // padded-row arrays
  const float* left = part == 0 ? a.d_o + ((size_t)bh * L + (size_t)c * C) * dv
                                : (part == 1 ? a.dR : a.E) + row0 * dv;
  const float* S0c = a.S0s + ((size_t)bh * nch + c) * dk * dv;
  const float* right = STATE ? a.Gs + ((size_t)bh * nch + c) * dk * dv : S0c;
  const float* Ec = a.E + row0 * dv;
  const int w = tid >> 6, r = tid & 15, q = (tid & 63) >> 4;
  floatx4 m[8] = {}, p[4] = {};
  float gs = 0.f;
  for (int jb = 0; jb < dv; jb += VW) {
    Frag<C * VW / NT> fl, fe;
    Frag<DP * VW / NT> fr, fs0;
    fetch_tile<NT, VW>(fl, left, n, dv, jb);
    if (!STATE) fetch_tile<NT, VW>(fe, Ec, n, dv, jb);
#pragma unroll
    for (int u = 0; u < DP * VW / NT; ++u) {
      const int idx = tid + u * NT, d = idx / VW, j = idx % VW;
      const bool ok = d < dk && jb + j < dv;
      fr.x[u] = ok ? right[(size_t)d * dv + jb + j] : 0.f;
      if (STATE) fs0.x[u] = ok ? S0c[(size_t)d * dv + jb + j] : 0.f;
    }
    __syncthreads();
    put_tile<NT, LJ, VW>(fl, sL, nullptr);
    if (!STATE) put_tile<NT, LJ, VW>(fe, sE, nullptr);
#pragma unroll
    for (int u = 0; u < DP * VW / NT; ++u) {
      const int idx = tid + u * NT, d = idx / VW, j = idx % VW;
      sR[d * LJ + j] = fr.x[u];
      if (STATE) gs = fmaf(fr.x[u], fs0.x[u], gs);
    }
    __syncthreads();
    mfma_row<8>(m, sL, LJ, 1, nullptr, sR, 1, LJ, 16 * w, VW);
    if (!STATE) mfma_row<4>(p, sL, LJ, 1, nullptr, sE, 1, LJ, 16 * w, VW);
  }
  float* M = (part == 0 ? a.M1 : part == 1 ? a.M2 : a.M3) + row0 * dk;
#pragma unroll
  for (int b = 0; b < 8; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 16 * b + r;
      if (d < dk) M[(size_t)(16 * w + 4 * q + i) * dk + d] = m[b][i];
    }
  if (!STATE) {
    float* P = (part == 0 ? a.dPm : a.dA) + cc_off(bh, nch, c);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) P[(16 * w + 4 * q + i) * C + 16 * b + r] = p[b][i];
  } else {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) gs += __shfl_xor(gs, off, 64);
    if ((tid & 63) == 0) sRed[tid >> 6] = gs;
    __syncthreads();
    if (tid == 0) a.gs0[(size_t)bh * nch + c] = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
  }
}

__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 1, 16);
  x += __shfl_xor(x, 2, 16);
  x += __shfl_xor(x, 4, 16);
  x += __shfl_xor(x, 8, 16);
  return x;
}

// ---------------------------------------------------------------------------
// per-token gradients of one chunk; wavefront w takes tokens 16 w .. 16 w + 15
// of the [C][d_k] products
__global__ __launch_bounds__(NT) void bwd_grad_kernel(BwdArgs a) {
  extern __shared__ __align__(16) float lds[];
  constexpr int LQ = DP + 1;
  constexpr int LX = C + 1;
  float* sQ = lds;               // [C][LQ]
  float* sK = sQ + C * LQ;       // [C][LQ]
  float* sXp = sK + C * LQ;      // [C][LX] lower_incl(dO E^T) * D
  float* sXa = sXp + C * LX;     // [C][LX] dA * D
  double* sLg = reinterpret_cast<double*>(sXa + C * LX);  // [C] (8-byte aligned)
  float* sB = reinterpret_cast<float*>(sLg + C);
  float* sAl = sB + C;
  float* sRow = sAl + C;         // [6][C] per-token sums
  float* sCs = sRow + 6 * C;     // [NT / 64][C] partial column sums
  float* sGn = sCs + (NT / 64) * C;  // [C][LQ] gain rows (gain mode)
  const int bh = blockIdx.x, c = blockIdx.y, tid = threadIdx.x, nch = gridDim.y;
  const int L = a.L, dk = a.dk, dv = a.dv;
  const int n = min(C, L - c * C);
  const size_t tok = (size_t)bh * L + (size_t)c * C;
  const size_t row0 = (size_t)bh * nch * C + (size_t)c * C;
  const bool erase = a.resid != 2, plain = a.resid == 1, gain = a.gain != nullptr;
  {
    Frag<C * DP / NT> fq, fk, fg;
    fetch_rows<NT>(fq, a.q + tok * dk, n, dk);
    fetch_rows<NT>(fk, a.k + tok * dk, n, dk);
    if (gain) fetch_rows<NT>(fg, a.gain + tok * dk, n, dk);
    const Scal sc = fetch_scalars(a, tok, n);
    put_rows<NT, LQ>(fq, sQ);
    put_rows<NT, LQ>(fk, sK);
    if (gain) put_rows<NT, LQ>(fg, sGn);
    put_scalars(a, sc, sLg, sB, sAl);
  }
  const size_t o = cc_off(bh, nch, c);
  Frag<C * C / NT> fP, fA, fdP, fdA;
  fetch_cc<NT>(fP, a.Pm + o);
  fetch_cc<NT>(fdP, a.dPm + o);
  if (erase) {
    fetch_cc<NT>(fA, a.Am + o);
    fetch_cc<NT>(fdA, a.dA + o);
  }
  // this lane's elements of dO S0^T, dR S0^T and E G^T (tokens 16 w + 4 q + i,
  // columns 16 b + r), in flight during the elementwise pass
  const int w = tid >> 6, r = tid & 15, q = (tid & 63) >> 4;
  float m1v[4][8], m2v[4][8], m3v[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int d = 16 * b + r;
      const size_t e = (row0 + 16 * w + 4 * q + i) * dk + d;
      m1v[i][b] = d < dk ? a.M1[e] : 0.f;
      m2v[i][b] = (erase && d < dk) ? a.M2[e] : 0.f;
      m3v[i][b] = d < dk ? a.M3[e] : 0.f;
    }
  __syncthreads();
  // Xp, Xa, and the row and column sums of W = dPm * Pm + dA * A (lane = s)
  {
    const int s = tid & 63;
    float cs = 0.f;
#pragma unroll
    for (int u = 0; u < C * C / NT; ++u) {
      const int t = (tid >> 6) + u * (NT / 64);
      const bool lo = s <= t, st = erase && s < t;
      const float D = lo ? expf((float)(sLg[t] - sLg[s])) : 0.f;
      const float dp = lo ? fdP.x[u] : 0.f;
      const float da = st ? -fdA.x[u] : 0.f;
      sXp[t * LX + s] = dp * D;
      sXa[t * LX + s] = da * D;
      const float wv = dp * (lo ? fP.x[u] : 0.f) + (st ? da * fA.x[u] : 0.f);
      cs += wv;
      float rs = wv;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) rs += __shfl_xor(rs, off, 64);
      if (s == 0) sRow[5 * C + t] = rs;
    }
    sCs[(tid >> 6) * C + s] = cs;
  }
  __syncthreads();
  const double lgC = sLg[C - 1];
  float pq[4] = {}, kr[4] = {}, wv[4] = {}, dbv[4] = {}, vv[4] = {};
  // the write vectors: rows b_t k_t (sB scaling sK), or the gain rows
  const float* sW = gain ? sGn : sK;
  const float* sWs = gain ? nullptr : sB;
  {  // dQ = diag(g) dO S0^T + Xp diag(b) K
    floatx4 acc[8] = {};
    mfma_row<8>(acc, sXp, LX, 1, sWs, sW, LQ, 1, 16 * w, C);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * w + 4 * q + i;
      const float g = expf((float)sLg[t]);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int d = 16 * b + r;
        const float x = m1v[i][b];
        pq[i] = fmaf(x, sQ[t * LQ + d], pq[i]);
        if (t < n && d < dk) a.dq[(tok + t) * dk + d] = fmaf(g, x, acc[b][i]);
      }
      pq[i] *= g;
    }
  }
  {  // dB = Xp^T Q + Xa^T K + diag(Lambda) E G^T;  dK = Xa diag(b) K - diag(g) dR S0^T + diag(b) dB
    floatx4 db[8] = {}, dkk[8] = {};
    mfma_row<8>(db, sXp, 1, LX, nullptr, sQ, LQ, 1, 16 * w, C);
    if (erase) {
      mfma_row<8>(db, sXa, 1, LX, nullptr, sK, LQ, 1, 16 * w, C);
      mfma_row<8>(dkk, sXa, LX, 1, sWs, sW, LQ, 1, 16 * w, C);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * w + 4 * q + i;
      const float lam = expf((float)(lgC - sLg[t])), g = expf((float)sLg[t]), b = sB[t];
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
        const int d = 16 * bb + r;
        const float kv = sK[t * LQ + d];
        const float x3 = m3v[i][bb];
        const float x2 = m2v[i][bb];
        wv[i] = fmaf(sW[t * LQ + d], x3, wv[i]);
        const float dbb = fmaf(lam, x3, db[bb][i]);
        dbv[i] = fmaf(dbb, kv, dbv[i]);
        const float dkr = -g * x2;
        kr[i] = fmaf(dkr, kv, kr[i]);
        if (t < n && d < dk) {
          if (gain) {
            a.dgain[(tok + t) * dk + d] = dbb;
            a.dk_out[(tok + t) * dk + d] = dkk[bb][i] + dkr;
          } else {
            a.dk_out[(tok + t) * dk + d] = fmaf(b, dbb, dkk[bb][i] + dkr);
          }
        }
      }
      wv[i] *= lam * b;
      if (plain && t < n) {
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) {
          const int col = 16 * bb + r;
          if (col < dv) vv[i] = fmaf(a.dR[(row0 + t) * dv + col], a.v[(tok + t) * dv + col], vv[i]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pq[i] = sum16(pq[i]);
    kr[i] = sum16(kr[i]);
    wv[i] = sum16(wv[i]);
    dbv[i] = sum16(dbv[i]);
    vv[i] = sum16(vv[i]);
    if (r == 0) {
      const int t = 16 * w + 4 * q + i;
      sRow[t] = pq[i];
      sRow[C + t] = kr[i];
      sRow[2 * C + t] = wv[i];
      sRow[3 * C + t] = dbv[i];
      sRow[4 * C + t] = vv[i];
    }
  }
  __syncthreads();
  if (tid < C) {
    const int t = tid;
    float cs = 0.f;
#pragma unroll
    for (int p = 0; p < NT / 64; ++p) cs += sCs[p * C + t];
    const float w_t = sRow[2 * C + t];
    float dl = (sRow[5 * C + t] - cs) + sRow[t] + sRow[C + t] - w_t;
    float wsum = w_t;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) wsum += __shfl_xor(wsum, off, 64);
    if (t == n - 1) dl += expf((float)lgC) * a.gs0[(size_t)bh * nch + c] + wsum;
    float suf = dl;  // sum over t' >= t (tokens past the end hold 0)
#pragma unroll
    for (int off = 1; off < C; off <<= 1) {
      const float y = __shfl_down(suf, off, 64);
      if (t + off < C) suf += y;
    }
    if (t < n) {
      const float al = sAl[t], dbp = sRow[3 * C + t];
      float dal = suf / al, dbe = dbp;
      if (plain) {
        dal += -dbp * sB[t] / al + sRow[4 * C + t];
        dbe = dbp / al;
      }
      if (a.dalpha) a.dalpha[tok + t] = dal;
      if (a.dbeta) a.dbeta[tok + t] = dbe;
    }
  }
}

struct BwdPlan {
  size_t off[14];
  size_t total;
};

BwdPlan plan_bwd(int BH, int L, int dk, int dv) {
  const size_t nch = ((size_t)L + C - 1) / C, Lp = nch * C;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t sz[14] = {
      (size_t)BH * nch * dk * dv, (size_t)BH * nch * dk * dv,           // S0s, Gs
      (size_t)BH * Lp * dv,       (size_t)BH * Lp * dv,                 // E, dR
      (size_t)BH * nch * C * C,   (size_t)BH * nch * C * C,             // Am, Tm
      (size_t)BH * nch * C * C,                                         // Pm
      (size_t)BH * Lp * dk,       (size_t)BH * Lp * dk, (size_t)BH * Lp * dk,  // M1..M3
      (size_t)BH * nch * C * C,   (size_t)BH * nch * C * C,             // dPm, dA
      (size_t)BH * nch,           0};                                   // gs0
  BwdPlan p{};
  size_t o = 0;
  for (int i = 0; i < 14; ++i) {
    p.off[i] = o;
    o += up(sz[i] * 4);
  }
  p.total = o;
  return p;
}

template <typename K>
hipError_t launch_lds(const char* name, K kern, dim3 grid, int threads, size_t lds, const BwdArgs& a,
                      hipStream_t s) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  KDN_LAUNCH_NAMED(name, kern, grid, dim3(threads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

size_t scan_bwd_workspace_bytes(int BH, int L, int dk, int dv) {
  return plan_bwd(BH, L, dk, dv).total;
}

hipError_t launch_scan_bwd(BwdArgs a, void* ws, hipStream_t s) {
  if (a.dk > DP || a.dv > 128) return hipErrorInvalidValue;
  const BwdPlan p = plan_bwd(a.BH, a.L, a.dk, a.dv);
  char* b = static_cast<char*>(ws);
  float** parts[13] = {&a.S0s, &a.Gs, &a.E, &a.dR, &a.Am, &a.Tm, &a.Pm,
                       &a.M1,  &a.M2, &a.M3, &a.dPm, &a.dA, &a.gs0};
  for (int i = 0; i < 13; ++i) *parts[i] = reinterpret_cast<float*>(b + p.off[i]);
  const int nch = (a.L + C - 1) / C, ntw = (a.dv + TW - 1) / TW;
  const size_t f = sizeof(float);
  hipError_t e;
  const int ng = a.gain ? 1 : 0;  // gain mode: one more [C][d_k] tile per kernel
  e = launch_lds("bwd_prep_kernel", bwd_prep_kernel, dim3(a.BH, nch), NT,
                 ((2 + ng) * C * (DP + 1) + 4 * C) * f, a, s);
  if (e != hipSuccess) return e;
  e = launch_lds("bwd_fwd_kernel", bwd_fwd_kernel, dim3(a.BH, ntw), NTC,
                 ((1 + ng) * C * LKC + C * LCC + DP * LOC + 2 * C * LOC + 4 * C) * f, a, s);
  if (e != hipSuccess) return e;
  const size_t lds_rev = (2 * C * LKC + 2 * C * LCC + DP * LOC + 3 * C * LOC + 4 * C) * f;
  e = a.gain ? launch_lds("bwd_rev_kernel<true>", bwd_rev_kernel<true>, dim3(a.BH, ntw), NTC,
                          lds_rev, a, s)
             : launch_lds("bwd_rev_kernel<false>", bwd_rev_kernel<false>, dim3(a.BH, ntw), NTC,
                          lds_rev, a, s);
  if (e != hipSuccess) return e;
  const size_t lds_c = (2 * C * (VW + 1) + DP * (VW + 1) + NT / 64) * f;
  e = launch_lds("bwd_contract_kernel<false>", bwd_contract_kernel<false>, dim3(a.BH, nch, 2), NT,
                 lds_c, a, s);
  if (e != hipSuccess) return e;
  e = launch_lds("bwd_contract_kernel<true>", bwd_contract_kernel<true>, dim3(a.BH, nch), NT, lds_c,
                 a, s);
  if (e != hipSuccess) return e;
  return launch_lds("bwd_grad_kernel", bwd_grad_kernel, dim3(a.BH, nch), NT,
                    ((2 + ng) * C * (DP + 1) + 2 * C * (C + 1) + 4 * C + 6 * C + (NT / 64) * C) * f,
                    a, s);
}

}  // namespace kdn
