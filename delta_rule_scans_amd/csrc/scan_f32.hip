// scan_f32.hip -- chunkwise-parallel scan on the float32 vector units.
//
// The general path: any d_k, d_v <= 128, chunk 16/32/64, float32 or bf16
// inputs and outputs, every write mode. All arithmetic is float32.
//
// Recurrence ("A Hippocampus for Linear Attention", sec. 3.3 eq. (5), sec. 3.5):
//   e_t = v_t - alpha_t S_{t-1}^T k_t,  S_t = alpha_t S_{t-1} + b_t e_t^T,  o_t = S_t^T q_t
// with write vector b_t = beta_t k_t (delta) or the Kalman gain (precomputed).
// Chunk form (derived by unrolling the recurrence over a chunk of n tokens with
// incoming state S0 and chunk-local decay g_i = prod_{l<=i} alpha_l):
//   A = strict_lower((K B^T) * G), G_il = g_i / g_l;   (I + A) U = V - diag(g) K S0
//   O = diag(g) Q S0 + lower_incl((Q B^T) * G) U;      S = g_n S0 + (diag(g_n / g) B)^T U
// U are exactly the per-token residuals e_t. Without the erase term (e_t = v_t)
// A = 0 and the K S0 term drops: U = V. The plain residual e_t = v_t -
// S_{t-1}^T k_t unrolls to the same form with the exclusive decay g_{t-1} =
// g_t / alpha_t in the rows of A and in the K S0 term (every ratio <= 1).
//
// One workgroup per (head, d_v tile): grid (heads, d_v tiles). The state tile lives in LDS; the loop
// over chunks is sequential inside the workgroup.
#include "kdn_internal.h"

namespace kdn {
namespace {

constexpr int NT = 256;

struct F32Plan {
  int dvt;
  size_t lds;
};

__host__ __device__ inline size_t f32_lds_floats(int dk, int C, int dvt) {
  return (size_t)3 * C * (dk + 1) + (size_t)2 * C * dvt + (size_t)2 * C * (C + 1) +
         (size_t)dk * dvt + 5 * (size_t)C;
}

constexpr size_t kMaxLds = 160 * 1024;

F32Plan plan_f32(int dk, int C) {
  for (int dvt : {32, 16}) {
    size_t b = f32_lds_floats(dk, C, dvt) * sizeof(float);
    if (b <= kMaxLds) return {dvt, b};
  }
  return {0, 0};
}

template <typename Tin, typename Tout, typename Tg>
__global__ __launch_bounds__(NT) void scan_f32_kernel(ScanArgs a, int dvt) {
  extern __shared__ __align__(16) float lds[];
  const int C = a.chunk, dk = a.dk, dv = a.dv, L = a.L;
  const int KP = dk + 1, CP = C + 1;
  const int bh = blockIdx.x;
  const int j0 = blockIdx.y * dvt;
  const int nj = min(dvt, dv - j0);
  const int tid = threadIdx.x;

  float* sK = lds;              // [C][KP] keys
  float* sQ = sK + C * KP;      // [C][KP] queries
  float* sB = sQ + C * KP;      // [C][KP] write directions (k or gain)
  float* sX = sB + C * KP;      // [C][dvt] values, then residuals U
  float* sO = sX + C * dvt;     // [C][dvt] inter-chunk part of the output
  float* sA = sO + C * dvt;     // [C][CP]
  float* sP = sA + C * CP;      // [C][CP]
  float* sS = sP + C * CP;      // [dk][dvt] state tile
  // [C] chunk-local prefix of log alpha in float64 (8-byte aligned: every
  // region before it is an even number of floats). Decay ratios come from
  // differences of these prefixes, which reach about -1000 in a chunk of
  // tokens with alpha near 1e-8: in float32 they would keep only ~6e-5 of
  // each ratio.
  double* sLg = reinterpret_cast<double*>(sS + dk * dvt);
  float* sBs = reinterpret_cast<float*>(sLg + C);  // [C] write scale (beta, or 1 for a gain)
  float* sLa = sBs + C;         // [C] log alpha_t when the residual decay is exclusive, else 0
  float* sW = sLa + C;          // [C] state-update weights (g_n / g_l) * scale_l

  const Tin* qp = static_cast<const Tin*>(a.q);
  const Tin* kp = static_cast<const Tin*>(a.k);
  const Tin* vp = static_cast<const Tin*>(a.v);
  const Tg* gp = static_cast<const Tg*>(a.gain);
  Tout* op = static_cast<Tout*>(a.o);
  const size_t tok0 = (size_t)bh * L;

  for (int idx = tid; idx < dk * dvt; idx += NT) {
    const int i = idx / dvt, j = idx - i * dvt;
    float s = 0.f;
    if (a.state_in && j < nj) s = a.state_in[((size_t)bh * dk + i) * dv + j0 + j];
    sS[idx] = s;
  }

  for (int c0 = 0; c0 < L; c0 += C) {
    const int n = min(C, L - c0);
    __syncthreads();
    // every global read of the chunk in one round: keys, queries, write
    // directions, values, and (wavefront 0, lane t = token t) the decays and
    // write scales, whose chunk-local prefix of log alpha is a wavefront scan
    for (int idx = tid; idx < C * dk; idx += NT) {
      const int t = idx / dk, i = idx - t * dk;
      float kv = 0.f, qv = 0.f, bv = 0.f;
      if (t < n) {
        const size_t g = (tok0 + c0 + t) * dk + i;
        kv = Elem<Tin>::load(kp, g);
        qv = Elem<Tin>::load(qp, g);
        bv = gp ? Elem<Tg>::load(gp, g) : kv;
      }
      sK[t * KP + i] = kv;
      sQ[t * KP + i] = qv;
      sB[t * KP + i] = bv;
    }
    for (int idx = tid; idx < C * dvt; idx += NT) {
      const int t = idx / dvt, j = idx - t * dvt;
      float x = 0.f;
      if (t < n && j < nj) x = Elem<Tin>::load(vp, (tok0 + c0 + t) * dv + j0 + j);
      sX[idx] = x;
    }
    if (tid < 64) {  // C <= 64
      float la = 0.f, bs = 0.f;
      if (tid < n) {
        const size_t g = tok0 + c0 + tid;
        const float al = a.alpha ? a.alpha[g] : 1.f;
        la = logf(al);
        bs = gp ? 1.f : a.beta[g];
      }
      double pre = la;  // inclusive prefix over the chunk's tokens (0 past n)
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(pre, off, 64);
        if (tid >= off) pre += y;
      }
      if (tid < C) {
        sLg[tid] = pre;
        sBs[tid] = bs;
        sLa[tid] = a.plain ? la : 0.f;
      }
    }
    __syncthreads();
    if (tid < n) sW[tid] = expf((float)(sLg[n - 1] - sLg[tid])) * sBs[tid];
    // Gram blocks: A strictly lower, P lower including the diagonal.
    for (int idx = tid; idx < n * n; idx += NT) {
      const int i = idx / n, l = idx - i * n;
      float av = 0.f, pv = 0.f;
      if (l <= i) {
        float dkb = 0.f, dqb = 0.f;
#pragma unroll 4
        for (int r = 0; r < dk; ++r) {
          const float b = sB[l * KP + r];
          dkb = fmaf(sK[i * KP + r], b, dkb);
          dqb = fmaf(sQ[i * KP + r], b, dqb);
        }
        const float f = expf((float)(sLg[i] - sLg[l])) * sBs[l];
        av = (l < i) ? dkb * expf((float)((sLg[i] - sLa[i]) - sLg[l])) * sBs[l] : 0.f;
        pv = dqb * f;
      }
      sA[i * CP + l] = av;
      sP[i * CP + l] = pv;
    }
    // X = V - diag(g) K S0 and the inter-chunk output diag(g) Q S0.
    for (int idx = tid; idx < n * dvt; idx += NT) {
      const int i = idx / dvt, j = idx - i * dvt;
      float ks = 0.f, qs = 0.f;
#pragma unroll 4
      for (int r = 0; r < dk; ++r) {
        const float s = sS[r * dvt + j];
        ks = fmaf(sK[i * KP + r], s, ks);
        qs = fmaf(sQ[i * KP + r], s, qs);
      }
      if (!a.noerase) sX[idx] -= expf((float)(sLg[i] - sLa[i])) * ks;
      sO[idx] = expf((float)sLg[i]) * qs;
    }
    __syncthreads();
    // Forward substitution (I + A) U = X: one lane per column, rows in order
    // (no barrier between rows; row i of A is read by every lane at once)
    if (!a.noerase && tid < dvt) {
      const int j = tid;
      for (int i = 1; i < n; ++i) {
        const float* ar = sA + i * CP;
        float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
        int l = 0;
        for (; l + 4 <= i; l += 4) {
          s0 = fmaf(ar[l], sX[l * dvt + j], s0);
          s1 = fmaf(ar[l + 1], sX[(l + 1) * dvt + j], s1);
          s2 = fmaf(ar[l + 2], sX[(l + 2) * dvt + j], s2);
          s3 = fmaf(ar[l + 3], sX[(l + 3) * dvt + j], s3);
        }
        for (; l < i; ++l) s0 = fmaf(ar[l], sX[l * dvt + j], s0);
        sX[i * dvt + j] -= (s0 + s1) + (s2 + s3);
      }
    }
    __syncthreads();
    // per-tile squared residual norms for the write scores
    if (a.esq && tid < n) {
      float ss = 0.f;
      for (int j = 0; j < nj; ++j) ss = fmaf(sX[tid * dvt + j], sX[tid * dvt + j], ss);
      a.esq[((size_t)bh * gridDim.y + blockIdx.y) * L + c0 + tid] = ss;
    }
    // O = diag(g) Q S0 + P U
    for (int idx = tid; idx < n * dvt; idx += NT) {
      const int i = idx / dvt, j = idx - i * dvt;
      float acc = sO[idx];
#pragma unroll 4
      for (int l = 0; l <= i; ++l) acc = fmaf(sP[i * CP + l], sX[l * dvt + j], acc);
      if (j < nj) Elem<Tout>::store(op, (tok0 + c0 + i) * dv + j0 + j, acc);
    }
    // S <- g_n S0 + sum_l w_l b_l U_l^T
    const float gn = expf((float)sLg[n - 1]);
    for (int idx = tid; idx < dk * dvt; idx += NT) {
      const int r = idx / dvt, j = idx - r * dvt;
      float acc = 0.f;
#pragma unroll 4
      for (int l = 0; l < n; ++l) acc = fmaf(sW[l] * sB[l * KP + r], sX[l * dvt + j], acc);
      sS[idx] = fmaf(gn, sS[idx], acc);
    }
  }
  __syncthreads();
  if (a.state_out) {
    for (int idx = tid; idx < dk * dvt; idx += NT) {
      const int i = idx / dvt, j = idx - i * dvt;
      if (j < nj) a.state_out[((size_t)bh * dk + i) * dv + j0 + j] = sS[idx];
    }
  }
}

template <typename Tin, typename Tout, typename Tg>
hipError_t launch_typed(const ScanArgs& a, hipStream_t s) {
  const F32Plan p = plan_f32(a.dk, a.chunk);
  if (p.dvt == 0) return hipErrorInvalidValue;
  auto kern = scan_f32_kernel<Tin, Tout, Tg>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds);
  if (e != hipSuccess) return e;
  dim3 grid(a.BH, (a.dv + p.dvt - 1) / p.dvt);
  KDN_LAUNCH_NAMED("scan_f32_kernel", kern, grid, dim3(NT), p.lds, s, a, p.dvt);
  return hipGetLastError();
}

template <typename Tin, typename Tout>
hipError_t launch_gain_typed(const ScanArgs& a, bool gain_f16, hipStream_t s) {
  return gain_f16 ? launch_typed<Tin, Tout, _Float16>(a, s) : launch_typed<Tin, Tout, float>(a, s);
}

__global__ void bf16_to_f32_kernel(const uint16_t* src, float* dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = bf16_to_f32(src[i]);
}

__global__ void copy_f32_kernel(const float* src, float* dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src ? src[i] : 0.f;
}

}  // namespace

size_t scan_f32_lds_bytes(int dk, int chunk) { return plan_f32(dk, chunk).lds; }
int scan_f32_tile_cols(int dk, int chunk) { return plan_f32(dk, chunk).dvt; }

hipError_t launch_scan_f32(const ScanArgs& a, bool in_bf16, bool out_bf16, bool gain_f16,
                           hipStream_t s) {
  if (in_bf16)
    return out_bf16 ? launch_gain_typed<uint16_t, uint16_t>(a, gain_f16, s)
                    : launch_gain_typed<uint16_t, float>(a, gain_f16, s);
  return out_bf16 ? launch_gain_typed<float, uint16_t>(a, gain_f16, s)
                  : launch_gain_typed<float, float>(a, gain_f16, s);
}

hipError_t launch_bf16_to_f32(const uint16_t* src, float* dst, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  KDN_LAUNCH(bf16_to_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t s) {
  if (n == 0 || dst == nullptr) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  KDN_LAUNCH(copy_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

}  // namespace kdn
