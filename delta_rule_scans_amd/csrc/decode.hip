// decode.hip -- one decoding token per head: state read-modify-write.
//
// "A Hippocampus for Linear Attention", sec. 3.3 eqs. (5)-(6) and sec. 3.5:
//   e = v - alpha S^T k,  S <- alpha S + b e^T,  o = S^T q (after the write),
//   m = ||b e^T||_F  (= beta ||e|| for the delta write with unit keys).
// The plain residual is e = v - S^T k with the same update.
// b = beta k (delta), the diagonal Kalman gain or the isotropic one ("Kalman
// Delta Networks", abstract; the isotropic gain is p- k / (p- ||k||^2 + r) with
// one variance per head, 1/p = 1/p- + ||k||^2 / (d_k r)). The read-out is
// computed in the same pass over S as o = alpha S_old^T q + (b . q) e, so S is
// read once and written once.
//
// One workgroup (256 lanes) per head. Lane (rg, cg): column group cg (4
// columns), rows rg, rg + 8, ... The state row is read with 16-byte loads, so a
// wavefront touches two contiguous 512-byte rows per load.
#include "kdn_internal.h"

namespace kdn {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ float wave_sum(float x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Sum over the whole workgroup; every lane gets the result.
__device__ __forceinline__ float block_sum(float x, float* scratch) {
  x = wave_sum(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = x;
  __syncthreads();
  return scratch[0] + scratch[1] + scratch[2] + scratch[3];
}

template <bool VEC>
__global__ __launch_bounds__(NT) void decode_kernel(const float* __restrict__ q,
                                                    const float* __restrict__ k,
                                                    const float* __restrict__ v,
                                                    const float* __restrict__ alpha,
                                                    const float* __restrict__ beta,
                                                    const float* __restrict__ r,
                                                    float* __restrict__ cov, float qvar,
                                                    float* __restrict__ state,
                                                    float* __restrict__ o, float* __restrict__ m,
                                                    int dk, int dv, int gmode, int resid,
                                                    int score_kind) {
  __shared__ float sk[128], sq[128], sv[128], sb[128], se[128];
  __shared__ float red1[8][128], red2[8][128];
  __shared__ float scratch[4];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int cg = tid & 31, rg = tid >> 5;

  const bool diag = gmode == 1, iso = gmode == 2;
  const bool plain = resid == 1, noerase = resid == 2;
  const float a = alpha ? alpha[bh] : 1.f;
  float bscale = gmode == 0 ? beta[bh] : 1.f;
  const float pscale = plain ? 1.f : a;  // decay of the prediction in the residual
  if (tid < dk) {
    sk[tid] = k[(size_t)bh * dk + tid];
    sq[tid] = q[(size_t)bh * dk + tid];
  }
  if (tid < dv) sv[tid] = v[(size_t)bh * dv + tid];
  __syncthreads();

  // write vector
  if (diag) {
    const float rt = r ? r[bh] : 1.f;
    float pm = 0.f, kv = 0.f;
    if (tid < dk) {
      kv = sk[tid];
      pm = fmaf(a * a, cov[(size_t)bh * dk + tid], (1.f - a) * (1.f + a) * qvar);
    }
    const float s = rt + block_sum(pm * kv * kv, scratch);
    if (tid < dk) {
      sb[tid] = pm * kv / s;
      cov[(size_t)bh * dk + tid] = pm * rt / fmaf(pm * kv, kv, rt);
    }
  } else if (iso) {
    const float rt = r ? r[bh] : 1.f;
    const float pm = fmaf(a * a, cov[bh], (1.f - a) * (1.f + a) * qvar);
    const float kv = tid < dk ? sk[tid] : 0.f;
    const float kk = block_sum(kv * kv, scratch);
    bscale = pm / fmaf(pm, kk, rt);
    if (tid < dk) sb[tid] = bscale * kv;
    if (tid == 0) cov[bh] = pm * (dk * rt) / fmaf(pm, kk, dk * rt);
  } else if (tid < dk) {
    sb[tid] = bscale * sk[tid];
  }
  __syncthreads();

  // S^T k and S^T q over this lane's rows; the state is read and written once
  // per step, so both directions stream (measured: 10% faster step)
  float* S = state + (size_t)bh * dk * dv;
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(S, (size_t)dk * dv * sizeof(float));
  float reg[16][4];
  float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int i = rg + 8 * s;
#pragma unroll
    for (int c = 0; c < 4; ++c) reg[s][c] = 0.f;
    if (i < dk) {
      if (VEC) {
        if (4 * cg < dv) {
          const float4 x = stream_load16(rS, (i * dv + 4 * cg) * (int)sizeof(float));
          reg[s][0] = x.x;
          reg[s][1] = x.y;
          reg[s][2] = x.z;
          reg[s][3] = x.w;
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = cg + 32 * c;
          if (j < dv) reg[s][c] = S[(size_t)i * dv + j];
        }
      }
      const float ki = sk[i], qi = sq[i];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pk[c] = fmaf(reg[s][c], ki, pk[c]);
        pq[c] = fmaf(reg[s][c], qi, pq[c]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j = VEC ? 4 * cg + c : cg + 32 * c;
    if (j < 128) {
      red1[rg][j] = pk[c];
      red2[rg][j] = pq[c];
    }
  }
  __syncthreads();
  float e = 0.f, oq = 0.f;
  if (tid < dv) {
    float pred = 0.f, qp = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      pred += red1[g][tid];
      qp += red2[g][tid];
    }
    e = noerase ? sv[tid] : sv[tid] - pscale * pred;
    oq = a * qp;
    se[tid] = e;
  }
  const float bq = block_sum(tid < dk ? sb[tid] * sq[tid] : 0.f, scratch);
  const float ee = block_sum(e * e, scratch);
  const float bb = gmode ? block_sum(tid < dk ? sb[tid] * sb[tid] : 0.f, scratch) : 0.f;
  const float vv = score_kind == 2 ? block_sum(tid < dv ? sv[tid] * sv[tid] : 0.f, scratch) : 0.f;
  if (tid < dv) o[(size_t)bh * dv + tid] = fmaf(bq, e, oq);
  if (m && tid == 0) {
    const float ws = gmode ? sqrtf(bb) : bscale;
    m[bh] = score_kind == 1 ? sqrtf(ee) : (score_kind == 2 ? ws * sqrtf(vv) : ws * sqrtf(ee));
  }

  // S <- alpha S + b e^T
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    const int i = rg + 8 * s;
    if (i < dk) {
      const float bi = sb[i];
      if (VEC) {
        if (4 * cg < dv) {
          float4 x;
          x.x = fmaf(a, reg[s][0], bi * se[4 * cg + 0]);
          x.y = fmaf(a, reg[s][1], bi * se[4 * cg + 1]);
          x.z = fmaf(a, reg[s][2], bi * se[4 * cg + 2]);
          x.w = fmaf(a, reg[s][3], bi * se[4 * cg + 3]);
          stream_store16(rS, (i * dv + 4 * cg) * (int)sizeof(float), x);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int j = cg + 32 * c;
          if (j < dv) S[(size_t)i * dv + j] = fmaf(a, reg[s][c], bi * se[j]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_decode(const float* q, const float* k, const float* v, const float* alpha,
                         const float* beta, const float* r, float* cov, float q_noise_var,
                         float* state, float* o, float* m, int BH, int dk, int dv, int gmode,
                         int resid, int score_kind, hipStream_t s) {
  const bool vec = (dv % 4 == 0) && ((reinterpret_cast<uintptr_t>(state) & 15) == 0);
  if (vec)
    KDN_LAUNCH(decode_kernel<true>, dim3(BH), dim3(NT), 0, s, q, k, v, alpha, beta, r, cov,
                       q_noise_var, state, o, m, dk, dv, gmode, resid, score_kind);
  else
    KDN_LAUNCH(decode_kernel<false>, dim3(BH), dim3(NT), 0, s, q, k, v, alpha, beta, r,
                       cov, q_noise_var, state, o, m, dk, dv, gmode, resid, score_kind);
  return hipGetLastError();
}

}  // namespace kdn
