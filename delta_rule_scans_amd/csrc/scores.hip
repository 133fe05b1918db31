// scores.hip -- per-token write scores of a scan.
//
// "A Hippocampus for Linear Attention", sec. 3.3 eq. (6): the score of token t
// is the Frobenius norm of its rank-one write, m_t = ||b_t e_t^T||_F =
// ||b_t|| ||e_t||; for the delta write the page uses beta_t ||e_t|| (equal for
// unit keys). The residuals e_t are the rows of U in the chunk form, so the
// scan kernels leave them (or their per-tile squared norms) behind and this
// kernel combines the d_v tiles in a fixed order and applies the scale.
//
// The ablation scores of the same section replace the product by the residual
// alone (||e_t||) or by the write strength alone (s_t ||v_t||).
//
// One thread per token, one workgroup per (head, 64 tokens).
#include "kdn_internal.h"

namespace kdn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

// Squared residual norm of token t (0..63) of chunk cc from the matrix-core
// residual buffer: per (head, tile, chunk) four 64-lane blocks of 8 fp16 in the
// state kernel's register order. Token t = 32 b + 8 g + 4 h + r sits in block
// 2 b + g / 2, element 4 (g % 2) + r, of the 32 lanes 32 h .. 32 h + 31 (one
// value column each).
// The residuals of a (head, tile, chunk) are stored times 2^e_S (uexp).
__device__ float ubuf_sq(const half8* ub, const int* uexp, int bh, int ntiles, int nchunks, int cc,
                         int t) {
  const int b = t >> 5, g = (t >> 3) & 3, h = (t >> 2) & 1, r = t & 3;
  const int blk = 2 * b + (g >> 1), e = 4 * (g & 1) + r;
  float ss = 0.f;
  for (int tile = 0; tile < ntiles; ++tile) {
    const size_t rec = (size_t)(bh * ntiles + tile) * nchunks + cc;
    const half8* p = ub + rec * 256 + blk * 64 + 32 * h;
    float st = 0.f;
    for (int c = 0; c < 32; ++c) {
      const float x = (float)p[c][e];
      st = fmaf(x, x, st);
    }
    const float f = __int_as_float((127 - uexp[rec]) << 23);  // 2^-e_S
    ss = fmaf(st * f, f, ss);
  }
  return ss;
}

__global__ __launch_bounds__(64) void scores_kernel(ScoreArgs a) {
  const int bh = blockIdx.x, cc = blockIdx.y, t = threadIdx.x;
  const int tok = cc * 64 + t;
  if (tok >= a.L) return;
  const size_t g = (size_t)bh * a.L + tok;
  float ss = 0.f;
  if (a.ubuf) {
    const int nchunks = (a.L + 63) / 64;
    ss = ubuf_sq(static_cast<const half8*>(a.ubuf), a.uexp, bh, a.dv / 32, nchunks, cc, t);
  } else {
    for (int tile = 0; tile < a.ntiles; ++tile) ss += a.esq[((size_t)bh * a.ntiles + tile) * a.L + tok];
  }
  if (a.kind == 1) {  // ||e||
    a.m[g] = sqrtf(ss);
    return;
  }
  float scale;
  if (a.gains) {
    float gg = 0.f;
    for (int i = 0; i < a.dk; ++i) {
      const float x = a.gains_f16 ? (float)static_cast<const _Float16*>(a.gains)[g * a.dk + i]
                                  : static_cast<const float*>(a.gains)[g * a.dk + i];
      gg = fmaf(x, x, gg);
    }
    scale = sqrtf(gg);
  } else if (a.iso_beta) {
    scale = a.iso_beta[g] * sqrtf(a.iso_kk[g]);
  } else {
    scale = a.beta[g];
  }
  if (a.kind == 2) {  // write strength times ||v|| of the input value
    float vv = 0.f;
    for (int c = 0; c < a.dv; ++c) {
      const float x = a.v_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(a.v)[g * a.dv + c])
                               : static_cast<const float*>(a.v)[g * a.dv + c];
      vv = fmaf(x, x, vv);
    }
    a.m[g] = scale * sqrtf(vv);
    return;
  }
  a.m[g] = scale * sqrtf(ss);
}

}  // namespace

hipError_t launch_scores(const ScoreArgs& a, hipStream_t s) {
  const int nblk = (a.L + 63) / 64;
  KDN_LAUNCH(scores_kernel, dim3(a.BH, nblk), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace kdn
